"""float64 CPU oracle of LCSA. Test infrastructure only: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the library."""
