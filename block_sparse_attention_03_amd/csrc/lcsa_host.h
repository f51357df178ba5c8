// Host-side helpers shared by the C-ABI entry points: argument validation,
// the k rule, the local-window bounds and the ring bookkeeping. This header
// and lcsa_host.cpp use no HIP API, so they also build with a plain C++
// compiler.
#pragma once

#include <cstdint>

#include "../../include/lcsa.h"

namespace lcsa {

// Record `st` with a printf-style message as this thread's last error and
// return it.
lcsa_status fail(lcsa_status st, const char* fmt, ...);
// Clear the last error and return LCSA_OK.
lcsa_status ok();

// Inclusive block range [lo, hi] along one spatial axis of n blocks that
// block i may see under window size r and the border rule ([FN] Key
// design 3; [HW] 2.2 step 2).
void window_bounds(int32_t i, int32_t n, int32_t r, int32_t border, int32_t* lo,
                   int32_t* hi);

// k rule of lcsa_select_params (no validation of p).
int32_t topk_rule(const lcsa_select_params& p, int64_t n_allowed, int64_t n_keys);

lcsa_status check_geom(const lcsa_geom* g, const char* what);
lcsa_status check_params(const lcsa_select_params* p);
lcsa_status check_cache(const lcsa_kv_cache* c);
lcsa_status check_ptr(const void* p, const char* name, bool allow_null = false);
lcsa_status check_matches_cache(const lcsa_geom* g, const lcsa_kv_cache* c);

// Number of held TBs whose absolute index is <= tb (held TBs ascend).
int32_t visible_tbs(const lcsa_kv_cache& c, int64_t tb);

// Largest k over the query rows of a chunk against the held TBs; also the
// largest candidate count when n_allowed_max is non-null.
int32_t max_topk(const lcsa_geom& gq, int64_t q_first_abs_tb, const lcsa_kv_cache& c,
                 const lcsa_select_params& p, int64_t* n_allowed_max);

}  // namespace lcsa
