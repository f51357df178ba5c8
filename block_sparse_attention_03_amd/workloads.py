"""The LCSA workloads: shapes of the pages' 768x1408 to 4K streaming runs and
of the parallel (all frames at once) training forward.

Token geometry ([HW] "How FlashVSR works" 5.3): one token is 16x16 output
pixels, one block 8x8 tokens of 2 latent frames, 2 latent frames are 8 output
frames. A 768x1408 video is a 48x88 token grid; 1536x2688 is 96x168; 4K
(2176x3840 with padding) is 136x240. The local window is 11x11 blocks
([HW] 2.2 step 2). k is 20 % of a row's candidates, scaled by
768*1280/(H*W) for the two large resolutions ([HW] 2.2, topk_ratio rule).
The streaming cache keeps 6 latent frames = 3 temporal blocks ([HW] 2.3).
The parallel forward takes a whole training clip at once ([FN] Key design 1:
Stage 1 trains on 89-frame 768x1280 clips, and the student is trained on
all frames in parallel under the block-sparse causal mask).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    height: int                # token rows
    width: int                 # token cols
    frames: int                # latent frames of query chunk
    cache_frames: int          # latent frames primed into the cache before the first step
    cap_tb: int                # cache capacity kept after each step, in temporal blocks
    local_range: int = 11
    border: int = 0            # 0 Boundary-Preserved, 1 Boundary-Truncated
    topk_fixed: int = 0
    ratio: tuple = (1, 5)
    scale_by_resolution: bool = False
    out_hw: tuple = (768, 1280)
    ratio_base: int = 0        # 0: ratio of a row's candidates, 1: of all key blocks
    steps: int = 1
    seed: int = 2026
    batch: int = 1
    frame_seg: tuple | None = None  # Stage-1 segment id per latent frame (segment-masked path)
    lists: str = "draft"           # "draft": top-k selection; "local": every allowed key block
    layers: tuple = ()             # a stack of workloads run one after another per step
    backward: bool = False         # also run dq, dk, dv over the same lists (training shape)

    @property
    def n_slots(self) -> int:
        return self.cache_frames // 2 + self.frames // 2

    @property
    def nS(self) -> int:
        return (self.height // 8) * (self.width // 8)

    @property
    def nq(self) -> int:
        return (self.frames // 2) * self.nS


WORKLOADS = {
    "tiny": Workload("tiny LCSA 4x16x16 tokens, 2 heads, d64, fp32", 2, 64, "f32", 16, 16,
                     frames=4, cache_frames=0, cap_tb=2, topk_fixed=3, seed=1001),
    "cold_768x1408": Workload("cold-start chunk 768x1408 (6 latent frames x 48x88 tokens)", 12, 128,
                              "bf16", 48, 88, frames=6, cache_frames=0, cap_tb=3, seed=1002),
    "step_768x1408": Workload("streaming step 768x1408 (2 new latent frames x 48x88 tokens, "
                              "6-frame KV cache)", 12, 128, "bf16", 48, 88, frames=2,
                              cache_frames=6, cap_tb=3, steps=100, seed=1003),
    "step_1536x2688": Workload("streaming step 1536x2688 (2 new latent frames x 96x168 tokens, "
                               "6-frame KV cache)", 12, 128, "bf16", 96, 168, frames=2,
                               cache_frames=6, cap_tb=3, scale_by_resolution=True,
                               out_hw=(1536, 2688), steps=50, seed=1004),
    # Stage-1/2 training shape: 89-frame 768x1280 clips give 23 latent frames,
    # padded to 24 (12 temporal blocks of 6x10 blocks); every query block
    # sees its own and all earlier temporal blocks, lists grow with the TB
    "longT_768x1280": Workload("long-T parallel forward 768x1280 (24 latent frames x 48x80 "
                               "tokens, block-causal over 12 temporal blocks)", 12, 128, "bf16",
                               48, 80, frames=24, cache_frames=0, cap_tb=12, steps=10, seed=1006),
    "train_longT_768x1280": Workload("training step 768x1280: long-T forward + backward (24 "
                                     "latent frames, 12 TBs, dq/dk/dv over the same lists)", 12,
                                     128, "bf16", 48, 80, frames=24, cache_frames=0, cap_tb=12,
                                     steps=10, seed=1006, backward=True),
    # Stage-1 joint video-image training shape: an 89-frame 768x1280 clip
    # (23 latent frames) and one image as a one-frame segment, 24 frames
    "stage1_768x1280": Workload("Stage-1 segment-masked attention 768x1280 (23-frame video "
                                "segment + 1 image segment, 48x80 tokens)", 12, 128, "bf16",
                                48, 80, frames=24, cache_frames=0, cap_tb=12, steps=10,
                                seed=1007, frame_seg=(0,) * 23 + (1,)),
    # FlashVSR+ hybrid attention at 4K: local layers attend every causal key
    # block of a 3x3-block window over the current and previous TB (18 of the
    # 2,040 valid key blocks, about 1 %); global layers keep the draft top-k
    # over every causal key block (no spatial window), k = 20 % scaled by
    # resolution; one global layer every 4
    "hybrid_local_4k": Workload("FlashVSR+ local layer 4K (3x3 blocks x 2 TBs, every block)", 12,
                                128, "bf16", 136, 240, frames=2, cache_frames=2, cap_tb=1,
                                local_range=3, ratio=(1, 1), lists="local", steps=50, seed=1008),
    "hybrid_global_4k": Workload("FlashVSR+ global layer 4K (draft top-k over all causal key "
                                 "blocks)", 12, 128, "bf16", 136, 240, frames=2, cache_frames=6,
                                 cap_tb=3, local_range=255, scale_by_resolution=True,
                                 out_hw=(2176, 3840), steps=50, seed=1008),
    "hybrid_4k": Workload("FlashVSR+ hybrid stack 4K (3 local layers + 1 global layer per "
                          "step)", 12, 128, "bf16", 136, 240, frames=2, cache_frames=6, cap_tb=3,
                          steps=30, seed=1008,
                          layers=("hybrid_local_4k",) * 3 + ("hybrid_global_4k",)),
    "step_4k": Workload("streaming step 4K 2176x3840 padded (2 new latent frames x 136x240 "
                        "tokens, 6-frame KV cache)", 12, 128, "bf16", 136, 240, frames=2,
                        cache_frames=6, cap_tb=3, scale_by_resolution=True,
                        out_hw=(2176, 3840), steps=50, seed=1005),
}

ORDER = ["tiny", "cold_768x1408", "step_768x1408", "step_1536x2688", "step_4k", "longT_768x1280",
         "stage1_768x1280", "hybrid_local_4k", "hybrid_global_4k", "hybrid_4k",
         "train_longT_768x1280"]


def segment_pair_quarters(frame_seg) -> dict:
    """(query TB a, key TB p) -> number of (query frame, key frame) pairs of
    the two blocks that share a segment (0..4); each is a quarter of a
    block pair's attention work."""
    n = len(frame_seg) // 2
    out = {}
    for a in range(n):
        for p in range(n):
            qn = sum(frame_seg[2 * a + dq] == frame_seg[2 * p + dk]
                     for dq in range(2) for dk in range(2))
            if qn:
                out[(a, p)] = qn
    return out


def attention_flops_per_pair(head_dim: int) -> int:
    """QK^T and PV of one 128 x 128 block pair: 2 * 2 * 128 * 128 * D."""
    return 4 * 128 * 128 * head_dim


def backward_flops_per_pair(head_dim: int) -> int:
    """The five products of the backward of one block pair (S recomputed,
    dP, dV, dQ, dK): 5 * 2 * 128 * 128 * D."""
    return 10 * 128 * 128 * head_dim
