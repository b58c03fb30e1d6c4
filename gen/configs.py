"""The five workloads the library is checked and measured on.

Shapes follow the worked example and the tables of the English notes page
"AFFMAE: Scalable Vision Pre-Training for High-Resolution Microscopy
Segmentation on Desktop Hardware": 512x512 images cut into 8x8 patches give a
64x64 token grid, about half of it visible after Perlin masking (2048
tokens); stage 1 is 128-dim, stage 2 256-dim with about 819 tokens, stage 3
512-dim with about 328 and stage 4 768-dim with about 131 after merges at
retention 0.4 ("A Complete Example"); pre-training runs
at batch 32 ("Key Experimental Results", pre-training efficiency table) and
high-resolution fine-tuning at batch 4.  Heads of 32 dims, clusters of 8 and
6 neighbour clusters are the readings taken where the pages are silent.
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    seed: int
    B: int
    N: int            # tokens per image
    G: int            # grid side passed to the neighbour build
    H: int
    D: int
    dtype: str        # "f32" | "bf16" | "f16"
    geometry: str     # "cells" | "perlin" | "merged" | "jitter"
    passes: str       # "fwd" | "fwd+bwd"
    qkv_scale: float = 1.0
    dup_frac: float = 0.0
    cs: int = 8
    k: int = 6

    @property
    def C(self) -> int:
        return -(-self.N // self.cs)     # a partial last cluster when cs does not divide N

    @property
    def nk(self) -> int:
        return self.cs * self.k

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def with_batch(self, B: int) -> "WorkloadConfig":
        return replace(self, B=B)


CONFIGS = {
    # 256 distinct integer cells of a 32x32 grid, one head, fp32, forward only.
    "tiny": WorkloadConfig("tiny", 1001, 1, 256, 32, 1, 32, "f32", "cells", "fwd"),
    # Stage-1 pre-training shape: 64x64 grid, Perlin mask keeps 2048 cells.
    "stage1": WorkloadConfig("stage1", 1002, 32, 2048, 64, 4, 32, "bf16", "perlin", "fwd+bwd"),
    # Stage-3 shape: 328 merged tokens at real-valued coordinates, 16 heads.
    "stage3": WorkloadConfig("stage3", 1003, 32, 328, 64, 16, 32, "bf16", "merged", "fwd+bwd"),
    # High-resolution fine-tune shape: full 256x256 grid with jitter.
    "highres": WorkloadConfig("highres", 1004, 4, 65536, 256, 4, 32, "bf16", "jitter", "fwd+bwd"),
    # Stage-2 and stage-4 shapes of the worked example: 819 and 131 merged
    # tokens (neither a multiple of 8: each image ends with a partial
    # cluster), 256-dim = 8 heads and 768-dim = 24 heads.
    "stage2": WorkloadConfig("stage2", 1006, 32, 819, 64, 8, 32, "bf16", "merged", "fwd+bwd"),
    "stage4": WorkloadConfig("stage4", 1007, 32, 131, 64, 24, 32, "bf16", "merged", "fwd+bwd"),
    # Large-logit stress: stage-1 geometry, fp16 Q/K/V scaled by 8, 10% of
    # keys duplicated into extra cluster lists.
    "stress": WorkloadConfig("stress", 1005, 32, 2048, 64, 4, 32, "f16", "perlin", "fwd+bwd",
                             qkv_scale=8.0, dup_frac=0.1),
}


def get_config(name: str) -> WorkloadConfig:
    return CONFIGS[name]
