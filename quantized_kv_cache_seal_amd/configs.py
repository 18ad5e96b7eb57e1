"""The five synthetic workloads, as shapes and distributions only.

Shapes follow the models the pages measure: a Qwen 27B-class hybrid model
with 16 full-attention layers of 4 KV heads x 256 (SJ-KVaRN section 1 and
section 8), Gemma 4 31B-class 512-wide heads split into two 256-point halves
(SJ-KVaRN section 9), and the Qwen2.5-14B-1M class with 48 layers of 8 KV
heads x 128 (HAL #582 section 1).  No weights or datasets are involved: every
key, value and query comes from the seeded generator in ``inputs``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_kv_heads: int
    head_dim: int
    n_q_heads: int
    ctx: int                 # tokens per sequence at measurement
    n_seqs: int = 1
    passes: int = 16         # Sinkhorn passes
    k_bits: int = 4
    v_bits: int = 4
    tail_min: int = 4096
    tail_max: int = 8192
    margin: int = 512        # ring slack beyond tail_max (one micro-batch)
    k_dist: str = "normal"
    stage: str = "tq6"       # staging ring: "tq6" (rotated 6-bit) or "f16" (exact, original domain)
    outliers: int = 0
    outlier_scale: float = 1.0
    seed: int = 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny-1x1x256-ctx2048", n_layers=1, n_kv_heads=1, head_dim=256, n_q_heads=4,
                ctx=2048, passes=8, tail_min=256, tail_max=512, outliers=4, outlier_scale=20.0, seed=1)

QWEN27B = Workload("qwen27b-like-16x4x256-ctx110592", n_layers=16, n_kv_heads=4, head_dim=256,
                   n_q_heads=24, ctx=110_592, outliers=5, outlier_scale=15.0, seed=2)

GEMMA31B = Workload("gemma31b-like-16x2x512-ctx32768", n_layers=16, n_kv_heads=2, head_dim=512,
                    n_q_heads=16, ctx=32_768, tail_min=1024, tail_max=2048, k_dist="student_t3", seed=3)

QWEN14B1M = Workload("qwen14b1m-like-48x8x128-ctx262144-k8v4", n_layers=48, n_kv_heads=8, head_dim=128,
                     n_q_heads=40, ctx=262_144, k_bits=8, v_bits=4, outliers=8, outlier_scale=25.0, seed=4)

BATCHED = Workload("batched-16seq-16x4x256-ctx65536", n_layers=16, n_kv_heads=4, head_dim=256,
                   n_q_heads=24, ctx=65_536, n_seqs=16, tail_min=4096, tail_max=4352,
                   outliers=5, outlier_scale=15.0, seed=5)

# config 1 again with the KVarN-style f16 staging ring (SJ-KVaRN section 4.1)
TINY_F16 = TINY.scaled(name="tiny-1x1x256-ctx2048-f16stage", stage="f16")

ALL = [TINY, QWEN27B, GEMMA31B, QWEN14B1M, BATCHED]
