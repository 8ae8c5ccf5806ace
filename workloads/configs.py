"""The five MonarchAttention forward workloads, by short name.

Shapes follow the pages' speed workloads: N = 256, 4K and 16K sequences for
language and vision ([MA] abstract: speed-ups at N = 256, 4K and 16K), and a
3D video latent with Monarch blocks aligned to its (f, h, w) axes ([MRT] "Key
claims", section 4.1) plus its tiled c1 x c2 variant ([MRT] Theorem 4.1).
The video latent 21 x 30 x 52 with 12 heads and d = 128 is this project's
stand-in for the 480p latents the MonarchRT page times (the page does not give
the latent shape).
"""

from dataclasses import dataclass, field, asdict
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    key: str                   # short name of the workload
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    b1: int
    b2: int
    steps: int
    dtype: str                 # "f32" or "bf16"
    data: str                  # generator recipe, see generators.py
    seed: int
    c1: int = 1
    c2: int = 1
    layout: str = "flat"
    fhw: Optional[Tuple[int, int, int]] = None
    pad: str = "post"          # padding side when seq_len < b1*b2 (flat only)
    kv_heads: int = 0          # heads of K and V (0: heads); fewer = grouped-query attention

    @property
    def kv_group(self):
        """Query heads per K/V head."""
        return self.heads // (self.kv_heads or self.heads)

    @property
    def slices(self):
        return self.batch * self.heads

    def algorithmic_flops(self):
        """2*N*d*[3*c1*b2 + 2*c2*b1 + (T-1)*2*(c1*b2 + c2*b1)] per slice:
        stage 1 forms c1*b2 scores per query row and two aggregates (R K, R V);
        stage 2 forms c2*b1 scores per row and one aggregate (L U); every extra
        step adds the stage-1 scores and aggregate R K again plus the stage-2
        scores and the reduction L^T Q."""
        N, d, b1, b2, c1, c2, T = (self.seq_len, self.head_dim, self.b1, self.b2,
                                   self.c1, self.c2, self.steps)
        per = 2 * N * d * (3 * c1 * b2 + 2 * c2 * b1 + (T - 1) * 2 * (c1 * b2 + c2 * b1))
        return per * self.slices

    def algorithmic_bytes(self):
        """Q, K, V read once and Y written once (K and V once per K/V head)."""
        elt = 4 if self.dtype == "f32" else 2
        return (2 + 2 / self.kv_group) * self.seq_len * self.head_dim * elt * self.slices

    def describe(self):
        d = asdict(self)
        d["slices"] = self.slices
        return d


WORKLOADS = {
    "n256": WorkloadConfig("n256", "N=256 16x16 d=64 T=1 fp32, 1 slice",
                      batch=1, heads=1, seq_len=256, head_dim=64, b1=16, b2=16,
                      steps=1, dtype="f32", data="iid", seed=1001),
    "n4k_t3": WorkloadConfig("n4k_t3", "N=4096 64x64 d=64 T=3 bf16, batch 8 x 12 heads",
                      batch=8, heads=12, seq_len=4096, head_dim=64, b1=64, b2=64,
                      steps=3, dtype="bf16", data="lowrank", seed=1002),
    "n16k": WorkloadConfig("n16k", "N=16384 128x128 d=64 T=1 bf16, 12 heads",
                      batch=1, heads=12, seq_len=16384, head_dim=64, b1=128, b2=128,
                      steps=1, dtype="bf16", data="normed", seed=1003),
    "video": WorkloadConfig("video", "video f,h,w=21,30,52 (fh,w)=(630,52) d=128 T=1 bf16, 12 heads",
                      batch=1, heads=12, seq_len=32760, head_dim=128, b1=630, b2=52,
                      steps=1, dtype="bf16", data="video", seed=1004,
                      layout="fh_w", fhw=(21, 30, 52)),
    # the headline shape with the two generalisations: 100 tokens short of the
    # grid (padding in front), and 12 query heads sharing 4 K/V heads
    "n16k_pad": WorkloadConfig("n16k_pad", "N=16284 padded to 128x128 (pre) d=64 T=1 bf16, 12 heads",
                      batch=1, heads=12, seq_len=16384 - 100, head_dim=64, b1=128, b2=128,
                      steps=1, dtype="bf16", data="normed", seed=1003, pad="pre"),
    "n16k_gqa": WorkloadConfig("n16k_gqa", "N=16384 128x128 d=64 T=1 bf16, 12 query heads over 4 K/V heads",
                      batch=1, heads=12, seq_len=16384, head_dim=64, b1=128, b2=128,
                      steps=1, dtype="bf16", data="normed", seed=1003, kv_heads=4),
    "video_tiled": WorkloadConfig("video_tiled", "video (630,52) tiled c1=c2=2 d=128 T=1 bf16, 12 heads",
                      batch=1, heads=12, seq_len=32760, head_dim=128, b1=630, b2=52,
                      steps=1, dtype="bf16", data="video", seed=1004,
                      layout="fh_w", fhw=(21, 30, 52), c1=2, c2=2),
}


def get_workload(key):
    return WORKLOADS[key]
