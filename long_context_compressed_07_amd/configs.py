"""The five workloads of the compressed-attention layer, plus scaled-down variants for tests.

Sizes follow the pages' shapes: m = 4 CSA compression and top-1024 selection
(yudonglee.me "DeepSeek-V4 详解" 2.2 Steps 1-3), m' = 128 HCA compression of a 1M-token context
into 8192 summaries (2.3 Step 1; hongke120.com/20112.html 2.3), 128 query heads in BF16
(2.2 Step 4), a 512-wide latent plus 64 RoPE dims per cached token (deepseek.csdn.net
"一文搞懂 DeepSeek" MLA section), and fp8 cache rows with bf16 RoPE dims (jaylab-temp.pages.dev
"DeepSeek-V4 — 百万 Token 上下文的高效 MoE 模型", 其他技术细节).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "csa_decode" | "csa_prefill" | "hca_prefill" | "hybrid_decode"
    B: int               # sequences
    T: int               # context tokens per sequence (decode: includes the new token)
    d_c: int             # latent (value) dims of a cache row
    d_r: int             # RoPE dims of a cache row (bf16 whenever d_r > 0)
    H: int               # query heads
    m: int               # compression ratio of the attention layer (CSA m or HCA m')
    k: int = 0           # top-k (CSA)
    window: int = 0      # raw sliding window (CSA)
    H_I: int = 0         # indexer heads
    d_I: int = 0         # indexer head dim
    kv_dtype: str = "bf16"    # "f32" | "bf16" | "e4m3" (dtype of the c part of cache rows)
    idx_dtype: str = "bf16"   # "f32" | "bf16" | "e4m3" (indexer q and k)
    q_dtype: str = "bf16"     # "f32" | "bf16"
    nq: int = 1               # queries per sequence: the last nq positions of the context
    d_model: int = 0          # > 0: project x, g from a hidden state (fp32 workload)
    m_hca: int = 0            # hybrid: HCA compression ratio of the paired layer
    compress_on_path: bool = True   # prefill: pooling runs inside the step

    @property
    def d(self) -> int:
        return self.d_c + self.d_r

    @property
    def n_entries(self) -> int:
        return self.T // self.m

    @property
    def n_hca(self) -> int:
        return self.T // self.m_hca if self.m_hca else 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Full-size workloads.
C1 = Workload("csa_decode_f32_b1_4k", "csa_decode", B=1, T=4096, d_c=128, d_r=0, H=16, m=4,
              k=64, window=128, H_I=4, d_I=64, kv_dtype="f32", idx_dtype="f32", q_dtype="f32",
              nq=1, d_model=1024)
C2 = Workload("csa_prefill_bf16_32k", "csa_prefill", B=1, T=32768, d_c=512, d_r=64, H=64, m=4,
              k=1024, window=128, H_I=8, d_I=64, kv_dtype="bf16", idx_dtype="bf16",
              q_dtype="bf16", nq=32768)
C3 = Workload("hca_prefill_bf16_1m_q4096", "hca_prefill", B=1, T=1 << 20, d_c=512, d_r=64,
              H=128, m=128, kv_dtype="bf16", q_dtype="bf16", nq=4096)
C4 = Workload("csa_decode_fp8_b64_128k", "csa_decode", B=64, T=1 << 17, d_c=512, d_r=64, H=128,
              m=4, k=1024, window=128, H_I=8, d_I=64, kv_dtype="e4m3", idx_dtype="e4m3",
              q_dtype="bf16", nq=1, compress_on_path=False)
C5 = Workload("hybrid_decode_fp8_b8_1m", "hybrid_decode", B=8, T=1 << 20, d_c=512, d_r=64,
              H=128, m=4, k=1024, window=128, H_I=8, d_I=64, kv_dtype="e4m3",
              idx_dtype="e4m3", q_dtype="bf16", nq=1, m_hca=128, compress_on_path=False)

FULL = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}

# Scaled-down variants: same dtypes and layouts, sizes the oracle finishes in seconds, chosen to
# span several kernel tiles and to leave ragged tails (T not a multiple of m, n_vis not a
# multiple of any tile, k not a power of two where allowed), and, for the fp8 decode variants, key
# lists long enough to be split over workgroups (584 CSA keys, 600 HCA entries: 2 splits each).
SMALL = {
    "C1": C1.replace(name="csa_decode_f32_small", T=1027, d_model=256),
    "C2": C2.replace(name="csa_prefill_bf16_small", T=1502, nq=1502, k=96, window=40, H=64),
    "C3": C3.replace(name="hca_prefill_bf16_small", T=128 * 300 + 77, nq=37, H=128),
    "C4": C4.replace(name="csa_decode_fp8_small", B=3, T=4 * 1500 + 2, k=520, window=64),
    "C5": C5.replace(name="hybrid_decode_fp8_small", B=2, T=128 * 600 + 5, k=128, window=128),
}

SEED_BASE = {"C1": 7001, "C2": 7002, "C3": 7003, "C4": 7004, "C5": 7005}
