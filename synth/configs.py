"""Workload shapes of the batch-1 verify step (one MoE decoder layer, or a stack).

Every shape is a plain description of sizes and storage formats; no arithmetic
of the layer lives here.  The five named workloads are the single-layer and
stack configurations the project is measured on; the small ones exist for
tests that the CPU oracle finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerShape:
    name: str
    d: int            # hidden size
    n_h: int          # attention heads
    d_h: int          # per-head content dim
    d_c: int          # latent KV rank
    d_r: int          # decoupled RoPE dim
    E: int            # routed experts
    top_k: int        # experts per token
    n_shared: int     # shared experts
    f: int            # expert FFN width
    T: int            # verify rows (k drafts + 1)
    L: int            # cached positions before the step
    attn_fmt: str     # "f32" | "bf16"  (W_Q, W_DKV, W_UK, W_UV, W_O, W_R)
    exp_fmt: str      # "f32" | "bf16" | "fp8" | "mxfp4"  (W1, W3, W2; fp8 = E4M3 + fp32 128x128 scales,
                      #   mxfp4 = E2M1 + an E8M0 scale per 32 elements of a row)
    kv_fmt: str       # "f32" | "bf16" | "fp8row" (E4M3 codes + an fp32 power-of-two scale per row)
    routing: str = "uniform"   # "uniform" | "skew" (hot experts get a router bias)
    n_layers: int = 1
    V: int = 0                 # vocabulary (stacks only)
    steps: int = 1             # verify steps (stacks only)
    kv_capacity: int = 0       # 0 -> L + T
    n_pools: int = 0           # distinct routed-expert weight pools in a stack (0 = one per layer)
    head_fmt: str = "bf16"     # LM head: "bf16" | "fp8" (E4M3 + fp32 128x128 scales)
    q_lora: int = 0            # 0: one W_Q; > 0: low-rank query W_DQ -> q-norm -> W_UQ of this rank
    kv_norm: bool = False      # RMSNorm (gain gamma_kv) on the latent before it is cached
    idx_heads: int = 0         # sparse attention (idx_topk > 0): indexer heads, index key dim, rows kept
    idx_dim: int = 0
    idx_topk: int = 0
    eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def kvw(self) -> int:
        return self.d_c + self.d_r

    @property
    def kv_row(self) -> int:
        """Values per cache row: latent, RoPE key, and the index key with sparse attention."""
        return self.kvw + (self.idx_dim if self.idx_topk else 0)

    @property
    def qw(self) -> int:
        return self.d_h + self.d_r

    @property
    def capacity(self) -> int:
        return self.kv_capacity or (self.L + self.T)

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


# A micro shape for fp64 brute-force checks.
C0 = LayerShape("micro_f32", d=64, n_h=2, d_h=16, d_c=32, d_r=8, E=4, top_k=2, n_shared=1, f=32,
                T=3, L=5, attn_fmt="f32", exp_fmt="f32", kv_fmt="f32")
# Single tiny fp32 layer, T=1, 128 cached positions.
C1 = LayerShape("tiny_f32_T1_L128", d=512, n_h=8, d_h=64, d_c=128, d_r=32, E=16, top_k=2,
                n_shared=1, f=256, T=1, L=128, attn_fmt="f32", exp_fmt="f32", kv_fmt="f32")
# One bf16 layer, 128 experts, T=6, 2048 cached positions.
C2 = LayerShape("bf16_E128_T6_L2048", d=4096, n_h=32, d_h=128, d_c=512, d_r=64, E=128, top_k=8,
                n_shared=1, f=1024, T=6, L=2048, attn_fmt="bf16", exp_fmt="bf16", kv_fmt="bf16")
# One layer, 384 fp8 experts, T=8, 8192 cached positions.
C3 = LayerShape("fp8_E384_T8_L8192", d=4096, n_h=32, d_h=128, d_c=512, d_r=64, E=384, top_k=8,
                n_shared=1, f=2048, T=8, L=8192, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16")
# C3 at 65536 cached positions, T=6, skewed routing.
C4 = C3.with_(name="fp8_E384_T6_L65536_skew", T=6, L=65536, routing="skew")
# 32-layer stack of C3-type layers, vocab 129280, T=6, 512 steps from 4096 cached positions.
C5 = C3.with_(name="stack32_fp8_E384_T6_L4096", T=6, L=4096, n_layers=32, V=129280, steps=512,
              kv_capacity=8192, n_pools=16)

# The C3 layer with MXFP4 experts (the expert format of the pages' serving stack).
C3X = C3.with_(name="mxfp4_E384_T8_L8192", exp_fmt="mxfp4")
# The C5 stack with MXFP4 experts: at half a byte per weight all 32 layers keep
# routed experts of their own (about 165 GB).
C5X = C5.with_(name="stack32_mxfp4_E384_T6_L4096", exp_fmt="mxfp4", n_pools=0)

# The serving formats of the MXFP4 stack: MXFP4 experts with an fp8 (E4M3) KV
# cache, one power-of-two scale per row.
C3XK = C3X.with_(name="mxfp4_fp8kv_E384_T8_L8192", kv_fmt="fp8row")
C5XK = C5X.with_(name="stack32_mxfp4_fp8kv_E384_T6_L4096", kv_fmt="fp8row")
# The layer variant with a low-rank query (rank 1536, q-norm) and the latent norm.
C3Q = C3.with_(name="fp8_lowrankq_E384_T8_L8192", q_lora=1536, kv_norm=True)
# The long-context layer with sparse attention: an indexer of 64 heads x 128
# dims, each verify row attends to its top 2048 cache rows.
C4S = C4.with_(name="fp8_sparse2048_E384_T6_L65536_skew", idx_heads=64, idx_dim=128, idx_topk=2048)
# The same in the serving formats: MXFP4 experts and the fp8 cache, whose rows
# then carry the index key under the row's scale.
C4SXK = C4S.with_(name="mxfp4_fp8kv_sparse2048_E384_T6_L65536_skew", exp_fmt="mxfp4", kv_fmt="fp8row")
PRESETS = {s.name: s for s in (C0, C1, C2, C3, C4, C5, C3X, C5X, C3XK, C5XK, C3Q, C4S, C4SXK)}
BY_KEY = {"C0": C0, "C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5, "C3X": C3X, "C5X": C5X,
          "C3XK": C3XK, "C5XK": C5XK, "C3Q": C3Q, "C4S": C4S, "C4SXK": C4SXK}

# Skewed routing: the hot set is the first ceil(0.2 E) experts of a seeded permutation.
HOT_FRACTION = 0.2
HOT_SHARE_TARGET = 0.8
