"""Input recipe: which seeded tensors a layer (or stack) is fed, in canonical layout.

Distributions: weights N(0, 0.02); RMSNorm gains N(1, 0.1); hidden states and
prefilled KV rows N(0, 1) (rounded to the cache format); token ids uniform over
the vocabulary.  All are Irwin-Hall(4) draws from the counter-based generator
(synth.h), one stream per tensor.  Expert slot e < E is routed expert e; slot
E + s is shared expert s.  In a stack with n_pools > 0, routed experts of layer
l are drawn from pool l mod n_pools (attention, router, gains and shared experts
stay distinct per layer).  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from . import fp8_blocks, fp8row_kv, mxfp4_blocks, normal_bf16, normal_f32, permutation, stream_id, uniform_ints
from .configs import HOT_FRACTION, LayerShape

W_SIGMA = 0.02
GAIN_SIGMA = 0.1
ACT_SIGMA = 1.0

_GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")


def _attn_tensor(shape_rc, fmt, seed, stream):
    if fmt == "f32":
        return normal_f32(shape_rc, seed, stream, W_SIGMA)
    if fmt == "bf16":
        return normal_bf16(shape_rc, seed, stream, W_SIGMA)
    raise ValueError(fmt)


def attn_shapes(s: LayerShape):
    """Attention-format tensors of a layer; with a low-rank query, W_DQ and W_UQ
    take the place of W_Q."""
    q = {"wdq": (s.q_lora, s.d), "wuq": (s.n_h * s.qw, s.q_lora)} if s.q_lora else {"wq": (s.n_h * s.qw, s.d)}
    idx = {"widx": (s.idx_heads * s.idx_dim + s.idx_heads + s.idx_dim, s.d)} if s.idx_topk else {}
    return {
        **q,
        **idx,
        "wdkv": (s.kvw, s.d),
        "wuk": (s.n_h, s.d_h, s.d_c),
        "wuv": (s.n_h, s.d_h, s.d_c),
        "wo": (s.d, s.n_h * s.d_h),
        "wr": (s.E, s.d),
    }


def expert_pool_layer(s: LayerShape, layer: int) -> int:
    return layer % s.n_pools if s.n_pools else layer


def expert_host(s: LayerShape, seed: int, layer: int, slot: int):
    """(w1, w3, w2, s1, s3, s2) of expert slot `slot`; scales are None unless fp8
    (fp32 per 128x128 block) or mxfp4 (E8M0 codes per 32 elements of a row)."""
    lay = expert_pool_layer(s, layer) if slot < s.E else layer
    out = []
    scales = []
    for tag, (R, K) in (("w1", (s.f, s.d)), ("w3", (s.f, s.d)), ("w2", (s.d, s.f))):
        st = stream_id(tag, lay, slot)
        if s.exp_fmt == "fp8":
            q, sc = fp8_blocks(R, K, seed, st, W_SIGMA)
            out.append(q)
            scales.append(sc)
        elif s.exp_fmt == "mxfp4":
            q, sc = mxfp4_blocks(R, K, seed, st, W_SIGMA)
            out.append(q)
            scales.append(sc)
        elif s.exp_fmt == "bf16":
            out.append(normal_bf16((R, K), seed, st, W_SIGMA))
            scales.append(None)
        else:
            out.append(normal_f32((R, K), seed, st, W_SIGMA))
            scales.append(None)
    return out[0], out[1], out[2], scales[0], scales[1], scales[2]


def router_bias(s: LayerShape, seed: int, layer: int):
    if s.routing != "skew":
        return None
    beta = skew_beta(s)
    hot = permutation(s.E, seed, stream_id("hot_perm", layer))[: int(math.ceil(HOT_FRACTION * s.E))]
    b = np.zeros(s.E, dtype=np.float32)
    b[hot] = np.float32(beta)
    return b


def skew_beta(s: LayerShape) -> float:
    path = os.path.join(_GOLDEN, "router_skew_bias.json")
    with open(path) as fh:
        table = json.load(fh)
    key = "E%d_k%d_d%d" % (s.E, s.top_k, s.d)
    if key not in table:
        raise KeyError("no stored router skew bias for %s in %s" % (key, path))
    return float(table[key]["beta"])


def layer_weights_host(s: LayerShape, seed: int = 0, layer: int = 0, experts=None) -> dict:
    """Canonical weights of one layer.  `experts`: iterable of expert slots to
    materialise (default: all E + n_shared)."""
    w = {
        "gamma1": normal_f32(s.d, seed, stream_id("gamma1", layer), GAIN_SIGMA, mean=1.0),
        "gamma2": normal_f32(s.d, seed, stream_id("gamma2", layer), GAIN_SIGMA, mean=1.0),
    }
    if s.q_lora:
        w["gamma_q"] = normal_f32(s.q_lora, seed, stream_id("gamma_q", layer), GAIN_SIGMA, mean=1.0)
    if s.kv_norm:
        w["gamma_kv"] = normal_f32(s.d_c, seed, stream_id("gamma_kv", layer), GAIN_SIGMA, mean=1.0)
    for name, shp in attn_shapes(s).items():
        w[name] = _attn_tensor(shp, s.attn_fmt, seed, stream_id(name, layer))
    w["router_bias"] = router_bias(s, seed, layer)
    slots = range(s.E + s.n_shared) if experts is None else experts
    w["experts"] = {int(e): expert_host(s, seed, layer, int(e)) for e in slots}
    return w


def hidden_host(s: LayerShape, seed: int = 0, layer: int = 0, step: int = 0) -> np.ndarray:
    """H [T][d] fp32, N(0, 1)."""
    return normal_f32((s.T, s.d), seed, stream_id("H", layer, step), ACT_SIGMA)


def kv_row_bytes(s: LayerShape) -> int:
    """Bytes of one cache row of kv_row values (kvw, plus idx_dim with sparse
    attention): fp32 / bf16 elements, or for fp8 rows kv_row E4M3 codes and one
    fp32 scale, padded to a multiple of 16 bytes."""
    if s.kv_fmt == "f32":
        return 4 * s.kv_row
    if s.kv_fmt == "bf16":
        return 2 * s.kv_row
    return (s.kv_row + 4 + 15) // 16 * 16


def kv_prefill_host(s: LayerShape, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Cache of `capacity` rows; rows [0, L) hold N(0,1) values in the cache format,
    rows [L, capacity) are zero.  fp8 rows are uint8 [capacity][kv_row_bytes]."""
    cap = s.capacity
    if s.kv_fmt == "fp8row":
        kv = np.zeros((cap, kv_row_bytes(s)), dtype=np.uint8)
        kv[: s.L] = fp8row_kv(s.L, s.kv_row, kv_row_bytes(s), seed, stream_id("kv_prefill", layer),
                              stream_id("kv_scale", layer), ACT_SIGMA)
        return kv
    if s.kv_fmt == "f32":
        kv = np.zeros((cap, s.kv_row), dtype=np.float32)
        kv[: s.L] = normal_f32((s.L, s.kv_row), seed, stream_id("kv_prefill", layer), ACT_SIGMA)
    else:
        kv = np.zeros((cap, s.kv_row), dtype=np.uint16)
        kv[: s.L] = normal_bf16((s.L, s.kv_row), seed, stream_id("kv_prefill", layer), ACT_SIGMA)
    return kv


def stack_tables_host(s: LayerShape, seed: int = 0):
    """(embedding [V][d] bf16 bits, LM head, final gain [d] fp32).  The head is
    [V][d] bf16 bits, or for an fp8 head (E4M3 codes [V][d], fp32 128x128 block
    scales) drawn as the fp8 experts are."""
    emb = normal_bf16((s.V, s.d), seed, stream_id("emb"), W_SIGMA)
    if s.head_fmt == "fp8":
        head = fp8_blocks(s.V, s.d, seed, stream_id("head"), W_SIGMA)
    else:
        head = normal_bf16((s.V, s.d), seed, stream_id("head"), W_SIGMA)
    gf = normal_f32(s.d, seed, stream_id("gamma_f"), GAIN_SIGMA, mean=1.0)
    return emb, head, gf


def tokens_host(s: LayerShape, seed: int = 0, step: int = 0) -> np.ndarray:
    """T token ids (t0 then drafts), uniform over [0, V)."""
    return uniform_ints(s.T, s.V, seed, stream_id("tokens", 0, step)).astype(np.int32)
