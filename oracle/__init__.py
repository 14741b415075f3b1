"""CPU ORACLE -- TEST INFRASTRUCTURE ONLY.

Python driver around the plain-C oracle (``oracle.c``; what it computes and the
passages it follows are written out in ``oracle.h``).  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import this package.  It
shares no code with the GPU library; the only module both sides use is the
seeded input generator ``synth``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from synth import recipe
from synth.configs import LayerShape

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liborc.so")

ORC_F32, ORC_BF16, ORC_FP8B128, ORC_MXFP4 = 0, 1, 2, 3
ORC_FP8ROW = 4
_FMT = {"f32": ORC_F32, "bf16": ORC_BF16, "fp8": ORC_FP8B128, "mxfp4": ORC_MXFP4, "fp8row": ORC_FP8ROW}

_vp = ctypes.c_void_p
_i = ctypes.c_int


def build() -> None:
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
           os.path.join(_HERE, "oracle.c"), "-o", LIB, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stderr)


class Cfg(ctypes.Structure):
    _fields_ = [("d", _i), ("n_h", _i), ("d_h", _i), ("d_c", _i), ("d_r", _i), ("E", _i),
                ("top_k", _i), ("n_shared", _i), ("f", _i), ("attn_fmt", _i), ("exp_fmt", _i),
                ("kv_fmt", _i), ("eps", ctypes.c_float), ("rope_base", ctypes.c_double),
                ("q_lora", _i), ("kv_norm", _i), ("idx_heads", _i), ("idx_dim", _i), ("idx_topk", _i)]


class Weights(ctypes.Structure):
    _fields_ = [("gamma1", _vp), ("gamma2", _vp), ("wq", _vp), ("wdkv", _vp), ("wuk", _vp),
                ("wuv", _vp), ("wo", _vp), ("wr", _vp), ("router_bias", _vp),
                ("w1", _vp), ("w3", _vp), ("w2", _vp), ("s1", _vp), ("s3", _vp), ("s2", _vp),
                ("wdq", _vp), ("wuq", _vp), ("gamma_q", _vp), ("gamma_kv", _vp), ("widx", _vp),
                ("force_isel", _vp)]


class AttnTaps(ctypes.Structure):
    _fields_ = [("x", _vp), ("q", _vp), ("ckv", _vp), ("qabs", _vp), ("z", _vp), ("o", _vp), ("sel", _vp),
                ("iscore", _vp)]


class MoeTaps(ctypes.Structure):
    _fields_ = [("xp", _vp), ("logits", _vp), ("sel", _vp), ("gate", _vp), ("y_sel", _vp),
                ("y_shared", _vp)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        for name in ("orc_attn_block", "orc_router", "orc_moe_block", "orc_layer_step",
                     "orc_layer_step_f64", "orc_embed", "orc_head", "orc_greedy_accept"):
            getattr(L, name).restype = _i
        L.orc_attn_block.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _vp, _vp]
        L.orc_router.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp]
        L.orc_moe_block.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp]
        L.orc_layer_step.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp]
        L.orc_layer_step_f64.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp]
        L.orc_embed.argtypes = [_vp, _i, _i, _vp, _i, _vp]
        L.orc_head.argtypes = [_vp, _i, _i, _vp, ctypes.c_float, _vp, _i, _vp, _vp]
        L.orc_greedy_accept.argtypes = [_vp, _vp, _i, _vp]
        L.orc_head_fmt.restype = _i
        L.orc_head_fmt.argtypes = [_vp, _i, _vp, _i, _i, _vp, ctypes.c_float, _vp, _i, _vp, _vp]
        L.orc_verify_sampled.restype = _i
        L.orc_verify_sampled.argtypes = [_vp, _i, _i, _vp, ctypes.c_float, ctypes.c_uint64, _vp, _vp]
        L.orc_splitmix64_mix.restype = ctypes.c_uint64
        L.orc_splitmix64_mix.argtypes = [ctypes.c_uint64]
        L.orc_sample_key.restype = ctypes.c_uint64
        L.orc_sample_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        L.orc_sample_uniform.restype = ctypes.c_float
        L.orc_sample_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_e4m3_to_f32.restype = ctypes.c_float
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_f32.restype = ctypes.c_float
        L.orc_e2m1_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_f32.restype = ctypes.c_float
        L.orc_e8m0_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_f32_to_e4m3.restype = ctypes.c_uint8
        L.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.orc_fp8_row_scale.restype = ctypes.c_float
        L.orc_fp8_row_scale.argtypes = [_vp, _i]
        L.orc_kv_row_bytes.restype = _i
        L.orc_kv_row_bytes.argtypes = [_i, _i]
        L.orc_kv_decode_rows.restype = _i
        L.orc_kv_decode_rows.argtypes = [_vp, _i, _i, _i, _vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def cfg_of(s: LayerShape) -> Cfg:
    return Cfg(s.d, s.n_h, s.d_h, s.d_c, s.d_r, s.E, s.top_k, s.n_shared, s.f, _FMT[s.attn_fmt],
               _FMT[s.exp_fmt], _FMT[s.kv_fmt], s.eps, s.rope_base, s.q_lora, 1 if s.kv_norm else 0,
               s.idx_heads, s.idx_dim, s.idx_topk)


class _WeightsHolder:
    """Keeps the numpy arrays alive while the C struct points at them."""

    def __init__(self, s: LayerShape, w: dict):
        n = s.E + s.n_shared
        self.arrays = []
        self.ptr_arrays = []

        def keep(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            self.arrays.append(a)
            return a.ctypes.data

        ptrs = {k: (ctypes.c_void_p * n)() for k in ("w1", "w3", "w2", "s1", "s3", "s2")}
        for slot, tup in w["experts"].items():
            for k, a in zip(("w1", "w3", "w2", "s1", "s3", "s2"), tup):
                ptrs[k][slot] = keep(a)
        self.ptr_arrays.extend(ptrs.values())
        self.struct = Weights(keep(w["gamma1"]), keep(w["gamma2"]), keep(w.get("wq")), keep(w["wdkv"]),
                              keep(w["wuk"]), keep(w["wuv"]), keep(w["wo"]), keep(w["wr"]),
                              keep(w.get("router_bias")),
                              ctypes.cast(ptrs["w1"], _vp), ctypes.cast(ptrs["w3"], _vp),
                              ctypes.cast(ptrs["w2"], _vp), ctypes.cast(ptrs["s1"], _vp),
                              ctypes.cast(ptrs["s3"], _vp), ctypes.cast(ptrs["s2"], _vp),
                              keep(w.get("wdq")), keep(w.get("wuq")), keep(w.get("gamma_q")),
                              keep(w.get("gamma_kv")), keep(w.get("widx")),
                              keep(None if w.get("force_isel") is None
                                   else np.ascontiguousarray(w["force_isel"], dtype=np.int32)))


def _chk(rc, what):
    if rc != 0:
        raise RuntimeError("%s returned %d" % (what, rc))


def attn_block(s: LayerShape, w: dict, H: np.ndarray, kv: np.ndarray, L: int):
    """Returns (Hp, taps).  Writes KV rows [L, L+T) of `kv` in place."""
    T = H.shape[0]
    H = np.ascontiguousarray(H, dtype=np.float32)
    Hp = np.empty_like(H)
    taps = {"x": np.empty((T, s.d), np.float32), "q": np.empty((T, s.n_h, s.qw), np.float32),
            "ckv": np.empty((T, s.kvw), np.float32), "qabs": np.empty((T, s.n_h, s.d_c), np.float32),
            "z": np.empty((T, s.n_h, s.d_c), np.float32), "o": np.empty((T, s.n_h * s.d_h), np.float32)}
    if s.idx_topk:
        taps["isel"] = np.full((T, s.idx_topk), -1, np.int32)      # kept cache rows (sparse attention)
        taps["iscore"] = np.full((T, L + T), np.nan, np.float32)
    at = AttnTaps(*[taps[k].ctypes.data if k in taps else None
                    for k in ("x", "q", "ckv", "qabs", "z", "o", "isel", "iscore")])
    wh = _WeightsHolder(s, w)
    c = cfg_of(s)
    _chk(lib().orc_attn_block(ctypes.byref(c), ctypes.byref(wh.struct), _p(H), T, _p(kv), L,
                              _p(Hp), ctypes.byref(at)), "orc_attn_block")
    return Hp, taps


def router(s: LayerShape, w: dict, Hp: np.ndarray):
    T = Hp.shape[0]
    Hp = np.ascontiguousarray(Hp, dtype=np.float32)
    xp = np.empty((T, s.d), np.float32)
    lg = np.empty((T, s.E), np.float32)
    sel = np.empty((T, s.top_k), np.int32)
    g = np.empty((T, s.top_k), np.float32)
    wh = _WeightsHolder(s, dict(w, experts={}))
    c = cfg_of(s)
    _chk(lib().orc_router(ctypes.byref(c), ctypes.byref(wh.struct), _p(Hp), T, _p(xp), _p(lg),
                          _p(sel), _p(g)), "orc_router")
    return xp, lg, sel, g


def moe_block(s: LayerShape, w: dict, Hp: np.ndarray, force_sel=None):
    T = Hp.shape[0]
    Hp = np.ascontiguousarray(Hp, dtype=np.float32)
    out = np.empty_like(Hp)
    taps = {"xp": np.empty((T, s.d), np.float32), "logits": np.empty((T, s.E), np.float32),
            "sel": np.empty((T, s.top_k), np.int32), "gate": np.empty((T, s.top_k), np.float32),
            "y_sel": np.empty((T, s.top_k, s.d), np.float32), "y_shared": np.empty((T, s.d), np.float32)}
    mt = MoeTaps(*[taps[k].ctypes.data for k in ("xp", "logits", "sel", "gate", "y_sel", "y_shared")])
    fs = None if force_sel is None else np.ascontiguousarray(force_sel, dtype=np.int32)
    wh = _WeightsHolder(s, w)
    c = cfg_of(s)
    _chk(lib().orc_moe_block(ctypes.byref(c), ctypes.byref(wh.struct), _p(Hp), T, _p(fs), _p(out),
                             ctypes.byref(mt)), "orc_moe_block")
    return out, taps


def layer_step(s: LayerShape, w: dict, H: np.ndarray, kv: np.ndarray, L: int, force_sel=None):
    """Whole layer in fp32.  Returns (out, taps) with attention and MoE taps merged."""
    Hp, at = attn_block(s, w, H, kv, L)
    out, mt = moe_block(s, w, Hp, force_sel)
    taps = dict(at)
    taps.update(mt)
    taps["Hp"] = Hp
    return out, taps


def layer_step_lazy(s: LayerShape, seed: int, layer: int, H: np.ndarray, kv: np.ndarray, L: int,
                    base_weights: dict | None = None, force_sel=None, expert_cache: dict | None = None,
                    expert_fn=None):
    """Layer step that materialises only the experts the router picks (for the
    384-expert shapes).  `expert_fn(layer, slot)`, when given, supplies an
    expert's canonical tensors (the seeded generator's draws) instead of
    synth.recipe.expert_host.  Returns (out, taps, weights_used)."""
    w = base_weights if base_weights is not None else recipe.layer_weights_host(s, seed, layer, experts=[])
    Hp, at = attn_block(s, w, H, kv, L)
    if force_sel is None:
        _, _, sel, _ = router(s, w, Hp)
    else:
        sel = np.asarray(force_sel, dtype=np.int32)
    need = sorted(set(int(e) for e in sel.ravel())) + [s.E + i for i in range(s.n_shared)]
    experts = {}
    for e in need:
        key = (recipe.expert_pool_layer(s, layer) if e < s.E else layer, e)
        if expert_cache is not None and key in expert_cache:
            experts[e] = expert_cache[key]
        else:
            experts[e] = expert_fn(layer, e) if expert_fn is not None else recipe.expert_host(s, seed, layer, e)
            if expert_cache is not None:
                expert_cache[key] = experts[e]
    wx = dict(w, experts=experts)
    out, mt = moe_block(s, wx, Hp, force_sel)
    taps = dict(at)
    taps.update(mt)
    taps["Hp"] = Hp
    return out, taps, wx


def layer_step_f64(s: LayerShape, w: dict, H: np.ndarray, kv: np.ndarray, L: int, force_sel=None):
    T = H.shape[0]
    H = np.ascontiguousarray(H, dtype=np.float32)
    out = np.empty((T, s.d), np.float64)
    hp = np.empty((T, s.d), np.float64)
    kvn = np.empty((T, s.kvw), np.float64)
    lg = np.empty((T, s.E), np.float64)
    sel = np.empty((T, s.top_k), np.int32)
    fs = None if force_sel is None else np.ascontiguousarray(force_sel, dtype=np.int32)
    wh = _WeightsHolder(s, w)
    c = cfg_of(s)
    _chk(lib().orc_layer_step_f64(ctypes.byref(c), ctypes.byref(wh.struct), _p(H), T, _p(kv), L,
                                  _p(fs), _p(out), _p(hp), _p(kvn), _p(lg), _p(sel)),
         "orc_layer_step_f64")
    return {"out": out, "Hp": hp, "kv_new": kvn, "logits": lg, "sel": sel}


def embed(emb: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    V, d = emb.shape
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    h = np.empty((len(t), d), np.float32)
    _chk(lib().orc_embed(_p(np.ascontiguousarray(emb)), V, d, _p(t), len(t), _p(h)), "orc_embed")
    return h


def head(headw: np.ndarray, gamma_f: np.ndarray, h: np.ndarray, eps: float = 1e-6, want_logits=True):
    V, d = headw.shape
    T = h.shape[0]
    h = np.ascontiguousarray(h, dtype=np.float32)
    lg = np.empty((T, V), np.float32) if want_logits else None
    am = np.empty(T, np.int32)
    _chk(lib().orc_head(_p(np.ascontiguousarray(headw)), V, d, _p(gamma_f), eps, _p(h), T, _p(lg),
                        _p(am)), "orc_head")
    return lg, am


def head_fp8(codes: np.ndarray, scales: np.ndarray, gamma_f: np.ndarray, h: np.ndarray, eps: float = 1e-6):
    """LM head with E4M3 codes [V][d] and fp32 128x128 block scales."""
    V, d = codes.shape
    T = h.shape[0]
    h = np.ascontiguousarray(h, dtype=np.float32)
    lg = np.empty((T, V), np.float32)
    am = np.empty(T, np.int32)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    _chk(lib().orc_head_fmt(_p(np.ascontiguousarray(codes)), ORC_FP8B128, _p(sc), V, d, _p(gamma_f), eps, _p(h), T,
                            _p(lg), _p(am)), "orc_head_fmt")
    return lg, am


def sample_key(seed: int, step: int) -> int:
    return int(lib().orc_sample_key(seed, step))


def splitmix64_mix(z: int) -> int:
    return int(lib().orc_splitmix64_mix(z))


def sample_uniform(key: int, i: int) -> float:
    return float(lib().orc_sample_uniform(key, i))


def verify_sampled(logits: np.ndarray, tokens, tau: float, key: int):
    """Returns (sample [T], committed tokens)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, V = lg.shape
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    smp = np.empty(T, np.int32)
    com = np.empty(T + 1, np.int32)
    n = lib().orc_verify_sampled(_p(lg), V, T, _p(t), tau, key, _p(smp), _p(com))
    if n <= 0:
        raise RuntimeError("orc_verify_sampled failed")
    return smp, com[1:n + 1].copy()


def greedy_accept(tokens, argmax):
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    a = np.ascontiguousarray(argmax, dtype=np.int32)
    com = np.empty(len(t), np.int32)
    n = lib().orc_greedy_accept(_p(t), _p(a), len(t), _p(com))
    if n <= 0:
        raise RuntimeError("orc_greedy_accept failed")
    return com[:n].copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def kv_row_bytes(fmt: str, kvw: int) -> int:
    return int(lib().orc_kv_row_bytes(_FMT[fmt], kvw))


def kv_decode(kv: np.ndarray, fmt: str, kvw: int, nrows: int) -> np.ndarray:
    """Rows [0, nrows) of a cache buffer (any dtype, the format's row layout) as fp32 [nrows][kvw]."""
    buf = np.ascontiguousarray(kv)
    out = np.empty((nrows, kvw), np.float32)
    _chk(lib().orc_kv_decode_rows(_p(buf), _FMT[fmt], kvw, nrows, _p(out)), "orc_kv_decode_rows")
    return out


def f32_to_e4m3(x: float) -> int:
    return int(lib().orc_f32_to_e4m3(float(x)))


def fp8_row_scale(row: np.ndarray) -> float:
    r = np.ascontiguousarray(row, dtype=np.float32)
    return float(lib().orc_fp8_row_scale(_p(r), len(r)))
