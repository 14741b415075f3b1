"""Python binding of the mk C ABI (include/mk.h): argument marshalling only.

Every step of the verify path runs in the HIP kernels of ``libmk.so``; this
module only converts Python values to C arguments and raises ``MkError`` on a
non-zero status.  Importing it fails loudly if the library has not been built:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_ABI_VERSION = 4
MK_MAX_T = 8   # verify rows per step
MK_STATIC_SCRATCH_BYTES = 32 << 20

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_ABI_MISMATCH = -2
MK_ERR_UNSUPPORTED_DEVICE = -3
MK_ERR_NOT_CORESIDENT = -4
MK_ERR_HIP = -5
MK_ERR_TIMEOUT = -6
MK_ERR_DEVICE_FAULT = -7
MK_ERR_UNSUPPORTED_SHAPE = -8

MK_FMT_F32, MK_FMT_BF16, MK_FMT_FP8_B128, MK_FMT_MXFP4, MK_FMT_FP8_ROW = 0, 1, 2, 3, 4
FORMATS = {"f32": MK_FMT_F32, "bf16": MK_FMT_BF16, "fp8": MK_FMT_FP8_B128, "mxfp4": MK_FMT_MXFP4,
           "fp8row": MK_FMT_FP8_ROW}
MK_T_WQ, MK_T_WDKV, MK_T_WUK, MK_T_WUV, MK_T_WO, MK_T_WR, MK_T_EXPERT, MK_T_WDQ, MK_T_WUQ, MK_T_WIDX = range(10)

# Every entry point the header declares (checked by the CPU tests).
EXPORTS = (
    "mk_abi_version", "mk_last_error", "mk_query_device", "mk_check_config", "mk_packed_bytes",
    "mk_kv_bytes", "mk_layer_state_bytes", "mk_layer_workspace_bytes", "mk_pack_tensor", "mk_pack_expert",
    "mk_layer_init", "mk_decode_step", "mk_decode_step_static", "mk_debug_tap", "mk_get_stats", "mk_set_trace", "mk_read_trace",
    "mk_set_barrier_timeout_us", "mk_sync_status", "mk_layer_reset", "mk_layer_destroy",
    "mk_head_packed_bytes", "mk_pack_head", "mk_head_packed_bytes_fmt", "mk_pack_head_fp8",
    "mk_model_state_bytes", "mk_model_init", "mk_model_init_ex", "mk_model_set_sampling", "mk_model_set_length",
    "mk_model_length_ptr", "mk_model_step", "mk_model_sync_status", "mk_model_reset",
    "mk_model_set_hidden_record", "mk_model_destroy",
)


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("mk error %d: %s" % (code, msg))
        self.code = code


_i32 = ctypes.c_int32
_int = ctypes.c_int
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class LayerConfig(ctypes.Structure):
    _fields_ = [("abi_version", _i32), ("d_model", _i32), ("n_heads", _i32), ("d_head", _i32),
                ("d_latent", _i32), ("d_rope", _i32), ("n_experts", _i32), ("top_k", _i32),
                ("n_shared", _i32), ("d_ff", _i32), ("attn_format", _i32), ("expert_format", _i32),
                ("kv_format", _i32), ("has_router_bias", _i32), ("rms_eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("q_lora_rank", _i32), ("kv_norm", _i32), ("idx_heads", _i32),
                ("idx_dim", _i32), ("idx_topk", _i32), ("idx_max_rows", _i32),
                ("kv_max_rows", _i32)]


class DeviceInfo(ctypes.Structure):
    _fields_ = [("hip_device", _i32), ("is_gfx950", _i32), ("n_cus", _i32), ("wgs_per_cu", _i32),
                ("grid_wgs", _i32), ("threads_per_wg", _i32), ("lds_bytes_per_wg", _i32), ("pad", _i32),
                ("hbm_bytes", ctypes.c_int64), ("arch_name", ctypes.c_char * 64)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("gamma1", _vp), ("gamma2", _vp), ("wq", _vp), ("wdkv", _vp), ("wuk", _vp), ("wuv", _vp),
                ("wo", _vp), ("wr", _vp), ("router_bias", _vp), ("experts", _vp),
                ("wdq", _vp), ("wuq", _vp), ("gamma_q", _vp), ("gamma_kv", _vp), ("widx", _vp)]


class KvCache(ctypes.Structure):
    _fields_ = [("rows", _vp), ("capacity", _i32), ("length", _i32)]


class Stats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("launches", ctypes.c_int64), ("grid_wgs", _i32),
                ("threads_per_wg", _i32), ("barriers_per_step", _i32), ("trace_enabled", _i32),
                ("device_launches", ctypes.c_int64), ("expert_blocks_sum", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmk.so is not built at %s; run __graft_entry__.build() "
                          "(there is no fallback implementation)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "mk_abi_version": (_int, []),
        "mk_last_error": (ctypes.c_char_p, []),
        "mk_query_device": (_int, [_int, _vp]),
        "mk_check_config": (_int, [_vp]),
        "mk_packed_bytes": (_int, [_vp, _int, _vp]),
        "mk_kv_bytes": (_int, [_vp, _i32, _vp]),
        "mk_layer_state_bytes": (_int, [_vp, _int, _vp]),
        "mk_layer_workspace_bytes": (_int, [_vp, _int, _vp]),
        "mk_pack_tensor": (_int, [_vp, _int, _vp, _vp, _vp]),
        "mk_pack_expert": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "mk_layer_init": (_int, [_vp, _vp, _vp, _vp, _int, _vp]),
        "mk_decode_step": (_int, [_vp, _vp, _int, _vp, _vp, _vp]),
        "mk_decode_step_static": (_int, [_vp, _vp, _int, _vp, _vp, _vp]),
        "mk_debug_tap": (_int, [_vp, _int, _vp, _sz, _vp]),
        "mk_get_stats": (_int, [_vp, _vp]),
        "mk_set_trace": (_int, [_vp, _int]),
        "mk_read_trace": (_int, [_vp, _vp, _sz, _vp]),
        "mk_set_barrier_timeout_us": (_int, [_vp, ctypes.c_int64]),
        "mk_sync_status": (_int, [_vp]),
        "mk_layer_reset": (_int, [_vp]),
        "mk_layer_destroy": (None, [_vp]),
        "mk_head_packed_bytes": (_int, [_i32, _i32, _vp]),
        "mk_pack_head": (_int, [_i32, _i32, _vp, _vp, _vp]),
        "mk_model_state_bytes": (_int, [_i32, _i32, _int, _vp]),
        "mk_head_packed_bytes_fmt": (_int, [_i32, _i32, _i32, _vp]),
        "mk_pack_head_fp8": (_int, [_i32, _i32, _vp, _vp, _vp, _vp]),
        "mk_model_init": (_int, [_vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp]),
        "mk_model_init_ex": (_int, [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp]),
        "mk_model_set_sampling": (_int, [_vp, ctypes.c_float, ctypes.c_uint64]),
        "mk_model_set_length": (_int, [_vp, _i32]),
        "mk_model_length_ptr": (_vp, [_vp]),
        "mk_model_step": (_int, [_vp, _vp, _int, _vp, _vp, _vp, _vp, _vp]),
        "mk_model_sync_status": (_int, [_vp]),
        "mk_model_reset": (_int, [_vp]),
        "mk_model_set_hidden_record": (_int, [_vp, _vp]),
        "mk_model_destroy": (None, [_vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    m = lib.mk_last_error()
    return m.decode() if m else ""


def _chk(rc: int) -> None:
    if rc != MK_OK:
        raise MkError(rc, last_error())


def abi_version() -> int:
    return lib.mk_abi_version()


def query_device(hip_device: int = 0) -> DeviceInfo:
    info = DeviceInfo()
    _chk(lib.mk_query_device(hip_device, ctypes.byref(info)))
    return info


def make_config(d_model, n_heads, d_head, d_latent, d_rope, n_experts, top_k, n_shared, d_ff,
                attn_format, expert_format, kv_format, has_router_bias=0, rms_eps=1e-6, rope_base=10000.0,
                abi_version=MK_ABI_VERSION, q_lora_rank=0, kv_norm=0, idx_heads=0, idx_dim=0, idx_topk=0,
                idx_max_rows=0, kv_max_rows=0) -> LayerConfig:
    fm = lambda f: FORMATS[f] if isinstance(f, str) else int(f)
    return LayerConfig(abi_version, d_model, n_heads, d_head, d_latent, d_rope, n_experts, top_k, n_shared, d_ff,
                       fm(attn_format), fm(expert_format), fm(kv_format), int(has_router_bias), rms_eps, rope_base,
                       int(q_lora_rank), int(kv_norm), int(idx_heads), int(idx_dim), int(idx_topk), int(idx_max_rows),
                       int(kv_max_rows))


def check_config(cfg: LayerConfig) -> None:
    _chk(lib.mk_check_config(ctypes.byref(cfg)))


def _size_out(fn, *args) -> int:
    out = _sz(0)
    _chk(fn(*args, ctypes.byref(out)))
    return out.value


def packed_bytes(cfg: LayerConfig, tensor: int) -> int:
    return _size_out(lib.mk_packed_bytes, ctypes.byref(cfg), tensor)


def kv_bytes(cfg: LayerConfig, capacity: int) -> int:
    return _size_out(lib.mk_kv_bytes, ctypes.byref(cfg), capacity)


def layer_state_bytes(cfg: LayerConfig, hip_device: int = 0) -> int:
    return _size_out(lib.mk_layer_state_bytes, ctypes.byref(cfg), hip_device)


def layer_workspace_bytes(cfg: LayerConfig, hip_device: int = 0) -> int:
    return _size_out(lib.mk_layer_workspace_bytes, ctypes.byref(cfg), hip_device)


def pack_tensor(cfg: LayerConfig, tensor: int, src: int, dst: int, stream: int = 0) -> None:
    _chk(lib.mk_pack_tensor(ctypes.byref(cfg), tensor, src, dst, stream))


def pack_expert(cfg: LayerConfig, w1: int, w3: int, w2: int, s1, s3, s2, dst: int, stream: int = 0) -> None:
    _chk(lib.mk_pack_expert(ctypes.byref(cfg), w1, w3, w2, s1, s3, s2, dst, stream))


class Layer:
    """Owns an mk_layer handle (device buffers stay owned by the caller)."""

    def __init__(self, cfg: LayerConfig, weights: LayerWeights, expert_ptrs, state: int, workspace: int,
                 hip_device: int = 0):
        self.cfg = cfg
        self._experts = (ctypes.c_void_p * len(expert_ptrs))(*expert_ptrs)
        weights.experts = ctypes.cast(self._experts, _vp)
        self._weights = weights
        h = _vp()
        _chk(lib.mk_layer_init(ctypes.byref(cfg), ctypes.byref(weights), state, workspace, hip_device,
                               ctypes.byref(h)))
        self.handle = h

    def decode_step(self, hidden_in: int, T: int, kv_rows: int, capacity: int, length: int, hidden_out: int,
                    stream: int = 0) -> None:
        kv = KvCache(kv_rows, capacity, length)
        _chk(lib.mk_decode_step(self.handle, hidden_in, T, ctypes.byref(kv), hidden_out, stream))

    def decode_step_static(self, hidden_in: int, T: int, kv_rows: int, capacity: int, length: int,
                           hidden_out: int, stream: int = 0) -> None:
        kv = KvCache(kv_rows, capacity, length)
        _chk(lib.mk_decode_step_static(self.handle, hidden_in, T, ctypes.byref(kv), hidden_out, stream))

    def debug_tap(self, tap: int, host_buf, stream: int = 0) -> None:
        _chk(lib.mk_debug_tap(self.handle, tap, host_buf.ctypes.data, host_buf.nbytes, stream))

    def stats(self) -> Stats:
        s = Stats()
        _chk(lib.mk_get_stats(self.handle, ctypes.byref(s)))
        return s

    def set_trace(self, enabled: bool) -> None:
        _chk(lib.mk_set_trace(self.handle, 1 if enabled else 0))

    def read_trace(self, host_buf, stream: int = 0) -> None:
        _chk(lib.mk_read_trace(self.handle, host_buf.ctypes.data, host_buf.nbytes, stream))

    def set_barrier_timeout_us(self, us: int) -> None:
        _chk(lib.mk_set_barrier_timeout_us(self.handle, us))

    def sync_status(self) -> int:
        return lib.mk_sync_status(self.handle)

    def reset(self) -> None:
        _chk(lib.mk_layer_reset(self.handle))

    def destroy(self) -> None:
        if self.handle:
            lib.mk_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def head_packed_bytes(vocab: int, d_model: int, fmt=MK_FMT_BF16) -> int:
    return _size_out(lib.mk_head_packed_bytes_fmt, vocab, d_model, FORMATS[fmt] if isinstance(fmt, str) else fmt)


def pack_head_fp8(vocab: int, d_model: int, codes: int, scales: int, dst: int, stream: int = 0) -> None:
    _chk(lib.mk_pack_head_fp8(vocab, d_model, codes, scales, dst, stream))


def pack_head(vocab: int, d_model: int, src: int, dst: int, stream: int = 0) -> None:
    _chk(lib.mk_pack_head(vocab, d_model, src, dst, stream))


def model_state_bytes(n_layers: int, vocab: int, hip_device: int = 0) -> int:
    return _size_out(lib.mk_model_state_bytes, n_layers, vocab, hip_device)


class Model:
    def __init__(self, layers, embedding: int, head_packed: int, gamma_final: int, vocab: int, kv_rows,
                 capacity: int, state: int, hidden: int, head_fmt=MK_FMT_BF16):
        self.layers = list(layers)
        self._lh = (ctypes.c_void_p * len(layers))(*[l.handle.value for l in layers])
        self._kv = (ctypes.c_void_p * len(kv_rows))(*kv_rows)
        h = _vp()
        hf = FORMATS[head_fmt] if isinstance(head_fmt, str) else head_fmt
        _chk(lib.mk_model_init_ex(self._lh, len(layers), embedding, head_packed, hf, gamma_final, vocab, self._kv,
                                  capacity, state, hidden, ctypes.byref(h)))
        self.handle = h

    def set_sampling(self, temperature: float, seed: int) -> None:
        _chk(lib.mk_model_set_sampling(self.handle, temperature, seed))

    def set_length(self, length: int) -> None:
        _chk(lib.mk_model_set_length(self.handle, length))

    def length_ptr(self) -> int:
        return lib.mk_model_length_ptr(self.handle)

    def step(self, tokens: int, T: int, next_drafts, argmax: int, committed: int, logits=None,
             stream: int = 0) -> None:
        _chk(lib.mk_model_step(self.handle, tokens, T, next_drafts, argmax, committed, logits, stream))

    def sync_status(self) -> int:
        return lib.mk_model_sync_status(self.handle)

    def reset(self) -> None:
        _chk(lib.mk_model_reset(self.handle))

    def set_hidden_record(self, record_dev) -> None:
        _chk(lib.mk_model_set_hidden_record(self.handle, record_dev))

    def destroy(self) -> None:
        if self.handle:
            lib.mk_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
