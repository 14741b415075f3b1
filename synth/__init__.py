"""Seeded synthetic inputs shared by the CPU oracle side and the GPU side.

This package only draws numbers and encodes them into storage formats (fp32,
bf16, OCP fp8 E4M3 with 128x128 block scales, OCP MXFP4 with E8M0 scales per
32 elements); it holds none of the decoder
layer's arithmetic.  The generator definition is written out in ``synth.h``.
Two builds implement it: ``libmksynth_host.so`` (C, OpenMP) and
``libmksynth_dev.so`` (HIP); a GPU test checks that they agree bit for bit.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libmksynth_host.so")
DEV_LIB = os.path.join(_HERE, "libmksynth_dev.so")

_u64 = ctypes.c_uint64
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float


def build(verbose: bool = False) -> None:
    """Compile both generator builds in place (gcc for the host, hipcc for gfx950)."""
    host = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
            os.path.join(_HERE, "synth_host.c"), "-o", HOST_LIB, "-lm"]
    dev = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "synth_dev.hip"), "-o", DEV_LIB]
    for cmd in (host, dev):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), r.stderr))
        if verbose and r.stderr:
            print(r.stderr)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build()
        lib = ctypes.CDLL(HOST_LIB)
        lib.mks_host_raw.restype = _u64
        lib.mks_host_raw.argtypes = [_u64, _u64, _u64]
        lib.mks_host_raw_fill.argtypes = [_vp, _u64, _u64, _u64, _u64]
        lib.mks_host_normal_f32.argtypes = [_vp, _u64, _u64, _u64, _u64, _f32, _f32]
        lib.mks_host_normal_bf16.argtypes = [_vp, _u64, _u64, _u64, _u64, _f32, _f32]
        lib.mks_host_fp8_blocks.argtypes = [_vp, _vp, _i64, _i64, _u64, _u64, _f32]
        lib.mks_host_e4m3_encode.restype = ctypes.c_uint8
        lib.mks_host_e4m3_encode.argtypes = [_f32]
        lib.mks_host_e2m1_encode.restype = ctypes.c_uint8
        lib.mks_host_e2m1_encode.argtypes = [_f32]
        lib.mks_host_mxfp4_blocks.argtypes = [_vp, _vp, _i64, _i64, _u64, _u64, _f32]
        lib.mks_host_fp8row_kv.argtypes = [_vp, _i64, _i64, _i64, _u64, _u64, _u64, _f32]
        lib.mks_host_bf16_encode.restype = ctypes.c_uint16
        lib.mks_host_bf16_encode.argtypes = [_f32]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError("libmksynth_dev.so is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEV_LIB)
        lib.mks_dev_raw_fill.argtypes = [_vp, _u64, _u64, _u64, _u64, _vp]
        lib.mks_dev_normal_f32.argtypes = [_vp, _u64, _u64, _u64, _u64, _f32, _f32, _vp]
        lib.mks_dev_normal_bf16.argtypes = [_vp, _u64, _u64, _u64, _u64, _f32, _f32, _vp]
        lib.mks_dev_fp8_blocks.argtypes = [_vp, _vp, _i64, _i64, _u64, _u64, _f32, _vp]
        lib.mks_dev_mxfp4_blocks.argtypes = [_vp, _vp, _i64, _i64, _u64, _u64, _f32, _vp]
        lib.mks_dev_fp8row_kv.argtypes = [_vp, _i64, _i64, _i64, _u64, _u64, _u64, _f32, _vp]
        for f in (lib.mks_dev_raw_fill, lib.mks_dev_normal_f32, lib.mks_dev_normal_bf16,
                  lib.mks_dev_fp8_blocks, lib.mks_dev_mxfp4_blocks, lib.mks_dev_fp8row_kv):
            f.restype = ctypes.c_int
        _dev = lib
    return _dev


# ---------------------------------------------------------------- constants
def sigma_c(sigma: float) -> float:
    """The fp32 multiplier c that turns an Irwin-Hall(4) integer into N(0, sigma)-like values."""
    return float(np.float32(sigma * math.sqrt(3.0) / 65536.0))


# Stream ids: tag in the top 16 bits, layer in the next 16, index in the low 32.
TAGS = {
    "H": 1, "kv_prefill": 2, "gamma1": 3, "gamma2": 4, "wq": 5, "wdkv": 6, "wuk": 7,
    "wuv": 8, "wo": 9, "wr": 10, "w1": 11, "w3": 12, "w2": 13, "emb": 14, "head": 15,
    "gamma_f": 16, "tokens": 17, "hot_perm": 18, "kv_scale": 19, "wdq": 20, "wuq": 21, "gamma_q": 22,
    "gamma_kv": 23, "widx": 24,
}


def stream_id(tag: str, layer: int = 0, index: int = 0) -> int:
    return (TAGS[tag] << 48) | ((layer & 0xFFFF) << 32) | (index & 0xFFFFFFFF)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------- host draws
def raw(n: int, seed: int, stream: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _host_lib().mks_host_raw_fill(_ptr(out), n, seed, stream, offset)
    return out


def normal_f32(shape, seed: int, stream: int, sigma: float, mean: float = 0.0,
               offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _host_lib().mks_host_normal_f32(_ptr(out), out.size, seed, stream, offset,
                                    sigma_c(sigma), float(np.float32(mean)))
    return out


def normal_bf16(shape, seed: int, stream: int, sigma: float, mean: float = 0.0,
                offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16)."""
    out = np.empty(shape, dtype=np.uint16)
    _host_lib().mks_host_normal_bf16(_ptr(out), out.size, seed, stream, offset,
                                     sigma_c(sigma), float(np.float32(mean)))
    return out


def fp8_blocks(R: int, K: int, seed: int, stream: int, sigma: float):
    """(codes uint8 [R][K], scales float32 [ceil(R/128)][ceil(K/128)])."""
    codes = np.empty((R, K), dtype=np.uint8)
    scales = np.empty(((R + 127) // 128, (K + 127) // 128), dtype=np.float32)
    _host_lib().mks_host_fp8_blocks(_ptr(codes), _ptr(scales), R, K, seed, stream, sigma_c(sigma))
    return codes, scales


def mxfp4_blocks(R: int, K: int, seed: int, stream: int, sigma: float):
    """(codes uint8 [R][K/2], two E2M1 codes per byte; E8M0 scale codes uint8 [R][K/32])."""
    if K % 32:
        raise ValueError("MXFP4 rows must be a multiple of 32 long")
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 32), dtype=np.uint8)
    _host_lib().mks_host_mxfp4_blocks(_ptr(codes), _ptr(scales), R, K, seed, stream, sigma_c(sigma))
    return codes, scales


def fp8row_kv(rows: int, kvw: int, row_bytes: int, seed: int, stream: int, scale_stream: int,
              sigma: float) -> np.ndarray:
    """uint8 [rows][row_bytes]: per row kvw E4M3 codes, the fp32 scale, zero padding."""
    out = np.empty((rows, row_bytes), dtype=np.uint8)
    if rows:
        _host_lib().mks_host_fp8row_kv(_ptr(out), rows, kvw, row_bytes, seed, stream, scale_stream,
                                       sigma_c(sigma))
    return out


def e2m1_encode(x: float) -> int:
    return int(_host_lib().mks_host_e2m1_encode(float(x)))


def e4m3_encode(x: float) -> int:
    return int(_host_lib().mks_host_e4m3_encode(float(x)))


def bf16_encode(x: float) -> int:
    return int(_host_lib().mks_host_bf16_encode(float(x)))


def uniform_ints(n: int, modulus: int, seed: int, stream: int) -> np.ndarray:
    return (raw(n, seed, stream) % np.uint64(modulus)).astype(np.int64)


def permutation(n: int, seed: int, stream: int) -> np.ndarray:
    """Fisher-Yates shuffle of range(n) driven by raw(); j = r mod (i+1)."""
    r = raw(n, seed, stream)
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int(r[i] % np.uint64(i + 1))
        p[i], p[j] = p[j], p[i]
    return p


# ---------------------------------------------------------------- device draws
def _chk(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("%s failed with HIP error %d" % (what, rc))


def dev_raw(dst_ptr: int, n: int, seed: int, stream: int, offset: int = 0, hip_stream: int = 0):
    _chk(_dev_lib().mks_dev_raw_fill(dst_ptr, n, seed, stream, offset, hip_stream), "mks_dev_raw_fill")


def dev_normal_f32(dst_ptr: int, n: int, seed: int, stream: int, sigma: float, mean: float = 0.0,
                   offset: int = 0, hip_stream: int = 0):
    _chk(_dev_lib().mks_dev_normal_f32(dst_ptr, n, seed, stream, offset, sigma_c(sigma),
                                       float(np.float32(mean)), hip_stream), "mks_dev_normal_f32")


def dev_normal_bf16(dst_ptr: int, n: int, seed: int, stream: int, sigma: float, mean: float = 0.0,
                    offset: int = 0, hip_stream: int = 0):
    _chk(_dev_lib().mks_dev_normal_bf16(dst_ptr, n, seed, stream, offset, sigma_c(sigma),
                                        float(np.float32(mean)), hip_stream), "mks_dev_normal_bf16")


def dev_mxfp4_blocks(codes_ptr: int, scales_ptr: int, R: int, K: int, seed: int, stream: int,
                     sigma: float, hip_stream: int = 0):
    _chk(_dev_lib().mks_dev_mxfp4_blocks(codes_ptr, scales_ptr, R, K, seed, stream, sigma_c(sigma),
                                         hip_stream), "mks_dev_mxfp4_blocks")


def dev_fp8row_kv(dst_ptr: int, rows: int, kvw: int, row_bytes: int, seed: int, stream: int,
                  scale_stream: int, sigma: float, hip_stream: int = 0):
    _chk(_dev_lib().mks_dev_fp8row_kv(dst_ptr, rows, kvw, row_bytes, seed, stream, scale_stream,
                                      sigma_c(sigma), hip_stream), "mks_dev_fp8row_kv")


def dev_fp8_blocks(codes_ptr: int, scales_ptr: int, R: int, K: int, seed: int, stream: int,
                   sigma: float, hip_stream: int = 0):
    _chk(_dev_lib().mks_dev_fp8_blocks(codes_ptr, scales_ptr, R, K, seed, stream, sigma_c(sigma),
                                       hip_stream), "mks_dev_fp8_blocks")
