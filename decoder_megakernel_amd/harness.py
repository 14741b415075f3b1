"""Device-side set-up used by the tests and the benchmark: draws the seeded
synthetic weights straight into GPU memory (synth's device generator), packs
them through the C ABI and initialises layers.  PyTorch only provides device
memory and streams here; nothing of the layer's arithmetic runs in Python.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import synth
from synth import recipe
from synth.configs import LayerShape

from . import (FORMATS, MK_T_EXPERT, MK_T_WDKV, MK_T_WDQ, MK_T_WIDX, MK_T_WO, MK_T_WQ, MK_T_WR, MK_T_WUK, MK_T_WUQ,
               MK_T_WUV, Layer,
               LayerWeights, Model, head_packed_bytes, kv_bytes, layer_state_bytes, layer_workspace_bytes,
               make_config, model_state_bytes, pack_expert, pack_head, pack_head_fp8, pack_tensor, packed_bytes)


def config_of(s: LayerShape):
    return make_config(s.d, s.n_h, s.d_h, s.d_c, s.d_r, s.E, s.top_k, s.n_shared, s.f, s.attn_fmt, s.exp_fmt,
                       s.kv_fmt, has_router_bias=1 if s.routing == "skew" else 0, rms_eps=s.eps,
                       rope_base=s.rope_base, q_lora_rank=s.q_lora, kv_norm=1 if s.kv_norm else 0,
                       idx_heads=s.idx_heads, idx_dim=s.idx_dim, idx_topk=s.idx_topk,
                       idx_max_rows=(s.capacity + 7) // 8 * 8 if s.idx_topk else 0, kv_max_rows=s.capacity)


def _dev(device):
    return torch.device("cuda", device)


def _bytes(n, device):
    return torch.empty(int(n), dtype=torch.uint8, device=_dev(device))


def _gen_attn_tensor(s: LayerShape, name, shape, seed, layer, device):
    n = int(np.prod(shape))
    st = synth.stream_id(name, layer)
    if s.attn_fmt == "f32":
        t = torch.empty(n, dtype=torch.float32, device=_dev(device))
        synth.dev_normal_f32(t.data_ptr(), n, seed, st, recipe.W_SIGMA)
    else:
        t = torch.empty(n, dtype=torch.int16, device=_dev(device))
        synth.dev_normal_bf16(t.data_ptr(), n, seed, st, recipe.W_SIGMA)
    return t


class ExpertStager:
    """Reusable canonical buffers for drawing one expert at a time on the device."""

    def __init__(self, s: LayerShape, device):
        self.s = s
        self.device = device
        n = s.f * s.d
        if s.exp_fmt == "mxfp4":
            # codes [R][K/2] (two per byte) and E8M0 scale bytes [R][K/32]
            self.w = [_bytes(n // 2, device) for _ in range(3)]
            self.sc = [_bytes(n // 32, device) for _ in range(3)]
            return
        es = {"f32": 4, "bf16": 2, "fp8": 1}[s.exp_fmt]
        self.w = [_bytes(n * es, device) for _ in range(3)]
        nsc = ((s.f + 127) // 128) * ((s.d + 127) // 128)
        self.sc = [torch.empty(nsc, dtype=torch.float32, device=_dev(device)) for _ in range(3)]

    def draw_and_pack(self, cfg, seed, layer, slot, dst_ptr):
        s = self.s
        lay = recipe.expert_pool_layer(s, layer) if slot < s.E else layer
        dims = ((s.f, s.d), (s.f, s.d), (s.d, s.f))
        for i, (tag, (R, K)) in enumerate(zip(("w1", "w3", "w2"), dims)):
            st = synth.stream_id(tag, lay, slot)
            if s.exp_fmt == "mxfp4":
                synth.dev_mxfp4_blocks(self.w[i].data_ptr(), self.sc[i].data_ptr(), R, K, seed, st, recipe.W_SIGMA)
            elif s.exp_fmt == "fp8":
                synth.dev_fp8_blocks(self.w[i].data_ptr(), self.sc[i].data_ptr(), R, K, seed, st, recipe.W_SIGMA)
            elif s.exp_fmt == "bf16":
                synth.dev_normal_bf16(self.w[i].data_ptr(), R * K, seed, st, recipe.W_SIGMA)
            else:
                synth.dev_normal_f32(self.w[i].data_ptr(), R * K, seed, st, recipe.W_SIGMA)
        scp = [t.data_ptr() for t in self.sc] if s.exp_fmt in ("fp8", "mxfp4") else [None, None, None]
        pack_expert(cfg, self.w[0].data_ptr(), self.w[1].data_ptr(), self.w[2].data_ptr(), scp[0], scp[1], scp[2],
                    dst_ptr)


class ExpertPool:
    """Packed blocks of the routed experts of one pool (all E of them)."""

    def __init__(self, s: LayerShape, seed: int, pool_layer: int, device=0, stager=None):
        cfg = config_of(s)
        self.block = packed_bytes(cfg, MK_T_EXPERT)
        self.buf = _bytes(self.block * s.E, device)
        stager = stager or ExpertStager(s, device)
        for e in range(s.E):
            stager.draw_and_pack(cfg, seed, pool_layer, e, self.buf.data_ptr() + e * self.block)
        self.ptrs = [self.buf.data_ptr() + e * self.block for e in range(s.E)]


class DeviceLayer:
    """One layer's packed weights, state and handle on the GPU."""

    def __init__(self, s: LayerShape, seed: int = 0, layer: int = 0, device: int = 0, workspace=None,
                 pool: ExpertPool | None = None, stager: ExpertStager | None = None):
        self.s = s
        self.cfg = config_of(s)
        self.device = device
        cfg = self.cfg
        self.packed = {}
        shapes = recipe.attn_shapes(s)
        for name, tid in (("wq", MK_T_WQ), ("wdq", MK_T_WDQ), ("wuq", MK_T_WUQ), ("widx", MK_T_WIDX),
                          ("wdkv", MK_T_WDKV), ("wuk", MK_T_WUK), ("wuv", MK_T_WUV), ("wo", MK_T_WO), ("wr", MK_T_WR)):
            if name not in shapes:
                continue
            src = _gen_attn_tensor(s, name, shapes[name], seed, layer, device)
            dst = _bytes(packed_bytes(cfg, tid), device)
            pack_tensor(cfg, tid, src.data_ptr(), dst.data_ptr())
            self.packed[name] = dst
        self.g1 = torch.empty(s.d, dtype=torch.float32, device=_dev(device))
        self.g2 = torch.empty(s.d, dtype=torch.float32, device=_dev(device))
        synth.dev_normal_f32(self.g1.data_ptr(), s.d, seed, synth.stream_id("gamma1", layer), recipe.GAIN_SIGMA, 1.0)
        synth.dev_normal_f32(self.g2.data_ptr(), s.d, seed, synth.stream_id("gamma2", layer), recipe.GAIN_SIGMA, 1.0)
        self.gq = self.gkv = None
        if s.q_lora:
            self.gq = torch.empty(s.q_lora, dtype=torch.float32, device=_dev(device))
            synth.dev_normal_f32(self.gq.data_ptr(), s.q_lora, seed, synth.stream_id("gamma_q", layer),
                                 recipe.GAIN_SIGMA, 1.0)
        if s.kv_norm:
            self.gkv = torch.empty(s.d_c, dtype=torch.float32, device=_dev(device))
            synth.dev_normal_f32(self.gkv.data_ptr(), s.d_c, seed, synth.stream_id("gamma_kv", layer),
                                 recipe.GAIN_SIGMA, 1.0)
        rb = recipe.router_bias(s, seed, layer)
        self.rbias = None if rb is None else torch.from_numpy(rb).to(_dev(device))
        block = packed_bytes(cfg, MK_T_EXPERT)
        stager = stager or ExpertStager(s, device)
        if pool is None:
            self.pool_buf = _bytes(block * (s.E + s.n_shared), device)
            for e in range(s.E + s.n_shared):
                stager.draw_and_pack(cfg, seed, layer, e, self.pool_buf.data_ptr() + e * block)
            ptrs = [self.pool_buf.data_ptr() + e * block for e in range(s.E + s.n_shared)]
        else:
            self.pool = pool
            self.shared_buf = _bytes(block * s.n_shared, device)
            for i in range(s.n_shared):
                stager.draw_and_pack(cfg, seed, layer, s.E + i, self.shared_buf.data_ptr() + i * block)
            ptrs = list(pool.ptrs) + [self.shared_buf.data_ptr() + i * block for i in range(s.n_shared)]
        self.expert_ptrs = ptrs
        self.state = _bytes(layer_state_bytes(cfg, device), device)
        self.workspace = workspace if workspace is not None else _bytes(layer_workspace_bytes(cfg, device), device)
        torch.cuda.synchronize(_dev(device))
        ptr = lambda k: self.packed[k].data_ptr() if k in self.packed else None
        w = LayerWeights(self.g1.data_ptr(), self.g2.data_ptr(), ptr("wq"),
                         self.packed["wdkv"].data_ptr(), self.packed["wuk"].data_ptr(),
                         self.packed["wuv"].data_ptr(), self.packed["wo"].data_ptr(), self.packed["wr"].data_ptr(),
                         None if self.rbias is None else self.rbias.data_ptr(), None,
                         ptr("wdq"), ptr("wuq"), None if self.gq is None else self.gq.data_ptr(),
                         None if self.gkv is None else self.gkv.data_ptr(), ptr("widx"))
        self.layer = Layer(cfg, w, ptrs, self.state.data_ptr(), self.workspace.data_ptr(), device)

    def step(self, hin: torch.Tensor, T: int, kv: torch.Tensor, length: int, hout: torch.Tensor, stream: int = 0):
        cap = kv.shape[0]
        self.layer.decode_step(hin.data_ptr(), T, kv.data_ptr(), cap, length, hout.data_ptr(), stream)


def kv_cache(s: LayerShape, seed: int = 0, layer: int = 0, device: int = 0, capacity: int | None = None):
    """KV rows [capacity][kvw] (fp8 rows: uint8 [capacity][row bytes]); rows [0, L)
    drawn as synth.recipe.kv_prefill_host draws them."""
    cap = capacity or s.capacity
    n = s.L * s.kv_row
    st = synth.stream_id("kv_prefill", layer)
    if s.kv_fmt == "fp8row":
        rb = recipe.kv_row_bytes(s)
        kv = torch.zeros((cap, rb), dtype=torch.uint8, device=_dev(device))
        if s.L:
            synth.dev_fp8row_kv(kv.data_ptr(), s.L, s.kv_row, rb, seed, st, synth.stream_id("kv_scale", layer),
                                recipe.ACT_SIGMA)
        return kv
    if s.kv_fmt == "f32":
        kv = torch.zeros((cap, s.kv_row), dtype=torch.float32, device=_dev(device))
        if n:
            synth.dev_normal_f32(kv.data_ptr(), n, seed, st, recipe.ACT_SIGMA)
    else:
        kv = torch.zeros((cap, s.kv_row), dtype=torch.int16, device=_dev(device))
        if n:
            synth.dev_normal_bf16(kv.data_ptr(), n, seed, st, recipe.ACT_SIGMA)
    return kv


def hidden(s: LayerShape, seed: int = 0, layer: int = 0, step: int = 0, device: int = 0):
    t = torch.empty((s.T, s.d), dtype=torch.float32, device=_dev(device))
    synth.dev_normal_f32(t.data_ptr(), s.T * s.d, seed, synth.stream_id("H", layer, step), recipe.ACT_SIGMA)
    return t


class DeviceStack:
    """A stack of layers (expert pools shared as the shape says) plus embedding and LM head."""

    def __init__(self, s: LayerShape, seed: int = 0, device: int = 0, n_layers: int | None = None,
                 capacity: int | None = None, private_workspaces: bool = False):
        """private_workspaces: one workspace per layer (so every layer's debug
        taps survive a model step) instead of one shared by all layers."""
        self.s = s
        n_layers = n_layers or s.n_layers
        cfg = config_of(s)
        self.cfg = cfg
        dev = _dev(device)
        self.workspace = _bytes(layer_workspace_bytes(cfg, device), device)
        stager = ExpertStager(s, device)
        self.pools = {}
        self.layers = []
        for l in range(n_layers):
            pool = None
            if s.n_pools:
                pl = recipe.expert_pool_layer(s, l)
                if pl not in self.pools:
                    self.pools[pl] = ExpertPool(s, seed, pl, device, stager)
                pool = self.pools[pl]
            ws = None if private_workspaces else self.workspace
            self.layers.append(DeviceLayer(s, seed, l, device, workspace=ws, pool=pool, stager=stager))
        V, d = s.V, s.d
        self.emb = torch.empty((V, d), dtype=torch.int16, device=dev)
        synth.dev_normal_bf16(self.emb.data_ptr(), V * d, seed, synth.stream_id("emb"), recipe.W_SIGMA)
        self.head = _bytes(head_packed_bytes(V, d, s.head_fmt), device)
        if s.head_fmt == "fp8":
            # E4M3 codes with 128x128 block scales, drawn as the fp8 experts are
            codes = torch.empty((V, d), dtype=torch.uint8, device=dev)
            scales = torch.empty(((V + 127) // 128) * ((d + 127) // 128), dtype=torch.float32, device=dev)
            synth.dev_fp8_blocks(codes.data_ptr(), scales.data_ptr(), V, d, seed, synth.stream_id("head"),
                                 recipe.W_SIGMA)
            pack_head_fp8(V, d, codes.data_ptr(), scales.data_ptr(), self.head.data_ptr())
            torch.cuda.synchronize(dev)
            del codes, scales
        else:
            head_src = torch.empty((V, d), dtype=torch.int16, device=dev)
            synth.dev_normal_bf16(head_src.data_ptr(), V * d, seed, synth.stream_id("head"), recipe.W_SIGMA)
            pack_head(V, d, head_src.data_ptr(), self.head.data_ptr())
            del head_src
        self.gf = torch.empty(d, dtype=torch.float32, device=dev)
        synth.dev_normal_f32(self.gf.data_ptr(), d, seed, synth.stream_id("gamma_f"), recipe.GAIN_SIGMA, 1.0)
        self.capacity = capacity or s.capacity
        self.kv = [kv_cache(s, seed, l, device, self.capacity) for l in range(n_layers)]
        self.state = _bytes(model_state_bytes(n_layers, V, device), device)
        self.hidden = torch.empty((2, 8, d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize(dev)
        self.model = Model([dl.layer for dl in self.layers], self.emb.data_ptr(), self.head.data_ptr(),
                           self.gf.data_ptr(), V, [k.data_ptr() for k in self.kv], self.capacity,
                           self.state.data_ptr(), self.hidden.data_ptr(), head_fmt=s.head_fmt)
        self.model.set_length(s.L)
