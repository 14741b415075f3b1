"""Helpers of the stack parity tests: one GPU verify step of a stack of layers
(embedding, layers, final norm + LM head + argmax + greedy acceptance) against
the CPU oracle, in two ways.

Per layer, teacher-forced on the GPU's own state: layer l's oracle step is fed
the GPU's input rows of that layer (kept by mk_model_set_hidden_record) and
the GPU's cache rows [0, L), and its output, its new KV rows and its expert
selection are compared with the GPU's by the single-layer rules of parity.py
(selection identical unless the oracle's k-th and (k+1)-th logits are within
TAU_SEL).  The head is compared the same way on the GPU's final rows.

Free-running: the oracle composes the layers on its own hidden rows and its
own caches, as the stack runs from the embedding of the tokens.  Its inputs
drift from the GPU's by what the earlier layers' rounding accumulated, so a
selection (or argmax) that differs is judged by a band derived from the drift
actually measured at that point: if both sides rank the same candidates by
logits that differ by at most delta, every candidate one side selects lies
within 2 delta of the other side's k-th largest (plus TAU_SEL for the rounding
of the comparison itself).  Where a selection differs, the oracle follows the
GPU's (teacher forcing), and where an argmax differs, the oracle continues
from the GPU's committed tokens.  Near-ties and forcings are counted and
printed.
"""
from __future__ import annotations

from collections import OrderedDict

import numpy as np
import torch

import oracle
import parity
import synth
from synth import recipe

TAU_SEL = parity.TAU_SEL


class DeviceExpertDraws:
    """Canonical expert tensors drawn by the seeded generator's device build and
    copied to host memory.  The device and host builds give identical bits
    (tests/test_gpu_generator.py), so these are the oracle's own inputs drawn
    faster; nothing here comes from the layer kernels.  Least-recently-used
    cache of `cap` experts, keyed by (expert pool, slot)."""

    def __init__(self, s, seed=0, cap=512):
        self.s, self.seed, self.cap = s, seed, cap
        self.cache = OrderedDict()
        es = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 1}[s.exp_fmt]
        self.buf = torch.empty(s.f * s.d * es, dtype=torch.uint8, device="cuda")
        nsc = max(((s.f + 127) // 128) * ((s.d + 127) // 128) * 4, s.f * s.d // 32)
        self.sbuf = torch.empty(nsc, dtype=torch.uint8, device="cuda")

    def _draw(self, tag, R, K, lay, slot):
        s = self.s
        st = synth.stream_id(tag, lay, slot)
        n = R * K
        if s.exp_fmt == "mxfp4":
            synth.dev_mxfp4_blocks(self.buf.data_ptr(), self.sbuf.data_ptr(), R, K, self.seed, st, recipe.W_SIGMA)
            torch.cuda.synchronize()
            q = self.buf[:n // 2].cpu().numpy().reshape(R, K // 2)
            sc = self.sbuf[:n // 32].cpu().numpy().reshape(R, K // 32)
            return q, sc
        if s.exp_fmt == "fp8":
            synth.dev_fp8_blocks(self.buf.data_ptr(), self.sbuf.data_ptr(), R, K, self.seed, st, recipe.W_SIGMA)
            torch.cuda.synchronize()
            nsc = ((R + 127) // 128) * ((K + 127) // 128)
            q = self.buf[:n].cpu().numpy().reshape(R, K)
            sc = self.sbuf[:4 * nsc].cpu().numpy().view(np.float32).reshape((R + 127) // 128, (K + 127) // 128)
            return q, sc
        if s.exp_fmt == "bf16":
            synth.dev_normal_bf16(self.buf.data_ptr(), n, self.seed, st, recipe.W_SIGMA)
            torch.cuda.synchronize()
            return self.buf[:2 * n].cpu().numpy().view(np.uint16).reshape(R, K), None
        synth.dev_normal_f32(self.buf.data_ptr(), n, self.seed, st, recipe.W_SIGMA)
        torch.cuda.synchronize()
        return self.buf[:4 * n].cpu().numpy().view(np.float32).reshape(R, K), None

    def __call__(self, layer, slot):
        s = self.s
        lay = recipe.expert_pool_layer(s, layer) if slot < s.E else layer
        key = (lay, slot)
        if key in self.cache:
            self.cache.move_to_end(key)
            return self.cache[key]
        ws, ss = [], []
        for tag, (R, K) in (("w1", (s.f, s.d)), ("w3", (s.f, s.d)), ("w2", (s.d, s.f))):
            w, sc = self._draw(tag, R, K, lay, slot)
            ws.append(w)
            ss.append(sc)
        val = (ws[0], ws[1], ws[2], ss[0], ss[1], ss[2])
        self.cache[key] = val
        while len(self.cache) > self.cap:
            self.cache.popitem(last=False)
        return val


def read_i32(dev_ptr):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    out = ctypes.c_int32(0)
    rc = hip.hipMemcpy(ctypes.byref(out), ctypes.c_void_p(dev_ptr), ctypes.c_size_t(4), ctypes.c_int(2))
    assert rc == 0
    return out.value


def attach_record(st, s):
    """Keeps every layer's input rows of a step on the device."""
    rec = torch.zeros((len(st.layers) + 1, 8, s.d), dtype=torch.float32, device="cuda")
    st.model.set_hidden_record(rec.data_ptr())
    return rec


def gpu_step(st, s, rec, tokens, next_drafts=None):
    """One GPU stack step; returns everything the comparisons use."""
    from decoder_megakernel_amd import MK_OK
    dev = torch.device("cuda")
    L = read_i32(st.model.length_ptr())
    tok = torch.from_numpy(np.asarray(tokens, np.int32)).to(dev)
    am = torch.empty(s.T, dtype=torch.int32, device=dev)
    com = torch.zeros(s.T + 1, dtype=torch.int32, device=dev)
    lg = torch.empty((s.T, s.V), dtype=torch.float32, device=dev)
    nd = None if next_drafts is None else torch.from_numpy(np.asarray(next_drafts, np.int32)).to(dev)
    st.model.step(tok.data_ptr(), s.T, None if nd is None else nd.data_ptr(), am.data_ptr(), com.data_ptr(),
                  lg.data_ptr())
    torch.cuda.synchronize()
    assert st.model.sync_status() == MK_OK
    g = {"L": L, "am": am.cpu().numpy(), "com": com.cpu().numpy(), "logits": lg.cpu().numpy(),
         "len": read_i32(st.model.length_ptr()), "tok": tok.cpu().numpy(),
         "hidden": rec[:, : s.T].cpu().numpy().astype(np.float32),
         "sel": [], "rlogits": [], "Hp": [], "kv_new": [], "kv_raw": []}
    for l, dl in enumerate(st.layers):
        assert dl.layer.sync_status() == MK_OK
        sel = np.empty((s.T, s.top_k), np.int32)
        dl.layer.debug_tap(6, sel)
        rl = np.empty((s.T, s.E), np.float32)
        dl.layer.debug_tap(5, rl)
        hp = np.empty((s.T, s.d), np.float32)
        dl.layer.debug_tap(4, hp)
        g["sel"].append(sel)
        g["rlogits"].append(rl)
        g["Hp"].append(hp)
        if s.idx_topk:
            # sparse attention: the layer's kept rows and index scores
            isel = np.empty((s.T, s.idx_topk), np.int32)
            dl.layer.debug_tap(8, isel)
            isc = np.empty((s.T, (s.capacity + 7) // 8 * 8), np.float32)
            dl.layer.debug_tap(9, isc)
            g.setdefault("isel", []).append(isel)
            g.setdefault("iscore", []).append(isc)
        raw = st.kv[l][L:L + s.T].cpu().numpy()
        g["kv_raw"].append(raw)
        g["kv_new"].append(parity.kv_to_f32(raw, s.kv_fmt, s.kv_row))
    return g


def gpu_cache_host(st, s, l, L):
    """Host copy of the GPU's cache rows [0, L) of layer l (rows past L zero)."""
    rows = s.capacity if s.capacity > L + s.T else L + s.T
    if s.kv_fmt == "fp8row":
        kv = np.zeros((rows, recipe.kv_row_bytes(s)), np.uint8)
    else:
        kv = np.zeros((rows, s.kv_row), np.uint16 if s.kv_fmt == "bf16" else np.float32)
    src = st.kv[l][:L].cpu().numpy()
    kv[:L] = src.view(np.uint16) if s.kv_fmt == "bf16" else src
    return kv


def check_layers_teacher_forced(st, s, ws, g, expert_fn=None, seed=0, layers=None, tag=""):
    """Every layer's oracle step on the GPU's input rows and cache rows."""
    L = g["L"]
    out = []
    for l in (range(len(st.layers)) if layers is None else layers):
        H = g["hidden"][l]
        kvh = gpu_cache_host(st, s, l, L)
        taps = {"Hp": g["Hp"][l], "sel": g["sel"][l], "kv_raw": g["kv_raw"][l]}
        if s.idx_topk:
            taps.update(isel=g["isel"][l], iscore=g["iscore"][l])
        kw = dict(full_weights=ws[l]) if "experts" in ws[l] and ws[l]["experts"] else \
            dict(base_weights=ws[l], expert_fn=expert_fn)
        errs = parity.check_layer(s, seed, l, g["hidden"][l + 1], g["kv_new"][l], taps, H, L, kv_host=kvh, **kw)
        print("[stack%s] layer %d teacher-forced: %s" % (tag, l, {k: (round(v, 6) if isinstance(v, float) else v)
                                                               for k, v in errs.items()}), flush=True)
        out.append(errs)
    return out


def oracle_head(s, tables, h):
    """The oracle's head (bf16 or fp8 table) on hidden rows h: (logits, argmax)."""
    _, head, gf = tables
    if s.head_fmt == "fp8":
        return oracle.head_fp8(head[0], head[1], gf, h, s.eps)
    return oracle.head(head, gf, h, s.eps)


def check_head_teacher_forced(s, tables, g, tag="", argmax=True):
    """The oracle's head on the GPU's final rows: logits, and the argmax rule
    (argmax=False for a sampled step, whose argmax output holds the draws)."""
    o_lg, o_am = oracle_head(s, tables, g["hidden"][-1])
    err = parity.normwise(g["logits"], o_lg)
    near = 0
    for i in range(s.T if argmax else 0):
        if g["am"][i] != o_am[i]:
            lg = o_lg[i].astype(np.float64)
            assert lg[g["am"][i]] >= lg[o_am[i]] - TAU_SEL, (i, g["am"][i], o_am[i])
            near += 1
    print("[stack%s] head teacher-forced: logits normwise %.3e, argmax near-ties %d" % (tag, err, near), flush=True)
    assert err <= parity.TOL["fp8" if s.head_fmt == "fp8" else "bf16"], err
    return err, near


def oracle_stack_step(s, ws, tables, kvs, tokens, L, g=None, expert_fn=None, seed=0, tag=""):
    """Free-running oracle step of the stack on its own rows and caches (kvs is
    written in place).  With g (the GPU's step), a layer whose GPU selection
    differs is checked against the drift band and then follows the GPU's."""
    emb, head, gf = tables
    h = oracle.embed(emb, tokens)
    forced = near = 0
    drift = []
    for l, w in enumerate(ws):
        kw = dict(expert_fn=expert_fn, base_weights=w) if not w.get("experts") else {}
        if kw:
            out, taps, _ = oracle.layer_step_lazy(s, seed, l, h, kvs[l], L, **kw)
        else:
            out, taps = oracle.layer_step(s, w, h, kvs[l], L)
        if g is not None:
            gs = g["sel"][l]
            d = float(np.abs(g["rlogits"][l].astype(np.float64) - taps["logits"]).max())
            drift.append(d)
            diff = False
            for t in range(s.T):
                if set(gs[t].tolist()) == set(taps["sel"][t].tolist()):
                    continue
                lg = taps["logits"][t].astype(np.float64)
                kth = np.sort(lg)[::-1][s.top_k - 1]
                for e in gs[t]:
                    assert lg[e] >= kth - 2 * d - TAU_SEL, (l, t, int(e), lg[e], kth, d)
                diff = True
                near += 1
            if diff:
                forced += 1
                if kw:
                    out, taps, _ = oracle.layer_step_lazy(s, seed, l, h, kvs[l], L, force_sel=gs, **kw)
                else:
                    out, taps = oracle.layer_step(s, w, h, kvs[l], L, force_sel=gs)
        h = out
    logits, am = oracle_head(s, tables, h)
    if g is not None:
        print("[stack%s] free-running: router-logit drift max %.3e (last layer %.3e), tokens with a differing "
              "selection %d, layers forced %d" % (tag, max(drift), drift[-1], near, forced), flush=True)
    return logits, am, h


def compare_free_running(s, g, o_lg, o_am, tokens, tag=""):
    """Logits (normwise), argmax (rule with the measured drift) and the committed
    tokens.  Returns the tokens the GPU committed (the oracle continues from them)."""
    err = parity.normwise(g["logits"], o_lg)
    d = float(np.abs(g["logits"].astype(np.float64) - o_lg).max())
    near = 0
    for i in range(s.T):
        if g["am"][i] != o_am[i]:
            lg = o_lg[i].astype(np.float64)
            assert lg[g["am"][i]] >= lg[o_am[i]] - 2 * d - TAU_SEL, (i, g["am"][i], o_am[i], d)
            near += 1
    n = int(g["com"][0])
    g_com = list(g["com"][1:1 + n])
    assert g_com == list(oracle.greedy_accept(tokens, g["am"]))        # the GPU follows its own argmax
    o_com = list(oracle.greedy_accept(tokens, o_am))
    print("[stack%s] logits normwise %.3e (max abs diff %.3e), argmax gpu %s oracle %s, near-ties %d, commit gpu %s "
          "oracle %s" % (tag, err, d, g["am"].tolist(), o_am.tolist(), near, g_com, o_com), flush=True)
    assert err <= parity.TOL["fp8"], err
    if near == 0:
        assert g_com == o_com
    return g_com


def check_sampled_verification(s, g, tokens, tau, key, tag=""):
    """The GPU's sampled verification against the oracle's, both on the GPU's
    own logits (so that only the verification is compared; the logits are
    checked by check_head_teacher_forced).  A row's token draw may differ only
    where the oracle's two perturbed values are within 1e-4 of each other, and
    an acceptance decision only where the draw is within 1e-5 of p_i(draft);
    without such a near-tie the committed tokens, the count, the KV length and
    the next t0 must be identical.  Returns the number of committed tokens."""
    lg = g["logits"].astype(np.float32)
    o_smp, o_com = oracle.verify_sampled(lg, tokens, tau, key)
    T, V = lg.shape
    near = 0
    for i in range(T):
        if g["am"][i] != o_smp[i]:
            u = np.array([oracle.sample_uniform(key, i * (V + 1) + v) for v in (g["am"][i], o_smp[i])], np.float64)
            y = lg[i, [g["am"][i], o_smp[i]]].astype(np.float64) / tau - np.log(-np.log(u))
            assert abs(y[0] - y[1]) <= 1e-4 * max(1.0, abs(y[1])), (i, g["am"][i], o_smp[i], y)
            near += 1
    for i in range(T - 1):
        x = lg[i].astype(np.float64) / tau
        p = np.exp(x[tokens[i + 1]] - x.max()) / np.exp(x - x.max()).sum()
        ua = oracle.sample_uniform(key, i * (V + 1) + V)
        if abs(ua - p) < 1e-5:
            near += 1
    n = int(g["com"][0])
    gcom = list(g["com"][1:1 + n])
    print("[stack%s] sampled verification (tau %g): gpu %s oracle %s, near-ties %d"
          % (tag, tau, gcom, list(o_com), near), flush=True)
    if near == 0:
        assert gcom == list(o_com)
        assert list(g["am"]) == list(o_smp)
    assert g["len"] == g["L"] + n and g["tok"][0] == gcom[-1]
    for j in range(1, n):
        assert gcom[j - 1] == tokens[j]
    return n
