"""Helpers shared by the GPU parity tests: run one layer step on the GPU through
the C ABI and the same step in the CPU oracle, then compare.

Comparison rules:
  - floating outputs: normwise error per row, max_j |y_j - r_j| / max_j |r_j|,
    taken separately on the attention branch (H' - H), the MoE branch
    (out - H'), the output and the new KV rows, each held to the bound of the
    weights it is computed from: 1e-4 for fp32, 2e-2 for bf16, 5e-2 for fp8
    and MXFP4 (both decoded exactly on both sides, as fp8 is: what differs is
    the bf16 rounding of the activations, as for fp8).
    The attention branch and the new KV rows come from the attention weights
    and the cache (attn_fmt, kv_fmt); the MoE branch from the experts
    (exp_fmt); the output from both, so it takes the looser of the two;
  - expert selection: identical sets except at near-ties, where the oracle's
    k-th and (k+1)-th logits are within 1e-3; there every GPU pick must be
    within 1e-3 of the oracle's k-th logit, and the oracle is re-run with the
    GPU's picks forced before the outputs are compared.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import recipe

TAU_SEL = 1e-3
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2, "mxfp4": 5e-2, "fp8row": 5e-2}


def _loosest(*fmts):
    return max(TOL[f] for f in fmts)


def tols_of(s):
    """Bound of each compared branch, from the formats of the weights it is computed from."""
    attn = _loosest(s.attn_fmt, s.kv_fmt)
    moe = _loosest(s.exp_fmt, s.attn_fmt)       # the router (attention-format weights) picks the experts
    return {"attn_branch": attn, "kv_new": attn, "moe_branch": moe, "out": max(attn, moe)}


def normwise(a, ref):
    a = np.asarray(a, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    den = np.abs(ref).max(axis=1)
    den[den == 0] = 1.0
    return float((np.abs(a - ref).max(axis=1) / den).max())


def kv_to_f32(kv_np, fmt, kvw=None):
    if fmt == "fp8row":
        return oracle.kv_decode(kv_np, fmt, kvw, kv_np.shape[0])
    return oracle.bf16_to_f32(kv_np.view(np.uint16)) if fmt == "bf16" else kv_np.astype(np.float32)


def fp8row_kv_check(g_codes, o_codes, kvw):
    """New fp8 cache rows of the GPU against the oracle's.  The two sides quantize
    rows whose values differ by bf16 rounding of the activations, so a code may
    land one E4M3 step away and a row's power-of-two scale may differ by a factor
    of two where its maximum sits at a boundary.  Asserts: every scale a power of
    two and the smallest that fits the row (its largest code value is at least
    224 = 448 / 2), scales equal to the oracle's up to that factor, zero padding,
    and every decoded element within one code step of the oracle's at the larger
    of the two scales plus the activation tolerance.  Returns the fraction of
    codes identical to the oracle's (rows with equal scales)."""
    g = oracle.kv_decode(g_codes, "fp8row", kvw, g_codes.shape[0]).astype(np.float64)
    o = oracle.kv_decode(o_codes, "fp8row", kvw, o_codes.shape[0]).astype(np.float64)
    gs = g_codes[:, kvw:kvw + 4].copy().view(np.float32).astype(np.float64)[:, 0]
    os_ = o_codes[:, kvw:kvw + 4].copy().view(np.float32).astype(np.float64)[:, 0]
    assert np.all(np.frexp(gs)[0] == 0.5), gs
    top = np.abs(g).max(axis=1) / gs
    assert np.all((top >= 224.0) & (top <= 448.0)), top
    ratio = gs / os_
    assert np.all((ratio == 1.0) | (ratio == 2.0) | (ratio == 0.5)), ratio
    assert np.all(g_codes[:, kvw + 4:] == 0) and np.all(o_codes[:, kvw + 4:] == 0)
    sc = np.maximum(gs, os_)[:, None]
    # E4M3 step at magnitude a (in units of the row scale): 2^(floor(log2 a) - 3), 2^-9 below 2^-6
    a = np.maximum(np.abs(o), np.abs(g)) / sc
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    act = TOL["bf16"] * np.abs(o).max(axis=1, keepdims=True)
    assert np.all(np.abs(g - o) <= step * sc + act), float((np.abs(g - o) - step * sc - act).max())
    same = ratio == 1.0
    return float((g_codes[same, :kvw] == o_codes[same, :kvw]).mean()) if same.any() else 0.0


def gpu_step(dl, s, H_dev, kv_dev, L, T=None):
    """Runs one step; returns (out, new KV rows as float32, taps dict)."""
    from decoder_megakernel_amd import MK_OK
    T = T or s.T
    out = torch.empty((T, s.d), dtype=torch.float32, device=H_dev.device)
    dl.step(H_dev, T, kv_dev, L, out)
    torch.cuda.synchronize()
    assert dl.layer.sync_status() == MK_OK
    taps = {}
    o_dt = np.float32 if s.attn_fmt == "f32" else np.uint16     # o is kept in the operand format
    for name, tap, shape, dt in (("Hp", 4, (T, s.d), np.float32), ("logits", 5, (T, s.E), np.float32),
                                 ("sel", 6, (T, s.top_k), np.int32), ("gate", 7, (T, s.top_k), np.float32),
                                 ("z", 2, (T, s.n_h, s.d_c), np.float32), ("qabs", 1, (T, s.n_h, s.d_c), np.float32),
                                 ("o", 3, (T, s.n_h * s.d_h), o_dt), ("q", 0, (T, s.n_h, s.qw), np.float32)):
        buf = np.empty(shape, dt)
        dl.layer.debug_tap(tap, buf)
        taps[name] = oracle.bf16_to_f32(buf) if dt == np.uint16 else buf
    if s.idx_topk:
        imax = (s.capacity + 7) // 8 * 8
        for name, tap, shape, dt in (("isel", 8, (T, s.idx_topk), np.int32), ("iscore", 9, (T, imax), np.float32)):
            buf = np.empty(shape, dt)
            dl.layer.debug_tap(tap, buf)
            taps[name] = buf
    kvn = kv_dev[L:L + T].cpu().numpy()
    taps["kv_raw"] = kvn
    return out.cpu().numpy(), kv_to_f32(kvn, s.kv_fmt, s.kv_row), taps


def oracle_step(s, seed, layer, H, L, kv_host=None, force_sel=None, full_weights=None, base_weights=None,
                expert_fn=None, force_isel=None):
    """Oracle layer step on the host copies of the same seeded inputs (kv_host
    is written in place).  force_isel: sparse attention's kept rows to use.
    Returns (out, new KV rows float32, taps, weights used)."""
    kv = recipe.kv_prefill_host(s, seed, layer) if kv_host is None else kv_host
    if force_isel is not None:
        if full_weights is not None:
            full_weights = dict(full_weights, force_isel=force_isel)
        else:
            base = base_weights if base_weights is not None else recipe.layer_weights_host(s, seed, layer, experts=[])
            base_weights = dict(base, force_isel=force_isel)
    if full_weights is not None:
        out, taps = oracle.layer_step(s, full_weights, H, kv, L, force_sel=force_sel)
        w = full_weights
    else:
        out, taps, w = oracle.layer_step_lazy(s, seed, layer, H, kv, L, base_weights=base_weights,
                                              force_sel=force_sel, expert_fn=expert_fn)
    taps["kv_raw"] = kv[L:L + H.shape[0]].copy()
    return out, kv_to_f32(kv[L:L + H.shape[0]], s.kv_fmt, s.kv_row), taps, w


def compare_selection(s, gpu_sel, ora_logits, ora_sel):
    """Returns (n_near_ties, needs_forced_rerun); asserts the selection rule."""
    T, k = gpu_sel.shape
    near = 0
    forced = False
    for i in range(T):
        lg = ora_logits[i].astype(np.float64)
        srt = np.sort(lg)[::-1]
        gap = srt[k - 1] - srt[k] if k < len(srt) else np.inf
        if gap > TAU_SEL:
            assert set(gpu_sel[i].tolist()) == set(ora_sel[i].tolist()), (i, gpu_sel[i], ora_sel[i])
        else:
            near += 1
            kth = srt[k - 1]
            for e in gpu_sel[i]:
                assert lg[e] >= kth - TAU_SEL, (i, e, lg[e], kth)
            if set(gpu_sel[i].tolist()) != set(ora_sel[i].tolist()):
                forced = True
    return near, forced


def compare_kept_rows(s, g_taps, o_taps, L):
    """Sparse attention: the GPU's index scores against the oracle's (bf16 index
    queries on the GPU: the bf16 bound; with an fp8 cache the new rows' index
    keys may round to neighbouring codes: the fp8 row bound), and its kept rows
    (ascending, the right count per row).  Where the kept sets differ, every row
    the GPU keeps and the oracle drops must score within that bound of the
    oracle's k-th score.  Returns (rows kept differently, whether the oracle
    must follow the GPU)."""
    K = s.idx_topk
    tol = _loosest("bf16", s.kv_fmt)
    near, forced = 0, False
    for t in range(g_taps["isel"].shape[0]):
        n = L + t + 1
        cnt = min(K, n)
        g = g_taps["isel"][t][:cnt].tolist()
        o = o_taps["isel"][t][:cnt].tolist()
        assert g == sorted(g) and len(set(g)) == cnt and 0 <= g[0] and g[-1] < n, (t, g[:8], g[-8:])
        # exact: the kept rows are the top-k of the GPU's own scores, ties to the lower row
        gs = g_taps["iscore"][t][:n].astype(np.float64)
        own = np.sort(np.lexsort((np.arange(n), -gs))[:cnt]).tolist()
        assert g == own, (t, sorted(set(g) ^ set(own))[:8])
        osc = o_taps["iscore"][t][:n].astype(np.float64)
        assert normwise(g_taps["iscore"][t:t + 1, :n], osc[None]) <= tol, t
        if set(g) != set(o):
            kth = np.sort(osc)[::-1][cnt - 1]
            band = tol * np.abs(osc).max()
            for r in set(g) - set(o):
                assert osc[r] >= kth - band, (t, r, osc[r], kth, band)
            near += len(set(g) - set(o))
            forced = True
    return near, forced


def check_layer(s, seed, layer, g_out, g_kv, g_taps, H, L, kv_host=None, full_weights=None, report=None,
                base_weights=None, expert_fn=None):
    """Full parity check of one step against the oracle.  Returns a dict of errors."""
    kw = dict(full_weights=full_weights, base_weights=base_weights, expert_fn=expert_fn)
    kv0 = None if kv_host is None else kv_host.copy()
    o_out, o_kv, o_taps, w = oracle_step(s, seed, layer, H, L, kv_host=kv_host, **kw)
    rows_near, rows_forced = 0, False
    if s.idx_topk:
        rows_near, rows_forced = compare_kept_rows(s, g_taps, o_taps, L)
        if rows_forced:
            kvh = recipe.kv_prefill_host(s, seed, layer) if kv0 is None else kv0.copy()
            kw["force_isel"] = g_taps["isel"]
            o_out, o_kv, o_taps, w = oracle_step(s, seed, layer, H, L, kv_host=kvh, **kw)
    near, forced = compare_selection(s, g_taps["sel"], o_taps["logits"], o_taps["sel"])
    if forced:
        kvh = recipe.kv_prefill_host(s, seed, layer) if kv0 is None else kv0.copy()
        o_out, o_kv, o_taps, w = oracle_step(s, seed, layer, H, L, kv_host=kvh, force_sel=g_taps["sel"], **kw)
    tols = tols_of(s)
    errs = {
        "attn_branch": normwise(g_taps["Hp"].astype(np.float64) - H, o_taps["Hp"].astype(np.float64) - H),
        "moe_branch": normwise(g_out.astype(np.float64) - g_taps["Hp"], o_out.astype(np.float64) - o_taps["Hp"]),
        "out": normwise(g_out, o_out),
        "kv_new": normwise(g_kv, o_kv),
        "near_ties": near,
        "forced": bool(forced),
    }
    if s.idx_topk:
        errs["kept_rows_differing"] = rows_near
        errs["kept_rows_forced"] = bool(rows_forced)
    if report is not None:
        report.update(errs)
    if s.kv_fmt == "fp8row":
        # rows are compared code by code (fp8row_kv_check) where the GPU's raw rows are at hand
        if "kv_raw" in g_taps:
            errs["kv_new_same_codes"] = fp8row_kv_check(g_taps["kv_raw"], o_taps["kv_raw"], s.kv_row)
        checked = ("attn_branch", "moe_branch", "out")
    else:
        checked = ("attn_branch", "moe_branch", "out", "kv_new")
    for k in checked:
        assert errs[k] <= tols[k], (k, errs, tols)
    return errs
