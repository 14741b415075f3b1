"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks the oracle against a closed form, an invariant, a special case
that reduces to a textbook or library routine, the fp64 un-absorbed brute force,
or a published format table, chosen so that a plausible slip (a dropped term, a
wrong sign or index, a transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth import recipe
from synth.configs import C0, C1, LayerShape

GOLD = os.path.join(os.path.dirname(__file__), "golden")

# A small bf16/fp8 shape with several 128x128 scale blocks and ragged edges.
C0Q = LayerShape("micro_fp8", d=256, n_h=2, d_h=32, d_c=64, d_r=16, E=6, top_k=2, n_shared=1,
                 f=160, T=3, L=7, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16")


def normwise(a, ref):
    a = np.asarray(a, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    return (np.abs(a - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()


def fresh(s, seed=0):
    w = recipe.layer_weights_host(s, seed, 0)
    H = recipe.hidden_host(s, seed)
    kv = recipe.kv_prefill_host(s, seed)
    return w, H, kv


# ---------------------------------------------------------------- formats
def test_e4m3_decode_matches_ocp_table():
    g = json.load(open(os.path.join(GOLD, "ocp_e4m3_values.json")))
    L = oracle.lib()
    for code, val in g["values"].items():
        assert L.orc_e4m3_to_f32(int(code, 16)) == val, code
    for code in g["nan_codes"]:
        assert math.isnan(L.orc_e4m3_to_f32(int(code, 16)))


def test_e4m3_encoder_inverts_decoder_on_all_codes():
    """Generator encoder (synth) against the oracle's decoder: two implementations."""
    L = oracle.lib()
    for q in range(256):
        if q in (0x7F, 0xFF):
            continue
        v = L.orc_e4m3_to_f32(q)
        back = synth.e4m3_encode(v)
        if q == 0x80:          # -0 encodes with its sign
            assert back == 0x80
            continue
        assert back == q, (hex(q), v, hex(back))


def test_e4m3_encoder_rounding_and_saturation():
    L = oracle.lib()
    vals = sorted({L.orc_e4m3_to_f32(q) for q in range(0x7F) if q != 0x7F})
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = (lo + hi) / 2.0
        got = L.orc_e4m3_to_f32(synth.e4m3_encode(np.float32(mid)))
        qlo, qhi = synth.e4m3_encode(lo), synth.e4m3_encode(hi)
        want = lo if (qlo % 2 == 0) else hi            # ties to the even code
        assert got == want, (lo, hi, got)
        assert L.orc_e4m3_to_f32(synth.e4m3_encode(np.nextafter(np.float32(mid), np.float32(0)))) == lo
    assert synth.e4m3_encode(1e6) == 0x7E and synth.e4m3_encode(-500.0) == 0xFE
    assert synth.e4m3_encode(460.0) == 0x7E


def test_bf16_round_to_nearest_even():
    g = json.load(open(os.path.join(GOLD, "bf16_values.json")))
    L = oracle.lib()
    for e in g["encode"]:
        f = np.array([int(e["f32_bits"], 16)], np.uint32).view(np.float32)[0]
        assert L.orc_f32_to_bf16(float(f)) == int(e["bf16"], 16), e
        assert synth.bf16_encode(float(f)) == int(e["bf16"], 16), e
    # every finite bf16 value survives widen -> round
    for b in range(0, 0x10000, 7):
        if (b & 0x7F80) == 0x7F80:
            continue
        assert L.orc_f32_to_bf16(L.orc_bf16_to_f32(b)) == b


# ---------------------------------------------------------------- generator
def test_generator_moments_and_determinism():
    x = synth.normal_f32(1 << 20, 0, synth.stream_id("wq"), 0.02)
    assert abs(x.mean()) < 0.02 * 0.01
    assert abs(x.std() / 0.02 - 1.0) < 0.01
    assert np.array_equal(x, synth.normal_f32(1 << 20, 0, synth.stream_id("wq"), 0.02))
    y = synth.normal_f32(1 << 10, 0, synth.stream_id("wq", 0, 1), 0.02)
    assert not np.array_equal(x[: 1 << 10], y)
    # Irwin-Hall(4) is bounded by 2*sqrt(3) standard deviations
    assert np.abs(x).max() <= 2 * math.sqrt(3) * 0.02 * 1.0001
    # offset addressing is counter-based
    assert np.array_equal(x[100:200], synth.normal_f32(100, 0, synth.stream_id("wq"), 0.02, offset=100))


def test_generator_gain_mean():
    g = synth.normal_f32(1 << 16, 0, synth.stream_id("gamma1"), 0.1, mean=1.0)
    assert abs(g.mean() - 1.0) < 2e-3 and abs(g.std() - 0.1) < 2e-3


def test_fp8_blocks_dequantise_to_the_drawn_values():
    R, K = 300, 200
    q, s = synth.fp8_blocks(R, K, 0, synth.stream_id("w1"), 0.02)
    w = synth.normal_f32((R, K), 0, synth.stream_id("w1"), 0.02)
    L = oracle.lib()
    lut = np.array([L.orc_e4m3_to_f32(i) for i in range(256)], np.float32)
    deq = lut[q] * np.repeat(np.repeat(s, 128, 0), 128, 1)[:R, :K]
    # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 for normals
    big = np.abs(w) > 2 ** -6 * np.repeat(np.repeat(s, 128, 0), 128, 1)[:R, :K]
    assert np.all(np.abs(deq - w)[big] <= np.abs(w)[big] * 2 ** -4 + 1e-12)
    # the block maximum maps to +-448 exactly
    for br in range(s.shape[0]):
        for bk in range(s.shape[1]):
            blk = q[br * 128:(br + 1) * 128, bk * 128:(bk + 1) * 128]
            assert np.abs(lut[blk]).max() == 448.0


# ---------------------------------------------------------------- whole layer vs fp64 brute force
@pytest.mark.parametrize("shape", [C0, C1, C0Q], ids=lambda s: s.name)
def test_layer_matches_fp64_unabsorbed_bruteforce(shape):
    w, H, kv = fresh(shape)
    kv64 = kv.copy()
    out, taps = oracle.layer_step(shape, w, H, kv, shape.L)
    ref = oracle.layer_step_f64(shape, w, H, kv64, shape.L, force_sel=taps["sel"])
    assert normwise(out, ref["out"]) < 1e-5
    # the attention branch Hp - H is ~1% of H: fp32 rounding of Hp (half an ulp of
    # |H| <= 4, i.e. 2.4e-7) over a branch of ~1e-2 bounds this near 3e-5
    assert normwise(taps["Hp"].astype(np.float64) - H, ref["Hp"] - H) < 1e-4
    kvn = oracle.bf16_to_f32(kv[shape.L:shape.L + shape.T]) if shape.kv_fmt == "bf16" else kv[shape.L:shape.L + shape.T]
    # new rows: storage rounding may flip one bf16 ulp between fp32 and fp64 paths
    tol = 1e-5 if shape.kv_fmt == "f32" else 2 ** -7
    assert normwise(kvn, ref["kv_new"]) < tol
    # unforced fp64 selection agrees away from near-ties
    lg = ref["logits"]
    srt = -np.sort(-lg, axis=1)
    gap = srt[:, shape.top_k - 1] - srt[:, shape.top_k]
    for i in range(shape.T):
        if gap[i] > 1e-4:
            assert set(taps["sel"][i]) == set(np.argsort(-lg[i], kind="stable")[: shape.top_k])


# ---------------------------------------------------------------- causal invariant
@pytest.mark.parametrize("shape", [C0, C0Q], ids=lambda s: s.name)
def test_verify_rows_equal_sequential_single_token_steps_bitwise(shape):
    w, H, kv = fresh(shape)
    kv_seq = kv.copy()
    out, _ = oracle.layer_step(shape, w, H, kv, shape.L)
    one = shape.with_(T=1)
    outs = []
    for i in range(shape.T):
        o, _ = oracle.layer_step(one, w, H[i:i + 1], kv_seq, shape.L + i)
        outs.append(o)
    assert np.array_equal(out, np.concatenate(outs))
    assert np.array_equal(kv, kv_seq)


def test_later_rows_do_not_change_earlier_outputs():
    """Row i only sees cache rows <= L+i: perturbing row T-1's input leaves rows < T-1 alone."""
    s = C0
    w, H, kv = fresh(s)
    out1, _ = oracle.layer_step(s, w, H, kv.copy(), s.L)
    H2 = H.copy()
    H2[-1] += 1.0
    out2, _ = oracle.layer_step(s, w, H2, kv.copy(), s.L)
    assert np.array_equal(out1[:-1], out2[:-1])
    assert not np.array_equal(out1[-1], out2[-1])


# ---------------------------------------------------------------- attention special cases
def test_empty_cache_single_token_attends_to_its_own_row():
    s = C0.with_(T=1, L=0)
    w, H, kv = fresh(s)
    _, taps = oracle.layer_step(s, w, H, kv, 0)
    own = kv[0, : s.d_c]
    for h in range(s.n_h):
        assert np.array_equal(taps["z"][0, h], own)


def test_zero_query_gives_mean_of_latents():
    s = C0
    w, H, kv = fresh(s)
    w["wq"] = np.zeros_like(w["wq"])
    _, taps = oracle.layer_step(s, w, H, kv, s.L)
    for i in range(s.T):
        mean = kv[: s.L + i + 1, : s.d_c].astype(np.float64).mean(axis=0)
        for h in range(s.n_h):
            assert np.allclose(taps["z"][i, h], mean, rtol=0, atol=1e-6)


def test_absorbed_query_is_wuk_transpose_times_qc():
    s = C0
    w, H, kv = fresh(s)
    _, taps = oracle.layer_step(s, w, H, kv, s.L)
    for h in range(s.n_h):
        qc = taps["q"][:, h, : s.d_h].astype(np.float64)
        ref = qc @ w["wuk"][h].astype(np.float64)            # [T][d_c]
        assert np.allclose(taps["qabs"][:, h], ref, atol=1e-5)


# ---------------------------------------------------------------- norm / rope
def test_rmsnorm_constant_vector_closed_form():
    s = C0.with_(T=1, L=0)
    w, _, kv = fresh(s)
    a = -3.0
    H = np.full((1, s.d), a, np.float32)
    _, taps = oracle.layer_step(s, w, H, kv, 0)
    want = np.sign(a) * abs(a) / math.sqrt(a * a + s.eps) * w["gamma1"].astype(np.float64)
    assert np.allclose(taps["x"][0], want, rtol=2e-7, atol=0)


def test_rmsnorm_scale_invariance():
    s = C0.with_(T=1, L=0)
    w, H, kv = fresh(s)
    _, t1 = oracle.layer_step(s, w, H, kv.copy(), 0)
    _, t2 = oracle.layer_step(s, w, H * 8.0, kv.copy(), 0)   # power of two: exact scaling
    assert np.allclose(t1["x"], t2["x"], rtol=1e-6, atol=1e-7)


def test_rope_position_zero_is_identity_and_rotation_sign():
    s = C0.with_(T=2, L=0)
    w, H, kv = fresh(s)
    _, taps = oracle.layer_step(s, w, H, kv, 0)
    wd = w["wdkv"].astype(np.float64)
    for i, pos in enumerate((0, 1)):
        kr = wd[s.d_c:] @ taps["x"][i].astype(np.float64)      # pre-rotation key
        got = taps["ckv"][i, s.d_c:].astype(np.float64)
        # pair norms are preserved
        assert np.allclose(np.hypot(got[0::2], got[1::2]), np.hypot(kr[0::2], kr[1::2]), rtol=1e-5)
        # pair 0 has theta = 1: rotation by `pos` radians, counter-clockwise
        c, sn = math.cos(pos), math.sin(pos)
        assert np.allclose(got[:2], [kr[0] * c - kr[1] * sn, kr[0] * sn + kr[1] * c], atol=1e-5)
        if pos == 0:
            assert np.allclose(got, kr, atol=1e-5)


def test_rope_is_relative_same_token_inner_product_invariant_to_offset():
    s = C0.with_(T=1, L=0)
    w, H, kv = fresh(s)
    s2 = s.with_(L=1000, kv_capacity=1001)
    kv2 = np.zeros((1001, s.kvw), np.float32)
    _, t1 = oracle.layer_step(s, w, H, kv, 0)
    _, t2 = oracle.layer_step(s2, w, H, kv2, 1000)
    for h in range(s.n_h):
        ip1 = np.dot(t1["q"][0, h, s.d_h:].astype(np.float64), t1["ckv"][0, s.d_c:].astype(np.float64))
        ip2 = np.dot(t2["q"][0, h, s.d_h:].astype(np.float64), t2["ckv"][0, s.d_c:].astype(np.float64))
        assert abs(ip1 - ip2) < 1e-4 * (1 + abs(ip1))


# ---------------------------------------------------------------- router
@pytest.mark.parametrize("shape", [C1, C0Q], ids=lambda s: s.name)
def test_router_topk_set_and_gates(shape):
    w, H, kv = fresh(shape)
    _, taps = oracle.layer_step(shape, w, H, kv, shape.L)
    lg = taps["logits"].astype(np.float64)
    for i in range(shape.T):
        order = np.argsort(-lg[i], kind="stable")
        assert list(taps["sel"][i]) == list(order[: shape.top_k])
        g = taps["gate"][i].astype(np.float64)
        assert abs(g.sum() - 1.0) < 1e-6 and np.all(g > 0)
        assert np.all(np.diff(g) <= 0)                      # ordered like the logits
        p = np.exp(lg[i] - lg[i].max())
        p /= p.sum()
        ref = p[taps["sel"][i]] / p[taps["sel"][i]].sum()  # softmax then renormalise
        assert np.allclose(g, ref, rtol=1e-5)


def test_router_ties_go_to_lower_index():
    s = C0.with_(T=1, L=0)
    w, H, kv = fresh(s)
    w["wr"] = np.tile(w["wr"][:1], (s.E, 1))                # all logits equal
    _, taps = oracle.layer_step(s, w, H, kv, 0)
    assert list(taps["sel"][0]) == list(range(s.top_k))
    assert np.allclose(taps["gate"][0], 1.0 / s.top_k)


def test_router_bias_enters_selection():
    s = C0.with_(T=1, L=0)
    w, H, kv = fresh(s)
    w["router_bias"] = np.zeros(s.E, np.float32)
    w["router_bias"][s.E - 1] = 1e3
    _, taps = oracle.layer_step(s, w, H, kv, 0)
    assert taps["sel"][0][0] == s.E - 1
    assert taps["logits"][0][s.E - 1] > 900


# ---------------------------------------------------------------- MoE special cases
def test_single_expert_reduces_to_dense_swiglu_ffn():
    s = C0.with_(E=1, top_k=1, n_shared=0, T=2)
    w, H, kv = fresh(s)
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    w1, w3, w2 = (a.astype(np.float64) for a in w["experts"][0][:3])
    xp = taps["xp"].astype(np.float64)
    a = xp @ w1.T
    ffn = ((a / (1 + np.exp(-a))) * (xp @ w3.T)) @ w2.T
    assert np.allclose(taps["gate"], 1.0)
    assert np.allclose(out, taps["Hp"].astype(np.float64) + ffn, atol=1e-5)


def test_zero_down_projection_leaves_residual():
    s = C0
    w, H, kv = fresh(s)
    for e, t in w["experts"].items():
        w["experts"][e] = (t[0], t[1], np.zeros_like(t[2])) + t[3:]
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    assert np.array_equal(out, taps["Hp"])
    w["wo"] = np.zeros_like(w["wo"])
    out2, _ = oracle.layer_step(s, w, H, recipe.kv_prefill_host(s), s.L)
    assert np.array_equal(out2, H)


def test_fp8_block_scale_indexing_against_explicit_dense_matrix():
    """Codes all 1.0 and a distinct power-of-two scale per 128x128 block: the
    dequantised matrix is the block-constant scale map, known exactly."""
    s = C0Q.with_(E=1, top_k=1, n_shared=0, T=1, L=0)
    w, H, kv = fresh(s)
    one = 0x38
    mats = []
    tup = []
    for R, K in ((s.f, s.d), (s.f, s.d), (s.d, s.f)):
        nbr, nbk = (R + 127) // 128, (K + 127) // 128
        sc = np.array([[2.0 ** (-(i * nbk + j) - 6) for j in range(nbk)] for i in range(nbr)], np.float32)
        tup.append((np.full((R, K), one, np.uint8), sc))
        mats.append(np.repeat(np.repeat(sc.astype(np.float64), 128, 0), 128, 1)[:R, :K])
    w["experts"] = {0: (tup[0][0], tup[1][0], tup[2][0], tup[0][1], tup[1][1], tup[2][1])}
    out, taps = oracle.layer_step(s, w, H, kv, 0)
    xp = taps["xp"].astype(np.float64)
    a = xp @ mats[0].T
    ffn = ((a / (1 + np.exp(-a))) * (xp @ mats[1].T)) @ mats[2].T
    assert np.allclose(out - taps["Hp"], ffn, rtol=1e-5, atol=1e-9)


def test_forced_selection_equal_to_own_selection_is_identity():
    s = C0Q
    w, H, kv = fresh(s)
    out, taps = oracle.layer_step(s, w, H, kv.copy(), s.L)
    out2, _ = oracle.layer_step(s, w, H, kv.copy(), s.L, force_sel=taps["sel"])
    assert np.array_equal(out, out2)


# ---------------------------------------------------------------- stack pieces
def test_greedy_accept_cases():
    t = np.array([5, 7, 9, 11], np.int32)
    assert list(oracle.greedy_accept(t, [7, 9, 11, 13])) == [7, 9, 11, 13]     # all accepted
    assert list(oracle.greedy_accept(t, [1, 2, 3, 4])) == [1]                  # none
    assert list(oracle.greedy_accept(t, [7, 2, 11, 4])) == [7, 2]              # stops at first miss
    assert list(oracle.greedy_accept(t[:1], [8])) == [8]                       # T = 1


def test_head_argmax_ties_go_to_lower_id_and_embed_gathers_rows():
    V, d = 10, 64
    emb = synth.normal_bf16((V, d), 0, synth.stream_id("emb"), 0.02)
    head = np.tile(emb[3:4], (V, 1))
    gf = np.ones(d, np.float32)
    h = oracle.embed(emb, np.array([3, 3], np.int32))
    assert np.array_equal(h[0], oracle.bf16_to_f32(emb[3]))
    _, am = oracle.head(head, gf, h)
    assert list(am) == [0, 0]
    head2 = head.copy()
    head2[6] = emb[3] * 0 + synth.normal_bf16(d, 1, 1, 0.5)
    lg, am2 = oracle.head(head2, gf, h)
    assert am2[0] == int(np.argmax(lg[0]))


# ---------------------------------------------------------------- pins of the softmax scale, head norm/gain, biased gates
def test_two_key_softmax_scale_closed_form():
    """One verify row over two cache rows (the prefilled row 0 and its own row 1):
    z = p0 c0 + p1 c1 with p1 / p0 = exp((s1 - s0) / sqrt(d_h + d_r)), where
    s_j = q~ . c_j + q^R . k^R_j is computed here from the taps and the stored
    rows.  The ratio read back from z fixes the scale: 1/sqrt(d_h) (no RoPE
    dims in the scale) or no scale at all would be off by far more than the
    fp32 bound checked here."""
    s = C0.with_(T=1, L=1, kv_capacity=2)
    w, H, kv = fresh(s)
    _, taps = oracle.layer_step(s, w, H, kv, s.L)
    rows = kv.astype(np.float64)
    c0, c1 = rows[0, : s.d_c], rows[1, : s.d_c]
    k0, k1 = rows[0, s.d_c:], rows[1, s.d_c:]
    dc = c1 - c0
    for h in range(s.n_h):
        qa = taps["qabs"][0, h].astype(np.float64)
        qr = taps["q"][0, h, s.d_h:].astype(np.float64)
        ds = qa @ (c1 - c0) + qr @ (k1 - k0)
        z = taps["z"][0, h].astype(np.float64)
        p1 = (z - c0) @ dc / (dc @ dc)                      # z lies on the segment c0 -> c1
        assert np.allclose(z, c0 + p1 * dc, atol=1e-6)
        ratio = p1 / (1.0 - p1)
        want = math.exp(ds / math.sqrt(s.d_h + s.d_r))
        assert abs(ratio / want - 1.0) < 1e-4, (h, ratio, want)
        # the scale is not 1/sqrt(d_h) alone, and not 1
        for wrong in (math.exp(ds / math.sqrt(s.d_h)), math.exp(ds)):
            assert abs(wrong / want - 1.0) > 1e-3


def _rms_rows(h, gamma, eps):
    h = np.asarray(h, np.float64)
    return h / np.sqrt((h * h).mean(axis=1, keepdims=True) + eps) * np.asarray(gamma, np.float64)


def test_head_final_norm_and_gain():
    """LM head logits = W_head (RMSNorm(h) * gamma_f) with a non-unit gain, in three ways
    that each fail for a dropped norm or gain: (1) against fp64 arithmetic of the
    definition, (2) invariance under a positive scale of h, (3) linearity in the gain."""
    V, d, T = 96, 256, 3
    head = synth.normal_bf16((V, d), 0, synth.stream_id("head"), 0.02)
    gf = synth.normal_f32(d, 0, synth.stream_id("gamma_f"), 0.1, mean=1.0)
    h = synth.normal_f32((T, d), 0, synth.stream_id("H"), 3.0)
    eps = 1e-6
    lg, am = oracle.head(head, gf, h, eps)
    ref = _rms_rows(h, gf, eps) @ oracle.bf16_to_f32(head).astype(np.float64).T
    assert normwise(lg, ref) < 1e-5
    assert list(am) == list(np.argmax(ref, axis=1))
    lg2, _ = oracle.head(head, gf, h * np.float32(0.25), eps)      # exact scaling of h
    assert np.allclose(lg2, lg, rtol=1e-5, atol=1e-6)
    lg3, _ = oracle.head(head, (gf * np.float32(2.0)).astype(np.float32), h, eps)
    assert np.allclose(lg3, 2.0 * lg, rtol=1e-6, atol=1e-7)
    # a unit gain gives a different answer (the gain is applied at all)
    lg1, _ = oracle.head(head, np.ones(d, np.float32), h, eps)
    assert normwise(lg1, ref) > 1e-2


def test_gates_under_router_bias_use_the_biased_logits():
    """With a router bias (the skewed-routing workload) the logits tap is the
    unbiased logits plus the bias, and the gates are the softmax of the biased
    logits renormalised over the selection; a softmax of the unbiased logits
    would fail here."""
    s = C0Q.with_(E=16, top_k=4, T=3)
    w, H, kv = fresh(s)
    _, t0 = oracle.layer_step(s, w, H, kv.copy(), s.L)
    b = synth.normal_f32(s.E, 0, synth.stream_id("hot_perm"), 1.0)
    wb = dict(w, router_bias=b)
    _, tb = oracle.layer_step(s, wb, H, kv.copy(), s.L)
    assert np.array_equal(tb["Hp"], t0["Hp"])
    lb = tb["logits"].astype(np.float64)
    assert np.allclose(lb - t0["logits"].astype(np.float64), b.astype(np.float64), atol=1e-6)
    changed = 0
    for i in range(s.T):
        order = np.argsort(-lb[i], kind="stable")
        assert list(tb["sel"][i]) == list(order[: s.top_k])
        sel = tb["sel"][i]
        e = np.exp(lb[i][sel] - lb[i][sel].max())
        assert np.allclose(tb["gate"][i], e / e.sum(), rtol=1e-5)
        lu = t0["logits"][i].astype(np.float64)[sel]
        eu = np.exp(lu - lu.max())
        changed += not np.allclose(tb["gate"][i], eu / eu.sum(), rtol=1e-3)
    assert changed == s.T


# ---------------------------------------------------------------- MXFP4 experts (OCP MX: E2M1 + E8M0 per 32)
C0X = LayerShape("micro_mxfp4", d=256, n_h=2, d_h=32, d_c=64, d_r=16, E=6, top_k=2, n_shared=1,
                 f=160, T=3, L=7, attn_fmt="bf16", exp_fmt="mxfp4", kv_fmt="bf16")


def test_e2m1_and_e8m0_decode_match_the_mx_definitions():
    g = json.load(open(os.path.join(GOLD, "ocp_mx_e2m1_values.json")))
    L = oracle.lib()
    for code, val in g["e2m1"].items():
        got = L.orc_e2m1_to_f32(int(code))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)
    for code, val in g["e8m0"].items():
        assert L.orc_e8m0_to_f32(int(code)) == np.float32(val), code
    for code in g["e8m0_nan"]:
        assert math.isnan(L.orc_e8m0_to_f32(code))


def test_e2m1_encoder_rounds_to_nearest_even_code_and_saturates():
    L = oracle.lib()
    vals = [L.orc_e2m1_to_f32(c) for c in range(8)]
    for c in range(16):
        v = L.orc_e2m1_to_f32(c)
        assert synth.e2m1_encode(v) == c, (c, v)                  # every code round-trips (-0 keeps its sign)
    for i in range(7):
        lo, hi = vals[i], vals[i + 1]
        mid = (lo + hi) / 2
        want = i if i % 2 == 0 else i + 1                          # the even code wins a tie
        assert synth.e2m1_encode(mid) == want and synth.e2m1_encode(-mid) == 8 | want
        assert synth.e2m1_encode(np.nextafter(np.float32(mid), np.float32(0))) == i
        assert synth.e2m1_encode(np.nextafter(np.float32(mid), np.float32(9))) == i + 1
    assert synth.e2m1_encode(7.9) == 7 and synth.e2m1_encode(-100.0) == 15


def _mx_decode(codes, scales):
    """Dense fp64 matrix of MXFP4 codes [R][K/2] and E8M0 scales [R][K/32], written from the MX definitions."""
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    lo, hi = codes & 15, codes >> 4
    el = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    el[:, 0::2], el[:, 1::2] = lo, hi
    v = mag[el & 7] * np.where(el & 8, -1.0, 1.0)
    return v * np.repeat(2.0 ** (scales.astype(np.float64) - 127.0), 32, axis=1)


def test_mxfp4_blocks_quantise_by_the_mx_recipe():
    R, K = 40, 256
    q, sc = synth.mxfp4_blocks(R, K, 0, synth.stream_id("w2"), 0.02)
    w = synth.normal_f32((R, K), 0, synth.stream_id("w2"), 0.02).astype(np.float64)
    amax = np.abs(w).reshape(R, K // 32, 32).max(axis=2)
    mant, ex = np.frexp(amax)                                  # amax = mant * 2^ex, mant in [0.5, 1)
    assert np.array_equal(sc.astype(np.int64), (ex - 1) - 2 + 127)
    deq = _mx_decode(q, sc)
    X = np.repeat(2.0 ** (sc.astype(np.float64) - 127.0), 32, axis=1)
    # each element is the nearest E2M1 value of w / X (saturating at 6): error <= half the local spacing
    x = np.abs(w) / X
    spacing = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    err = np.abs(deq - w) / X
    assert np.all((err <= spacing / 2 + 1e-12) | (x > 6))
    assert np.all(np.abs(deq)[x > 6] == 6 * X[x > 6])
    assert np.array_equal(np.sign(deq)[deq != 0], np.sign(w)[deq != 0])


def test_mxfp4_nibble_order_and_scale_indexing_against_an_explicit_dense_matrix():
    """Distinct low and high nibbles and a distinct power-of-two scale per (row, 32-group):
    the oracle's expert output equals a dense fp64 SwiGLU over the explicitly decoded matrices."""
    s = C0X.with_(E=1, top_k=1, n_shared=0, T=2, L=0)
    w, H, kv = fresh(s)
    tup, mats = [], []
    for i, (R, K) in enumerate(((s.f, s.d), (s.f, s.d), (s.d, s.f))):
        r = np.arange(R)[:, None]
        j = np.arange(K // 2)[None, :]
        codes = (((r + j + i) % 16) | ((((r * 3 + j + 5) % 16)) << 4)).astype(np.uint8)
        scales = (118 + (np.arange(R)[:, None] + 2 * np.arange(K // 32)[None, :] + i) % 7).astype(np.uint8)
        tup.append((codes, scales))
        mats.append(_mx_decode(codes, scales))
    w["experts"] = {0: (tup[0][0], tup[1][0], tup[2][0], tup[0][1], tup[1][1], tup[2][1])}
    out, taps = oracle.layer_step(s, w, H, kv, 0)
    xp = taps["xp"].astype(np.float64)
    a = xp @ mats[0].T
    ffn = ((a / (1 + np.exp(-a))) * (xp @ mats[1].T)) @ mats[2].T
    assert np.allclose(out - taps["Hp"], ffn, rtol=2e-5, atol=1e-7)


def test_mxfp4_layer_matches_fp64_unabsorbed_bruteforce():
    s = C0X
    w, H, kv = fresh(s)
    out, taps = oracle.layer_step(s, w, H, kv.copy(), s.L)
    ref = oracle.layer_step_f64(s, w, H, kv, s.L, force_sel=taps["sel"])
    assert normwise(out, ref["out"]) < 1e-5


# ---------------------------------------------------------------- fp8 (E4M3) KV cache rows
# "DeepSeek-V4.1-Flash breaks 1,000 tokens per second for one user", section
# "Appendix: method": the cache may be held in fp8 E4M3.  Reading taken: one
# power-of-two fp32 scale per row (the smallest that fits the row's maximum in
# E4M3's +-448), codes by round-to-nearest-even of value / scale.
C0K = C0Q.with_(name="micro_fp8kv", kv_fmt="fp8row", L=9)


def _ocp_e4m3_table():
    """All finite codes from the E4M3 bit layout (bias 7; exponent field 0 is
    subnormal, m/8 * 2^-6), checked against the values the OCP document prints."""
    t = {}
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        e, m = (c >> 3) & 15, c & 7
        v = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        t[c] = -v if c & 0x80 else v
    g = json.load(open(os.path.join(GOLD, "ocp_e4m3_values.json")))
    for c, v in g["values"].items():
        assert t[int(c, 16)] == v, c
    return t


def _nearest_e4m3_bruteforce(x, table):
    """Nearest code of the published table, ties to the even code, saturating at +-448."""
    x = float(x)
    if abs(x) >= 448.0:
        return 0xFE if x < 0 else 0x7E
    best = None
    for c, v in table.items():
        if (c & 0x80) != (0x80 if math.copysign(1.0, x) < 0 else 0):
            continue
        dd = abs(v - x)
        if best is None or dd < best[0] or (dd == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (dd, c)
    return best[1]


def test_fp8_row_encoder_is_the_nearest_table_code_ties_to_even():
    table = _ocp_e4m3_table()
    vals = sorted(v for c, v in table.items() if c < 0x7F)
    probes = [0.0, 447.9, 448.0, 500.0, 2.0 ** -10, 2.0 ** -9 * 0.5, 2.0 ** -9 * 1.5]
    probes += [(a + b) / 2 for a, b in zip(vals, vals[1:])]            # every tie
    probes += list(np.random.default_rng(3).standard_normal(400) * 50)
    for x in probes:
        for sx in (x, -x):
            got = oracle.f32_to_e4m3(np.float32(sx))
            want = _nearest_e4m3_bruteforce(np.float32(sx), table)
            if want in (0x00, 0x80) and got in (0x00, 0x80):
                continue                                                   # +-0
            assert got == want, (sx, hex(got), hex(want))
    assert oracle.f32_to_e4m3(float("nan")) == 0x7F


def test_fp8_row_scale_is_the_smallest_fitting_power_of_two():
    rng = np.random.default_rng(5)
    for k in range(300):
        row = (rng.standard_normal(40) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        if k % 50 == 0:
            row[:] = 0
            row[k % 40] = np.float32(448.0 * 2.0 ** rng.integers(-20, 20))   # a boundary: exactly 448 s
        s = oracle.fp8_row_scale(row)
        m, e = math.frexp(s)
        assert m == 0.5, s                                                 # a power of two
        amax = float(np.abs(row).max())
        assert amax <= 448.0 * s and amax > 448.0 * s / 2, (amax, s)
    assert oracle.fp8_row_scale(np.zeros(7, np.float32)) == 1.0


def test_fp8_row_layout_and_decode_against_the_table():
    kvw = 21
    rb = oracle.kv_row_bytes("fp8row", kvw)
    assert rb == 32 and oracle.kv_row_bytes("fp8row", 576) == 592
    assert oracle.kv_row_bytes("bf16", 576) == 1152 and oracle.kv_row_bytes("f32", 576) == 2304
    table = _ocp_e4m3_table()
    rng = np.random.default_rng(7)
    buf = np.zeros((5, rb), np.uint8)
    want = np.zeros((5, kvw), np.float64)
    for r in range(5):
        codes = rng.integers(0, 256, kvw)
        codes[codes == 0x7F] = 0x7E
        codes[codes == 0xFF] = 0xFE
        sc = np.float32(2.0 ** int(rng.integers(-12, 4)))
        buf[r, :kvw] = codes
        buf[r, kvw:kvw + 4] = np.frombuffer(sc.tobytes(), np.uint8)
        want[r] = [table[int(c)] * float(sc) for c in codes]
    assert np.array_equal(oracle.kv_decode(buf, "fp8row", kvw, 5).astype(np.float64), want)


# With sparse attention an fp8 row holds the latent, the RoPE key and the index
# key as one run of kvw + idx_dim codes under the row's one scale (reading: the
# pages give one fp8 cache and no separate index-key format).
C0KS = C0K.with_(name="micro_fp8kv_sparse", idx_heads=4, idx_dim=32, idx_topk=5, L=12)


@pytest.mark.parametrize("shape", [C0K, C0KS], ids=lambda s: s.name)
def test_fp8_prefill_rows_decode_to_the_drawn_values(shape):
    """The generator's fp8 rows against the same N(0,1) draws the bf16 cache holds:
    each element within half an E4M3 step (at the row's scale) of its draw."""
    s = shape.with_(L=40)
    rw = s.kv_row
    kv = recipe.kv_prefill_host(s, seed=2)
    draws = synth.normal_f32((s.L, rw), 2, synth.stream_id("kv_prefill", 0), recipe.ACT_SIGMA).astype(np.float64)
    dec = oracle.kv_decode(kv, "fp8row", rw, s.L).astype(np.float64)
    sc = kv[: s.L, rw:rw + 4].copy().view(np.float32).astype(np.float64)
    a = np.abs(draws) / sc
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(dec - draws) <= step * sc / 2 + 1e-12)
    assert set(np.log2(sc[:, 0]).astype(int)) <= {-6, -5, -4}
    assert np.all(kv[s.L:] == 0) and np.all(kv[: s.L, rw + 4:] == 0)


@pytest.mark.parametrize("shape", [C0K, C0KS], ids=lambda s: s.name)
def test_fp8_cache_new_rows_are_the_f32_rows_quantised_per_row(shape):
    """Same layer with an f32 cache holding the decoded fp8 prefill: the new rows
    (which depend on H only) must come back as the f32 rows quantised by the
    row rule (scale and codes checked against the table by brute force), and
    the attention branch may differ only by that quantisation.  With sparse
    attention the index key shares the row's scale and the kept rows are those
    of the f32 layer wherever its scores are not within the quantisation of a tie."""
    s8 = shape
    rw = s8.kv_row
    w, H, kv8 = fresh(s8)
    s32 = s8.with_(kv_fmt="f32")
    kv32 = np.zeros((s32.capacity, rw), np.float32)
    kv32[: s8.L] = oracle.kv_decode(kv8, "fp8row", rw, s8.L)
    out8, t8 = oracle.layer_step(s8, w, H, kv8, s8.L)
    out32, t32 = oracle.layer_step(s32, w, H, kv32, s8.L)
    table = _ocp_e4m3_table()
    x = kv32[s8.L:s8.L + s8.T].astype(np.float64)
    for i in range(s8.T):
        row = kv8[s8.L + i]
        sc = float(row[rw:rw + 4].copy().view(np.float32)[0])
        amax = np.abs(x[i]).max()
        assert math.frexp(sc)[0] == 0.5 and 448 * sc / 2 < amax <= 448 * sc
        for m in range(rw):
            assert row[m] == _nearest_e4m3_bruteforce(np.float32(x[i, m] / sc), table), (i, m)
        assert np.all(row[rw + 4:] == 0)
    if s8.idx_topk:
        for i in range(s8.T):
            n = s8.L + i + 1
            a, b = t8["iscore"][i, :n].astype(np.float64), t32["iscore"][i, :n].astype(np.float64)
            # prefill rows score the same on both sides (same decoded values); the
            # new rows move by their index keys' quantisation, at most d
            assert np.array_equal(a[: s8.L], b[: s8.L])
            d = np.abs(a - b).max()
            sel8 = set(t8["isel"][i][t8["isel"][i] >= 0].tolist())
            sel32 = set(t32["isel"][i][t32["isel"][i] >= 0].tolist())
            # a row only the f32 layer keeps is within 2 d of the fp8 layer's cut
            for r in sel32 - sel8:
                assert a[r] >= min(a[list(sel8)]) - 2 * d, (i, r)
        # the branch compared on the same kept rows
        w32 = dict(w, force_isel=t8["isel"])
        kv32[s8.L:] = 0
        out32, t32 = oracle.layer_step(s32, w32, H, kv32, s8.L)
    # attention over mostly shared rows: the branch moves by the quantisation of the new rows only
    e = normwise(t8["Hp"].astype(np.float64) - H, t32["Hp"].astype(np.float64) - H)
    assert 0 < e < 5e-2, e


@pytest.mark.parametrize("shape", [C0K, C0KS], ids=lambda s: s.name)
def test_fp8_cache_layer_matches_fp64_unabsorbed_bruteforce(shape):
    s = shape
    rw = s.kv_row
    w, H, kv = fresh(s)
    kv64 = kv.copy()
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    ref = oracle.layer_step_f64(s, w, H, kv64, s.L, force_sel=taps["sel"])
    assert normwise(out, ref["out"]) < 1e-5
    assert normwise(taps["Hp"].astype(np.float64) - H, ref["Hp"] - H) < 1e-4
    # new rows (the latent and RoPE key the fp64 path returns): the fp32 and fp64
    # rows may round to neighbouring codes; the rows are otherwise equal after decoding
    kvn = oracle.kv_decode(kv[s.L:s.L + s.T], "fp8row", rw, s.T).astype(np.float64)[:, : s.kvw]
    sc = kv[s.L:s.L + s.T, rw:rw + 4].copy().view(np.float32).astype(np.float64)
    assert np.all(np.abs(kvn - ref["kv_new"]) <= 32 * sc)
    assert np.mean(kvn == ref["kv_new"]) > 0.99


def test_fp8_row_parity_rule_accepts_rounding_differences_and_rejects_a_loose_scale():
    """The GPU-side rule for new fp8 rows (tests/parity.py), exercised on the CPU:
    the oracle's rows against the rows of the same layer fed bf16-rounded hidden
    rows pass; the same rows with a scale twice too large (codes halved, values
    kept) fail the minimality check; codes moved by two steps fail."""
    import parity
    s = C0K
    w, H, kv = fresh(s)
    kv2 = kv.copy()
    oracle.layer_step(s, w, H, kv, s.L)
    Hb = oracle.bf16_to_f32(np.array([[oracle.lib().orc_f32_to_bf16(float(x)) for x in r] for r in H], np.uint16))
    oracle.layer_step(s, w, Hb.astype(np.float32), kv2, s.L)
    a, b = kv[s.L:s.L + s.T], kv2[s.L:s.L + s.T]
    assert parity.fp8row_kv_check(b, a, s.kvw) > 0.5
    loose = b.copy()
    table = _ocp_e4m3_table()
    for r in range(s.T):
        sc = loose[r, s.kvw:s.kvw + 4].copy().view(np.float32)[0]
        vals = [table[int(c)] for c in loose[r, :s.kvw]]
        loose[r, :s.kvw] = [_nearest_e4m3_bruteforce(np.float32(v / 2), table) for v in vals]
        loose[r, s.kvw:s.kvw + 4] = np.frombuffer(np.float32(sc * 2).tobytes(), np.uint8)
    with pytest.raises(AssertionError):
        parity.fp8row_kv_check(loose, a, s.kvw)
    off = b.copy()
    i = int(np.argmax(np.abs(oracle.kv_decode(b, "fp8row", s.kvw, s.T)[0])))
    off[0, i] = off[0, i] - 2 if off[0, i] & 0x7 >= 2 else off[0, i] + 2
    with pytest.raises(AssertionError):
        parity.fp8row_kv_check(off, a, s.kvw)


# ---------------------------------------------------------------- sampled verification and the fp8 head
# "DeepSeek-V4.1-Flash breaks 1,000 tokens per second for one user", section
# "The safety layer": sampling uses matched random draws; "Why one GB300 doesn't
# beat 4x RTX PRO 6000 at single-stream decode", section "Where the 11.2 ms goes":
# one rejection kernel per speculative step, and an fp8 head as a small item.
def test_splitmix64_matches_the_published_first_outputs():
    g = json.load(open(os.path.join(GOLD, "splitmix64_state0.json")))
    gamma = 0x9E3779B97F4A7C15
    for k, want in enumerate(g["outputs"]):
        assert oracle.splitmix64_mix(((k + 1) * gamma) % (1 << 64)) == int(want, 16)


def test_sample_uniform_is_an_odd_multiple_of_2_to_minus_24():
    key = oracle.sample_key(11, 3)
    u = np.array([oracle.sample_uniform(key, i) for i in range(50000)], np.float64)
    m = u * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(np.round(m) % 2 == 1)
    assert 0 < u.min() and u.max() < 1
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / len(u))
    assert abs(u.var() - 1 / 12) < 2e-3
    assert oracle.sample_key(11, 3) != oracle.sample_key(11, 4) != oracle.sample_key(12, 3)


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def test_sampled_verification_commits_tokens_distributed_as_the_target():
    """Speculative sampling's guarantee: the first committed token is a draw
    from the target p_0 = softmax(l_0 / tau) whatever the draft, the draft is
    accepted with probability p_0(draft), and after an acceptance the next
    token is a draw from p_1 (counts within 5 standard deviations)."""
    l = np.array([[1.0, 0.2, -0.5, 0.7, 0.0], [0.3, -1.0, 0.9, 0.1, 0.5]], np.float32)
    tau, draft = 0.8, 3
    p0, p1 = _softmax(l[0].astype(np.float64) / tau), _softmax(l[1].astype(np.float64) / tau)
    N = 20000
    first = np.zeros(5)
    second = np.zeros(5)
    acc = 0
    for k in range(N):
        _, com = oracle.verify_sampled(l, [4, draft], tau, oracle.sample_key(7, k))
        first[com[0]] += 1
        if len(com) == 2:
            acc += 1
            assert com[0] == draft
            second[com[1]] += 1
        else:
            assert com[0] != draft
    for v in range(5):
        assert abs(first[v] / N - p0[v]) < 5 * math.sqrt(p0[v] * (1 - p0[v]) / N), (v, first / N, p0)
        assert abs(second[v] / acc - p1[v]) < 5 * math.sqrt(p1[v] * (1 - p1[v]) / acc), (v, second / acc, p1)
    assert abs(acc / N - p0[draft]) < 5 * math.sqrt(p0[draft] * (1 - p0[draft]) / N)


def test_sampled_verification_at_low_temperature_is_greedy():
    rng = np.random.default_rng(4)
    V, T = 50, 6
    for trial in range(20):
        l = np.stack([rng.permutation(V) * 0.05 for _ in range(T)]).astype(np.float32)
        am = l.argmax(axis=1)
        toks = [int(rng.integers(V))] + [int(am[i]) if rng.random() < 0.7 else int(rng.integers(V))
                                         for i in range(T - 1)]
        smp, com = oracle.verify_sampled(l, toks, 1e-3, oracle.sample_key(1, trial))
        assert np.array_equal(smp, am)
        assert np.array_equal(com, oracle.greedy_accept(toks, am))


def test_sampled_verification_certain_and_impossible_drafts():
    l = np.zeros((3, 8), np.float32)
    l[0, 5] = 1e4           # draft 1 = 5 is certain
    l[1, 2] = -1e4          # draft 2 = 2 is impossible
    for k in range(200):
        smp, com = oracle.verify_sampled(l, [0, 5, 2], 1.0, oracle.sample_key(3, k))
        assert len(com) == 2 and com[0] == 5 and com[1] != 2
        assert smp[0] == 5


def test_fp8_head_against_an_explicit_dense_matrix():
    V, d, T = 300, 256, 3
    codes, scales = synth.fp8_blocks(V, d, 0, synth.stream_id("head", 0), 0.02)
    lut = np.array([oracle.lib().orc_e4m3_to_f32(i) for i in range(256)], np.float64)
    dense = lut[codes] * np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)[:V, :d]
    h = recipe.normal_f32((T, d), 0, synth.stream_id("H", 0), 1.0)
    gf = recipe.normal_f32(d, 0, synth.stream_id("gamma_f", 0), 0.1, mean=1.0)
    lg, am = oracle.head_fp8(codes, scales, gf, h, 1e-6)
    x = h.astype(np.float64)
    x = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + 1e-6) * gf
    ref = x @ dense.T
    assert np.abs(lg - ref).max() <= 1e-5 * np.abs(ref).max()
    assert np.array_equal(am, ref.argmax(axis=1))


# ---------------------------------------------------------------- low-rank query, q-norm, latent norm
# The low-rank query of the DeepSeek-V2 paper (section 2.1: c^Q = W_DQ x,
# q = W_UQ c^Q) with the q-norm the pages' "q-norm-rope-insert" kernel names
# ("Why one GB300 doesn't beat 4x RTX PRO 6000 at single-stream decode",
# section "Where the 11.2 ms goes"), and an RMSNorm of the cached latent.
C0L = C0.with_(name="micro_lowrank", q_lora=48, kv_norm=True)
C0QL = C0Q.with_(name="micro_fp8_lowrank", q_lora=64, kv_norm=True)


@pytest.mark.parametrize("shape", [C0L, C0QL], ids=lambda s: s.name)
def test_lowrank_layer_matches_fp64_unabsorbed_bruteforce(shape):
    w, H, kv = fresh(shape)
    kv64 = kv.copy()
    out, taps = oracle.layer_step(shape, w, H, kv, shape.L)
    ref = oracle.layer_step_f64(shape, w, H, kv64, shape.L, force_sel=taps["sel"])
    assert normwise(out, ref["out"]) < 1e-5
    assert normwise(taps["Hp"].astype(np.float64) - H, ref["Hp"] - H) < 1e-4


def test_lowrank_query_with_identity_down_projection_is_the_single_wq_layer():
    """W_DQ = I (rank d) and gamma_1 = 1: the normalised input x has unit RMS,
    so the q-norm returns x * gamma_q and q = (W_UQ diag(gamma_q)) x -- the
    one-W_Q layer with that matrix (up to eps / mean square ~ 1e-6)."""
    s = C0.with_(name="micro_lowrank_identity", q_lora=C0.d)
    w, H, kv = fresh(s)
    w["gamma1"] = np.ones_like(w["gamma1"])
    w["wdq"] = np.eye(s.d, dtype=np.float32)
    s1 = C0
    w1 = {k: v for k, v in w.items() if k not in ("wdq", "wuq", "gamma_q")}
    w1["wq"] = (w["wuq"].astype(np.float64) * w["gamma_q"].astype(np.float64)[None, :]).astype(np.float32)
    kv1 = kv.copy()
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    out1, taps1 = oracle.layer_step(s1, w1, H, kv1, s.L)
    assert normwise(taps["q"], taps1["q"]) < 1e-5
    assert normwise(taps["Hp"].astype(np.float64) - H, taps1["Hp"].astype(np.float64) - H) < 1e-4
    assert normwise(out, out1) < 1e-5
    # dropping the q-norm's gain is far outside that
    w2 = dict(w, gamma_q=np.ones_like(w["gamma_q"]))
    _, taps2 = oracle.layer_step(s, w2, H, kv.copy(), s.L)
    assert normwise(taps2["q"], taps1["q"]) > 3e-2


def test_latent_norm_gives_unit_rms_rows_before_the_gain_and_leaves_the_key():
    s = C0.with_(name="micro_kvnorm", kv_norm=True)
    w, H, kv = fresh(s)
    s0 = C0
    kv0 = kv.copy()
    oracle.layer_step(s, w, H, kv, s.L)
    oracle.layer_step(s0, {k: v for k, v in w.items() if k != "gamma_kv"}, H, kv0, s.L)
    c = kv[s.L:s.L + s.T, : s.d_c].astype(np.float64) / w["gamma_kv"].astype(np.float64)
    c0 = kv0[s.L:s.L + s.T, : s.d_c].astype(np.float64)
    ms0 = (c0 * c0).mean(axis=1)
    # closed form: RMS of c / gamma = sqrt(ms / (ms + eps)) for the un-normalised mean square ms
    assert np.allclose(np.sqrt((c * c).mean(axis=1)), np.sqrt(ms0 / (ms0 + s.eps)), rtol=1e-6)
    # the RoPE key is not normalised; the latent is the un-normalised one rescaled
    assert np.array_equal(kv[s.L:s.L + s.T, s.d_c:], kv0[s.L:s.L + s.T, s.d_c:])
    ratio = c / c0
    assert np.allclose(ratio, ratio[:, :1], rtol=1e-5)


# ---------------------------------------------------------------- sparse attention with an indexer
# The pages' sparse attention mode and indexer ("Why one GB300 ...", sections
# "Where the 11.2 ms goes" and "Corrections to things we said"), read as the
# lightning indexer of the DeepSeek-V3.2 report: score(t, s) = sum_j w_tj *
# relu(q_tj . k_s); each query row attends to its top-k cache rows.
C0S = C0.with_(name="micro_sparse", idx_heads=4, idx_dim=16, idx_topk=4, L=9)
C0QS = C0Q.with_(name="micro_bf16_sparse", idx_heads=4, idx_dim=32, idx_topk=5, L=12)


def _dense_of(s, kv):
    """The same layer without the indexer, on the same cache rows minus their index keys."""
    sd = s.with_(idx_heads=0, idx_dim=0, idx_topk=0)
    return sd, np.ascontiguousarray(kv[:, : s.kvw])


def test_sparse_with_topk_covering_every_row_is_the_dense_layer_bitwise():
    s = C0S.with_(idx_topk=64)
    w, H, kv = fresh(s)
    sd, kvd = _dense_of(s, kv)
    wd = {k: v for k, v in w.items() if k != "widx"}
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    outd, tapsd = oracle.layer_step(sd, wd, H, kvd, s.L)
    assert np.array_equal(taps["Hp"].view(np.uint32), tapsd["Hp"].view(np.uint32))
    assert np.array_equal(out.view(np.uint32), outd.view(np.uint32))
    for i in range(s.T):
        assert list(taps["isel"][i][: s.L + i + 1]) == list(range(s.L + i + 1))


def _decode(a, fmt, rw=None):
    if fmt == "fp8row":
        return oracle.kv_decode(a, fmt, rw, a.shape[0]).astype(np.float64)
    return oracle.bf16_to_f32(a).astype(np.float64) if fmt == "bf16" else a.astype(np.float64)


@pytest.mark.parametrize("shape", [C0S, C0QS, C0KS], ids=lambda s: s.name)
def test_sparse_selection_is_the_topk_of_independently_computed_index_scores(shape):
    s = shape
    w, H, kv = fresh(s)
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    HI, dI, k = s.idx_heads, s.idx_dim, s.idx_topk
    W = _decode(w["widx"], s.attn_fmt)
    x = taps["x"].astype(np.float64)
    rows = _decode(kv, s.kv_fmt, s.kv_row)[: s.L + s.T]
    kI = rows[:, s.kvw:]
    # the new rows carry W_IK x as their index key (stored at the cache's
    # precision; an fp8 row's index key is rounded at the row's scale, which its
    # latent may set, so the bound is an E4M3 half step at the row maximum)
    tol_k = {"f32": 1e-5, "bf16": 2 ** -8}.get(s.kv_fmt)
    if tol_k is None:
        amax = np.abs(rows[s.L:]).max(axis=1, keepdims=True)
        err = np.abs(kI[s.L:] - x @ W[HI * dI + HI:].T)
        assert np.all(err <= amax * 2.0 ** -4), float((err / amax).max())
        tol_k = np.inf
    assert normwise(kI[s.L:], x @ W[HI * dI + HI:].T) < tol_k
    for i in range(s.T):
        pos = s.L + i
        qI = (W[: HI * dI] @ x[i]).reshape(HI, dI)
        wI = W[HI * dI: HI * dI + HI] @ x[i]
        sc = (np.maximum(kI[: pos + 1] @ qI.T, 0.0) * wI[None, :]).sum(axis=1)
        got = taps["iscore"][i, : pos + 1].astype(np.float64)
        assert np.abs(got - sc).max() <= 1e-4 * np.abs(sc).max()
        sel = [j for j in taps["isel"][i] if j >= 0]
        assert sel == sorted(sel) and len(sel) == min(k, pos + 1)
        out_rows = sorted(set(range(pos + 1)) - set(sel))
        if out_rows:
            # every kept row scores at least as high as every dropped one (up to fp32 rounding)
            assert sc[sel].min() >= sc[out_rows].max() - 1e-5 * np.abs(sc).max()


@pytest.mark.parametrize("shape", [C0S, C0QS, C0KS], ids=lambda s: s.name)
def test_sparse_layer_matches_fp64_unabsorbed_bruteforce(shape):
    s = shape
    w, H, kv = fresh(s)
    kv64 = kv.copy()
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    ref = oracle.layer_step_f64(s, w, H, kv64, s.L, force_sel=taps["sel"])
    assert normwise(out, ref["out"]) < 1e-5
    assert normwise(taps["Hp"].astype(np.float64) - H, ref["Hp"] - H) < 1e-4


def test_sparse_attention_weights_only_the_kept_rows():
    """z of every (row, head) against numpy attention over the kept rows alone,
    from the oracle's absorbed query, rotated query and the stored cache rows."""
    s = C0S
    w, H, kv = fresh(s)
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    rows = kv[: s.L + s.T].astype(np.float64)
    scale = 1.0 / math.sqrt(s.d_h + s.d_r)
    for i in range(s.T):
        sel = [j for j in taps["isel"][i] if j >= 0]
        assert len(sel) == s.idx_topk < s.L + i + 1
        for h in range(s.n_h):
            qa = taps["qabs"][i, h].astype(np.float64)
            qr = taps["q"][i, h, s.d_h:].astype(np.float64)
            sc = (rows[sel, : s.d_c] @ qa + rows[sel, s.d_c:s.kvw] @ qr) * scale
            p = np.exp(sc - sc.max())
            p /= p.sum()
            z = p @ rows[sel, : s.d_c]
            assert np.abs(taps["z"][i, h] - z).max() <= 1e-5 * np.abs(z).max()


def test_sparse_ties_keep_the_lower_rows():
    """Indexer weights of zero make every index score 0: each row keeps the
    lowest idx_topk rows it may see (ties go to the lower row), in both the
    fp32 and the fp64 path."""
    s = C0S
    w, H, kv = fresh(s)
    w["widx"] = np.zeros_like(w["widx"])
    kv64 = kv.copy()
    out, taps = oracle.layer_step(s, w, H, kv, s.L)
    for i in range(s.T):
        assert not taps["iscore"][i, : s.L + i + 1].any()      # the rows row i may see
        assert list(taps["isel"][i][: s.idx_topk]) == list(range(s.idx_topk))
    ref = oracle.layer_step_f64(s, w, H, kv64, s.L, force_sel=taps["sel"])
    assert normwise(out, ref["out"]) < 1e-5
