"""GPU parity: the HIP verify step (through the C ABI) against the CPU oracle on
identical seeded inputs (rules in tests/parity.py)."""
import numpy as np
import pytest

from synth import recipe
from synth.configs import C1, C2, C3, C3X, C3XK, C4, LayerShape

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Several tiles in every dimension, ragged tails (L+T not a multiple of 16,
# T < 16 MFMA columns, expert counts not a multiple of the grid).
MID_BF16 = LayerShape("mid_bf16", d=512, n_h=4, d_h=64, d_c=128, d_r=32, E=32, top_k=4, n_shared=1, f=256,
                      T=5, L=77, attn_fmt="bf16", exp_fmt="bf16", kv_fmt="bf16")
MID_FP8 = LayerShape("mid_fp8", d=640, n_h=6, d_h=64, d_c=256, d_r=64, E=48, top_k=6, n_shared=1, f=384,
                     T=7, L=300, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16")
# MXFP4 experts: 5 and 3 tiles of 128 columns per row (ragged slices), and
# 16 and 8 (the streaming engines' chunked paths).
MID_MX = LayerShape("mid_mxfp4", d=640, n_h=6, d_h=64, d_c=256, d_r=64, E=48, top_k=6, n_shared=1, f=384,
                    T=7, L=300, attn_fmt="bf16", exp_fmt="mxfp4", kv_fmt="bf16")
MID_MX_WIDE = LayerShape("mid_mxfp4_wide", d=2048, n_h=4, d_h=64, d_c=128, d_r=32, E=32, top_k=4, n_shared=1,
                         f=1024, T=6, L=100, attn_fmt="bf16", exp_fmt="mxfp4", kv_fmt="bf16")
# d_model 4096 (32 MXFP4 tiles): ticket-fed gate/up with two units per workgroup;
# with d_ff 2048 also the ticket-fed down projections of eight row tiles (fused).
MID_MX_TICKET = LayerShape("mid_mxfp4_ticket", d=4096, n_h=4, d_h=64, d_c=128, d_r=32, E=16, top_k=3, n_shared=1,
                           f=1024, T=5, L=60, attn_fmt="bf16", exp_fmt="mxfp4", kv_fmt="bf16")
MID_MX_FUSED = MID_MX_TICKET.with_(name="mid_mxfp4_fused", f=2048, top_k=2, T=6, L=33)
# fp8 (E4M3, one scale per row) cache: generic shapes with each expert format.
MID_KV8 = MID_FP8.with_(name="mid_fp8_kv8", kv_fmt="fp8row")
MID_BF16_KV8 = MID_BF16.with_(name="mid_bf16_kv8", kv_fmt="fp8row")
MID_MX_KV8 = MID_MX_TICKET.with_(name="mid_mxfp4_kv8", kv_fmt="fp8row")
MID_F32 = LayerShape("mid_f32", d=384, n_h=4, d_h=32, d_c=96, d_r=32, E=16, top_k=3, n_shared=1, f=256,
                     T=3, L=45, attn_fmt="f32", exp_fmt="f32", kv_fmt="f32")
# Expert widths of 32 tiles, d_model of 64 tiles and d_model >= 2 d_ff: the
# expert phases run fused (ticket-fed gate/up counted per slot, then ticket-fed
# four-row-tile down projections with the expert rows double-buffered in LDS).
MID_F32_DOWN = LayerShape("mid_f32_down", d=2048, n_h=4, d_h=64, d_c=128, d_r=32, E=16, top_k=2, n_shared=1,
                          f=512, T=5, L=50, attn_fmt="f32", exp_fmt="f32", kv_fmt="f32")
MID_BF16_DOWN = LayerShape("mid_bf16_down", d=2048, n_h=4, d_h=64, d_c=128, d_r=32, E=16, top_k=4, n_shared=1,
                           f=1024, T=6, L=100, attn_fmt="bf16", exp_fmt="bf16", kv_fmt="bf16")


def _run(s, seed=0, layer=0, L=None, T=None, full_weights=True):
    from decoder_megakernel_amd import harness
    import parity
    L = s.L if L is None else L
    T = s.T if T is None else T
    s2 = s.with_(L=L, T=T, kv_capacity=max(s.capacity, L + T))
    print("[parity] %s seed=%d L=%d T=%d" % (s.name, seed, L, T), flush=True)
    dl = harness.DeviceLayer(s2, seed, layer)
    kv = harness.kv_cache(s2, seed, layer)
    H = recipe.hidden_host(s2, seed, layer)
    Hd = torch.from_numpy(H).cuda()
    g_out, g_kv, g_taps = parity.gpu_step(dl, s2, Hd, kv, L, T)
    w = recipe.layer_weights_host(s2, seed, layer) if full_weights else None
    rep = {}
    errs = parity.check_layer(s2, seed, layer, g_out, g_kv, g_taps, H, L, full_weights=w, report=rep)
    print("[parity] %s errors %s" % (s.name, errs), flush=True)
    return dl, kv, Hd, g_out, g_kv, errs


@pytest.mark.parametrize("shape", [C1, MID_F32, MID_BF16, MID_FP8, MID_F32_DOWN, MID_BF16_DOWN, MID_MX, MID_MX_WIDE,
                                   MID_MX_TICKET, MID_MX_FUSED, MID_KV8, MID_BF16_KV8, MID_MX_KV8],
                         ids=lambda s: s.name)
def test_small_shapes_match_oracle(shape):
    _run(shape)


def test_single_row_empty_cache():
    _run(MID_BF16, L=0, T=1)


def test_single_row_empty_fp8_cache():
    _run(MID_KV8, L=0, T=1)


def test_max_rows():
    _run(MID_FP8, T=8, L=13)


def test_max_rows_fp8_cache():
    _run(MID_KV8, T=8, L=13)


def test_full_size_bf16_E128_T6_L2048():
    _run(C2, full_weights=False)


def test_full_size_fp8_E384_T8_L8192():
    _run(C3, full_weights=False)


def test_full_size_mxfp4_E384_T8_L8192():
    _run(C3X, full_weights=False)


def test_full_size_mxfp4_fp8kv_E384_T8_L8192():
    _run(C3XK, full_weights=False)


def test_full_size_fp8_E384_T6_L65536_skew():
    _run(C4, full_weights=False)


@pytest.mark.parametrize("s", [MID_FP8, MID_KV8], ids=lambda s: s.name)
def test_run_twice_bitwise_identical(s):
    from decoder_megakernel_amd import harness
    dl = harness.DeviceLayer(s, 0, 0)
    H = harness.hidden(s)
    outs = []
    for _ in range(2):
        kv = harness.kv_cache(s)
        out = torch.empty_like(H)
        dl.step(H, s.T, kv, s.L, out)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().view(np.uint32), kv.cpu().numpy().view(np.uint8)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_back_to_back_layers_sharing_a_workspace():
    """Two layers launched back to back on one stream, sharing one workspace,
    with no host synchronisation in between, give bitwise the results each
    gives alone (a stale cached line of the first launch would show here)."""
    from decoder_megakernel_amd import harness
    s = MID_FP8.with_(T=6, L=40, kv_capacity=64)
    H1 = torch.from_numpy(recipe.hidden_host(s, 0, 0, step=0)).cuda()
    H2 = torch.from_numpy(recipe.hidden_host(s, 0, 1, step=1)).cuda()
    alone = harness.DeviceLayer(s, 0, 1)
    kva = harness.kv_cache(s, 0, 1)
    ref = torch.empty_like(H2)
    alone.step(H2, s.T, kva, s.L, ref)
    torch.cuda.synchronize()
    l0 = harness.DeviceLayer(s, 0, 0)
    l1 = harness.DeviceLayer(s, 0, 1, workspace=l0.workspace)
    for _ in range(2):
        kv0, kv1 = harness.kv_cache(s, 0, 0), harness.kv_cache(s, 0, 1)
        o0, o1 = torch.empty_like(H1), torch.empty_like(H2)
        l0.step(H1, s.T, kv0, s.L, o0)
        l1.step(H2, s.T, kv1, s.L, o1)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
        assert np.array_equal(kv1.cpu().numpy().view(np.uint16), kva.cpu().numpy().view(np.uint16))


def test_verify_rows_match_sequential_single_row_steps():
    """Causal invariant on the GPU: row i of a T-row step equals (to tolerance)
    a single-row step at position L+i on the cache the earlier rows built."""
    from decoder_megakernel_amd import harness
    import parity
    s = MID_BF16
    dl = harness.DeviceLayer(s, 0, 0)
    H = harness.hidden(s)
    kv = harness.kv_cache(s)
    out = torch.empty_like(H)
    dl.step(H, s.T, kv, s.L, out)
    kv2 = harness.kv_cache(s)
    outs = []
    for i in range(s.T):
        o = torch.empty((1, s.d), dtype=torch.float32, device="cuda")
        dl.step(H[i:i + 1].contiguous(), 1, kv2, s.L + i, o)
        outs.append(o)
    torch.cuda.synchronize()
    seq = torch.cat(outs).cpu().numpy()
    assert parity.normwise(out.cpu().numpy(), seq) < 2e-2
    kvs = parity.kv_to_f32(kv2[s.L:s.L + s.T].cpu().numpy(), "bf16")
    kvb = parity.kv_to_f32(kv[s.L:s.L + s.T].cpu().numpy(), "bf16")
    assert parity.normwise(kvb, kvs) < 2e-2


# The low-rank query variant (W_DQ, q-norm, W_UQ) with the latent norm, on each
# expert format and cache format; one without the latent norm.
MID_LR_BF16 = MID_BF16.with_(name="mid_bf16_lowrank", q_lora=256, kv_norm=True)
MID_LR_FP8 = MID_FP8.with_(name="mid_fp8_lowrank", q_lora=384, kv_norm=True)
MID_LR_FP8_NOKVN = MID_FP8.with_(name="mid_fp8_lowrank_no_kvnorm", q_lora=224)
MID_LR_MX_KV8 = MID_MX_TICKET.with_(name="mid_mxfp4_kv8_lowrank", kv_fmt="fp8row", q_lora=512, kv_norm=True)


@pytest.mark.parametrize("shape", [MID_LR_BF16, MID_LR_FP8, MID_LR_FP8_NOKVN, MID_LR_MX_KV8], ids=lambda s: s.name)
def test_lowrank_query_shapes_match_oracle(shape):
    _run(shape)


def test_lowrank_query_single_row_empty_cache():
    _run(MID_LR_FP8, L=0, T=1)


def test_full_size_lowrank_query_fp8_E384_T8_L8192():
    from synth.configs import C3Q
    _run(C3Q, full_weights=False)


def test_full_size_lowrank_query_mxfp4_fp8kv_E384_T8_L8192():
    from synth.configs import C3XK
    _run(C3XK.with_(name="mxfp4_fp8kv_lowrankq_E384_T8_L8192", q_lora=1536, kv_norm=True), full_weights=False)


# Sparse attention (indexer + top-k kept rows): 16 heads per query tile, 100
# rows kept of ~300; with a low-rank query; with MXFP4 experts; and a top-k
# that covers every row (the dense attention).
MID_SP = LayerShape("mid_sparse", d=1024, n_h=16, d_h=64, d_c=128, d_r=32, E=32, top_k=4, n_shared=1, f=256,
                    T=6, L=300, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16", idx_heads=16, idx_dim=64, idx_topk=100)
MID_SP_LR = MID_SP.with_(name="mid_sparse_lowrank", q_lora=256, kv_norm=True)
MID_SP_MX = MID_SP.with_(name="mid_sparse_mxfp4", exp_fmt="mxfp4")
MID_SP_ALL = MID_SP.with_(name="mid_sparse_topk_covers_all", idx_topk=512)
# fp8 cache rows carrying the index key under the row's scale
MID_SP_K = MID_SP.with_(name="mid_sparse_fp8kv", kv_fmt="fp8row")
MID_SP_K_LR = MID_SP_LR.with_(name="mid_sparse_fp8kv_lowrank", kv_fmt="fp8row", exp_fmt="mxfp4")
MID_SP_K_ALL = MID_SP_K.with_(name="mid_sparse_fp8kv_topk_covers_all", idx_topk=512)
MID_SP_K_BF = MID_SP_K.with_(name="mid_sparse_fp8kv_bf16_experts", exp_fmt="bf16")


@pytest.mark.parametrize("shape", [MID_SP, MID_SP_LR, MID_SP_MX, MID_SP_ALL, MID_SP_K, MID_SP_K_LR, MID_SP_K_ALL,
                                   MID_SP_K_BF],
                         ids=lambda s: s.name)
def test_sparse_attention_shapes_match_oracle(shape):
    _run(shape)


def test_sparse_attention_fp8kv_single_row_empty_cache():
    _run(MID_SP_K, L=0, T=1)


def test_sparse_attention_single_row_empty_cache():
    _run(MID_SP, L=0, T=1)


def test_sparse_attention_rows_just_past_topk():
    _run(MID_SP, L=97, T=6)


@pytest.mark.parametrize("L", [9000, 16384])
def test_sparse_attention_all_scores_equal(L):
    """Indexer weights of zero: every index score is 0 and the kept rows are the
    lowest idx_topk rows (ties go to the lower row).  At L = 9000 every row is a
    candidate of the first digit's bin and still fits the workgroup's list; at
    L = 16384 it does not, and the top-k reads the row again for each digit."""
    from decoder_megakernel_amd import harness
    import parity
    s = MID_SP.with_(name="mid_sparse_ties", L=L, idx_topk=2048)
    s = s.with_(kv_capacity=max(s.capacity, L + s.T))
    print("[parity] %s L=%d" % (s.name, L), flush=True)
    dl = harness.DeviceLayer(s, 0, 0)
    dl.packed["widx"].zero_()
    kv = harness.kv_cache(s, 0, 0)
    H = recipe.hidden_host(s, 0, 0)
    g_out, g_kv, g_taps = parity.gpu_step(dl, s, torch.from_numpy(H).cuda(), kv, L, s.T)
    assert not g_taps["iscore"][:, :L + s.T].any()
    for t in range(s.T):
        assert g_taps["isel"][t].tolist() == list(range(2048)), t
    w = recipe.layer_weights_host(s, 0, 0)
    w["widx"] = np.zeros_like(w["widx"])
    errs = parity.check_layer(s, 0, 0, g_out, g_kv, g_taps, H, L, full_weights=w)
    print("[parity] %s errors %s" % (s.name, errs), flush=True)
    assert errs["kept_rows_differing"] == 0 and not errs["kept_rows_forced"]


@pytest.mark.parametrize("s", [MID_SP.with_(name="mid_sparse_L20000", L=20000, idx_topk=2048),
                               MID_SP_K.with_(name="mid_sparse_fp8kv_L20000", L=20000, idx_topk=2048)],
                         ids=lambda s: s.name)
def test_sparse_run_twice_bitwise_identical(s):
    """Two runs of the same sparse step (the top-k over ten parts of the row, its
    sums of part histograms made with atomics) give bitwise the same output, new
    cache rows, index scores and kept rows."""
    from decoder_megakernel_amd import harness
    import parity
    print("[parity] %s L=%d" % (s.name, s.L), flush=True)
    dl = harness.DeviceLayer(s, 0, 0)
    H = harness.hidden(s)
    res = []
    for _ in range(2):
        kv = harness.kv_cache(s)
        out, kvn, taps = parity.gpu_step(dl, s, H, kv, s.L, s.T)
        res.append((out.view(np.uint32), taps["kv_raw"].view(np.uint8), taps["iscore"].view(np.uint32), taps["isel"]))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


def test_full_size_sparse_fp8_E384_T6_L65536_skew():
    from synth.configs import C4S
    _run(C4S, full_weights=False)


def test_full_size_sparse_mxfp4_fp8kv_E384_T6_L65536_skew():
    from synth.configs import C4SXK
    _run(C4SXK, full_weights=False)
