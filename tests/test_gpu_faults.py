"""Failure handling on the GPU, every condition forced from the host so that
all kernels still leave normally:

  - a bounded wait given a 1 us limit on a healthy step: every workgroup's
    wait gives up (or passes), the launch ends, the layer reports
    MK_ERR_TIMEOUT, later launches of the layer do nothing until
    mk_layer_reset, and the next step is clean (bitwise equal to a fresh
    layer's step, and within tolerance of the oracle);
  - a stack step with a token id outside [0, vocab): nothing committed, KV
    length and token buffer unchanged, MK_ERR_INVALID_ARG from
    mk_model_sync_status, sticky until mk_model_reset, then a clean step;
  - a stack step whose KV length + T passes the capacity: the same.

The wait bound is the pages' watchdog idea ("DeepSeek-V4.1-Flash breaks 1,000
tokens per second for one user", section "The safety layer": a possible hang
turned into a fast, visible stop)."""
import ctypes

import numpy as np
import pytest

from synth import recipe
from synth.configs import LayerShape

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHAPE = LayerShape("fault_fp8", d=640, n_h=6, d_h=64, d_c=256, d_r=64, E=48, top_k=6, n_shared=1, f=384,
                   T=6, L=60, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16", kv_capacity=96)
STACK = SHAPE.with_(name="fault_stack", n_layers=2, V=512, n_pools=0, kv_capacity=80)


def _read_i32(dev_ptr):
    hip = ctypes.CDLL("libamdhip64.so")
    out = ctypes.c_int32(0)
    assert hip.hipMemcpy(ctypes.byref(out), ctypes.c_void_p(dev_ptr), ctypes.c_size_t(4), ctypes.c_int(2)) == 0
    return out.value


def test_timeout_then_reset_gives_a_clean_step():
    from decoder_megakernel_amd import MK_ERR_TIMEOUT, MK_OK, harness
    import parity
    s = SHAPE
    print("[fault] timeout on %s" % s.name, flush=True)
    dl = harness.DeviceLayer(s, 0, 0)
    H = torch.from_numpy(recipe.hidden_host(s, 0, 0)).cuda()
    out = torch.empty_like(H)
    dl.layer.set_barrier_timeout_us(1)
    kv = harness.kv_cache(s)
    dl.step(H, s.T, kv, s.L, out)
    torch.cuda.synchronize()
    assert dl.layer.sync_status() == MK_ERR_TIMEOUT
    # sticky: the next launch leaves at its first barrier, still reporting the fault
    dl.layer.set_barrier_timeout_us(2_000_000)
    dl.step(H, s.T, kv, s.L, out)
    torch.cuda.synchronize()
    assert dl.layer.sync_status() == MK_ERR_TIMEOUT
    dl.layer.reset()
    assert dl.layer.sync_status() == MK_OK
    kv = harness.kv_cache(s)
    g_out, g_kv, g_taps = parity.gpu_step(dl, s, H, kv, s.L)
    # bitwise what a layer that never faulted computes
    fresh = harness.DeviceLayer(s, 0, 0)
    kv2 = harness.kv_cache(s)
    ref = torch.empty_like(H)
    fresh.step(H, s.T, kv2, s.L, ref)
    torch.cuda.synchronize()
    assert np.array_equal(g_out.view(np.uint32), ref.cpu().numpy().view(np.uint32))
    assert np.array_equal(kv.cpu().numpy().view(np.uint16), kv2.cpu().numpy().view(np.uint16))
    errs = parity.check_layer(s, 0, 0, g_out, g_kv, g_taps, recipe.hidden_host(s, 0, 0), s.L,
                              full_weights=recipe.layer_weights_host(s, 0, 0))
    print("[fault] clean step after reset: %s" % errs, flush=True)


def _stack_step(st, s, tokens, nd=None):
    dev = torch.device("cuda")
    am = torch.full((s.T,), 77, dtype=torch.int32, device=dev)
    com = torch.full((s.T + 1,), 55, dtype=torch.int32, device=dev)
    st.model.step(tokens.data_ptr(), s.T, None if nd is None else nd.data_ptr(), am.data_ptr(), com.data_ptr())
    torch.cuda.synchronize()
    return am.cpu().numpy(), com.cpu().numpy()


@pytest.mark.parametrize("case", ["bad_token", "kv_capacity"])
def test_stack_fault_commits_nothing_until_reset(case):
    from decoder_megakernel_amd import MK_ERR_INVALID_ARG, MK_OK, harness
    s = STACK
    print("[fault] stack %s" % case, flush=True)
    st = harness.DeviceStack(s, 0)
    good = recipe.tokens_host(s, 0, 0)
    tok = torch.from_numpy(good.copy()).cuda()
    L0 = s.L
    if case == "bad_token":
        bad = good.copy()
        bad[2] = s.V + 5
        tok = torch.from_numpy(bad).cuda()
    else:
        L0 = s.capacity - s.T + 1           # one row short
        st.model.set_length(L0)
    before = tok.cpu().numpy().copy()
    am, com = _stack_step(st, s, tok)
    assert st.model.sync_status() == MK_ERR_INVALID_ARG
    assert com[0] == 0 and np.all(am == -1)
    assert _read_i32(st.model.length_ptr()) == L0
    assert np.array_equal(tok.cpu().numpy(), before)
    # sticky until reset, even for a valid step
    tok = torch.from_numpy(good.copy()).cuda()
    st.model.set_length(s.L)
    am, com = _stack_step(st, s, tok)
    assert st.model.sync_status() == MK_ERR_INVALID_ARG and com[0] == 0
    assert _read_i32(st.model.length_ptr()) == s.L
    st.model.reset()
    assert st.model.sync_status() == MK_OK
    am, com = _stack_step(st, s, tok)
    assert st.model.sync_status() == MK_OK
    for dl in st.layers:
        assert dl.layer.sync_status() == MK_OK
    n = int(com[0])
    assert 1 <= n <= s.T and np.all(am >= 0) and np.all(am < s.V)
    assert _read_i32(st.model.length_ptr()) == s.L + n
