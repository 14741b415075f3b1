"""mk_decode_step_static, the step for callers that cannot allocate (its scratch
is a device array inside the library), against mk_decode_step on the same
layer: two calls in a row, the second with a smaller input (fewer rows,
shorter cache) on the scratch the first one left behind.  Each is compared
bitwise with the workspace step (same kernels) and with the oracle by the
parity rules; a layer whose scratch would not fit is refused."""
import numpy as np
import pytest

from synth import recipe
from synth.configs import LayerShape

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHAPE = LayerShape("noalloc_fp8", d=640, n_h=6, d_h=64, d_c=256, d_r=64, E=48, top_k=6, n_shared=1, f=384,
                   T=7, L=300, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16", kv_capacity=320)
# sparse attention over the fp8 cache (the top-k's histograms and counters live in the scratch too)
SHAPE_SP = SHAPE.with_(name="noalloc_sparse_fp8kv", n_h=16, kv_fmt="fp8row", idx_heads=16, idx_dim=64, idx_topk=100)


@pytest.mark.parametrize("s", [SHAPE, SHAPE_SP], ids=lambda s: s.name)
def test_static_scratch_step_matches_workspace_step_twice_second_smaller(s):
    from decoder_megakernel_amd import MK_OK, harness
    import parity
    dl = harness.DeviceLayer(s, 0, 0)
    w = recipe.layer_weights_host(s, 0, 0)
    for T, L in ((7, 300), (3, 120)):
        print("[no-alloc] %s T=%d L=%d" % (s.name, T, L), flush=True)
        s2 = s.with_(T=T, L=L)
        H = recipe.hidden_host(s2, 0, 0)
        Hd = torch.from_numpy(H).cuda()
        kv_a, kv_b = harness.kv_cache(s2), harness.kv_cache(s2)
        out_a, out_b = torch.empty_like(Hd), torch.empty_like(Hd)
        dl.layer.decode_step(Hd.data_ptr(), T, kv_a.data_ptr(), kv_a.shape[0], L, out_a.data_ptr())
        dl.layer.decode_step_static(Hd.data_ptr(), T, kv_b.data_ptr(), kv_b.shape[0], L, out_b.data_ptr())
        torch.cuda.synchronize()
        assert dl.layer.sync_status() == MK_OK
        assert np.array_equal(out_a.cpu().numpy().view(np.uint32), out_b.cpu().numpy().view(np.uint32))
        assert np.array_equal(kv_a.cpu().numpy().view(np.uint8), kv_b.cpu().numpy().view(np.uint8))
        # the static step's taps and outputs against the oracle
        taps = {}
        pairs = [("Hp", 4, (T, s.d), np.float32), ("sel", 6, (T, s.top_k), np.int32)]
        if s.idx_topk:
            pairs += [("isel", 8, (T, s.idx_topk), np.int32), ("iscore", 9, (T, (s.capacity + 7) // 8 * 8), np.float32)]
        for name, tap, shape, dt in pairs:
            buf = np.empty(shape, dt)
            dl.layer.debug_tap(tap, buf)
            taps[name] = buf
        taps["kv_raw"] = kv_b[L:L + T].cpu().numpy()
        g_kv = parity.kv_to_f32(kv_b[L:L + T].cpu().numpy(), s.kv_fmt, s.kv_row)
        errs = parity.check_layer(s2, 0, 0, out_b.cpu().numpy(), g_kv, taps, H, L, full_weights=w)
        print("[no-alloc] T=%d L=%d errors %s" % (T, L, errs), flush=True)


class _OneBlockPool:
    """Every routed expert slot points at one packed block (cheap to build)."""

    def __init__(self, s, device=0):
        from decoder_megakernel_amd import MK_T_EXPERT, harness, packed_bytes
        cfg = harness.config_of(s)
        block = packed_bytes(cfg, MK_T_EXPERT)
        self.buf = torch.empty(block, dtype=torch.uint8, device="cuda")
        harness.ExpertStager(s, device).draw_and_pack(cfg, 0, 0, 0, self.buf.data_ptr())
        self.ptrs = [self.buf.data_ptr()] * s.E


def test_scratch_larger_than_the_static_array_is_refused():
    from decoder_megakernel_amd import MK_ERR_UNSUPPORTED_SHAPE, MK_STATIC_SCRATCH_BYTES, MkError, harness
    from decoder_megakernel_amd import layer_workspace_bytes
    s = LayerShape("noalloc_big", d=4096, n_h=32, d_h=128, d_c=512, d_r=64, E=128, top_k=16, n_shared=1,
                   f=2048, T=8, L=16, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16")
    assert layer_workspace_bytes(harness.config_of(s)) > MK_STATIC_SCRATCH_BYTES
    dl = harness.DeviceLayer(s, 0, 0, pool=_OneBlockPool(s))
    kv = harness.kv_cache(s)
    H = harness.hidden(s)
    out = torch.empty_like(H)
    with pytest.raises(MkError) as ei:
        dl.layer.decode_step_static(H.data_ptr(), s.T, kv.data_ptr(), kv.shape[0], s.L, out.data_ptr())
    assert ei.value.code == MK_ERR_UNSUPPORTED_SHAPE
