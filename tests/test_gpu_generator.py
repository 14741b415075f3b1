"""The seeded generator's two builds agree bit for bit: the device build
(libmksynth_dev.so), which draws every weight the GPU path is fed, and the
host build (libmksynth_host.so), which draws the same tensors for the CPU
oracle.  Covered: raw 64-bit outputs, fp32 normals (with and without a mean),
bf16 normals, fp8 E4M3 blocks with their fp32 scales, and MXFP4 rows (E2M1
codes with an E8M0 scale per 32 elements), on ragged shapes (edges of partial
128x128 blocks) and at the full size of one expert matrix."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _dev(n, dtype):
    return torch.empty(n, dtype=dtype, device="cuda")


def test_raw_outputs_identical():
    n, seed, st = 1 << 20, 7, synth.stream_id("tokens", 3, 11)
    d = _dev(n, torch.int64)
    synth.dev_raw(d.data_ptr(), n, seed, st, offset=12345)
    torch.cuda.synchronize()
    h = synth.raw(n, seed, st, offset=12345)
    assert np.array_equal(d.cpu().numpy().view(np.uint64), h)


@pytest.mark.parametrize("sigma,mean", [(0.02, 0.0), (1.0, 0.0), (0.1, 1.0)])
def test_normal_f32_identical(sigma, mean):
    n, st = 3_000_017, synth.stream_id("wq", 5)
    d = _dev(n, torch.float32)
    synth.dev_normal_f32(d.data_ptr(), n, 0, st, sigma, mean=mean, offset=99)
    torch.cuda.synchronize()
    h = synth.normal_f32(n, 0, st, sigma, mean=mean, offset=99)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), h.view(np.uint32))


def test_normal_bf16_identical():
    n, st = 2_000_003, synth.stream_id("head")
    d = _dev(n, torch.int16)
    synth.dev_normal_bf16(d.data_ptr(), n, 0, st, 0.02)
    torch.cuda.synchronize()
    h = synth.normal_bf16(n, 0, st, 0.02)
    assert np.array_equal(d.cpu().numpy().view(np.uint16), h)
    d2 = _dev(4099, torch.int16)
    synth.dev_normal_bf16(d2.data_ptr(), 4099, 0, st, 1.0, mean=1.0)
    torch.cuda.synchronize()
    assert np.array_equal(d2.cpu().numpy().view(np.uint16), synth.normal_bf16(4099, 0, st, 1.0, mean=1.0))


@pytest.mark.parametrize("R,K", [(2048, 4096), (4096, 2048), (300, 200), (129, 1), (1, 257), (384, 640)])
def test_fp8_blocks_identical(R, K):
    st = synth.stream_id("w1", 2, 17)
    q = _dev(R * K, torch.uint8)
    nsc = ((R + 127) // 128) * ((K + 127) // 128)
    sc = _dev(nsc, torch.float32)
    synth.dev_fp8_blocks(q.data_ptr(), sc.data_ptr(), R, K, 0, st, 0.02)
    torch.cuda.synchronize()
    hq, hs = synth.fp8_blocks(R, K, 0, st, 0.02)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), hs.ravel().view(np.uint32))
    dq = q.cpu().numpy()
    bad = np.flatnonzero(dq != hq.ravel())
    assert bad.size == 0, (bad[:8], dq[bad[:8]], hq.ravel()[bad[:8]])


@pytest.mark.parametrize("R,K", [(2048, 4096), (4096, 2048), (300, 224), (1, 32), (17, 96)])
def test_mxfp4_blocks_identical(R, K):
    st = synth.stream_id("w2", 9, 3)
    q = _dev(R * K // 2, torch.uint8)
    sc = _dev(R * K // 32, torch.uint8)
    synth.dev_mxfp4_blocks(q.data_ptr(), sc.data_ptr(), R, K, 0, st, 0.02)
    torch.cuda.synchronize()
    hq, hs = synth.mxfp4_blocks(R, K, 0, st, 0.02)
    assert np.array_equal(sc.cpu().numpy(), hs.ravel())
    dq = q.cpu().numpy()
    bad = np.flatnonzero(dq != hq.ravel())
    assert bad.size == 0, (bad[:8], dq[bad[:8]], hq.ravel()[bad[:8]])


@pytest.mark.parametrize("rows,kvw,rb", [(1, 21, 32), (77, 576, 592), (300, 80, 96)])
def test_fp8row_kv_identical(rows, kvw, rb):
    st, ss = synth.stream_id("kv_prefill", 4), synth.stream_id("kv_scale", 4)
    d = _dev(rows * rb, torch.uint8)
    synth.dev_fp8row_kv(d.data_ptr(), rows, kvw, rb, 1, st, ss, 1.0)
    torch.cuda.synchronize()
    h = synth.fp8row_kv(rows, kvw, rb, 1, st, ss, 1.0)
    dd = d.cpu().numpy()
    bad = np.flatnonzero(dd != h.ravel())
    assert bad.size == 0, (bad[:8], dd[bad[:8]], h.ravel()[bad[:8]])
