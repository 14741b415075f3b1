"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and validates arguments without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_header_function():
    import decoder_megakernel_amd as mk
    lib = ctypes.CDLL(mk.LIB_PATH)
    names = _header_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mk.EXPORTS) == names


def test_abi_version():
    import decoder_megakernel_amd as mk
    assert mk.abi_version() == mk.MK_ABI_VERSION == 4


def _cfg(**kw):
    import decoder_megakernel_amd as mk
    base = dict(d_model=4096, n_heads=32, d_head=128, d_latent=512, d_rope=64, n_experts=384, top_k=8,
                n_shared=1, d_ff=2048, attn_format="bf16", expert_format="fp8", kv_format="bf16")
    base.update(kw)
    return mk.make_config(**base)


def test_valid_configs_pass_and_sizes():
    import decoder_megakernel_amd as mk
    mk.check_config(_cfg())
    cfg = _cfg()
    assert mk.packed_bytes(cfg, mk.MK_T_WQ) == 32 * 192 * 4096 * 2
    assert mk.packed_bytes(cfg, mk.MK_T_WDKV) == 576 * 4096 * 2
    assert mk.packed_bytes(cfg, mk.MK_T_WO) == 4096 * 4096 * 2
    exp = mk.packed_bytes(cfg, mk.MK_T_EXPERT)
    scales = 3 * 16 * 32 * 4
    assert exp == 3 * 2048 * 4096 + ((scales + 255) // 256) * 256
    assert mk.kv_bytes(cfg, 8192) == 8192 * 576 * 2
    f32 = _cfg(d_model=512, n_heads=8, d_head=64, d_latent=128, d_rope=32, n_experts=16, top_k=2, d_ff=256,
               attn_format="f32", expert_format="f32", kv_format="f32")
    mk.check_config(f32)
    assert mk.packed_bytes(f32, mk.MK_T_WR) == 16 * 512 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(abi_version=0), -2),
    (dict(d_model=4000), -8),
    (dict(d_rope=48), -8),
    (dict(n_experts=100), -8),
    (dict(top_k=17), -8),
    (dict(n_shared=2), -8),
    (dict(expert_format=7), -1),
    (dict(attn_format="f32"), -8),
    (dict(d_latent=1024), -8),
    (dict(d_head=0), -1),
    (dict(q_lora_rank=-32), -1),
    (dict(q_lora_rank=100), -8),
    (dict(q_lora_rank=8192), -8),
    (dict(kv_norm=1), -8),
    (dict(kv_norm=2, q_lora_rank=256), -1),
    (dict(idx_topk=-1), -1),
    (dict(idx_topk=2048, idx_heads=64, idx_dim=128, idx_max_rows=0), -1),
    (dict(idx_topk=2048, idx_heads=60, idx_dim=128, idx_max_rows=70000), -8),
    (dict(idx_topk=2048, idx_heads=64, idx_dim=128, idx_max_rows=70001), -1),
    (dict(idx_topk=2048, idx_heads=64, idx_dim=128, idx_max_rows=70000, kv_format="f32"), -8),
    (dict(idx_topk=2048, idx_heads=32, idx_dim=160, idx_max_rows=70000), -8),
    (dict(kv_max_rows=-1), -1),
])
def test_invalid_configs_are_refused(kw, code):
    import decoder_megakernel_amd as mk
    with pytest.raises(mk.MkError) as ei:
        mk.check_config(_cfg(**kw))
    assert ei.value.code == code
    assert mk.last_error()


def test_null_arguments_are_refused_without_a_device():
    import decoder_megakernel_amd as mk
    lib = mk.lib
    assert lib.mk_decode_step(None, None, 6, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_layer_init(None, None, None, None, 0, None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_model_step(None, None, 6, None, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_get_stats(None, None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_sync_status(None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_model_sync_status(None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_model_reset(None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_model_set_hidden_record(None, None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_layer_reset(None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_head_packed_bytes(129280, 4096, None) == mk.MK_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.mk_head_packed_bytes(129280, 4096, ctypes.byref(n)) == 0
    assert n.value == 129280 * 4096 * 2
    assert lib.mk_head_packed_bytes(129281, 4096, ctypes.byref(n)) == mk.MK_ERR_INVALID_ARG
    # fp8 head: E4M3 tiles, then the 128x128 block scales at a 256-byte boundary
    assert lib.mk_head_packed_bytes_fmt(129280, 4096, mk.MK_FMT_FP8_B128, ctypes.byref(n)) == 0
    assert n.value == 129280 * 4096 + 1010 * 32 * 4
    assert lib.mk_head_packed_bytes_fmt(129280, 4096, mk.MK_FMT_MXFP4, ctypes.byref(n)) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_pack_head_fp8(129280, 4096, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_model_set_sampling(None, 1.0, 0) == mk.MK_ERR_INVALID_ARG
    assert lib.mk_model_init_ex(None, 1, None, None, mk.MK_FMT_BF16, None, 16, None, 8, None, None, None) \
        == mk.MK_ERR_INVALID_ARG


def test_no_device_is_an_error_not_a_crash():
    import decoder_megakernel_amd as mk
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(mk.MkError):
        mk.query_device(0)


def test_lowrank_query_config_and_packed_sizes():
    import decoder_megakernel_amd as mk
    cfg = _cfg(q_lora_rank=1536, kv_norm=1)
    mk.check_config(cfg)
    assert mk.packed_bytes(cfg, mk.MK_T_WDQ) == 1536 * 4096 * 2
    assert mk.packed_bytes(cfg, mk.MK_T_WUQ) == 32 * 192 * 1536 * 2
    with pytest.raises(mk.MkError) as ei:
        mk.packed_bytes(_cfg(), mk.MK_T_WDQ)
    assert ei.value.code == mk.MK_ERR_INVALID_ARG


def test_sparse_attention_config_and_sizes():
    import decoder_megakernel_amd as mk
    cfg = _cfg(idx_heads=64, idx_dim=128, idx_topk=2048, idx_max_rows=70000)
    mk.check_config(cfg)
    assert mk.packed_bytes(cfg, mk.MK_T_WIDX) == (64 * 128 + 64 + 128) * 4096 * 2
    assert mk.kv_bytes(cfg, 1000) == 1000 * (512 + 64 + 128) * 2
    # an fp8 row holds the 704 codes, the scale and padding to 16 bytes
    k8 = _cfg(idx_heads=64, idx_dim=128, idx_topk=2048, idx_max_rows=70000, kv_format="fp8row")
    mk.check_config(k8)
    assert mk.kv_bytes(k8, 1000) == 1000 * 720
    mk.check_config(_cfg(idx_heads=64, idx_dim=128, idx_topk=2048, idx_max_rows=70000, kv_format="fp8row",
                         expert_format="mxfp4", q_lora_rank=1536, kv_norm=1))
    mk.check_config(_cfg(idx_heads=64, idx_dim=128, idx_topk=2048, idx_max_rows=70000, kv_format="fp8row",
                         expert_format="bf16"))
