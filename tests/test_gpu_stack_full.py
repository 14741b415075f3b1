"""GPU parity of the 32-layer stack at its real shape: 32 layers of the fp8
384-expert layer (16 routed-expert pools), d_model 4096, vocab 129,280,
T = 6, cache from 4096 positions (capacity 8192) -- the same stack and launch
configuration bench.py times -- and the same stack with MXFP4 experts, every
layer with routed experts of its own, with a bf16 and with an fp8 (E4M3, one
scale per row) cache.

  - steps 0-3 against the oracle composed layer by layer on its own rows and
    caches (free-running): logits normwise <= 5e-2, argmax and expert selection
    by the measured-drift band, committed tokens exact wherever no argmax is a
    near-tie (rules in tests/stack_parity.py);
  - step 0 also layer by layer, each layer's oracle step teacher-forced on the
    GPU's input rows and cache rows at the single-layer bands, and the head
    (129,280 rows: every workgroup streams about 31 row tiles and the argmax is
    merged across the grid) on the GPU's final rows;
  - step 3 runs with every cache row at and past the committed length set to
    NaN: nothing past the step's own rows is read.

The oracle's expert weights are the seeded generator's draws made on the
device and copied to the host (identical bits to the host build, checked in
tests/test_gpu_generator.py), which keeps the oracle's share of the test to
about two minutes."""
import numpy as np
import pytest

import stack_parity as sp
from synth import recipe
from synth.configs import C5, C5X, C5XK

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("s", [C5, C5X, C5XK], ids=lambda s: s.name)
def test_full_stack_32_layers_vocab_129280(s):
    from decoder_megakernel_amd import harness
    print("[stack] building %s on the GPU" % s.name, flush=True)
    st = harness.DeviceStack(s, 0, private_workspaces=True)
    rec = sp.attach_record(st, s)
    print("[stack] host tables", flush=True)
    ws = [recipe.layer_weights_host(s, 0, l, experts=[]) for l in range(s.n_layers)]
    kvs = [recipe.kv_prefill_host(s, 0, l) for l in range(s.n_layers)]
    tables = recipe.stack_tables_host(s, 0)
    draws = sp.DeviceExpertDraws(s, 0, cap=1600)
    L = s.L
    tokens = recipe.tokens_host(s, 0, 0)
    for step in range(4):
        nxt = recipe.tokens_host(s, 0, step + 1)[1:]
        if step == 3:
            for l in range(s.n_layers):
                if s.kv_fmt == "fp8row":
                    st.kv[l][L:] = torch.tensor(0x7F, dtype=torch.uint8)    # E4M3 NaN codes
                else:
                    st.kv[l][L:] = torch.tensor(0x7FC0, dtype=torch.int16)  # bf16 quiet NaN
            torch.cuda.synchronize()
        g = sp.gpu_step(st, s, rec, tokens, nxt)
        assert g["L"] == L
        tag = " %s step %d" % (s.name, step)
        assert np.isfinite(g["logits"]).all() and np.isfinite(g["hidden"]).all()
        o_lg, o_am, _ = sp.oracle_stack_step(s, ws, tables, kvs, tokens, L, g=g, expert_fn=draws, tag=tag)
        com = sp.compare_free_running(s, g, o_lg, o_am, tokens, tag=tag)
        if step == 0:
            sp.check_layers_teacher_forced(st, s, ws, g, expert_fn=draws, tag=tag)
            sp.check_head_teacher_forced(s, tables, g, tag=tag)
        n = len(com)
        assert g["len"] == L + n
        assert g["tok"][0] == com[-1] and list(g["tok"][1:]) == list(nxt)
        L += n
        tokens = np.concatenate([[com[-1]], nxt]).astype(np.int32)


def test_fp8_head_and_sampled_verification_at_vocab_129280():
    """One layer of the stack's shape with an fp8 LM head of 129,280 rows
    (about 31 row tiles per workgroup, the cross-grid merges): a greedy step
    against the oracle (head teacher-forced, then the free-running step), then
    two sampled steps at temperature 1 whose verification matches the oracle's
    on the GPU's logits."""
    import oracle
    from decoder_megakernel_amd import harness
    s = C5.with_(name="stack1_fp8head_V129280", n_layers=1, head_fmt="fp8")
    print("[stack] building %s on the GPU" % s.name, flush=True)
    st = harness.DeviceStack(s, 0, private_workspaces=True)
    rec = sp.attach_record(st, s)
    ws = [recipe.layer_weights_host(s, 0, 0, experts=[])]
    kvs = [recipe.kv_prefill_host(s, 0, 0)]
    tables = recipe.stack_tables_host(s, 0)
    draws = sp.DeviceExpertDraws(s, 0, cap=400)
    L = s.L
    tokens = recipe.tokens_host(s, 0, 0)
    nxt = recipe.tokens_host(s, 0, 1)[1:]
    g = sp.gpu_step(st, s, rec, tokens, nxt)
    sp.check_head_teacher_forced(s, tables, g, tag=" fp8 head")
    o_lg, o_am, _ = sp.oracle_stack_step(s, ws, tables, kvs, tokens, L, g=g, expert_fn=draws, tag=" fp8 head")
    com = sp.compare_free_running(s, g, o_lg, o_am, tokens, tag=" fp8 head")
    assert g["len"] == L + len(com)
    tokens = np.concatenate([[com[-1]], nxt]).astype(np.int32)
    seed, tau = 77, 1.0
    st.model.set_sampling(tau, seed)
    for step in range(2):
        nxt = recipe.tokens_host(s, 0, step + 2)[1:]
        g = sp.gpu_step(st, s, rec, tokens, nxt)
        tag = " fp8 head sampled step %d" % step
        sp.check_head_teacher_forced(s, tables, g, tag=tag, argmax=False)
        sp.check_sampled_verification(s, g, tokens, tau, oracle.sample_key(seed, step), tag=tag)
        tokens = np.concatenate([[g["tok"][0]], nxt]).astype(np.int32)
