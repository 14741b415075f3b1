"""GPU parity of the stack step (embedding, layers, final norm + LM head +
argmax + greedy acceptance or sampled verification, bf16 or fp8 head,
device-resident KV length) against the CPU oracle, at a small shape: 3 layers
sharing 2 routed-expert pools, vocab 2048.  Rules in
tests/stack_parity.py (per-layer checks teacher-forced on the GPU's state at
the single-layer selection band; free-running composition with the measured
drift band; the oracle follows the GPU at a near-tie instead of giving up)."""
import numpy as np
import pytest

import oracle
import stack_parity as sp
from synth import recipe
from synth.configs import LayerShape

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# 3 layers sharing 2 routed-expert pools (layer 2 reuses layer 0's pool).
STACK_SMALL = LayerShape("stack3_fp8", d=640, n_h=6, d_h=64, d_c=256, d_r=64, E=48, top_k=6, n_shared=1,
                         f=384, T=6, L=40, attn_fmt="bf16", exp_fmt="fp8", kv_fmt="bf16", n_layers=3, V=2048,
                         steps=3, kv_capacity=128, n_pools=2)


def _setup(s, seed=0):
    from decoder_megakernel_amd import harness
    print("[stack] building %s" % s.name, flush=True)
    st = harness.DeviceStack(s, seed, private_workspaces=True)
    rec = sp.attach_record(st, s)
    ws = [recipe.layer_weights_host(s, seed, l) for l in range(s.n_layers)]
    kvs = [recipe.kv_prefill_host(s, seed, l) for l in range(s.n_layers)]
    tables = recipe.stack_tables_host(s, seed)
    return st, rec, ws, kvs, tables


def test_stack_steps_match_oracle():
    s = STACK_SMALL
    st, rec, ws, kvs, tables = _setup(s)
    L = s.L
    tokens = recipe.tokens_host(s, 0, 0)
    for step in range(s.steps):
        nxt = recipe.tokens_host(s, 0, step + 1)[1:]
        g = sp.gpu_step(st, s, rec, tokens, nxt)
        assert g["L"] == L
        tag = " step %d" % step
        sp.check_layers_teacher_forced(st, s, ws, g, tag=tag)
        sp.check_head_teacher_forced(s, tables, g, tag=tag)
        o_lg, o_am, _ = sp.oracle_stack_step(s, ws, tables, kvs, tokens, L, g=g, tag=tag)
        com = sp.compare_free_running(s, g, o_lg, o_am, tokens, tag=tag)
        n = len(com)
        assert g["len"] == L + n
        assert g["tok"][0] == com[-1] and list(g["tok"][1:]) == list(nxt)
        L += n
        tokens = np.concatenate([[com[-1]], nxt]).astype(np.int32)


# Sparse attention over the fp8 cache in the stack: 16 heads (a query tile per
# verify row), each verify row keeps 24 of its 41..58 visible rows.
STACK_SPARSE = STACK_SMALL.with_(name="stack3_sparse_fp8kv", n_h=16, kv_fmt="fp8row", idx_heads=16, idx_dim=64,
                                 idx_topk=24)


def test_sparse_fp8kv_stack_steps_match_oracle_teacher_forced():
    """The stack step with sparse-attention layers over the fp8 cache (the
    device-resident length feeding the indexer and the top-k): every layer
    against the oracle on the GPU's own input rows and cache (kept rows checked
    as in the single-layer tests), the head on the GPU's final rows, and the
    length advanced by the committed count."""
    s = STACK_SPARSE
    st, rec, ws, kvs, tables = _setup(s)
    L = s.L
    tokens = recipe.tokens_host(s, 0, 0)
    for step in range(s.steps):
        nxt = recipe.tokens_host(s, 0, step + 1)[1:]
        g = sp.gpu_step(st, s, rec, tokens, nxt)
        assert g["L"] == L
        tag = " sparse step %d" % step
        errs = sp.check_layers_teacher_forced(st, s, ws, g, tag=tag)
        assert all("kept_rows_differing" in e for e in errs)
        sp.check_head_teacher_forced(s, tables, g, tag=tag)
        n = int(g["com"][0])
        com = list(g["com"][1:1 + n])
        assert com == list(oracle.greedy_accept(tokens, g["am"])) and g["len"] == L + n
        assert g["tok"][0] == com[-1] and list(g["tok"][1:]) == list(nxt)
        L += n
        tokens = np.concatenate([[com[-1]], nxt]).astype(np.int32)


def test_all_drafts_accepted_when_drafts_follow_greedy_decoding():
    """Drafts built by single-token greedy oracle steps: the oracle accepts every
    one of them (causal invariant), and so does the GPU unless an argmax is a
    near-tie within the measured logit difference (asserted)."""
    s = STACK_SMALL
    st, rec, ws, kvs, tables = _setup(s)
    kv_chain = [k.copy() for k in kvs]
    one = s.with_(T=1)
    chain = [int(recipe.tokens_host(s, 0, 0)[0])]
    for i in range(s.T - 1):
        _, am, _ = sp.oracle_stack_step(one, ws, tables, kv_chain, np.array([chain[-1]], np.int32), s.L + i)
        chain.append(int(am[0]))
    tokens = np.array(chain, np.int32)
    g = sp.gpu_step(st, s, rec, tokens)
    o_lg, o_am, _ = sp.oracle_stack_step(s, ws, tables, kvs, tokens, s.L, g=g, tag=" chain")
    o_com = list(oracle.greedy_accept(tokens, o_am))
    assert len(o_com) == s.T            # the oracle accepts every draft (causal invariant)
    com = sp.compare_free_running(s, g, o_lg, o_am, tokens, tag=" chain")
    if com == o_com:
        assert g["com"][0] == s.T and g["len"] == s.L + s.T
    else:
        # only a near-tie argmax may cut the chain (compare_free_running asserted the band)
        assert g["len"] == s.L + len(com)


def test_poisoned_rows_past_the_committed_length_are_never_read():
    """Cache rows at and beyond the committed length hold NaN before a step: the
    step overwrites its own T rows and reads nothing past them, so no NaN
    reaches the logits, and the step matches the oracle (which never had NaN)."""
    s = STACK_SMALL
    st, rec, ws, kvs, tables = _setup(s)
    L = s.L
    for l in range(s.n_layers):
        st.kv[l][L:] = torch.tensor(0x7FC0, dtype=torch.int16)      # bf16 quiet NaN
    torch.cuda.synchronize()
    tokens = recipe.tokens_host(s, 0, 0)
    g = sp.gpu_step(st, s, rec, tokens)
    assert np.isfinite(g["logits"]).all() and np.isfinite(g["hidden"]).all()
    for l in range(s.n_layers):
        assert np.isfinite(g["kv_new"][l]).all()
    sp.check_layers_teacher_forced(st, s, ws, g, tag=" poisoned")
    o_lg, o_am, _ = sp.oracle_stack_step(s, ws, tables, kvs, tokens, L, g=g, tag=" poisoned")
    sp.compare_free_running(s, g, o_lg, o_am, tokens, tag=" poisoned")


def test_fp8_head_stack_steps_match_oracle():
    s = STACK_SMALL.with_(name="stack3_fp8_fp8head", head_fmt="fp8", steps=2)
    st, rec, ws, kvs, tables = _setup(s)
    L = s.L
    tokens = recipe.tokens_host(s, 0, 0)
    for step in range(s.steps):
        nxt = recipe.tokens_host(s, 0, step + 1)[1:]
        g = sp.gpu_step(st, s, rec, tokens, nxt)
        tag = " fp8 head step %d" % step
        sp.check_head_teacher_forced(s, tables, g, tag=tag)
        o_lg, o_am, _ = sp.oracle_stack_step(s, ws, tables, kvs, tokens, L, g=g, tag=tag)
        com = sp.compare_free_running(s, g, o_lg, o_am, tokens, tag=tag)
        assert g["len"] == L + len(com)
        L += len(com)
        tokens = np.concatenate([[com[-1]], nxt]).astype(np.int32)


@pytest.mark.parametrize("head_fmt", ["bf16", "fp8"])
def test_sampled_verification_matches_oracle(head_fmt):
    """Temperature 1 with seeded drafts (rejected: each step commits one draw
    from the target without the draft), three steps in a row: the device step
    counter keys each step's draws."""
    s = STACK_SMALL.with_(name="stack3_sampled_" + head_fmt, head_fmt=head_fmt)
    st, rec, ws, kvs, tables = _setup(s)
    seed, tau = 123, 1.0
    st.model.set_sampling(tau, seed)
    tokens = recipe.tokens_host(s, 0, 0)
    for step in range(3):
        nxt = recipe.tokens_host(s, 0, step + 1)[1:]
        g = sp.gpu_step(st, s, rec, tokens, nxt)
        tag = " sampled %s step %d" % (head_fmt, step)
        sp.check_head_teacher_forced(s, tables, g, tag=tag, argmax=False)
        n = sp.check_sampled_verification(s, g, tokens, tau, oracle.sample_key(seed, step), tag=tag)
        tokens = np.concatenate([[g["tok"][0]], nxt]).astype(np.int32)
        assert n >= 1


def test_sampled_verification_accepts_a_greedy_chain_at_low_temperature():
    """Drafts that follow greedy decoding, verified at temperature 0.01: the
    target puts almost all its mass on the greedy token, so the drafts are
    accepted (as the oracle decides on the same logits)."""
    s = STACK_SMALL
    st, rec, ws, kvs, tables = _setup(s)
    kv_chain = [k.copy() for k in kvs]
    one = s.with_(T=1)
    chain = [int(recipe.tokens_host(s, 0, 0)[0])]
    for i in range(s.T - 1):
        _, am, _ = sp.oracle_stack_step(one, ws, tables, kv_chain, np.array([chain[-1]], np.int32), s.L + i)
        chain.append(int(am[0]))
    tokens = np.array(chain, np.int32)
    seed, tau = 5, 0.01
    st.model.set_sampling(tau, seed)
    g = sp.gpu_step(st, s, rec, tokens)
    n = sp.check_sampled_verification(s, g, tokens, tau, oracle.sample_key(seed, 0), tag=" low-temperature chain")
    assert n >= 2
    st.model.set_sampling(0.0, 0)
