"""GPU parity of multi-token decode (kda_decode_tokens: n_tok consecutive tokens
per sequence, one state read and one write) against the CPU oracle, through the
C ABI.  The oracle runs the same tokens as packed sequences of n_tok tokens, so
its packed layout [B * n_tok, H, d] is the decode layout [B, n_tok, H, d]."""
import numpy as np
import pytest
import torch

import workloads
from kda_testutil import (TOL_BF16, TOL_F32, dev, gpu_or_skip, np64, oracle_on,
                          assert_parity, rel_fro)

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def as_tokens(x, B, n_tok):
    """[B * n_tok, ...] packed sequence-major -> [B, n_tok, ...]."""
    return x.reshape((B, n_tok) + tuple(x.shape[1:]))


def run_tokens(m, inp, B, n_tok, state, slot_idx=None, token_states=None):
    t = lambda x: dev(as_tokens(x, B, n_tok))
    return m.kda_decode_tokens(t(inp.q), t(inp.k), t(inp.v), t(inp.g), t(inp.beta), state,
                               slot_idx=slot_idx, token_states=token_states)


@pytest.mark.parametrize("n_tok", [1, 4])
@pytest.mark.parametrize("d,dtype", [(16, "f32"), (16, "bf16"), (32, "f32"), (64, "bf16"),
                                     (128, "bf16"), (128, "f32")])
def test_decode_tokens_matches_oracle(d, dtype, n_tok):
    """B sequences advanced by n_tok tokens through a slot permutation into a
    larger pool: outputs of every token and the final states match the oracle;
    every other slot is untouched, bit for bit."""
    m = kda()
    B, H, n_slots = 5, 3, 9
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype=dtype, s0_std=0.3,
                                      seed=60 + d + n_tok)
    pool = torch.randn((n_slots, H, d, d), generator=torch.Generator().manual_seed(d)) * 0.3
    slots = torch.tensor([7, 0, 4, 2, 8], dtype=torch.int32)
    pool[slots.long()] = inp.S0
    state = dev(pool)
    o, _ = run_tokens(m, inp, B, n_tok, state, slot_idx=dev(slots))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_on(inp)
    st = state.cpu()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o).reshape(B * n_tok, H, d), o_ref, np64(st[slots.long()]), S_ref,
                  inp.cu_seqlens, tol, f"decode_tokens d={d} {dtype} n_tok={n_tok}")
    untouched = [s for s in range(n_slots) if s not in slots.tolist()]
    assert torch.equal(st[untouched], pool[untouched])


@pytest.mark.parametrize("dtype,n_tok", [("bf16", 6), ("f32", 9), ("bf16", 64)])
def test_decode_tokens_several_groups(dtype, n_tok):
    """d = 128 over more tokens than the four of the speculative-decoding
    workload, up to the 64-token maximum, through a slot permutation: outputs
    and final states match the oracle, other slots are untouched."""
    m = kda()
    B, H, n_slots, d = 3, 2, 5, 128
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype=dtype, s0_std=0.3,
                                      seed=80 + n_tok)
    pool = torch.randn((n_slots, H, d, d), generator=torch.Generator().manual_seed(81)) * 0.3
    slots = torch.tensor([4, 0, 2], dtype=torch.int32)
    pool[slots.long()] = inp.S0
    state = dev(pool)
    o, _ = run_tokens(m, inp, B, n_tok, state, slot_idx=dev(slots))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_on(inp)
    st = state.cpu()
    assert_parity(np64(o).reshape(B * n_tok, H, d), o_ref, np64(st[slots.long()]), S_ref,
                  inp.cu_seqlens, TOL_F32 if dtype == "f32" else TOL_BF16,
                  f"decode_tokens d=128 {dtype} n_tok={n_tok}")
    untouched = [s for s in range(n_slots) if s not in slots.tolist()]
    assert torch.equal(st[untouched], pool[untouched])


@pytest.mark.parametrize("d,dtype", [(16, "f32"), (128, "bf16")])
def test_decode_tokens_snapshots_match_prefixes(d, dtype):
    """token_states[b, j] is sequence b's state after token j: it matches the
    oracle run on the first j + 1 tokens, and the last one is the final state."""
    m = kda()
    B, n_tok, H = 3, 4, 2
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype=dtype, s0_std=0.3,
                                      seed=71 + d)
    state = dev(inp.S0)
    o, snaps = run_tokens(m, inp, B, n_tok, state, token_states=True)
    torch.cuda.synchronize()
    snaps = snaps.cpu()
    for j in range(n_tok):
        rows = torch.tensor([b * n_tok + i for b in range(B) for i in range(j + 1)])
        pre = workloads.RecurrenceInputs(inp.q[rows], inp.k[rows], inp.v[rows], inp.g[rows],
                                         inp.beta[rows],
                                         torch.arange(0, B * (j + 1) + 1, j + 1,
                                                      dtype=torch.int32),
                                         inp.S0, dtype, inp.chunk)
        _, S_ref = oracle_on(pre)
        assert_parity(None, None, np64(snaps[:, j]), S_ref, range(B + 1),
                      TOL_F32 if dtype == "f32" else TOL_BF16,
                      f"d={d} {dtype}, snapshot after token {j}")
    assert torch.equal(snaps[:, -1], state.cpu())


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_decode_tokens_equals_single_steps(state_dtype):
    """One call over n_tok tokens against n_tok single-token decode steps.
    fp32 states: the call keeps the state in fp32 registers between tokens,
    exactly what a round trip through memory holds, so the two agree to fp32
    rounding (at d = 128 the single-token kernel sums columns over 32 row
    groups of 4 rows, the multi-token kernel over 8 of 16).  bf16 states:
    single steps round the state after every token and the call only once at
    its end, so only the first token's outputs are comparable (64 row groups
    against 16: fp32 rounding, then one bf16 rounding of o)."""
    m = kda()
    B, n_tok, H, d = 4, 3, 2, 128
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype="bf16", s0_std=0.3, seed=72)
    s_multi = dev(inp.S0).to(state_dtype)
    o_multi, _ = run_tokens(m, inp, B, n_tok, s_multi)
    s_single = dev(inp.S0).to(state_dtype)
    outs = []
    for j in range(n_tok):
        rows = torch.arange(B) * n_tok + j
        outs.append(m.kda_decode_step(dev(inp.q[rows]), dev(inp.k[rows]), dev(inp.v[rows]),
                                      dev(inp.g[rows]), dev(inp.beta[rows]), s_single))
    torch.cuda.synchronize()
    o_single = torch.stack(outs, dim=1)
    # outputs are bf16: fp32 regrouping may move one across a rounding boundary
    if state_dtype == torch.bfloat16:
        o_multi, o_single = o_multi[:, :1], o_single[:, :1]
    assert torch.allclose(o_multi.float(), o_single.float(), rtol=2.0 ** -7, atol=1e-6)
    eo = rel_fro(np64(o_multi), np64(o_single))
    print(f"multi vs single steps, {state_dtype} state: o {eo:.2e}")
    assert eo <= 1e-4
    if state_dtype == torch.float32:
        es = rel_fro(np64(s_multi), np64(s_single))
        print(f"  S {es:.2e}")
        assert es <= 1e-6


def test_decode_tokens_out_of_range_slot():
    """A slot outside the pool: all n_tok outputs of that sequence are NaN and no
    state changes."""
    m = kda()
    B, n_tok, H, d = 2, 3, 2, 64
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype="bf16", seed=73)
    state = torch.randn((2, H, d, d), device="cuda")
    before = state.clone()
    slots = torch.tensor([1, 5], dtype=torch.int32, device="cuda")
    o, _ = run_tokens(m, inp, B, n_tok, state, slot_idx=slots)
    torch.cuda.synchronize()
    assert torch.isnan(o[1].float()).all() and not torch.isnan(o[0].float()).any()
    assert torch.equal(state[0], before[0])
