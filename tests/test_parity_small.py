"""GPU parity against the CPU oracle on small inputs that still span several
chunks/tiles and ragged tails: prefill (vector and MFMA kernels), decode, state
init, short conv.  Every call goes through libkda.so's C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from kda_testutil import (TOL_BF16, TOL_F32, dev, gpu_or_skip, gpu_prefill, np64, oracle_on,
                          assert_parity, rel_fro)

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def test_tiny_f32_prefill():
    """Tiny fp32 recurrence: B=1, H=2, T=64, d=16, chunk 16."""
    kda()
    inp = workloads.tiny_f32()
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_F32,
                  f"tiny f32 prefill")


def test_tiny_f32_as_decode_steps():
    """The same workload run as 64 successive one-token decode steps."""
    m = kda()
    inp = workloads.tiny_f32()
    state = torch.zeros((1, inp.H, inp.d, inp.d), device="cuda")
    m.kda_state_init(state)
    outs = []
    for t in range(inp.T):
        sl = slice(t, t + 1)
        outs.append(m.kda_decode_step(dev(inp.q[sl]), dev(inp.k[sl]), dev(inp.v[sl]),
                                      dev(inp.g[sl]), dev(inp.beta[sl]), state))
    torch.cuda.synchronize()
    o = torch.cat(outs)
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(state), S_ref, inp.cu_seqlens, TOL_F32,
                  f"tiny f32 decode steps")


RAGGED = [37, 0, 100, 1, 64, 129]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_prefill_ragged(d, chunk, dtype):
    """Packed ragged sequences (incl. empty and 1-token), nonzero initial states."""
    kda()
    inp = workloads.recurrence_inputs(RAGGED, H=3, d=d, dtype=dtype, chunk=chunk, g_mu=2.0,
                                      g_sigma=0.5, s0_std=0.5, seed=7 + d + chunk)
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_on(inp)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, tol, f"d={d} C={chunk} {dtype}")


# workspace argument of the binding: "auto" runs the two-kernel matrix-core path
# (chunk-parallel operand kernel, then the state pass), None the fused kernel
PATHS = {"split": "auto", "fused": None}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("H", [8, 3])
def test_mfma_prefill_multichunk(H, path):
    """bf16, d=128, chunk 64 (matrix-core kernels): lengths around chunk multiples,
    nonzero states; H=8 uses the XCD-grouped placement, H=3 the plain one."""
    kda()
    inp = workloads.recurrence_inputs([64, 65, 127, 128, 1, 300], H=H, d=128, dtype="bf16",
                                      chunk=64, g_mu=3.0, g_sigma=1.0, s0_std=0.5, seed=99 + H)
    o, S = gpu_prefill(inp, workspace=PATHS[path])
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16,
                  f"mfma {path} H={H}")


@pytest.mark.parametrize("path", list(PATHS))
def test_mfma_prefill_multiwindow(path):
    """Sequences longer than one 32-chunk window of the two-kernel path (state
    carried across windows), next to empty, 1-token and ragged ones."""
    kda()
    inp = workloads.recurrence_inputs([4480, 2100, 64, 0, 1, 130], H=2, d=128, dtype="bf16",
                                      chunk=64, g_mu=3.0, g_sigma=1.0, s0_std=0.5, seed=123)
    o, S = gpu_prefill(inp, workspace=PATHS[path])
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16,
                  f"mfma {path} multiwindow")


@pytest.mark.parametrize("path", list(PATHS))
def test_mfma_prefill_many_short_sequences(path):
    """600 packed sequences of 0..600 tokens, H=2: the two-kernel path's window
    shrinks to 2 chunks (the tile budget is shared by every sequence and head),
    so most sequences span several windows; every sequence checked."""
    kda()
    lens = np.random.default_rng(5).integers(0, 601, size=600).tolist()
    inp = workloads.recurrence_inputs(lens, H=2, d=128, dtype="bf16", chunk=64, g_mu=3.0,
                                      g_sigma=1.0, s0_std=0.3, seed=125)
    o, S = gpu_prefill(inp, workspace=PATHS[path])
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16,
                  f"mfma {path} 600 sequences")


@pytest.mark.parametrize("path", list(PATHS))
def test_prefill_empty_sequences_keep_state(path):
    """Zero-length sequences: final state equals the initial state, bit for bit."""
    kda()
    inp = workloads.recurrence_inputs([0, 5, 0], H=2, d=128, dtype="bf16", chunk=64,
                                      s0_std=1.0, seed=5)
    o, S = gpu_prefill(inp, workspace=PATHS[path])
    S0 = inp.S0
    assert torch.equal(S.cpu()[0], S0[0]) and torch.equal(S.cpu()[2], S0[2])


def test_prefill_all_empty():
    """Only empty sequences (T = 0): final states are copies of the initial ones."""
    kda()
    inp = workloads.recurrence_inputs([0, 0], H=2, d=128, dtype="bf16", chunk=64,
                                      s0_std=1.0, seed=6)
    o, S = gpu_prefill(inp)
    assert o.numel() == 0 and torch.equal(S.cpu(), inp.S0)


def test_state_init():
    m = kda()
    st = torch.full((3, 2, 32, 32), 7.0, device="cuda")
    m.kda_state_init(st)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st).item() == 0
    src = torch.randn((3, 2, 32, 32), device="cuda")
    m.kda_state_init(st, src)
    torch.cuda.synchronize()
    assert torch.equal(st, src)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_decode_slots(d, dtype):
    """Decode with a slot permutation into a larger state pool: the addressed slots
    match the oracle; every other slot is untouched, bit for bit."""
    m = kda()
    B, H, n_slots = 5, 3, 9
    inp = workloads.recurrence_inputs([1] * B, H=H, d=d, dtype=dtype, s0_std=0.3, seed=40 + d)
    pool = torch.randn((n_slots, H, d, d), generator=torch.Generator().manual_seed(d)) * 0.3
    slots = torch.tensor([7, 0, 4, 2, 8], dtype=torch.int32)
    pool[slots.long()] = inp.S0
    state = dev(pool)
    o = m.kda_decode_step(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state,
                          slot_idx=dev(slots))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_on(inp)
    st = state.cpu()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o), o_ref, np64(st[slots.long()]), S_ref, inp.cu_seqlens, tol,
                  f"decode d={d} {dtype}")
    untouched = [s for s in range(n_slots) if s not in slots.tolist()]
    assert torch.equal(st[untouched], pool[untouched])


def test_decode_out_of_range_slot():
    """A slot outside the pool leaves every state untouched and gives NaN output."""
    m = kda()
    B, H, d = 2, 2, 128
    inp = workloads.recurrence_inputs([1] * B, H=H, d=d, dtype="bf16", seed=3)
    state = torch.randn((2, H, d, d), device="cuda")
    before = state.clone()
    slots = torch.tensor([1, 5], dtype=torch.int32, device="cuda")
    o = m.kda_decode_step(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state,
                          slot_idx=slots)
    torch.cuda.synchronize()
    assert torch.isnan(o[1].float()).all() and not torch.isnan(o[0].float()).any()
    assert torch.equal(state[0], before[0])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("C,l2", [(512, 0), (512, 128), (2560, 128), (384, 96)])
def test_short_conv_prefill(C, l2, dtype):
    """Conv (+ per-head L2) over packed ragged sequences with incoming tails;
    outgoing tails are copies of inputs, so they must match bit for bit.  Heads
    of 128 channels run the 16-byte-per-lane kernel (2560 channels: a partly
    filled last workgroup); heads of 96, not a power of two in lanes, the
    general one."""
    m = kda()
    lens = [1, 40, 0, 2, 33]
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = workloads.normal((T, C), 11, 0).to(tdt)
    w = workloads.normal((C, 4), 11, 1, 0.0, 0.5)
    tail = workloads.normal((len(lens), 3, C), 11, 2).to(tdt)
    tail_out = torch.empty_like(tail).cuda()
    y = m.kda_short_conv_prefill(dev(x), dev(w), cu_seqlens=dev(cu), cu_seqlens_host=cu,
                                 l2_head_dim=l2, conv_tail_in=dev(tail),
                                 conv_tail_out=tail_out)
    torch.cuda.synchronize()
    y_ref, tail_ref = oracle.short_conv(np64(x), np64(w), cu_seqlens=cu.numpy(),
                                        tail=np64(tail))
    if l2:
        y_ref = oracle.l2norm_heads(y_ref, l2, eps=1e-6)
    err = rel_fro(np64(y), y_ref)
    print(f"conv prefill C={C} l2={l2} {dtype}: {err:.2e}")
    assert err <= (1e-6 if dtype == "f32" else 1e-2)
    assert np.array_equal(np64(tail_out), tail_ref)


def test_short_conv_prefill_long_runs():
    """131072 tokens x 2048 bf16 channels: enough tokens that each workgroup of
    the 16-byte kernel walks 128 of them, over ragged sequences (empty ones
    included) that start and end inside those runs.  Checked on sampled tokens
    (every sequence's first four, the ends, and random ones); output token t
    needs only inputs t-3..t of its sequence, or the incoming tail."""
    m = kda()
    C, l2 = 2048, 128
    rng = np.random.default_rng(14)
    lens = rng.integers(1, 700, size=400)
    lens[::37] = 0
    lens[-1] += 131072 - int(lens.sum())
    assert lens[-1] > 0
    T = int(lens.sum())
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    x = workloads.normal((T, C), 14, 0).to(torch.bfloat16)
    w = workloads.normal((C, 4), 14, 1, 0.0, 0.5)
    tail = workloads.normal((len(lens), 3, C), 14, 2).to(torch.bfloat16)
    y = m.kda_short_conv_prefill(dev(x), dev(w), cu_seqlens=dev(cu), cu_seqlens_host=cu,
                                 l2_head_dim=l2, conv_tail_in=dev(tail))
    torch.cuda.synchronize()
    y = y.cpu()
    cuv = cu.numpy().astype(np.int64)
    picks = set(rng.integers(0, T, size=200).tolist())
    for n in range(len(lens)):
        for t in range(cuv[n], min(cuv[n] + 4, cuv[n + 1])):
            picks.add(t)
        if cuv[n + 1] > cuv[n]:
            picks.add(int(cuv[n + 1] - 1))
    w64 = np64(w)
    worst = 0.0
    for t in sorted(picks):
        n = int(np.searchsorted(cuv, t, side="right") - 1)
        lo = max(int(cuv[n]), t - 3)
        y_ref, _ = oracle.short_conv(np64(x[lo:t + 1]), w64,
                                     tail=np64(tail[n:n + 1]) if lo == cuv[n] else None)
        y_ref = oracle.l2norm_heads(y_ref[-1:], l2, eps=1e-6)
        worst = max(worst, rel_fro(np64(y[t:t + 1]), y_ref))
    print(f"conv prefill {T} x {C}, {len(picks)} sampled tokens: worst {worst:.2e}")
    assert worst <= 1e-2


def test_short_conv_prefill_in_place_tail():
    """conv_tail_out may be the same buffer as conv_tail_in."""
    m = kda()
    lens = [2, 9]
    T, C = sum(lens), 256
    cu = torch.tensor([0, 2, 11], dtype=torch.int32)
    x = workloads.normal((T, C), 12, 0).to(torch.bfloat16)
    w = workloads.normal((C, 4), 12, 1)
    tail = workloads.normal((2, 3, C), 12, 2).to(torch.bfloat16)
    t_dev = dev(tail)
    m.kda_short_conv_prefill(dev(x), dev(w), cu_seqlens=dev(cu), cu_seqlens_host=cu,
                             conv_tail_in=t_dev, conv_tail_out=t_dev)
    torch.cuda.synchronize()
    _, tail_ref = oracle.short_conv(np64(x), np64(w), cu_seqlens=cu.numpy(), tail=np64(tail))
    assert np.array_equal(np64(t_dev), tail_ref)


@pytest.mark.parametrize("l2", [0, 128])
def test_short_conv_decode(l2):
    """Decode conv over a slot pool equals the prefill conv of the history plus the
    new token; the tail shifts in place."""
    m = kda()
    B, C, n_slots = 3, 384, 5
    slots = torch.tensor([4, 0, 2], dtype=torch.int32)
    pool = workloads.normal((n_slots, 3, C), 13, 0).to(torch.bfloat16)
    x = workloads.normal((B, C), 13, 1).to(torch.bfloat16)
    w = workloads.normal((C, 4), 13, 2)
    tail = dev(pool)
    y = m.kda_short_conv_decode(dev(x), dev(w), tail, slot_idx=dev(slots), l2_head_dim=l2)
    torch.cuda.synchronize()
    for b in range(B):
        s = int(slots[b])
        y_ref, t_ref = oracle.short_conv(np64(x[b:b + 1]), np64(w), tail=np64(pool[s:s + 1]))
        if l2:
            y_ref = oracle.l2norm_heads(y_ref, l2, eps=1e-6)
        assert rel_fro(np64(y[b:b + 1]), y_ref) <= 1e-2
        assert np.array_equal(np64(tail[s]), t_ref[0])
    untouched = [1, 3]
    assert torch.equal(tail.cpu()[untouched], pool[untouched])
