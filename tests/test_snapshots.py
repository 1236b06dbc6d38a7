"""GPU parity of chunk-aligned state snapshots taken during prefill (the states a
prefix cache keeps for recurrent layers) through the C ABI: snapshot [n, j] is
sequence n's state after its first (j + 1) * interval tokens, checked against
the oracle run on exactly that prefix; entries a sequence is too short for keep
their previous contents bit for bit; and taking snapshots changes neither the
outputs nor the final states."""
import pytest
import torch

import workloads
from kda_testutil import (TOL_BF16, TOL_F32, assert_parity, dev, gpu_or_skip, np64, oracle_on,
                          parity_stats)

pytestmark = pytest.mark.gpu

SENTINEL = 7.25

# (name, d, dtype, chunk, workspace): the two matrix-core paths (bf16, d = 128,
# chunk 64, with and without a workspace) and the fp32 vector kernel.
PATHS = [
    ("split", 128, "bf16", 64, "auto"),
    ("fused", 128, "bf16", 64, None),
    ("vector-bf16", 64, "bf16", 64, "auto"),
    ("vector-f32", 128, "f32", 32, "auto"),
]


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def prefix(inp, n, length):
    """Sequence n of inp cut to its first `length` tokens, as a one-sequence input."""
    b = int(inp.cu_seqlens[n])
    rows = slice(b, b + length)
    S0 = None if inp.S0 is None else inp.S0[n:n + 1]
    return workloads.RecurrenceInputs(inp.q[rows], inp.k[rows], inp.v[rows], inp.g[rows],
                                      inp.beta[rows],
                                      torch.tensor([0, length], dtype=torch.int32), S0,
                                      inp.dtype, inp.chunk)


def run(m, inp, workspace, snaps=None, interval=0):
    out = m.kda_prefill_chunked(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                                cu_seqlens=dev(inp.cu_seqlens), cu_seqlens_host=inp.cu_seqlens,
                                chunk=inp.chunk, initial_state=dev(inp.S0), workspace=workspace,
                                snapshots=snaps, snap_interval=interval)
    torch.cuda.synchronize()
    return out


def check(m, inp, workspace, interval, tol, label):
    lens = [int(inp.cu_seqlens[i + 1] - inp.cu_seqlens[i]) for i in range(len(inp.cu_seqlens) - 1)]
    H, d = inp.q.shape[1], inp.q.shape[2]
    cap = max(lens) // interval + 1  # one entry more than the longest sequence fills
    snaps = torch.full((len(lens), cap, H, d, d), SENTINEL, device="cuda")
    o, S, out = run(m, inp, workspace, snaps, interval)
    assert out is snaps
    o_plain, S_plain = run(m, inp, workspace)
    assert torch.equal(o, o_plain) and torch.equal(S, S_plain)
    snaps = snaps.cpu()
    worst, taken = 0.0, 0
    for n, L in enumerate(lens):
        for j in range(cap):
            done = (j + 1) * interval
            if done > L:
                assert torch.equal(snaps[n, j], torch.full_like(snaps[n, j], SENTINEL)), (n, j)
                continue
            _, S_ref = oracle_on(prefix(inp, n, done))
            # per state, per head and per key-channel row of the snapshot
            st = parity_stats(None, None, np64(snaps[n, j])[None], S_ref, [0, 0])
            worst = max(worst, st["seq_S"], st["head_S"], st["row_S"])
            taken += 1
            if done == L:
                assert torch.equal(snaps[n, j], S[n].cpu())
    print(f"{label}: {taken} snapshots, worst relative error {worst:.2e}")
    assert taken > 0 and worst <= tol


@pytest.mark.parametrize("name,d,dtype,chunk,workspace", PATHS, ids=[p[0] for p in PATHS])
def test_snapshots_match_prefix_oracle(name, d, dtype, chunk, workspace):
    """Ragged lengths (a full interval, an empty sequence, tails past the last
    snapshot, a length that ends exactly on one) and a nonzero initial state."""
    m = kda()
    inp = workloads.recurrence_inputs([300, 64, 130, 0, 256], H=2, d=d, dtype=dtype, chunk=chunk,
                                      s0_std=0.3, seed=80 + d)
    check(m, inp, workspace, 64 if chunk == 64 else 96, TOL_F32 if dtype == "f32" else TOL_BF16,
          name)


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_snapshots_across_windows(gate):
    """The two-kernel path runs a long sequence in windows of at most 32 chunks:
    snapshots every 8 chunks land inside windows and on the window boundary
    (2048 tokens) and the last one is the final state."""
    m = kda()
    inp = workloads.recurrence_inputs([2560, 700], H=2, d=128, dtype="bf16", s0_std=0.2,
                                      seed=90, gate=gate)
    check(m, inp, "auto", 512, TOL_BF16, f"windows {gate}")


def test_snapshot_capacity_zero_and_short_buffer():
    """Capacity 0 takes nothing; a buffer shorter than the sequence keeps only
    the snapshots it has room for."""
    m = kda()
    inp = workloads.recurrence_inputs([256], H=2, d=128, dtype="bf16", seed=91)
    empty = torch.zeros((1, 0, 2, 128, 128), device="cuda")
    o, S, _ = run(m, inp, "auto", empty, 64)
    o_plain, S_plain = run(m, inp, "auto")
    assert torch.equal(o, o_plain) and torch.equal(S, S_plain)
    two = torch.zeros((1, 2, 2, 128, 128), device="cuda")
    run(m, inp, "auto", two, 64)
    _, S_ref = oracle_on(prefix(inp, 0, 128))
    assert_parity(None, None, np64(two[0, 1:2]), S_ref, [0, 0], TOL_BF16,
                  "snapshot after 128 tokens, two-entry buffer")
