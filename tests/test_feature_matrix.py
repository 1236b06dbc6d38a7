"""GPU parity over combinations of features, through the C ABI.  The other
parity tests each pin one feature on chosen paths; here seeded draws combine
them, so that a feature that breaks only beside another one (an output gate
with snapshots on the static scratch, a per-head decay with bf16 states and
token snapshots through a slot permutation, ...) is still caught.

Prefill draws: the path (two-kernel with a workspace, the same on the static
scratch, the fused kernel, the vector kernel at every d and chunk in fp32 and
bf16), the decay input (per channel, per head, the fused gate prologue), the
output gate, an initial state, snapshots, 1-4 ragged sequences (empty, one
token, one chunk +- 1, a few chunks; on the matrix-core paths sometimes a
sequence longer than one 32-chunk window) and 1-3 heads.

Decode draws: d, the input dtype, the state dtype, the decay input, the output
gate, 1-9 tokens per call (one token sometimes through kda_decode_step), token
snapshots, and a slot permutation into a larger pool.

Every case is checked against the oracle with assert_parity (per sequence, per
(sequence, head) and per row); snapshots against the oracle run on the prefix
they hold; slots no sequence maps to must stay unchanged bit for bit."""
import random

import numpy as np
import pytest
import torch

import oracle
import workloads
from kda_testutil import (TOL_BF16, TOL_F32, assert_parity, dev, gpu_or_skip, np64, oracle_on,
                          parity_stats)

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


# ------------------------------------------------------------------ prefill

def _prefill_cases(n=30, seed=2024):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        path = rng.choice(["split", "static", "fused", "vector", "vector"])
        if path == "vector":
            dtype = rng.choice(["f32", "bf16"])
            d = rng.choice([16, 32, 64, 128])
            chunk = rng.choice([16, 32, 64])
            if dtype == "bf16" and d == 128 and chunk == 64:
                chunk = 32  # that shape runs on the matrix cores
        else:
            dtype, d, chunk = "bf16", 128, 64
        pool = [0, 1, chunk - 1, chunk, chunk + 1, rng.randint(2, 4 * chunk)]
        lens = [rng.choice(pool) for _ in range(rng.randint(1, 4))]
        if path in ("split", "static") and rng.random() < 0.3:
            lens[rng.randrange(len(lens))] = 32 * 64 + rng.randint(1, 150)  # two windows
        if sum(lens) == 0:
            lens[0] = chunk + 3
        cases.append(dict(
            id=i, path=path, dtype=dtype, d=d, chunk=chunk, lens=lens,
            H=rng.randint(1, 3), gate=rng.choice(["channel", "head", "proj"]),
            out_gate=rng.random() < 0.5, s0=rng.random() < 0.6,
            snap=rng.choice([0, 0, chunk, 2 * chunk]), seed=rng.randrange(1 << 20)))
    return cases


PREFILL = _prefill_cases()


def _pid(c):
    return (f"{c['id']}-{c['path']}-{c['dtype']}-d{c['d']}-C{c['chunk']}-{c['gate']}"
            f"{'-og' if c['out_gate'] else ''}{'-s0' if c['s0'] else ''}"
            f"{'-snap' + str(c['snap']) if c['snap'] else ''}-L{'.'.join(map(str, c['lens']))}")


def _prefix(inp, n, length, g, beta):
    b = int(inp.cu_seqlens[n])
    rows = slice(b, b + length)
    S0 = None if inp.S0 is None else inp.S0[n:n + 1]
    return workloads.RecurrenceInputs(inp.q[rows], inp.k[rows], inp.v[rows], g[rows], beta[rows],
                                      torch.tensor([0, length], dtype=torch.int32), S0,
                                      inp.dtype, inp.chunk)


@pytest.mark.parametrize("c", PREFILL, ids=[_pid(c) for c in PREFILL])
def test_prefill_feature_combination(c):
    m = kda()
    H, d, chunk, dtype = c["H"], c["d"], c["chunk"], c["dtype"]
    gate = "head" if c["gate"] == "head" else "channel"
    inp = workloads.recurrence_inputs(c["lens"], H=H, d=d, dtype=dtype, chunk=chunk,
                                      s0_std=0.3 if c["s0"] else 0.0, seed=c["seed"], gate=gate)
    if c["gate"] == "proj":
        pr = workloads.gate_projections(inp.T, H, d, dtype=dtype, a_log_std=0.5, seed=c["seed"])
        g_ref, b_ref = (torch.from_numpy(x) for x in
                        oracle.gate_prologue(np64(pr.f), np64(pr.a_log), np64(pr.b)))
        g_in, b_in, a_log = pr.f, pr.b, dev(pr.a_log)
    else:
        g_ref, b_ref = inp.g, inp.beta
        g_in, b_in, a_log = inp.g, inp.beta, None
    z = workloads.output_gate_projection(inp.T, H, d, dtype=dtype, seed=c["seed"] + 1) \
        if c["out_gate"] else None
    ws = {"split": "auto", "static": "static", "fused": None, "vector": "auto"}[c["path"]]
    snaps = None
    if c["snap"]:
        cap = max(c["lens"]) // c["snap"] + 1
        snaps = torch.full((len(c["lens"]), cap, H, d, d), 7.25, device="cuda")
    out = m.kda_prefill_chunked(dev(inp.q), dev(inp.k), dev(inp.v), dev(g_in), dev(b_in),
                                cu_seqlens=dev(inp.cu_seqlens), cu_seqlens_host=inp.cu_seqlens,
                                chunk=chunk, initial_state=dev(inp.S0), workspace=ws,
                                snapshots=snaps, snap_interval=c["snap"], a_log=a_log,
                                out_gate=dev(z))
    torch.cuda.synchronize()
    o, S = out[0], out[1]
    ref = workloads.RecurrenceInputs(inp.q, inp.k, inp.v, g_ref, b_ref, inp.cu_seqlens, inp.S0,
                                     dtype, chunk)
    o_ref, S_ref = oracle_on(ref)
    if z is not None:
        o_ref = oracle.output_gate(o_ref, np64(z))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, tol, _pid(c))
    if snaps is None:
        return
    snaps = snaps.cpu()
    worst, taken = 0.0, 0
    for n, L in enumerate(c["lens"]):
        js = [j for j in range(snaps.shape[1]) if (j + 1) * c["snap"] <= L]
        for j in range(snaps.shape[1]):
            if j not in js:  # entries the sequence is too short for keep their contents
                assert torch.equal(snaps[n, j], torch.full_like(snaps[n, j], 7.25)), (n, j)
        # every snapshot of short sequences; first, middle and last of long ones
        pick = js if len(js) <= 6 else sorted({js[0], js[len(js) // 2], js[-1]})
        for j in pick:
            _, S_pre = oracle_on(_prefix(inp, n, (j + 1) * c["snap"], g_ref, b_ref))
            st = parity_stats(None, None, np64(snaps[n, j])[None], S_pre, [0, 0])
            worst = max(worst, st["seq_S"], st["head_S"], st["row_S"])
            taken += 1
    print(f"  {taken} snapshots, worst {worst:.2e}")
    assert worst <= tol


# ------------------------------------------------------------------ decode

def _decode_cases(n=24, seed=4048):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        n_tok = rng.choice([1, 1, 2, 3, 4, 5, 9])
        cases.append(dict(
            id=i, d=rng.choice([16, 32, 64, 128, 128]), dtype=rng.choice(["f32", "bf16"]),
            state=rng.choice(["f32", "bf16"]), gate=rng.choice(["channel", "head", "proj"]),
            out_gate=rng.random() < 0.5, n_tok=n_tok, step_api=n_tok == 1 and rng.random() < 0.5,
            snaps=rng.random() < 0.4, B=rng.randint(1, 5), H=rng.randint(1, 3),
            extra_slots=rng.randint(0, 3), seed=rng.randrange(1 << 20)))
        if cases[-1]["step_api"]:
            cases[-1]["snaps"] = False  # the one-token entry point takes no snapshots
    return cases


DECODE = _decode_cases()


def _did(c):
    return (f"{c['id']}-d{c['d']}-{c['dtype']}-state{c['state']}-{c['gate']}"
            f"{'-og' if c['out_gate'] else ''}-tok{c['n_tok']}{'-step' if c['step_api'] else ''}"
            f"{'-snaps' if c['snaps'] else ''}-B{c['B']}H{c['H']}")


@pytest.mark.parametrize("c", DECODE, ids=[_did(c) for c in DECODE])
def test_decode_feature_combination(c):
    m = kda()
    B, H, d, n_tok, dtype = c["B"], c["H"], c["d"], c["n_tok"], c["dtype"]
    gate = "head" if c["gate"] == "head" else "channel"
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype=dtype, s0_std=0.3,
                                      seed=c["seed"], gate=gate)
    bf16_state = c["state"] == "bf16"
    S0 = inp.S0
    if bf16_state:  # the stored values are what the kernel reads
        S0 = torch.from_numpy(oracle.round_bf16(S0.double().numpy())).float()
    if c["gate"] == "proj":
        pr = workloads.gate_projections(inp.T, H, d, dtype=dtype, a_log_std=0.5, seed=c["seed"])
        g_ref, b_ref = (torch.from_numpy(x) for x in
                        oracle.gate_prologue(np64(pr.f), np64(pr.a_log), np64(pr.b)))
        g_in, b_in, a_log = pr.f, pr.b, dev(pr.a_log)
    else:
        g_ref, b_ref = inp.g, inp.beta
        g_in, b_in, a_log = inp.g, inp.beta, None
    z = workloads.output_gate_projection(inp.T, H, d, dtype=dtype, seed=c["seed"] + 1) \
        if c["out_gate"] else None
    # slot permutation into a larger pool; the other slots hold other states
    rng = np.random.default_rng(c["seed"])
    n_slots = B + c["extra_slots"]
    slots = torch.from_numpy(rng.permutation(n_slots)[:B].astype(np.int32))
    pool = torch.randn((n_slots, H, d, d), generator=torch.Generator().manual_seed(c["seed"]))
    pool[slots.long()] = S0
    sdt = torch.bfloat16 if bf16_state else torch.float32
    state = dev(pool.to(sdt))
    before = state.clone()
    tok = lambda x: None if x is None else dev(x.reshape((B, n_tok) + tuple(x.shape[1:])))
    snaps = None
    if c["step_api"]:
        o = m.kda_decode_step(dev(inp.q), dev(inp.k), dev(inp.v), dev(g_in), dev(b_in), state,
                              slot_idx=dev(slots), a_log=a_log, out_gate=dev(z))
    else:
        o, snaps = m.kda_decode_tokens(tok(inp.q), tok(inp.k), tok(inp.v), tok(g_in), tok(b_in),
                                       state, slot_idx=dev(slots), a_log=a_log,
                                       out_gate=tok(z), token_states=True if c["snaps"] else None)
    torch.cuda.synchronize()
    ref = workloads.RecurrenceInputs(inp.q, inp.k, inp.v, g_ref, b_ref, inp.cu_seqlens, S0, dtype,
                                     inp.chunk)
    o_ref, S_ref = oracle_on(ref)
    if z is not None:
        o_ref = oracle.output_gate(o_ref, np64(z))
    tol = TOL_F32 if (dtype == "f32" and not bf16_state) else TOL_BF16
    S_gpu = state.float().cpu().double().numpy()[slots.long().numpy()]
    assert_parity(np64(o).reshape(B * n_tok, H, d), o_ref, S_gpu, S_ref, inp.cu_seqlens, tol,
                  _did(c))
    untouched = [s for s in range(n_slots) if s not in slots.tolist()]
    assert torch.equal(state[untouched], before[untouched])
    if snaps is None:
        return
    assert snaps.dtype == sdt
    assert torch.equal(snaps[:, -1], state[slots.long()])
    for j in range(n_tok):
        rows = torch.tensor([b * n_tok + i for b in range(B) for i in range(j + 1)])
        pre = workloads.RecurrenceInputs(inp.q[rows], inp.k[rows], inp.v[rows], g_ref[rows],
                                         b_ref[rows],
                                         torch.arange(0, B * (j + 1) + 1, j + 1,
                                                      dtype=torch.int32), S0, dtype, inp.chunk)
        _, S_pre = oracle_on(pre)
        st = parity_stats(None, None, snaps[:, j].float().cpu().double().numpy(), S_pre,
                          range(B + 1))
        assert max(st["seq_S"], st["head_S"], st["row_S"]) <= tol, (j, st)
