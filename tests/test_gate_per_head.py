"""The per-head-decay case (KDA_GATE_HEAD: one log decay per token and head,
broadcast over the key channels, the Gated DeltaNet layer that KDA refines)
through the C ABI: parity with the oracle on the broadcast decay, and equality,
bit for bit, with the per-channel path fed the broadcast values."""
import pytest
import torch

import workloads
from kda_testutil import (TOL_BF16, TOL_F32, dev, gpu_or_skip, gpu_prefill, np64, oracle_on,
                          assert_parity)

pytestmark = pytest.mark.gpu

LENS = [70, 0, 129, 1, 200]


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def broadcast(inp):
    """The same inputs with g expanded to one value per key channel."""
    g = inp.g[:, :, None].expand(-1, -1, inp.q.shape[2]).contiguous()
    return workloads.RecurrenceInputs(inp.q, inp.k, inp.v, g, inp.beta, inp.cu_seqlens, inp.S0,
                                      inp.dtype, inp.chunk)


CASES = [  # (d, dtype, chunk, workspace)
    (32, "f32", 16, "auto"), (64, "bf16", 64, "auto"),     # vector kernel
    (128, "bf16", 64, "auto"), (128, "bf16", 64, None),    # two-kernel, fused
]


@pytest.mark.parametrize("d,dtype,chunk,ws", CASES)
def test_prefill_head_gate(d, dtype, chunk, ws):
    kda()
    inp = workloads.recurrence_inputs(LENS, H=3, d=d, dtype=dtype, chunk=chunk, g_mu=3.0,
                                      g_sigma=1.0, s0_std=0.3, seed=300 + d + chunk, gate="head")
    o, S = gpu_prefill(inp, workspace=ws)
    o_ref, S_ref = oracle_on(inp)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, tol,
                  f"head gate d={d} {dtype} C={chunk} ws={ws}")
    # the per-channel path on the broadcast decay gives the same bits
    o2, S2 = gpu_prefill(broadcast(inp), workspace=ws)
    assert torch.equal(o, o2) and torch.equal(S, S2)


@pytest.mark.parametrize("d,dtype", [(32, "f32"), (128, "bf16")])
def test_decode_head_gate(d, dtype):
    m = kda()
    B, n_tok, H = 4, 3, 2
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype=dtype, s0_std=0.3,
                                      seed=310 + d, gate="head")
    t = lambda x: dev(x.reshape((B, n_tok) + tuple(x.shape[1:])))
    state = dev(inp.S0)
    o, _ = m.kda_decode_tokens(t(inp.q), t(inp.k), t(inp.v), t(inp.g), t(inp.beta), state)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_on(inp)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o).reshape(B * n_tok, H, d), o_ref, np64(state), S_ref,
                            inp.cu_seqlens, tol,
                  f"head gate decode d={d} {dtype}")
    # single-token step, per-head vs broadcast per-channel decay: same bits
    rows = torch.arange(B) * n_tok
    b = broadcast(inp)
    s1, s2 = dev(inp.S0), dev(inp.S0)
    o1 = m.kda_decode_step(dev(inp.q[rows]), dev(inp.k[rows]), dev(inp.v[rows]),
                           dev(inp.g[rows]), dev(inp.beta[rows]), s1)
    o2 = m.kda_decode_step(dev(b.q[rows]), dev(b.k[rows]), dev(b.v[rows]), dev(b.g[rows]),
                           dev(b.beta[rows]), s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
