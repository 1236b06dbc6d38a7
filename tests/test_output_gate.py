"""GPU parity of the output gate (out_gate: o * sigmoid(z), z the gate
projection per token, head and value channel) on every prefill path and on the
decode steps, through the C ABI, against the oracle's recurrence followed by
oracle.output_gate on the same inputs.  The gate does not touch the state, so
the final states equal those of the ungated call bit for bit; a gate wide open
(z = 60, sigmoid(z) = 1 in fp32) gives the ungated outputs bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from kda_testutil import (TOL_BF16, TOL_F32, assert_parity, dev, gpu_or_skip, np64, oracle_on)

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def prefill(m, inp, z, chunk=None, workspace="auto"):
    o, S = m.kda_prefill_chunked(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                                 cu_seqlens=dev(inp.cu_seqlens), cu_seqlens_host=inp.cu_seqlens,
                                 chunk=inp.chunk if chunk is None else chunk,
                                 initial_state=dev(inp.S0), workspace=workspace,
                                 out_gate=dev(z))
    torch.cuda.synchronize()
    return o, S


# (label, d, dtype, chunk, workspace): the two-kernel and fused matrix-core paths
# and the vector kernel (fp32, and bf16 at a chunk the matrix cores do not take)
PATHS = [("split", 128, "bf16", 64, "auto"), ("fused", 128, "bf16", 64, None),
         ("vector_f32", 32, "f32", 16, None), ("vector_bf16", 64, "bf16", 32, None)]


@pytest.mark.parametrize("label,d,dtype,chunk,ws", PATHS, ids=[p[0] for p in PATHS])
def test_prefill_output_gate(label, d, dtype, chunk, ws):
    m = kda()
    inp = workloads.recurrence_inputs([130, 0, 64, 301, 1], H=3, d=d, dtype=dtype, chunk=chunk,
                                      g_mu=3.0, g_sigma=1.0, s0_std=0.3, seed=500 + d)
    z = workloads.output_gate_projection(inp.T, inp.H, d, dtype=dtype, seed=501)
    o, S = prefill(m, inp, z, workspace=ws)
    o_plain, S_plain = prefill(m, inp, None, workspace=ws)
    assert torch.equal(S, S_plain), "the gate changed the state"
    o_ref, S_ref = oracle_on(inp)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o), oracle.output_gate(o_ref, np64(z)), np64(S), S_ref, inp.cu_seqlens,
                  tol, f"gated prefill, {label}")
    wide = torch.full_like(z, 60.0)
    o_open, _ = prefill(m, inp, wide, workspace=ws)
    assert torch.equal(o_open, o_plain), "an open gate changed the outputs"


@pytest.mark.parametrize("label,chunk,ws", [("split", 64, "auto"), ("fused", 64, None),
                                            ("vector", 16, None)])
def test_prefill_output_gate_ling_layer(label, chunk, ws):
    """The Ling-shaped layer (T = 8192, H = 64, d = 128, bf16) with the gate, on
    each path (chunk 16 runs the vector kernel); every head against the oracle."""
    m = kda()
    inp = workloads.ling_prefill()
    z = workloads.output_gate_projection(inp.T, inp.H, inp.d, seed=502)
    o, S = prefill(m, inp, z, chunk=chunk, workspace=ws)
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), oracle.output_gate(o_ref, np64(z)), np64(S), S_ref, inp.cu_seqlens,
                  TOL_BF16, f"gated Ling layer, {label}")


@pytest.mark.parametrize("n_tok", [1, 3])
@pytest.mark.parametrize("d,dtype,state", [(128, "bf16", torch.float32), (64, "f32", torch.float32),
                                           (128, "bf16", torch.bfloat16)])
def test_decode_output_gate(d, dtype, state, n_tok):
    m = kda()
    B, H = 5, 4
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype=dtype, s0_std=0.3,
                                      seed=510 + d + n_tok)
    S0 = torch.from_numpy(oracle.round_bf16(inp.S0.double().numpy())).float() \
        if state == torch.bfloat16 else inp.S0
    z = workloads.output_gate_projection(inp.T, H, d, dtype=dtype, seed=511)
    st = dev(S0.to(state))
    if n_tok == 1:
        o = m.kda_decode_step(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), st,
                              out_gate=dev(z))
    else:
        t = lambda x: dev(x.reshape((B, n_tok) + tuple(x.shape[1:])))
        o, _ = m.kda_decode_tokens(t(inp.q), t(inp.k), t(inp.v), t(inp.g), t(inp.beta), st,
                                   out_gate=t(z))
    torch.cuda.synchronize()
    ref = workloads.RecurrenceInputs(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, S0,
                                     dtype, inp.chunk)
    o_ref, S_ref = oracle_on(ref)
    if state == torch.bfloat16:
        S_ref = oracle.round_bf16(S_ref)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o).reshape(B * n_tok, H, d), oracle.output_gate(o_ref, np64(z)),
                  st.float().cpu().double().numpy(), S_ref, inp.cu_seqlens, tol,
                  f"gated decode d={d} {dtype} state {state} n_tok={n_tok}")
