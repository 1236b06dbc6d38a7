"""Helpers shared by the GPU parity tests: device plumbing, oracle calls on the
exact inputs the GPU sees, and the error measure.

Error measure: for each sequence n, separately for the outputs o and for the
final state, the relative Frobenius error ||X_gpu - X_ref||_F / ||X_ref||_F; a
case passes when the largest of these is within the tolerance (1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 state).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def dev(x):
    return None if x is None else x.cuda().contiguous()


def np64(x):
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()


def rel_fro(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def per_seq_errors(o_gpu, o_ref, S_gpu, S_ref, cu):
    """Max over sequences of the relative Frobenius errors of o and of S."""
    cu = [int(c) for c in cu]
    eo, es = 0.0, 0.0
    for n in range(len(cu) - 1):
        if cu[n + 1] > cu[n]:
            eo = max(eo, rel_fro(o_gpu[cu[n]:cu[n + 1]], o_ref[cu[n]:cu[n + 1]]))
        if S_ref is not None:
            es = max(es, rel_fro(S_gpu[n], S_ref[n]))
    return eo, es


def oracle_on(inp, heads=None, precision="f64"):
    """Oracle run on a workloads.RecurrenceInputs (optionally a subset of heads)."""
    import oracle

    sel = slice(None) if heads is None else list(heads)
    q = np64(inp.q[:, sel])
    k = np64(inp.k[:, sel])
    v = np64(inp.v[:, sel])
    g = np64(inp.g[:, sel])
    if g.ndim == 2:  # one decay per head: the same alpha on every key channel
        g = np.repeat(g[:, :, None], q.shape[2], axis=2)
    beta = np64(inp.beta[:, sel])
    S0 = None if inp.S0 is None else np64(inp.S0[:, sel])
    return oracle.recurrence(q, k, v, g, beta, cu_seqlens=inp.cu_seqlens.numpy(), S0=S0,
                             precision=precision)


def gpu_prefill(inp, chunk=None, workspace="auto"):
    """Prefill through the binding; workspace None selects the fused matrix-core
    kernel, "auto" the two-kernel path (bf16, d = 128, chunk 64)."""
    import gated_delta_rule_99_amd as kda

    o, S = kda.kda_prefill_chunked(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g),
                                   dev(inp.beta), cu_seqlens=dev(inp.cu_seqlens),
                                   cu_seqlens_host=inp.cu_seqlens,
                                   chunk=inp.chunk if chunk is None else chunk,
                                   initial_state=dev(inp.S0), workspace=workspace)
    torch.cuda.synchronize()
    return o, S
