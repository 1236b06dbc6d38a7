"""Helpers shared by the GPU parity tests: device plumbing, oracle calls on the
exact inputs the GPU sees, and the error measures.

The reference is the oracle's fp64 build run on exactly the values the GPU
reads (bf16 inputs widened exactly).  That is a stricter reading of "the fp32
CPU recurrence" than the fp32 build itself: the fp32 build is pinned to lie
within 1e-5 of the fp64 one (``pins.pin_f32_close_to_f64``), far inside every
tolerance below, so the GPU's error is measured against the exact recurrence
rather than against another rounding of it.

Error measures (``assert_parity``), all against one tolerance tol (1e-4 for
fp32 inputs, 2e-2 for bf16 inputs with fp32 state):
  * per sequence n, separately for o and the final state S:
    ||X_gpu - X_ref||_F / ||X_ref||_F  (the headline measure);
  * per (sequence, head), the same ratio for o and for S, so that one wrong
    head cannot hide among many right ones;
  * per row: every (token, head) row of o and every (sequence, head, key
    channel) row of S must satisfy ||x_gpu - x_ref|| <= tol * max(||x_ref||,
    median row norm of the case), so that one wrong token or chunk cannot hide
    in a long sequence.
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


def _row_ratio(x, ref):
    """max over rows (last axis) of ||x - ref|| / max(||ref||, median ||ref||)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rn = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=-1)
    en = np.linalg.norm((x - ref).reshape(-1, ref.shape[-1]), axis=-1)
    floor = float(np.median(rn))
    scale = np.maximum(rn, floor)
    if floor == 0.0:
        scale = np.where(scale == 0.0, 1.0, scale)
    return float(np.max(en / scale))


def parity_stats(o_gpu, o_ref, S_gpu, S_ref, cu):
    """Error measures of a case: o [T, H, dv] and S [n, H, dk, dv] (either
    reference may be None: not compared), cu the n + 1 sequence offsets.  Returns the maxima over sequences, over
    (sequence, head) pairs and over rows (see the module docstring)."""
    cu = [int(c) for c in cu]
    st = {"seq_o": 0.0, "seq_S": 0.0, "head_o": 0.0, "head_S": 0.0}
    if o_ref is not None:
        o_gpu = np.asarray(o_gpu, dtype=np.float64)
        o_ref = np.asarray(o_ref, dtype=np.float64)
        H = o_ref.shape[1]
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if b > a and o_ref is not None:
            st["seq_o"] = max(st["seq_o"], rel_fro(o_gpu[a:b], o_ref[a:b]))
            for h in range(H):
                st["head_o"] = max(st["head_o"], rel_fro(o_gpu[a:b, h], o_ref[a:b, h]))
        if S_ref is not None:
            st["seq_S"] = max(st["seq_S"], rel_fro(S_gpu[n], S_ref[n]))
            for h in range(S_ref.shape[1]):
                st["head_S"] = max(st["head_S"], rel_fro(S_gpu[n, h], S_ref[n, h]))
    st["row_o"] = _row_ratio(o_gpu, o_ref) if o_ref is not None else 0.0
    st["row_S"] = _row_ratio(S_gpu, S_ref) if S_ref is not None else 0.0
    return st


def assert_parity(o_gpu, o_ref, S_gpu, S_ref, cu, tol, label=""):
    """Assert every measure of ``parity_stats`` within tol; print them."""
    st = parity_stats(o_gpu, o_ref, S_gpu, S_ref, cu)
    print(f"{label}: " + " ".join(f"{k} {v:.2e}" for k, v in st.items()))
    bad = {k: v for k, v in st.items() if not v <= tol}
    assert not bad, f"{label}: above {tol:g}: {bad}"
    return st


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
