"""KDA oracle: plain CPU reference for the gated delta-rule mixer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and it
shares no code with them.

Contents
--------
* ``recurrence``    -- the sequential recurrence in C (``kda_oracle.c``), fp64 or
  fp32, OpenMP over independent (sequence, head) pairs.
* ``short_conv``    -- width-4 causal depthwise convolution (C, fp64).
* ``l2norm_heads``  -- per-head L2 normalisation (C, fp64).
* ``brute_force``   -- a second, independent formulation in numpy fp64: the
  dense transition matrices M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) multiplied
  out, for tiny inputs only.
* ``round_bf16``    -- rounding to the nearest bfloat16 value (ties to even), the
  storage rounding of a state kept in bf16 (numpy, integer arithmetic).
* ``gate_prologue`` -- the decay and write strength from the projections' raw
  outputs (numpy fp64): g = -exp(a_log) softplus(f), beta = sigmoid(b).  The
  same page names f_proj and A_log behind the per-channel decay and b_proj
  behind beta but prints no formula; this is the reading the library adopts.
* ``output_gate``   -- the output gate applied to the recurrence's outputs
  (numpy fp64): o * sigmoid(z), z the gate projection per (token, head, value
  channel).

Where each step comes from is stated in ``kda_oracle.c``'s header: page
"Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its safetensors
headers", section "How KDA and MLA split the work" (per-channel decay, per-head
write strength, width-4 causal convolution of q, k, v), whose display equation
did not survive extraction; the recurrence is the gated delta rule
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(out: str = LIB, src: str = SRC) -> str:
    """Compile the C oracle with gcc (``src``: this package's kda_oracle.c; the
    pin tests pass patched copies of it)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)


def _ptr(a, kind):
    if a is None:
        return None
    return a.ctypes.data_as(kind)


class Oracle:
    """ctypes view of one build of ``kda_oracle.c``."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        for name, fp in (("kda_oracle_recurrence_f64", _dp), ("kda_oracle_recurrence_f32", _fp)):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [fp, fp, fp, fp, fp, _ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int, fp, fp, fp, ctypes.c_int]
        lib.kda_oracle_short_conv_f64.restype = ctypes.c_int
        lib.kda_oracle_short_conv_f64.argtypes = [_dp, _dp, _ip, ctypes.c_int, ctypes.c_int, _dp,
                                                  _dp, _dp]
        lib.kda_oracle_l2norm_heads_f64.restype = ctypes.c_int
        lib.kda_oracle_l2norm_heads_f64.argtypes = [_dp, ctypes.c_int64, ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_double]
        self.lib = lib

    # ------------------------------------------------------------------ recurrence
    def recurrence(self, q, k, v, g, beta, cu_seqlens=None, S0=None, precision="f64",
                   n_threads=0):
        """Run the recurrence.

        q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H] (any real dtype; they are
        converted exactly to the working precision).  ``cu_seqlens`` [n+1] packs n
        sequences (default: one sequence of T tokens).  ``S0`` [n, H, dk, dv] or
        None (zeros).  Returns (o [T, H, dv], S_final [n, H, dk, dv]) in the working
        precision.
        """
        real = np.float64 if precision == "f64" else np.float32
        kind = _dp if precision == "f64" else _fp
        fn = self.lib.kda_oracle_recurrence_f64 if precision == "f64" else \
            self.lib.kda_oracle_recurrence_f32
        q, k, v, g = (np.ascontiguousarray(x, dtype=real) for x in (q, k, v, g))
        beta = np.ascontiguousarray(beta, dtype=real)
        T, H, dk = q.shape
        dv = v.shape[2]
        if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) \
                or beta.shape != (T, H):
            raise ValueError("oracle: inconsistent shapes")
        if cu_seqlens is None:
            cu_seqlens = np.array([0, T], dtype=np.int32)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        n = cu.shape[0] - 1
        if int(cu[-1]) != T:
            raise ValueError("oracle: cu_seqlens[-1] != T")
        if S0 is not None:
            S0 = np.ascontiguousarray(S0, dtype=real)
            if S0.shape != (n, H, dk, dv):
                raise ValueError("oracle: S0 shape")
        o = np.empty((T, H, dv), dtype=real)
        S = np.empty((n, H, dk, dv), dtype=real)
        rc = fn(_ptr(q, kind), _ptr(k, kind), _ptr(v, kind), _ptr(g, kind), _ptr(beta, kind),
                _ptr(cu, _ip), n, H, dk, dv, _ptr(S0, kind), _ptr(o, kind), _ptr(S, kind),
                int(n_threads))
        if rc != 0:
            raise RuntimeError(f"oracle recurrence failed: {rc}")
        return o, S

    # ------------------------------------------------------------------ conv + norm
    def short_conv(self, x, w, cu_seqlens=None, tail=None):
        """Width-4 causal depthwise convolution.  x [T, Cch], w [Cch, 4],
        tail [n, 3, Cch] or None.  Returns (y [T, Cch], tail_out [n, 3, Cch]) fp64."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        T, C = x.shape
        if w.shape != (C, 4):
            raise ValueError("oracle: conv weight shape")
        if cu_seqlens is None:
            cu_seqlens = np.array([0, T], dtype=np.int32)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        n = cu.shape[0] - 1
        if tail is not None:
            tail = np.ascontiguousarray(tail, dtype=np.float64)
            if tail.shape != (n, 3, C):
                raise ValueError("oracle: tail shape")
        y = np.empty((T, C), dtype=np.float64)
        tail_out = np.empty((n, 3, C), dtype=np.float64)
        rc = self.lib.kda_oracle_short_conv_f64(_ptr(x, _dp), _ptr(w, _dp), _ptr(cu, _ip), n, C,
                                                _ptr(tail, _dp), _ptr(y, _dp),
                                                _ptr(tail_out, _dp))
        if rc != 0:
            raise RuntimeError(f"oracle short_conv failed: {rc}")
        return y, tail_out

    def l2norm_heads(self, x, head_dim, eps=1e-6):
        """x / sqrt(sum x^2 + eps) over each run of ``head_dim`` channels of each
        row of x [rows, width].  Returns a new fp64 array."""
        y = np.array(x, dtype=np.float64, order="C", copy=True)
        rows = y.shape[0]
        width = int(np.prod(y.shape[1:]))
        rc = self.lib.kda_oracle_l2norm_heads_f64(_ptr(y, _dp), rows, width, int(head_dim),
                                                  float(eps))
        if rc != 0:
            raise RuntimeError(f"oracle l2norm failed: {rc}")
        return y


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default


def recurrence(*args, **kw):
    return default().recurrence(*args, **kw)


def short_conv(*args, **kw):
    return default().short_conv(*args, **kw)


def l2norm_heads(*args, **kw):
    return default().l2norm_heads(*args, **kw)


def brute_force(q, k, v, g, beta, S0=None):
    """Second formulation, numpy fp64, for one sequence and tiny sizes only.

    Builds each transition matrix M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) as a
    dense d_k x d_k matrix and expands the state as
        S_t = Phi_{t,0} S_0 + sum_{s<=t} Phi_{t,s} beta_s k_s v_s^T,
    Phi_{t,s} = M_t M_{t-1} ... M_{s+1} (Phi_{t,t} = I), reading o_t = S_t^T q_t.
    Every S_t is formed from scratch from that sum, with no carried state, so a
    mistake in the carried-state bookkeeping of the C oracle cannot repeat here.
    Shapes as ``Oracle.recurrence`` with one sequence; returns (o, S_T).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    S_T = np.zeros((H, dk, dv))
    eye = np.eye(dk)
    for h in range(H):
        S0h = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)[h]
        M = [(eye - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h]))
             for t in range(T)]
        for t in range(T):
            # Phi_{t,s} for s = t, t-1, ..., -1 built right to left
            phi = eye.copy()
            acc = np.zeros((dk, dv))
            for s in range(t, -1, -1):
                acc += phi @ (beta[s, h] * np.outer(k[s, h], v[s, h]))
                phi = phi @ M[s]
            St = phi @ S0h + acc
            o[t, h] = St.T @ q[t, h]
            if t == T - 1:
                S_T[h] = St
    return o, S_T


def round_bf16(x):
    """Round finite values in the normal binary32 range to the nearest bfloat16
    value, ties to even; returns float64 (exact).

    bfloat16 keeps a binary32 number's sign, its 8 exponent bits and the top 7 of
    its 23 fraction bits, so a value keeps 8 significant bits.  In binary64 that
    is the sign, the exponent and the top 7 of the 52 fraction bits: the low 45
    bits are rounded away.  Adding 2^44 - 1 plus the lowest kept bit and then
    clearing the 45 bits rounds to nearest with ties to even; a carry out of the
    fraction moves into the exponent, which is the correct result there too.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = a.view(np.uint64)
    drop = np.uint64(45)
    keep_lsb = (bits >> drop) & np.uint64(1)
    bias = (np.uint64(1) << np.uint64(44)) - np.uint64(1) + keep_lsb
    out = ((bits + bias) >> drop) << drop
    return out.view(np.float64).reshape(a.shape)


def gate_prologue(f, a_log, b):
    """Decay and write strength from the projections' outputs, in fp64.

    f: [..., H, d_k] decay projection; a_log: [H] log rate per head; b: [..., H]
    write-strength logits.  Returns (g, beta) with
        g    = -exp(a_log[h]) * softplus(f),  softplus(x) = log(1 + e^x),
        beta = 1 / (1 + e^{-b}),
    so alpha = exp(g) lies in (0, 1] and beta in (0, 1).  Page "Ling-3.1-flash:
    a 560B hybrid-attention MoE, counted from its safetensors headers", section
    "How KDA and MLA split the work", names the tensors (f_proj and A_log for the
    per-channel decay, b_proj for beta, one per head) without the formula; this
    is the plainest form in which a per-head log rate scales a per-channel
    projection into a negative log decay.  softplus uses numpy's logaddexp(0, x),
    exact for every finite x."""
    f = np.asarray(f, dtype=np.float64)
    a_log = np.asarray(a_log, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    rate = np.exp(a_log)[:, None]           # [H, 1], broadcast over d_k
    g = -rate * np.logaddexp(0.0, f)
    beta = 1.0 / (1.0 + np.exp(-b))
    return g, beta



def output_gate(o, z):
    """The output gate on the recurrence's outputs, in fp64: o * sigmoid(z).

    o: [..., H, d_v] outputs o_t = S_t^T q_t; z: the same shape, the gate
    projection's output.  Page "Ling-3.1-flash: a 560B hybrid-attention MoE,
    counted from its safetensors headers", section "How KDA and MLA split the
    work", lists a gate projection among each KDA layer's full-rank 4096 -> 8192
    matrices (one value per head and value channel) beside the output
    projection that follows it, without its activation; the same section's
    gated MLA scales its result by a sigmoid gate.  Taken here: the elementwise
    sigmoid gate, with no normalisation before it (the pages name none).
    sigmoid(z) = 1 / (1 + e^{-z}) is evaluated without overflow for any finite
    z (numpy's exp of a large -z gives inf, and 1 / inf = 0)."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    if o.shape != z.shape:
        raise ValueError("oracle: output gate shape")
    with np.errstate(over="ignore"):
        return o / (1.0 + np.exp(-z))
