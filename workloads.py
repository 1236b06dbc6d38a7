"""Seeded synthetic inputs for the KDA hot path.

This module only draws and shapes random inputs.  It holds none of the method's
arithmetic: no decay, no delta rule, no convolution.  Both the HIP path (through
its Python binding) and the CPU oracle consume the arrays it returns, so both see
bit-identical inputs.  bf16 inputs are produced by rounding fp32 draws to bf16
(round-to-nearest-even); the oracle widens them back to fp32/fp64 exactly.

Recipes (one per workload; N(mu, sigma) means mean mu and standard deviation
sigma):

* q, k ~ N(0, 1) per element, then every (token, head) row divided by its L2
  norm in fp32, then rounded to the input dtype.
* v ~ N(0, 1), rounded to the input dtype.
* g = log(sigmoid(N(mu_g, sigma_g))) per (token, head, key channel), fp32; the
  decay is alpha = exp(g) in (0, 1).  The per-head-decay variant draws one g
  per (token, head) from the same recipe.
* beta = sigmoid(N(0, 1)) per (token, head), fp32.
* initial states ~ N(0, s0_std) fp32 where a workload has one, else zero.
* mixer workload: pre-convolution streams x_q, x_k, x_v ~ N(0, 1) rounded to
  bf16, convolution weights ~ N(0, 0.5) fp32.
* output gate projection z ~ N(0, 1) per (token, head, value channel), rounded
  to the input dtype.

Random numbers come from numpy's PCG64 in fixed blocks of 2^22 elements, each
block seeded by (workload seed, tensor id, block index), so the values do not
depend on how many threads draw them.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_BLOCK = 1 << 22

# tensor ids: the order in which a workload's tensors are drawn
TID = {"q": 0, "k": 1, "v": 2, "g": 3, "beta": 4, "S0": 5, "conv_w": 6,
       "x_q": 7, "x_k": 8, "x_v": 9, "f": 10, "a_log": 11, "b": 12, "z": 13, "g_strong": 14}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, seed: int, tid: int, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    """fp32 N(mean, std) draws of the given shape as a CPU tensor."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nb = (n + _BLOCK - 1) // _BLOCK

    def fill(b):
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        rng = np.random.default_rng([int(seed), int(tid), int(b)])
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)

    if nb > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nb)))
    elif n:
        fill(0)
    t = torch.from_numpy(out).view(shape)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Divide each last-axis row by its L2 norm (input recipe, fp32)."""
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.to(torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16)  # round-to-nearest-even
    raise ValueError(dtype)


@dataclasses.dataclass
class RecurrenceInputs:
    """Inputs of the recurrence on packed sequences (CPU tensors)."""
    q: torch.Tensor          # [T, H, dk]  dtype
    k: torch.Tensor          # [T, H, dk]  dtype
    v: torch.Tensor          # [T, H, dv]  dtype
    g: torch.Tensor          # [T, H, dk] or [T, H]  fp32 (log of the decay)
    beta: torch.Tensor       # [T, H]      fp32
    cu_seqlens: torch.Tensor  # [n+1] int32
    S0: torch.Tensor | None  # [n, H, dk, dv] fp32
    dtype: str
    chunk: int

    @property
    def T(self):
        return int(self.q.shape[0])

    @property
    def H(self):
        return int(self.q.shape[1])

    @property
    def d(self):
        return int(self.q.shape[2])

    @property
    def n_seqs(self):
        return int(self.cu_seqlens.shape[0] - 1)


def recurrence_inputs(seqlens, H, d, dtype="bf16", chunk=64, g_mu=2.0, g_sigma=0.5,
                      s0_std=0.0, seed=0, dv=None, gate="channel") -> RecurrenceInputs:
    """gate "channel": g [T, H, d], one log decay per key channel; "head":
    g [T, H], one per head (drawn from the same recipe)."""
    dv = d if dv is None else dv
    if gate not in ("channel", "head"):
        raise ValueError(gate)
    seqlens = [int(s) for s in seqlens]
    T = sum(seqlens)
    cu = torch.tensor([0] + list(np.cumsum(seqlens)), dtype=torch.int32)
    q = to_dtype(_unit_rows(normal((T, H, d), seed, TID["q"])), dtype)
    k = to_dtype(_unit_rows(normal((T, H, d), seed, TID["k"])), dtype)
    v = to_dtype(normal((T, H, dv), seed, TID["v"]), dtype)
    g_shape = (T, H, d) if gate == "channel" else (T, H)
    g = torch.nn.functional.logsigmoid(normal(g_shape, seed, TID["g"], g_mu, g_sigma))
    beta = torch.sigmoid(normal((T, H), seed, TID["beta"]))
    S0 = None
    if s0_std > 0:
        S0 = normal((len(seqlens), H, d, dv), seed, TID["S0"], 0.0, s0_std)
    return RecurrenceInputs(q, k, v, g, beta, cu, S0, dtype, chunk)


@dataclasses.dataclass
class MixerInputs:
    """Front end + recurrence: pre-conv streams, conv weights, gates."""
    x_q: torch.Tensor   # [T, H*d] bf16 (pre-convolution)
    x_k: torch.Tensor
    x_v: torch.Tensor
    w_q: torch.Tensor   # [H*d, 4] fp32
    w_k: torch.Tensor
    w_v: torch.Tensor
    g: torch.Tensor     # [T, H, d] fp32
    beta: torch.Tensor  # [T, H] fp32
    H: int
    d: int
    t_prefill: int
    n_decode: int
    chunk: int


def mixer_inputs(t_prefill, n_decode, H, d, chunk=64, seed=0) -> MixerInputs:
    T = t_prefill + n_decode
    C = H * d
    w = normal((3 * C, 4), seed, TID["conv_w"], 0.0, 0.5)
    xq = normal((T, C), seed, TID["x_q"]).to(torch.bfloat16)
    xk = normal((T, C), seed, TID["x_k"]).to(torch.bfloat16)
    xv = normal((T, C), seed, TID["x_v"]).to(torch.bfloat16)
    g = torch.nn.functional.logsigmoid(normal((T, H, d), seed, TID["g"], 2.0, 0.5))
    beta = torch.sigmoid(normal((T, H), seed, TID["beta"]))
    return MixerInputs(xq, xk, xv, w[:C].contiguous(), w[C:2 * C].contiguous(),
                       w[2 * C:].contiguous(), g, beta, H, d, t_prefill, n_decode, chunk)


# --------------------------------------------------------------------------- the
# five workloads.  Seeds are 1000 + workload number.

def tiny_f32():
    """B=1, H=2, T=64, d=16, chunk 16, fp32; g = log sigmoid(N(2, 0.5))."""
    return recurrence_inputs([64], H=2, d=16, dtype="f32", chunk=16, g_mu=2.0, g_sigma=0.5,
                             seed=1001)


def ling_prefill(T=8192):
    """One Ling-shaped KDA layer prefill: B=1, H=64, T=8192, d=128, chunk 64, bf16
    q/k/v, g = log sigmoid(N(3, 1)), zero initial state."""
    return recurrence_inputs([T], H=64, d=128, dtype="bf16", chunk=64, g_mu=3.0, g_sigma=1.0,
                             seed=1002)


def decode_batch(B=256):
    """Batched decode step: B=256 sequences x H=64 heads, one token each, random
    fp32 initial states N(0, 0.02), bf16 q/k/v, g = log sigmoid(N(2, 0.5))."""
    return recurrence_inputs([1] * B, H=64, d=128, dtype="bf16", chunk=64, g_mu=2.0,
                             g_sigma=0.5, s0_std=0.02, seed=1003)


PACKED_LENGTHS = (131072, 65536, 16384, 1000)


def packed_long(lengths=PACKED_LENGTHS):
    """Long packed prefill: sequences of 131072, 65536, 16384 and 1000 tokens
    packed with cu_seqlens, H=64, d=128, bf16, g = log sigmoid(N(2, 0.5)),
    seeded nonzero initial states N(0, 0.02)."""
    return recurrence_inputs(list(lengths), H=64, d=128, dtype="bf16", chunk=64, g_mu=2.0,
                             g_sigma=0.5, s0_std=0.02, seed=1004)


@dataclasses.dataclass
class GateProjections:
    """Raw inputs of the fused gate prologue (CPU tensors)."""
    f: torch.Tensor       # [T, H, dk] dtype: decay projection
    a_log: torch.Tensor   # [H] fp32: log rate per head
    b: torch.Tensor       # [T, H] fp32: write-strength logits


def gate_projections(T, H, d, dtype="bf16", g_mu=2.0, g_sigma=0.5, a_log_std=0.0,
                     seed=0) -> GateProjections:
    """f = -N(g_mu, g_sigma) rounded to dtype, b = N(0, 1), a_log = N(0, a_log_std)
    per head (zeros for a_log_std = 0).  With a_log = 0 the decay sigmoid(-f) and
    the strength sigmoid(b) follow the per-channel recipe of recurrence_inputs."""
    f = to_dtype(-normal((T, H, d), seed, TID["f"], g_mu, g_sigma), dtype)
    a_log = (normal((H,), seed, TID["a_log"], 0.0, a_log_std) if a_log_std > 0
             else torch.zeros(H))
    b = normal((T, H), seed, TID["b"])
    return GateProjections(f, a_log, b)


def with_strong_decay(inp: RecurrenceInputs, channels, tokens=None, g_mu=-4.7, g_sigma=0.3,
                      seed=0) -> RecurrenceInputs:
    """A copy of inp whose log decay on the given key channels (of every head)
    is redrawn as log(sigmoid(N(g_mu, g_sigma))), on the given token range (all
    tokens by default).  With the default recipe alpha ~ e^-4.7 per token, so a
    64-token chunk decays by about e^-300 on those channels."""
    g = inp.g.clone()
    lo, hi = (0, inp.T) if tokens is None else tokens
    ch = list(channels)
    draw = torch.nn.functional.logsigmoid(
        normal((hi - lo, inp.H, len(ch)), seed, TID["g_strong"], g_mu, g_sigma))
    g[lo:hi, :, ch] = draw
    return RecurrenceInputs(inp.q, inp.k, inp.v, g, inp.beta, inp.cu_seqlens, inp.S0, inp.dtype,
                            inp.chunk)


def output_gate_projection(T, H, dv, dtype="bf16", seed=0) -> torch.Tensor:
    """The output gate's projection z ~ N(0, 1) per (token, head, value channel),
    rounded to dtype: [T, H, dv] (or any leading shape given as T)."""
    lead = tuple(T) if isinstance(T, (tuple, list)) else (T,)
    return to_dtype(normal(lead + (H, dv), seed, TID["z"]), dtype)


def mixer_conv_streams(t_prefill=32768, seed=1005):
    """The pre-conv q, k, v streams [t_prefill, 8192] bf16 and conv weights
    [8192, 4] of the mixer workload: the same draws as mixer() for its first
    t_prefill tokens, without the recurrence inputs."""
    C = 64 * 128
    w = normal((3 * C, 4), seed, TID["conv_w"], 0.0, 0.5)
    xs = [normal((t_prefill, C), seed, TID[n]).to(torch.bfloat16) for n in ("x_q", "x_k", "x_v")]
    return xs, [w[i * C:(i + 1) * C].contiguous() for i in range(3)]


def mixer(t_prefill=32768, n_decode=512):
    """Full mixer with state handoff: width-4 causal conv over 8192-channel q, k, v
    streams, per-head L2 norm of q and k, prefill of 32768 tokens then 512 decode
    steps, H=64, d=128, bf16 activations, fp32 state."""
    return mixer_inputs(t_prefill, n_decode, H=64, d=128, chunk=64, seed=1005)
