"""Pins for the CPU oracle: facts fixed by the definition of the recurrence, by
closed forms, by special cases that reduce to library routines, and by brute
force -- never by re-running the oracle's own formula.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees with the fact.  ``test_oracle_pins``
runs them on the real oracle; ``test_oracle_mutants`` runs them on builds with a
planted mistake and requires every planted mistake to fail at least one pin.

The recurrence (page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from
its safetensors headers", section "How KDA and MLA split the work"):
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,  alpha_t = exp(g_t) per key channel, beta_t per head.
"""
from __future__ import annotations

import numpy as np

import oracle as oracle_mod


def _rand_inputs(rng, T, H, d, unit_k=True, beta_range=(0.0, 1.0), g_scale=0.3, dv=None):
    dv = d if dv is None else dv
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.abs(rng.standard_normal((T, H, d))) * g_scale
    beta = rng.uniform(*beta_range, size=(T, H))
    return q, k, v, g, beta


def pin_identity(orc):
    """beta = 0 and alpha = 1 (g = 0) leave the state unchanged, bit for bit, and
    every output is the initial state read by q: o_t = S_0^T q_t."""
    rng = np.random.default_rng(11)
    T, H, d = 20, 3, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d)
    g[:] = 0.0
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, d, d))
    o, S = orc.recurrence(q, k, v, g, beta, S0=S0)
    assert np.array_equal(S, S0), "identity: state changed"
    ref = np.einsum("hij,thi->thj", S0[0], q)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12), "identity: o != S0^T q"


def pin_pure_decay(orc):
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S_0 -- rows (key channels) decay by
    the product of their own factors."""
    rng = np.random.default_rng(12)
    T, H, d = 17, 2, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, g_scale=0.5)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, d, d))
    _, S = orc.recurrence(q, k, v, g, beta, S0=S0)
    decay = np.exp(g.sum(axis=0))  # [H, d]
    ref = decay[:, :, None] * S0[0]
    assert np.allclose(S[0], ref, rtol=1e-12, atol=1e-14), "pure decay mismatch"


def _stepwise_states(orc, q, k, v, g, beta, S0):
    """S_0, S_1, ..., S_T by chaining one-token calls."""
    states = [S0]
    S = S0
    for t in range(q.shape[0]):
        sl = slice(t, t + 1)
        _, S = orc.recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], S0=S)
        states.append(S)
    return states


def pin_delta_interpolation(orc):
    """For unit k_t: S_t^T k_t = (1 - beta_t) (Diag(alpha_t) S_{t-1})^T k_t + beta_t v_t.
    At beta_t = 1 the last write is recalled exactly, whatever alpha and S."""
    rng = np.random.default_rng(13)
    T, H, d = 12, 2, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, g_scale=0.4)
    beta[5] = 1.0
    S0 = rng.standard_normal((1, H, d, d))
    states = _stepwise_states(orc, q, k, v, g, beta, S0)
    for t in range(T):
        for h in range(H):
            Sp = np.exp(g[t, h])[:, None] * states[t][0, h]
            lhs = states[t + 1][0, h].T @ k[t, h]
            rhs = (1 - beta[t, h]) * (Sp.T @ k[t, h]) + beta[t, h] * v[t, h]
            assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-12), f"interpolation t={t}"
            if beta[t, h] == 1.0:
                assert np.allclose(lhs, v[t, h], rtol=1e-12, atol=1e-12), "beta=1 recall"


def pin_orthonormal_recall(orc):
    """alpha = 1, beta = 1, orthonormal keys, S_0 = 0: S^T k_j = v_j for every
    written key; re-writing a key replaces its value; reading with q_t = k_t
    returns v_t (the read follows the write)."""
    rng = np.random.default_rng(14)
    d, H = 16, 2
    m = 10
    keys = np.empty((m, H, d))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        keys[:, h] = Qm[:, :m].T
    order = list(range(m)) + [3, 7]  # two re-writes at the end
    k = keys[order]
    T = len(order)
    v = rng.standard_normal((T, H, d))
    q = k.copy()
    g = np.zeros((T, H, d))
    beta = np.ones((T, H))
    o, S = orc.recurrence(q, k, v, g, beta)
    assert np.allclose(o, v, rtol=1e-12, atol=1e-12), "read-after-write recall"
    last = {}
    for t, j in enumerate(order):
        last[j] = t
    for j, t in last.items():
        for h in range(H):
            assert np.allclose(S[0, h].T @ keys[j, h], v[t, h], rtol=1e-12, atol=1e-12), \
                f"stored value of key {j}"


def pin_brute_force(orc):
    """Agreement with the dense transition-matrix expansion (numpy fp64) on tiny
    random inputs, nonzero S_0, keys not normalised, beta in (0, 1.5)."""
    rng = np.random.default_rng(15)
    for (T, H, d, dv) in ((9, 2, 4, 4), (24, 1, 8, 8), (16, 2, 16, 16), (7, 1, 6, 3)):
        q, k, v, g, beta = _rand_inputs(rng, T, H, d, unit_k=False, beta_range=(0.0, 1.5),
                                        dv=dv)
        k *= 0.5
        S0 = rng.standard_normal((1, H, d, dv))
        o, S = orc.recurrence(q, k, v, g, beta, S0=S0)
        ob, Sb = oracle_mod.brute_force(q, k, v, g, beta, S0=S0[0])
        assert np.allclose(o, ob, rtol=1e-9, atol=1e-10), f"brute force o {T,H,d,dv}"
        assert np.allclose(S[0], Sb, rtol=1e-9, atol=1e-10), f"brute force S {T,H,d,dv}"


def pin_linearity(orc):
    """For fixed q, k, g, beta the pair (o, S_T) is linear in (V, S_0)."""
    rng = np.random.default_rng(16)
    T, H, d = 15, 2, 8
    q, k, v1, g, beta = _rand_inputs(rng, T, H, d)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, d, d))
    s2 = rng.standard_normal((1, H, d, d))
    a, b = 0.7, -1.3
    o1, S1 = orc.recurrence(q, k, v1, g, beta, S0=s1)
    o2, S2 = orc.recurrence(q, k, v2, g, beta, S0=s2)
    o3, S3 = orc.recurrence(q, k, a * v1 + b * v2, g, beta, S0=a * s1 + b * s2)
    assert np.allclose(o3, a * o1 + b * o2, rtol=1e-10, atol=1e-11), "linearity o"
    assert np.allclose(S3, a * S1 + b * S2, rtol=1e-10, atol=1e-11), "linearity S"


def pin_norm_bound(orc):
    """|k| = 1, beta in [0,1], alpha in (0,1]: ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||
    (I - beta k k^T has eigenvalues 1 and 1 - beta; Diag(alpha) is a contraction)."""
    rng = np.random.default_rng(17)
    T, H, d = 30, 2, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, g_scale=0.2)
    S0 = rng.standard_normal((1, H, d, d)) * 3
    states = _stepwise_states(orc, q, k, v, g, beta, S0)
    for t in range(T):
        for h in range(H):
            n1 = np.linalg.norm(states[t + 1][0, h], 2)
            n0 = np.linalg.norm(states[t][0, h], 2)
            assert n1 <= n0 + beta[t, h] * np.linalg.norm(v[t, h]) + 1e-12, f"norm bound t={t}"


def pin_scalar_gate(orc):
    """A decay that is the same on every channel (scalar a_t per head) gives the
    scalar-gated delta rule S_t = a_t (S_{t-1} - beta_t k_t k_t^T S_{t-1}) + beta_t k_t v_t^T
    (Diag(a_t) = a_t I commutes with the erase)."""
    rng = np.random.default_rng(18)
    T, H, d = 14, 2, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d)
    gs = -np.abs(rng.standard_normal((T, H))) * 0.3
    g = np.repeat(gs[:, :, None], d, axis=2)
    S0 = rng.standard_normal((1, H, d, d))
    o, S = orc.recurrence(q, k, v, g, beta, S0=S0)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            St = np.exp(gs[t, h]) * (St - beta[t, h] * np.outer(k[t, h], k[t, h] @ St)) \
                + beta[t, h] * np.outer(k[t, h], v[t, h])
            assert np.allclose(o[t, h], St.T @ q[t, h], rtol=1e-10, atol=1e-12), "scalar o"
        assert np.allclose(S[0, h], St, rtol=1e-10, atol=1e-12), "scalar S"


def pin_padding(orc):
    """Tokens with beta = 0, g = 0 and k = 0 leave the state unchanged, so padding
    a sequence with them changes neither its outputs nor its final state."""
    rng = np.random.default_rng(19)
    T, H, d = 11, 2, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d)
    S0 = rng.standard_normal((1, H, d, d))
    o, S = orc.recurrence(q, k, v, g, beta, S0=S0)
    P = 5
    pad = lambda x, fill: np.concatenate([x, np.full((P,) + x.shape[1:], fill)], axis=0)
    qp = np.concatenate([q, rng.standard_normal((P, H, d))])
    vp = np.concatenate([v, rng.standard_normal((P, H, d))])
    op, Sp = orc.recurrence(qp, pad(k, 0.0), vp, pad(g, 0.0), pad(beta, 0.0), S0=S0)
    assert np.array_equal(Sp, S), "padding changed the state"
    assert np.array_equal(op[:T], o), "padding changed the outputs"


def pin_packing(orc):
    """A packed run equals separate runs, sequence by sequence, bit for bit
    (nothing crosses a sequence boundary)."""
    rng = np.random.default_rng(20)
    lens = [5, 0, 9, 1]
    T, H, d = sum(lens), 2, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, d)
    S0 = rng.standard_normal((len(lens), H, d, d))
    cu = np.array([0] + list(np.cumsum(lens)), dtype=np.int32)
    o, S = orc.recurrence(q, k, v, g, beta, cu_seqlens=cu, S0=S0)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, Sn = orc.recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], S0=S0[n:n + 1])
        assert np.array_equal(o[sl], on), f"packing o seq {n}"
        assert np.array_equal(S[n], Sn[0]), f"packing S seq {n}"


def pin_f32_close_to_f64(orc):
    """The fp32 build of the recurrence stays within 1e-5 (relative Frobenius) of
    the fp64 one on a 256-token run with d = 32."""
    rng = np.random.default_rng(21)
    T, H, d = 256, 2, 32
    q, k, v, g, beta = _rand_inputs(rng, T, H, d)
    o64, S64 = orc.recurrence(q, k, v, g, beta, precision="f64")
    o32, S32 = orc.recurrence(q, k, v, g, beta, precision="f32")
    assert np.linalg.norm(o32 - o64) / np.linalg.norm(o64) < 1e-5
    assert np.linalg.norm(S32 - S64) / np.linalg.norm(S64) < 1e-5


RECURRENCE_PINS = [pin_identity, pin_pure_decay, pin_delta_interpolation,
                   pin_orthonormal_recall, pin_brute_force, pin_linearity, pin_norm_bound,
                   pin_scalar_gate, pin_padding, pin_packing, pin_f32_close_to_f64]


# --------------------------------------------------------------------------- conv

def pin_conv_identity_tap(orc):
    """w[c] = (0, 0, 0, 1): the tap w[c][3] multiplies the current token, so y = x."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((13, 6))
    w = np.zeros((6, 4))
    w[:, 3] = 1.0
    y, _ = orc.short_conv(x, w)
    assert np.array_equal(y, x)


def pin_conv_numpy(orc):
    """Each channel equals numpy.convolve(x_c, reversed w_c) truncated to T (causal,
    zero history), including packed sequences restarting from zero history."""
    rng = np.random.default_rng(32)
    lens = [7, 1, 12]
    T, C = sum(lens), 5
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4))
    cu = np.array([0] + list(np.cumsum(lens)), dtype=np.int32)
    y, tail = orc.short_conv(x, w, cu_seqlens=cu)
    for n in range(len(lens)):
        for c in range(C):
            xs = x[cu[n]:cu[n + 1], c]
            ref = np.convolve(xs, w[c, ::-1])[:lens[n]]
            assert np.allclose(y[cu[n]:cu[n + 1], c], ref, rtol=1e-13, atol=1e-13)
            hist = np.concatenate([np.zeros(3), xs])
            assert np.array_equal(tail[n, :, c], hist[-3:])


def pin_conv_handoff(orc):
    """Convolving [a; b] equals convolving a, then b starting from a's tail."""
    rng = np.random.default_rng(33)
    C = 4
    a = rng.standard_normal((9, C))
    b = rng.standard_normal((2, C))
    w = rng.standard_normal((C, 4))
    y, tail = orc.short_conv(np.concatenate([a, b]), w)
    ya, ta = orc.short_conv(a, w)
    yb, tb = orc.short_conv(b, w, tail=ta)
    assert np.allclose(y, np.concatenate([ya, yb]), rtol=1e-14, atol=1e-14)
    assert np.array_equal(tail, tb)


def pin_l2norm(orc):
    """Per-head L2 norm: each head's row has unit norm (up to eps) and keeps its
    direction."""
    rng = np.random.default_rng(34)
    x = rng.standard_normal((6, 4 * 16)) * 3
    y = orc.l2norm_heads(x, 16, eps=0.0)
    yh = y.reshape(6, 4, 16)
    xh = x.reshape(6, 4, 16)
    assert np.allclose(np.linalg.norm(yh, axis=-1), 1.0, rtol=1e-14)
    cos = np.sum(yh * xh, axis=-1) / np.linalg.norm(xh, axis=-1)
    assert np.allclose(cos, 1.0, rtol=1e-14)


def pin_l2norm_eps(orc):
    """Where eps enters: inside the square root, x / sqrt(sum x^2 + eps).  Two
    rows whose sum of squares is comparable to eps, with values fixed by hand:
    (3, 4) with eps = 11 gives (3, 4) / sqrt(36) = (1/2, 2/3); four channels of
    0.05 with eps = 0.01 (sum of squares 0.01) give 0.05 / sqrt(0.02) = 1/sqrt(8)
    each.  eps added outside the root, or dropped, or squared, misses both."""
    y = orc.l2norm_heads(np.array([[3.0, 4.0]]), 2, eps=11.0)
    assert np.allclose(y, [[0.5, 2.0 / 3.0]], rtol=1e-15, atol=0), y
    y = orc.l2norm_heads(np.full((1, 8), 0.05), 4, eps=0.01)
    assert np.allclose(y, 1.0 / np.sqrt(8.0), rtol=1e-14, atol=0), y


CONV_PINS = [pin_conv_identity_tap, pin_conv_numpy, pin_conv_handoff, pin_l2norm,
             pin_l2norm_eps]


# --------------------------------------------------------------------------- output gate

def pin_output_gate(gate):
    """The output gate o * sigmoid(z) at values fixed by hand: sigmoid(0) = 1/2,
    sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4, sigmoid(-ln 3) = 1/4; far positive z
    passes o through, far negative z closes the gate; gate(o, z) + gate(o, -z)
    = o (sigmoid(z) + sigmoid(-z) = 1); elementwise, so each (token, head,
    channel) uses its own z."""
    o = np.array([[[2.0, -8.0, 4.0, 1.0]]])
    z = np.array([[[0.0, np.log(3.0), -np.log(3.0), 60.0]]])
    y = gate(o, z)
    assert np.allclose(y, [[[1.0, -6.0, 1.0, 1.0]]], rtol=1e-15, atol=0), y
    assert abs(gate(np.array([5.0]), np.array([-60.0]))[0]) < 1e-24
    assert gate(np.array([3.0]), np.array([-1000.0]))[0] == 0.0
    rng = np.random.default_rng(35)
    o = rng.standard_normal((7, 3, 16))
    z = rng.standard_normal((7, 3, 16)) * 4
    assert np.allclose(gate(o, z) + gate(o, -z), o, rtol=1e-14, atol=1e-14)
    # each element gated by its own z: permuting both the same way commutes
    perm = rng.permutation(16)
    assert np.array_equal(gate(o[..., perm], z[..., perm]), gate(o, z)[..., perm])
