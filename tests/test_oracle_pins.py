"""The CPU oracle against facts fixed by the definition, closed forms, library
routines and brute force (see ``pins.py``), plus the pages' printed sizes."""
import json
import os

import numpy as np
import pytest

import oracle
from pins import CONV_PINS, RECURRENCE_PINS

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIB)


@pytest.mark.parametrize("pin", RECURRENCE_PINS + CONV_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_state_size_matches_pages(orc):
    """The oracle's per-sequence state for the layer the pages describe (64 heads,
    128 x 128, fp32) times 63 KDA layers is the pages' 264.2 MB = 252 MiB."""
    gold = json.load(open(os.path.join(HERE, "golden", "state_sizes.json")))
    H, d = gold["heads"], gold["head_dim"]
    rng = np.random.default_rng(0)
    T = 2
    z = np.zeros((T, H, d))
    _, S = orc.recurrence(z, z, z, z, np.zeros((T, H)), precision="f32")
    per_layer = S[0].astype(np.float32).nbytes
    total = per_layer * gold["kda_layers"]
    assert total == gold["state_bytes_per_sequence_all_layers"]
    assert round(total / 1e6, 1) == gold["state_MB_printed"]
    assert total / 2 ** 20 == gold["state_MiB_printed"]
    assert H * d == gold["qkv_width"]


# ---- bfloat16 storage rounding (the bf16-state decode's write-back)
# (value, its nearest bfloat16 with ties to even): bfloat16 keeps 8 significant
# bits, so just above 1 its spacing is 2^-7 and in [128, 256) it is 1.
BF16_CASES = [
    (1.0 + 2.0 ** -8, 1.0),                        # tie: down to the even neighbour
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),        # tie: up to the even neighbour
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # just above a tie: up
    (1.0 + 2.0 ** -8 - 2.0 ** -30, 1.0),           # just below a tie: down
    (-(1.0 + 3 * 2.0 ** -8), -(1.0 + 2.0 ** -6)),  # sign kept
    (255.5, 256.0),                                # tie carried into the exponent
    (0.15625, 0.15625),                            # representable: unchanged
    (0.0, 0.0),
]


@pytest.mark.parametrize("x,want", BF16_CASES)
def test_round_bf16_cases(x, want):
    assert oracle.round_bf16(np.array([x]))[0] == want


def test_round_bf16_matches_torch_on_binary32():
    """On binary32 inputs the rounding equals torch's float32 -> bfloat16
    conversion, an independent implementation, bit for bit."""
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(7).standard_normal(200_000).astype(np.float32)
    x[::3] *= 1e-3
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_conv_tail_size_matches_pages():
    """A conv tail as the library keeps it, [3, channels] bf16 per sequence and
    layer for the q, k, v streams (3 x 8192 channels), over 63 KDA layers, is
    the pages' ~9 MB per sequence."""
    gold = json.load(open(os.path.join(HERE, "golden", "state_sizes.json")))
    assert gold["conv_channels"] == 3 * gold["qkv_width"]
    per_layer = gold["conv_history_tokens"] * gold["conv_channels"] * \
        gold["conv_tail_bytes_per_element"]
    total = per_layer * gold["kda_layers"]
    assert round(total / 1e6) == gold["conv_tail_MB_printed"]


# ---- gate prologue (decay and write strength from the projections' outputs)
def test_gate_prologue_unit_rate_is_logsigmoid():
    """With a_log = 0 (rate 1) the decay is alpha = sigmoid(-f), i.e. g equals
    torch's logsigmoid(-f), an independent implementation; beta equals
    torch.sigmoid(b)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    f = rng.standard_normal((50, 3, 8)) * 6
    b = rng.standard_normal((50, 3)) * 6
    g, beta = oracle.gate_prologue(f, np.zeros(3), b)
    want_g = torch.nn.functional.logsigmoid(-torch.from_numpy(f)).numpy()
    assert np.allclose(g, want_g, rtol=1e-13, atol=1e-300)
    assert np.allclose(beta, torch.sigmoid(torch.from_numpy(b)).numpy(), rtol=1e-14)


def test_gate_prologue_closed_forms():
    """f = 0 gives g = -exp(a_log) ln 2 per head (heads on the second-to-last
    axis, channels on the last); the decay scales linearly with the rate
    exp(a_log); far tails follow softplus's asymptotes; alpha lies in (0, 1]."""
    a_log = np.array([0.0, np.log(3.0), -1.5])
    g0, beta0 = oracle.gate_prologue(np.zeros((2, 3, 5)), a_log, np.zeros((2, 3)))
    assert np.allclose(g0, -np.exp(a_log)[None, :, None] * np.log(2.0) * np.ones((2, 3, 5)),
                       rtol=1e-15)
    assert np.all(beta0 == 0.5)
    rng = np.random.default_rng(22)
    f = rng.standard_normal((4, 3, 5))
    g_unit, _ = oracle.gate_prologue(f, np.zeros(3), np.zeros((4, 3)))
    g_rate, _ = oracle.gate_prologue(f, a_log, np.zeros((4, 3)))
    assert np.allclose(g_rate, g_unit * np.exp(a_log)[None, :, None], rtol=1e-14)
    lo, _ = oracle.gate_prologue(np.full((1, 1, 1), -40.0), np.zeros(1), np.zeros((1, 1)))
    hi, _ = oracle.gate_prologue(np.full((1, 1, 1), 40.0), np.zeros(1), np.zeros((1, 1)))
    assert abs(lo[0, 0, 0] / -np.exp(-40.0) - 1) < 1e-12
    assert abs(hi[0, 0, 0] / -40.0 - 1) < 1e-15
    alpha = np.exp(oracle.gate_prologue(rng.standard_normal((9, 3, 5)) * 20, a_log,
                                        np.zeros((9, 3)))[0])
    assert np.all((alpha > 0) & (alpha <= 1))


def test_output_gate_pin():
    from pins import pin_output_gate
    pin_output_gate(oracle.output_gate)


# plausible mistakes in an output gate, each of which the pin must reject
WRONG_GATES = {
    "gate_sign_flipped": lambda o, z: o / (1.0 + np.exp(z)),
    "raw_multiply": lambda o, z: o * z,
    "tanh_gate": lambda o, z: o * np.tanh(z),
    "additive": lambda o, z: o + 1.0 / (1.0 + np.exp(-z)),
    "swish_gate": lambda o, z: o * z / (1.0 + np.exp(-z)),
    "gate_per_head": lambda o, z: o / (1.0 + np.exp(-z.mean(axis=-1, keepdims=True))),
}


@pytest.mark.parametrize("name", list(WRONG_GATES))
def test_output_gate_pin_catches(name):
    from pins import pin_output_gate
    with np.errstate(over="ignore", invalid="ignore"):
        with pytest.raises(AssertionError):
            pin_output_gate(WRONG_GATES[name])
