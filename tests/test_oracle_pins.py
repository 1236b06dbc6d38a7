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
