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
