"""The stored tiny-config expectations (tests/golden/tiny_greedy.json, written
by tests/golden/make_golden.py from the oracle alone) still hold: guards the
oracle and the seeded input recipe against silent change."""
import json
import os

import numpy as np
import pytest

import workload
from oracle.decoder import greedy, prefill_prompt
from tests.helpers import oracle_model

GOLDEN = os.path.join(os.path.dirname(os.path.dirname(__file__)), "golden", "tiny_greedy.json")


@pytest.mark.parametrize("gains", ["ones", "random"])
def test_tiny_greedy_golden(gains):
    ref = json.load(open(GOLDEN))[gains]
    wl = workload.config(0)
    m = oracle_model(0, gains)
    prompt = workload.make_prompt(wl)
    assert prompt[0].tolist() == ref["prompt"]
    st = m.new_state(1, wl.max_seq)
    prefill_prompt(m, st, prompt)
    toks, margins, logits = greedy(m, st, prompt[:, -1], [prompt.shape[1] - 1], wl.steps, True)
    assert toks[:, 0].tolist() == ref["tokens"]
    assert np.allclose([lg[0, :8] for lg in logits], ref["logits_head"], rtol=0, atol=1e-12)
