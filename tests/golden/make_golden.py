"""Write the stored expected values for the tiny config (calls only the oracle).

Usage: python tests/golden/make_golden.py   (from the repository root)

Writes tests/golden/tiny_greedy.json: the oracle's 16 greedy token ids for the
tiny config's seeded 8-token prompt (norm gains 1.0 and random), the top-2
logit margin of each step, and the first 8 logits of each step.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workload  # noqa: E402
from oracle.decoder import Model, greedy, prefill_prompt  # noqa: E402


def to_u16(t):
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def run(gains):
    wl = workload.config(0)
    w = workload.make_weights(wl, gains=gains)
    m = Model(wl.shape, {k: to_u16(v) for k, v in w.items()}, cache=True)
    prompt = workload.make_prompt(wl)
    st = m.new_state(1, wl.max_seq)
    prefill_prompt(m, st, prompt)
    P = prompt.shape[1]
    toks, margins, logits = greedy(m, st, prompt[:, -1], [P - 1], wl.steps, keep_logits=True)
    return {"prompt": prompt[0].tolist(), "tokens": toks[:, 0].tolist(),
            "margins": margins[:, 0].tolist(),
            "logits_head": [lg[0, :8].tolist() for lg in logits]}


if __name__ == "__main__":
    out = {"config": workload.config(0).name,
           "source": "oracle.decoder greedy protocol; seeds per workload module",
           "ones": run("ones"), "random": run("random")}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_greedy.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)
