"""Shared test helpers: seeded workloads turned into oracle inputs."""
import functools

import numpy as np

import workload


def to_u16(t) -> np.ndarray:
    """torch.bfloat16 CPU tensor -> uint16 bit patterns (no arithmetic)."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=4)
def weights(cfg_index: int, gains: str = "ones"):
    wl = workload.config(cfg_index)
    return wl, workload.make_weights(wl, gains=gains)


def oracle_model(cfg_index: int, gains: str = "ones", cache: bool = True, kv_round: bool = True,
                 shape=None, w=None):
    from oracle.decoder import Model
    wl, wt = weights(cfg_index, gains) if w is None else (workload.config(cfg_index), w)
    u16 = {k: to_u16(v) for k, v in wt.items()}
    return Model(shape or wl.shape, u16, cache=cache, kv_round=kv_round)


def progress(msg: str) -> None:
    """Print a test's own progress line, and append it to
    gpurun_out/pytest_progress.log when that folder exists (long GPU tests
    run under pytest -q, which holds printed output until the test ends)."""
    import os
    import time
    print(msg, flush=True)
    d = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(d):
        with open(os.path.join(d, "pytest_progress.log"), "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')}   {msg}\n")
