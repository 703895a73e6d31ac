"""Seeded synthetic workloads for the persistent decode megakernel.

This module is shared by the oracle, the tests and the benchmark. It holds the
model shapes and the random-input recipe only: no step of the decoder's
arithmetic lives here.

Recipe (stated once, used everywhere):

* Every tensor ``k`` of config ``i`` is drawn from its own stream
  ``numpy.random.Generator(PCG64(SeedSequence([0, i, k])))`` where ``k`` is the
  tensor's index in :func:`tensor_index` (a fixed enumeration).
* Weight matrices (HF layout ``[out, in]``): ``standard_normal(float32) * 0.02``
  then rounded to bfloat16 (round to nearest even, done by torch's dtype cast).
* Norm gains (the per-head q/k norm gains of a qk_norm shape included) are 1.0
  (HF initialisation) unless ``gains="random"``, in which case they are
  ``1 + 0.1 * standard_normal`` rounded to bfloat16.
* Prompt / first tokens: ``integers(0, vocab)``.
* Prefilled KV (long-context and batch configs): ``standard_normal(float32)``
  rounded to bfloat16, for positions ``< kv_len[b]``; context lengths of the
  batch config are ``integers(512, 8193)`` per sequence.

The pages measure on no public benchmark or dataset; these inputs stand in for
their workload (a 39-token prompt followed by 512 greedy decode steps, batch 1).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "ModelShape", "Workload", "CONFIGS", "config", "tensor_index",
    "make_weights", "make_prompt", "make_prefill", "weight_names",
]


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    tied: bool
    rope_theta: float
    rms_eps: float = 1e-5
    qk_norm: bool = False     # per-head RMSNorm of queries and keys before RoPE

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int            # position in CONFIGS; part of every seed
    name: str
    shape: ModelShape
    batch: int
    max_seq: int
    prompt_len: int       # 0 when the KV cache is prefilled instead
    steps: int            # greedy decode steps
    kv_prefill: str       # "none" | "fixed" | "uniform"
    kv_len: int = 0       # fixed prefill length ("fixed")
    kv_lo: int = 0        # uniform prefill range [kv_lo, kv_hi] ("uniform")
    kv_hi: int = 0


_TINY = ModelShape(2, 256, 4, 2, 64, 688, 1024, False, 1e4)
_1B = ModelShape(16, 2048, 32, 8, 64, 8192, 128256, True, 5e5)
_8B = ModelShape(32, 4096, 32, 8, 128, 14336, 128256, False, 5e5)
_TINY_D128 = ModelShape(2, 512, 8, 2, 128, 1024, 2048, False, 1e4)

CONFIGS: List[Workload] = [
    Workload(0, "tiny-2L-h256", _TINY, 1, 64, 8, 16, "none"),
    Workload(1, "llama3.2-1b-shape", _1B, 1, 4096, 39, 512, "none"),
    Workload(2, "llama3-8b-shape", _8B, 1, 4096, 39, 512, "none"),
    Workload(3, "1b-shape-kv32768", _1B, 1, 32768 + 128, 0, 128, "fixed", kv_len=32768),
    Workload(4, "8b-shape-batch16", _8B, 16, 8192 + 128, 0, 128, "uniform",
             kv_lo=512, kv_hi=8192),
    # test-only: the tiny config's size with the 8B shape's head width (128),
    # four query heads per kv head and an untied LM head
    Workload(5, "tiny-2L-h512-d128", _TINY_D128, 1, 64, 8, 16, "none"),
    # test-only: the tiny config with per-head q/k RMSNorm (the attention of
    # the MPK walk-through's demo model)
    Workload(6, "tiny-2L-h256-qknorm", dataclasses.replace(_TINY, qk_norm=True), 1, 64, 8, 16, "none"),
    # test-only: the tiny config with an FFN width the matrix-core bodies take
    # (a multiple of 64), sixteen sequences: the batched (C4-like) path at a
    # size the oracle runs in seconds
    Workload(7, "tiny-2L-h256-f768-batch16", dataclasses.replace(_TINY, ffn=768), 16, 64, 8, 16, "none"),
]


def config(i: int) -> Workload:
    return CONFIGS[i]


def weight_names(s: ModelShape) -> List[str]:
    """Fixed enumeration of the model's tensors (the seed index is the position)."""
    names = ["embed"]
    for l in range(s.n_layers):
        names += [f"l{l}.{n}" for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd",
                                        "g_attn", "g_mlp")]
    names += ["lm_head", "g_final", "prompt", "first_token", "kv_len"]
    names += [f"l{l}.kcache" for l in range(s.n_layers)]
    names += [f"l{l}.vcache" for l in range(s.n_layers)]
    # appended last so that every earlier tensor keeps its seed index
    names += [f"l{l}.{n}" for l in range(s.n_layers) for n in ("q_norm", "k_norm")]
    return names


def tensor_index(s: ModelShape, name: str) -> int:
    return weight_names(s).index(name)


def _rng(wl: Workload, name: str) -> np.random.Generator:
    k = tensor_index(wl.shape, name)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, wl.index, k])))


def _shape_of(s: ModelShape, name: str):
    H, D, F = s.hidden, s.head_dim, s.ffn
    base = name.split(".")[-1]
    return {
        "embed": (s.vocab, H), "lm_head": (s.vocab, H),
        "wq": (s.n_q_heads * D, H), "wk": (s.n_kv_heads * D, H),
        "wv": (s.n_kv_heads * D, H), "wo": (H, s.n_q_heads * D),
        "wg": (F, H), "wu": (F, H), "wd": (H, F),
        "g_attn": (H,), "g_mlp": (H,), "g_final": (H,),
        "q_norm": (D,), "k_norm": (D,),
    }[base]


def _draw_bf16(wl: Workload, name: str, scale: float, offset: float = 0.0):
    import torch
    shape = _shape_of(wl.shape, name)
    g = _rng(wl, name)
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16)
    chunk = 1 << 24                      # fixed chunking: same stream order always
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        x = g.standard_normal(b - a, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        if offset != 0.0:
            x += np.float32(offset)
        out[a:b] = torch.from_numpy(x).to(torch.bfloat16)
    return out.view(*shape)


def make_weights(wl: Workload, gains: str = "ones", threads: int = 8) -> Dict[str, "object"]:
    """All weights as CPU torch.bfloat16 tensors in HF layout.

    ``lm_head`` is absent when the embedding is tied.
    """
    import torch
    s = wl.shape
    jobs = ["embed"]
    for l in range(s.n_layers):
        jobs += [f"l{l}.{n}" for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")]
    if not s.tied:
        jobs.append("lm_head")
    out: Dict[str, object] = {}
    with ThreadPoolExecutor(max(1, threads)) as ex:
        for name, t in zip(jobs, ex.map(lambda n: _draw_bf16(wl, n, 0.02), jobs)):
            out[name] = t
    norms = [f"l{l}.{n}" for l in range(s.n_layers) for n in ("g_attn", "g_mlp")] + ["g_final"]
    if s.qk_norm:
        norms += [f"l{l}.{n}" for l in range(s.n_layers) for n in ("q_norm", "k_norm")]
    for name in norms:
        if gains == "random":
            out[name] = _draw_bf16(wl, name, 0.1, 1.0)
        else:
            out[name] = torch.ones(_shape_of(s, name), dtype=torch.bfloat16)
    return out


def make_prompt(wl: Workload) -> np.ndarray:
    """Prompt token ids ``[batch, prompt_len]`` (int64), or the first token
    ``[batch, 1]`` when the cache is prefilled instead."""
    if wl.prompt_len > 0:
        return _rng(wl, "prompt").integers(0, wl.shape.vocab, size=(wl.batch, wl.prompt_len))
    return _rng(wl, "first_token").integers(0, wl.shape.vocab, size=(wl.batch, 1))


def kv_lengths(wl: Workload) -> np.ndarray:
    """Prefilled context length per sequence (0 for prompt configs)."""
    if wl.kv_prefill == "none":
        return np.zeros(wl.batch, dtype=np.int64)
    if wl.kv_prefill == "fixed":
        return np.full(wl.batch, wl.kv_len, dtype=np.int64)
    return _rng(wl, "kv_len").integers(wl.kv_lo, wl.kv_hi + 1, size=wl.batch)


def make_prefill(wl: Workload, layers: Optional[List[int]] = None):
    """Prefilled K and V caches as CPU bf16 tensors ``[L][B][Hkv][max_seq][D]``
    (zeros past each sequence's length). Returns (k, v) or (None, None)."""
    import torch
    s = wl.shape
    if wl.kv_prefill == "none":
        return None, None
    lens = kv_lengths(wl)
    layers = list(range(s.n_layers)) if layers is None else layers
    shape = (len(layers), wl.batch, s.n_kv_heads, wl.max_seq, s.head_dim)
    k = torch.zeros(shape, dtype=torch.bfloat16)
    v = torch.zeros(shape, dtype=torch.bfloat16)
    for li, l in enumerate(layers):
        for which, dst in (("kcache", k), ("vcache", v)):
            g = _rng(wl, f"l{l}.{which}")
            for b in range(wl.batch):
                n = int(lens[b]) * s.n_kv_heads * s.head_dim
                x = g.standard_normal(n, dtype=np.float32).reshape(s.n_kv_heads, int(lens[b]), s.head_dim)
                dst[li, b, :, : int(lens[b])] = torch.from_numpy(x).to(torch.bfloat16)
    return k, v
