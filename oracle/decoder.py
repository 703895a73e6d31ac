"""The plain decoder the megakernel must reproduce (test infrastructure only).

This is the textbook pre-norm Llama-style decoder, one token per sequence per
call, written out in float64. The megakernel reaches this same result (up to
rounding order), so the oracle is the definition itself, in the operator order
the pages wire up (MPK walk-through, section 3.3.1 "build_mirage_graph": embed,
then per layer RMSNorm+QKV, attention with RoPE and the KV cache, O-projection
+ residual, RMSNorm+gate/up, SiLU-multiply + down-projection + residual, then
the final RMSNorm + LM head and argmax; Hazy megakernel summary: the same fused
instruction list).

Where the pages leave a step open, the readings used are:

* RMSNorm: ``g_i * x_i / sqrt(mean_j x_j^2 + eps)`` (eps inside the root).
* RoPE: the HF half-split rotation, ``w_j = theta^(-2j/D)`` for ``j < D/2``,
  angle ``p * w_j``; no frequency scaling. Keys are cached after rotation.
* GQA: query head ``h`` reads kv head ``h // (Hq/Hkv)``.
* Attention: scale ``1/sqrt(D)``, causal over positions ``0..p`` inclusive.
* KV cache entries are stored as bf16 (round to nearest even) and read back
  from the cache, including the entry just written.
* Logits stay in full precision; argmax returns the lowest index among ties.
* SiLU: ``z / (1 + exp(-z))``.
* Optional per-head q/k RMSNorm (``shape.qk_norm``): the attention layer of the
  MPK walk-through's demo takes q_norm and k_norm weights (section 3.3.1,
  ``attention_layer``); each query and key head vector (length D) is RMS
  normalised with its [D] gain and the same eps, after the projection and
  before RoPE (the Qwen3 order; the pages name the weights only).

Numbers: float64 throughout; weights are bf16 bit patterns decoded exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import bf16


# ----------------------------------------------------------------------------
# elementwise / small building blocks (each pinned in tests/oracle)
# ----------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, times the gain."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def rope_angles(pos: int, head_dim: int, theta: float) -> np.ndarray:
    """Rotation angles ``pos * theta^(-2j/D)`` for ``j < D/2`` (float64)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -2.0 * j / head_dim)


def rope(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate each head vector (last axis, length D) by its position.

    Pairs are (j, j + D/2): ``u'_j = u_j cos - u_{j+D/2} sin`` and
    ``u'_{j+D/2} = u_{j+D/2} cos + u_j sin``.
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    a = rope_angles(pos, d, theta)
    c, s = np.cos(a), np.sin(a)
    lo, hi = u[..., : d // 2], u[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """One query head against ``n`` cached positions: softmax(k q / sqrt(D)) v."""
    d = q.shape[-1]
    s = (k @ q) / np.sqrt(float(d))
    return softmax(s) @ v


def argmax_first(x: np.ndarray) -> int:
    """Index of the maximum; the lowest index wins a tie."""
    return int(np.argmax(x))


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class State:
    """Per-sequence decode state: the bf16 KV cache (bit patterns)."""
    kcache: np.ndarray      # uint16 [L][B][Hkv][S][D]
    vcache: np.ndarray      # uint16 [L][B][Hkv][S][D]


class Model:
    """Decoder with bf16 weights given as bit patterns (HF ``[out, in]``).

    ``weights`` maps the names of ``workload.weight_names`` (``embed``,
    ``l{i}.wq`` ... ``l{i}.g_mlp``, ``lm_head`` when untied, ``g_final``) to
    uint16 arrays. Matrices are decoded to float64 on use (``cache=True`` keeps
    the decoded copies, for small models).
    """

    def __init__(self, shape, weights: Dict[str, np.ndarray], cache: bool = False,
                 kv_round: bool = True):
        self.s = shape
        self.w = weights
        self._cache = {} if cache else None
        # kv_round=False keeps K/V in float64 (cache arrays then hold float64);
        # it exists only to compare the rest of the definition with a
        # third-party decoder that has no bf16 cache.
        self.kv_round = kv_round

    def _store(self, x: np.ndarray) -> np.ndarray:
        return bf16.encode(x) if self.kv_round else np.asarray(x, dtype=np.float64)

    def _load(self, x: np.ndarray) -> np.ndarray:
        return bf16.decode(x) if self.kv_round else np.asarray(x, dtype=np.float64)

    # -- weights -------------------------------------------------------------
    def W(self, name: str) -> np.ndarray:
        if name == "lm_head" and self.s.tied:
            name = "embed"
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        m = bf16.decode(self.w[name])
        if self._cache is not None:
            self._cache[name] = m
        return m

    def _qk_norm(self, l: int, q: np.ndarray, k: np.ndarray):
        """Per-head RMSNorm of query and key head vectors (last axis, D), when
        the shape has it; identity otherwise."""
        if not getattr(self.s, "qk_norm", False):
            return q, k
        gq = bf16.decode(self.w[f"l{l}.q_norm"])
        gk = bf16.decode(self.w[f"l{l}.k_norm"])
        return rmsnorm(q, gq, self.s.rms_eps), rmsnorm(k, gk, self.s.rms_eps)

    def embed_row(self, tok: int) -> np.ndarray:
        return bf16.decode(self.w["embed"][int(tok)])

    # -- state ---------------------------------------------------------------
    def new_state(self, batch: int, max_seq: int) -> State:
        s = self.s
        shp = (s.n_layers, batch, s.n_kv_heads, max_seq, s.head_dim)
        dt = np.uint16 if self.kv_round else np.float64
        return State(np.zeros(shp, dt), np.zeros(shp, dt))

    # -- one decode step -----------------------------------------------------
    def decode_step(self, st: State, tokens: Sequence[int], pos: Sequence[int],
                    want_hidden: bool = False, kv_given: bool = False):
        """Feed ``tokens[b]`` at position ``pos[b]``; write K/V there; return
        float64 logits ``[B, V]`` (and the final hidden states if asked).

        ``kv_given=True`` leaves the cache entries at ``pos[b]`` as the state
        holds them (written by another implementation of the same step) and
        attends over those instead of this step's own rounding of K/V; the
        arithmetic is otherwise unchanged. Tests use it to compare logits over
        one identical cache."""
        s = self.s
        B = len(tokens)
        G, D = s.group, s.head_dim
        x = np.stack([self.embed_row(t) for t in tokens])          # [B, H]
        for l in range(s.n_layers):
            wq, wk, wv = self.W(f"l{l}.wq"), self.W(f"l{l}.wk"), self.W(f"l{l}.wv")
            wo = self.W(f"l{l}.wo")
            ga = bf16.decode(self.w[f"l{l}.g_attn"])
            gm = bf16.decode(self.w[f"l{l}.g_mlp"])
            attn = np.zeros((B, s.n_q_heads * D))
            h = rmsnorm(x, ga, s.rms_eps)                           # [B, H]
            qs = (h @ wq.T).reshape(B, s.n_q_heads, D)
            ks = (h @ wk.T).reshape(B, s.n_kv_heads, D)
            vs = (h @ wv.T).reshape(B, s.n_kv_heads, D)
            qs, ks = self._qk_norm(l, qs, ks)
            for b in range(B):
                p = int(pos[b])
                q = rope(qs[b], p, s.rope_theta)
                k = rope(ks[b], p, s.rope_theta)
                if not kv_given:
                    st.kcache[l, b, :, p] = self._store(k)
                    st.vcache[l, b, :, p] = self._store(vs[b])
                for g in range(s.n_kv_heads):
                    kk = self._load(st.kcache[l, b, g, : p + 1])
                    vv = self._load(st.vcache[l, b, g, : p + 1])
                    for hq in range(g * G, (g + 1) * G):
                        attn[b, hq * D:(hq + 1) * D] = attend(q[hq], kk, vv)
            x = x + attn @ wo.T
            wg, wu, wd = self.W(f"l{l}.wg"), self.W(f"l{l}.wu"), self.W(f"l{l}.wd")
            h2 = rmsnorm(x, gm, s.rms_eps)
            x = x + (silu(h2 @ wg.T) * (h2 @ wu.T)) @ wd.T
        gf = bf16.decode(self.w["g_final"])
        xf = rmsnorm(x, gf, s.rms_eps)
        logits = xf @ self.W("lm_head").T
        return (logits, x) if want_hidden else logits

    # -- whole prompt without a cache ------------------------------------------
    def forward_full(self, tokens: Sequence[int]):
        """Causal forward of one sequence over all its positions at once, with
        no cache (keys/values rounded to bf16 as the cache would hold them).
        Returns float64 logits ``[P, V]`` and the bf16 K/V it produced
        ``[L][Hkv][P][D]``."""
        s = self.s
        G, D = s.group, s.head_dim
        P = len(tokens)
        x = np.stack([self.embed_row(t) for t in tokens])          # [P, H]
        ks, vs = [], []
        for l in range(s.n_layers):
            ga = bf16.decode(self.w[f"l{l}.g_attn"])
            gm = bf16.decode(self.w[f"l{l}.g_mlp"])
            h = rmsnorm(x, ga, s.rms_eps)
            q = (h @ self.W(f"l{l}.wq").T).reshape(P, s.n_q_heads, D)
            k = (h @ self.W(f"l{l}.wk").T).reshape(P, s.n_kv_heads, D)
            v = (h @ self.W(f"l{l}.wv").T).reshape(P, s.n_kv_heads, D)
            q, k = self._qk_norm(l, q, k)
            q = np.stack([rope(q[p], p, s.rope_theta) for p in range(P)])
            k = np.stack([rope(k[p], p, s.rope_theta) for p in range(P)])
            kb = self._store(k).transpose(1, 0, 2)                  # [Hkv, P, D]
            vb = self._store(v).transpose(1, 0, 2)
            ks.append(kb)
            vs.append(vb)
            kd, vd = self._load(kb), self._load(vb)
            attn = np.zeros((P, s.n_q_heads * D))
            mask = np.triu(np.full((P, P), -np.inf), k=1)            # causal
            for hq in range(s.n_q_heads):
                g = hq // G
                sc = (q[:, hq] @ kd[g].T) / np.sqrt(float(D)) + mask
                attn[:, hq * D:(hq + 1) * D] = softmax(sc) @ vd[g]
            x = x + attn @ self.W(f"l{l}.wo").T
            h2 = rmsnorm(x, gm, s.rms_eps)
            x = x + (silu(h2 @ self.W(f"l{l}.wg").T) * (h2 @ self.W(f"l{l}.wu").T)) @ self.W(f"l{l}.wd").T
        gf = bf16.decode(self.w["g_final"])
        logits = rmsnorm(x, gf, s.rms_eps) @ self.W("lm_head").T
        return logits, np.stack(ks), np.stack(vs)


# ----------------------------------------------------------------------------
# decoding protocol
# ----------------------------------------------------------------------------

def top2_margin(logits: np.ndarray) -> float:
    """Gap between the largest and second-largest logit (near-tie diagnostics)."""
    part = np.partition(np.asarray(logits), -2)
    return float(part[-1] - part[-2])


def prefill_prompt(m: Model, st: State, prompt: np.ndarray):
    """Consume prompt tokens ``0..P-2`` as single-token steps at positions
    ``0..P-2`` (their logits are not needed). ``prompt`` is ``[B, P]``."""
    B, P = prompt.shape
    for p in range(P - 1):
        m.decode_step(st, prompt[:, p], [p] * B)


def greedy(m: Model, st: State, first_tokens: Sequence[int], first_pos: Sequence[int],
           steps: int, keep_logits: bool = False):
    """``steps`` greedy decode steps. Step 0 feeds ``first_tokens[b]`` at
    ``first_pos[b]``; step k feeds the previous argmax at ``first_pos[b] + k``.
    Returns token ids ``[steps, B]``, per-step top-2 margins and (optionally)
    the per-step logits."""
    B = len(first_tokens)
    toks = np.zeros((steps, B), dtype=np.int64)
    margins = np.zeros((steps, B))
    all_logits: List[np.ndarray] = []
    cur = [int(t) for t in first_tokens]
    for k in range(steps):
        lg = m.decode_step(st, cur, [int(p) + k for p in first_pos])
        if keep_logits:
            all_logits.append(lg)
        for b in range(B):
            toks[k, b] = argmax_first(lg[b])
            margins[k, b] = top2_margin(lg[b])
        cur = [int(t) for t in toks[k]]
    return toks, margins, all_logits
