"""Whole-decoder pins for the oracle.

* HF transformers' LlamaForCausalLM (a third-party implementation of the same
  textbook decoder) in float64 on the tiny config, with random norm gains, tied
  and untied: it has no bf16 KV cache, so it is compared with the oracle run
  with ``kv_round=False``. HF computes RMSNorm and softmax in float32, hence the
  1e-5 tolerance.
* Incremental decoding equals the no-cache causal forward on the same tokens
  (logits and the bf16 cache bit patterns).
* A layer whose O and down projections are zero is the identity on the
  residual stream.
* Grouped-query attention equals multi-head attention with the K/V heads
  repeated per query head.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workload
from oracle import bf16
from oracle.decoder import Model, greedy, prefill_prompt
from tests.helpers import oracle_model, to_u16, weights


def hf_model(shape, w, tied):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.hidden,
                      intermediate_size=shape.ffn, num_hidden_layers=shape.n_layers,
                      num_attention_heads=shape.n_q_heads, num_key_value_heads=shape.n_kv_heads,
                      head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps,
                      rope_theta=shape.rope_theta, tie_word_embeddings=tied,
                      attention_bias=False, mlp_bias=False, max_position_embeddings=128,
                      attn_implementation="eager")
    m = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": w["embed"], "model.norm.weight": w["g_final"]}
    for l in range(shape.n_layers):
        p = f"model.layers.{l}."
        sd.update({p + "self_attn.q_proj.weight": w[f"l{l}.wq"], p + "self_attn.k_proj.weight": w[f"l{l}.wk"],
                   p + "self_attn.v_proj.weight": w[f"l{l}.wv"], p + "self_attn.o_proj.weight": w[f"l{l}.wo"],
                   p + "mlp.gate_proj.weight": w[f"l{l}.wg"], p + "mlp.up_proj.weight": w[f"l{l}.wu"],
                   p + "mlp.down_proj.weight": w[f"l{l}.wd"],
                   p + "input_layernorm.weight": w[f"l{l}.g_attn"],
                   p + "post_attention_layernorm.weight": w[f"l{l}.g_mlp"]})
    sd["lm_head.weight"] = w["embed"] if tied else w["lm_head"]
    sd = {k: v.double() for k, v in sd.items()}
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    return m


@pytest.mark.parametrize("tied", [False, True])
def test_matches_transformers_llama(tied):
    wl, w = weights(0, "random")
    shape = dataclasses.replace(wl.shape, tied=tied)
    w = dict(w)
    if tied:
        w.pop("lm_head", None)
    toks = workload.make_prompt(wl)[0]
    with torch.no_grad():
        ref = hf_model(shape, w, tied)(torch.tensor(toks)[None], use_cache=False).logits[0].numpy()
    om = Model(shape, {k: to_u16(v) for k, v in w.items()}, cache=True, kv_round=False)
    full, _, _ = om.forward_full(toks)
    assert np.max(np.abs(full - ref)) < 1e-5, np.max(np.abs(full - ref))
    st = om.new_state(1, wl.max_seq)
    for p, t in enumerate(toks):
        lg = om.decode_step(st, [t], [p])[0]
        assert np.max(np.abs(lg - ref[p])) < 1e-5


def test_incremental_equals_full_forward():
    wl, _ = weights(0, "random")
    om = oracle_model(0, "random")
    toks = workload.make_prompt(wl)[0]
    full, ks, vs = om.forward_full(toks)
    st = om.new_state(1, wl.max_seq)
    for p, t in enumerate(toks):
        lg = om.decode_step(st, [t], [p])[0]
        assert np.allclose(lg, full[p], rtol=0, atol=1e-11)
    P = len(toks)
    assert np.array_equal(st.kcache[:, 0, :, :P], ks)
    assert np.array_equal(st.vcache[:, 0, :, :P], vs)


def test_zero_projection_layer_is_identity():
    wl, w = weights(0, "random")
    one = dataclasses.replace(wl.shape, n_layers=1)
    w2 = dict(w)
    w2["l1.wo"] = torch.zeros_like(w["l1.wo"])
    w2["l1.wd"] = torch.zeros_like(w["l1.wd"])
    m2 = Model(wl.shape, {k: to_u16(v) for k, v in w2.items()}, cache=True)
    m1 = Model(one, {k: to_u16(v) for k, v in w2.items()}, cache=True)
    toks = workload.make_prompt(wl)[0]
    s2, s1 = m2.new_state(1, 16), m1.new_state(1, 16)
    for p, t in enumerate(toks):
        assert np.array_equal(m2.decode_step(s2, [t], [p]), m1.decode_step(s1, [t], [p]))


def test_gqa_equals_mha_with_repeated_kv():
    wl, w = weights(0, "random")
    s = wl.shape
    G, D = s.group, s.head_dim
    mha = dataclasses.replace(s, n_kv_heads=s.n_q_heads)
    w2 = dict(w)
    for l in range(s.n_layers):
        for nm in ("wk", "wv"):
            t = w[f"l{l}.{nm}"].view(s.n_kv_heads, D, s.hidden)
            w2[f"l{l}.{nm}"] = t.repeat_interleave(G, dim=0).reshape(s.n_q_heads * D, s.hidden)
    a = Model(s, {k: to_u16(v) for k, v in w.items()}, cache=True)
    b = Model(mha, {k: to_u16(v) for k, v in w2.items()}, cache=True)
    toks = workload.make_prompt(wl)[0]
    sa, sb = a.new_state(1, 16), b.new_state(1, 16)
    for p, t in enumerate(toks):
        assert np.array_equal(a.decode_step(sa, [t], [p]), b.decode_step(sb, [t], [p]))


def test_batch_rows_are_independent():
    """Two sequences at different positions decode as they would alone."""
    wl, _ = weights(0, "ones")
    om = oracle_model(0)
    toks = workload.make_prompt(wl)[0]
    sb = om.new_state(2, 32)
    s0, s1 = om.new_state(1, 32), om.new_state(1, 32)
    for p in range(4):
        om.decode_step(s0, [toks[p]], [p])
        om.decode_step(sb, [toks[p], toks[p]], [p, p])
    om.decode_step(sb, [toks[4], toks[5]], [4, 4])   # rows diverge
    lg = om.decode_step(sb, [toks[5], toks[6]], [5, 5])
    for p in range(4):
        om.decode_step(s1, [toks[p]], [p])
    om.decode_step(s1, [toks[5]], [4])
    ref1 = om.decode_step(s1, [toks[6]], [5])[0]
    assert np.allclose(lg[1], ref1, rtol=0, atol=1e-12)   # BLAS row blocking differs


def test_greedy_protocol_and_kv_written():
    wl, _ = weights(0, "ones")
    om = oracle_model(0)
    prompt = workload.make_prompt(wl)
    st = om.new_state(1, wl.max_seq)
    prefill_prompt(om, st, prompt)
    P = prompt.shape[1]
    toks, margins, _ = greedy(om, st, prompt[:, -1], [P - 1], 4)
    assert toks.shape == (4, 1) and np.all(margins > 0)
    assert np.all(st.kcache[:, 0, :, : P - 1 + 4].any(axis=-1))   # every position written
    assert not st.kcache[:, 0, :, P - 1 + 4:].any()


def test_kv_given_reads_the_entries_it_is_given():
    """kv_given=True attends over the cache entries the state already holds at
    the fed position: with the entries the normal step writes there, the
    logits are identical; with other entries, they differ (so the option does
    not silently rewrite them)."""
    wl = workload.config(0)
    m = oracle_model(0, "random")
    prompt = workload.make_prompt(wl)[0]
    st = m.new_state(1, wl.max_seq)
    for p in range(4):
        m.decode_step(st, [int(prompt[p])], [p])
    import copy
    st2 = copy.deepcopy(st)
    ref = m.decode_step(st, [int(prompt[4])], [4])          # writes position 4
    st2.kcache[:, :, :, 4] = st.kcache[:, :, :, 4]
    st2.vcache[:, :, :, 4] = st.vcache[:, :, :, 4]
    got = m.decode_step(st2, [int(prompt[4])], [4], kv_given=True)
    assert np.array_equal(got, ref)
    st3 = copy.deepcopy(st)
    st3.vcache[:, :, :, 4] = bf16.encode(bf16.decode(st3.vcache[:, :, :, 4]) * 2.0)
    other = m.decode_step(st3, [int(prompt[4])], [4], kv_given=True)
    assert not np.allclose(other, ref)
    assert np.array_equal(st3.kcache, st.kcache)            # nothing written


def hf_qwen3(shape, w, tied):
    """HF Qwen3ForCausalLM in float64 with the workload's weights: the same
    pre-norm decoder with per-head q/k RMSNorm before RoPE."""
    from transformers import Qwen3Config, Qwen3ForCausalLM
    cfg = Qwen3Config(vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.ffn,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_theta, tie_word_embeddings=tied,
                      attention_bias=False, max_position_embeddings=128, use_sliding_window=False,
                      attn_implementation="eager")
    m = Qwen3ForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": w["embed"], "model.norm.weight": w["g_final"]}
    for l in range(shape.n_layers):
        p = f"model.layers.{l}."
        sd.update({p + "self_attn.q_proj.weight": w[f"l{l}.wq"], p + "self_attn.k_proj.weight": w[f"l{l}.wk"],
                   p + "self_attn.v_proj.weight": w[f"l{l}.wv"], p + "self_attn.o_proj.weight": w[f"l{l}.wo"],
                   p + "self_attn.q_norm.weight": w[f"l{l}.q_norm"], p + "self_attn.k_norm.weight": w[f"l{l}.k_norm"],
                   p + "mlp.gate_proj.weight": w[f"l{l}.wg"], p + "mlp.up_proj.weight": w[f"l{l}.wu"],
                   p + "mlp.down_proj.weight": w[f"l{l}.wd"],
                   p + "input_layernorm.weight": w[f"l{l}.g_attn"],
                   p + "post_attention_layernorm.weight": w[f"l{l}.g_mlp"]})
    sd["lm_head.weight"] = w["embed"] if tied else w["lm_head"]
    sd = {k: v.double() for k, v in sd.items()}
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    return m


def test_qk_norm_matches_transformers_qwen3():
    """The q/k-norm variant (MPK walk-through 3.3.1, attention_layer with
    q_norm and k_norm) against HF's Qwen3 decoder, which normalises each query
    and key head over head_dim before RoPE; random gains, so the [D] gains are
    pinned too. HF computes its norms in float32, hence the 1e-5 tolerance."""
    wl, w = weights(6, "random")
    toks = workload.make_prompt(wl)[0]
    with torch.no_grad():
        ref = hf_qwen3(wl.shape, w, False)(torch.tensor(toks)[None], use_cache=False).logits[0].numpy()
    om = Model(wl.shape, {k: to_u16(v) for k, v in w.items()}, cache=True, kv_round=False)
    full, _, _ = om.forward_full(toks)
    assert np.max(np.abs(full - ref)) < 1e-5, np.max(np.abs(full - ref))
    st = om.new_state(1, wl.max_seq)
    for p, t in enumerate(toks):
        lg = om.decode_step(st, [t], [p])[0]
        assert np.max(np.abs(lg - ref[p])) < 1e-5


def test_qk_norm_scale_invariance():
    """Per-head RMSNorm makes attention independent of the scale of W_q and
    W_k (up to eps): doubling both leaves the logits unchanged to ~1e-4, while
    the same change without the norm moves them far."""
    base = {}
    for cfg in (6, 0):
        wl, w = weights(cfg, "random")
        toks = workload.make_prompt(wl)[0]
        w2 = dict(w)
        for l in range(wl.shape.n_layers):
            w2[f"l{l}.wq"] = (w[f"l{l}.wq"].float() * 2).to(torch.bfloat16)
            w2[f"l{l}.wk"] = (w[f"l{l}.wk"].float() * 2).to(torch.bfloat16)
        a = Model(wl.shape, {k: to_u16(v) for k, v in w.items()}, cache=True).forward_full(toks)[0]
        b = Model(wl.shape, {k: to_u16(v) for k, v in w2.items()}, cache=True).forward_full(toks)[0]
        base[cfg] = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert base[6] < 1e-3, base
    assert base[0] > 1e-2, base
