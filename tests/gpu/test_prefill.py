"""GPU parity of prefill as graph steps (mk_prefill): a prompt's tokens go
through the graph as the columns of one step per launch group instead of one
step per token.

Bar: the logits at every prompt position against the oracle's causal
forward over the whole prompt (forward_full), within the logits bar of the
decode target; the sequence's KV-cache entries against forward_full's bf16
keys and values (kv_close); the next decode step after the prompt against the
oracle's decode step on the oracle's own cache. Other sequences' cache rows
stay untouched (zeros)."""
import numpy as np
import pytest

import workload
from tests.gpu.test_parity import check_logits, kv_close, session
from tests.helpers import oracle_model, progress

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def prompt_tokens(cfg, n, seed):
    wl = workload.config(cfg)
    return [int(t) for t in np.random.default_rng(seed).integers(0, wl.shape.vocab, size=n)]


def run_prefill_case(cfg, max_batch, n, seq, opts=None, gains="random", pos0=0):
    import decode_persistent_megakernel_amd as mk
    wl = workload.config(cfg)
    ss = session(cfg, gains, opts=opts, max_batch=max_batch, max_seq=64)
    om = oracle_model(cfg, gains)
    toks = prompt_tokens(cfg, n, 100 + cfg)
    progress(f"[prefill] cfg {cfg}: {n} tokens on sequence {seq}, {ss.batch_per_launch} per step, "
             f"use_mfma {ss.opts.use_mfma}")
    nxt, lg = ss.prefill(toks, seq=seq, pos0=pos0)
    ref, kref, vref = om.forward_full(toks)
    g = lg.double().cpu().numpy()
    for p in range(n):
        check_logits(g[p], ref[p], f"cfg {cfg} prefill pos {p}")
        assert int(nxt[p]) == int(np.argmax(g[p]))
    # the sequence's cache rows against forward_full's bf16 keys and values
    for name, dev, ref_kv in (("k", ss.k, kref), ("v", ss.v, vref)):
        got = dev[:, seq, :, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert kv_close(got, np.asarray(ref_kv), what=f"prefill cfg {cfg} {name} cache")
        others = [b for b in range(max_batch) if b != seq]
        if others:
            assert int(dev[:, others].abs().sum()) == 0, "prefill wrote another sequence's rows"
    # the next decode step after the prompt, against the oracle's decode over
    # its own prefilled cache
    st = om.new_state(1, 64)
    st.kcache[:, 0, :, :n] = np.asarray(kref)
    st.vcache[:, 0, :, :n] = np.asarray(vref)
    if seq == 0:
        t_next = int(np.argmax(ref[-1]))
        _, lg2 = ss.decode_step([t_next], [n])
        ref2 = om.decode_step(st, [t_next], [n])[0]
        check_logits(lg2[0].double().cpu().numpy(), ref2, f"cfg {cfg} decode after prefill")
    ss.check()
    ss.close()


@pytest.mark.parametrize("cfg,max_batch,n,seq", [(7, 16, 20, 3), (7, 16, 8, 0), (5, 16, 11, 0)])
def test_prefill_matrix_core(cfg, max_batch, n, seq):
    """Matrix-core bodies (16 columns per step): config 7 with a 20-token
    prompt on sequence 3 (two steps: 16 + 4 columns, the second attending over
    the first's cache entries) and an 8-token prompt on sequence 0 followed by
    a decode step; config 5 (head dim 128, four query heads per kv head)."""
    import decode_persistent_megakernel_amd as mk
    o = mk.GraphOpts()
    o.use_mfma = 2
    run_prefill_case(cfg, max_batch, n, seq, opts=o)


@pytest.mark.parametrize("cfg,max_batch,n,seq", [(0, 4, 9, 0), (6, 4, 7, 2)])
def test_prefill_vector_bodies(cfg, max_batch, n, seq):
    """Vector bodies (4 columns per step): config 0 with 9 tokens (steps of
    4, 4, 1) and the q/k-norm config 6 with 7 tokens on sequence 2."""
    run_prefill_case(cfg, max_batch, n, seq)


def test_prefill_after_decoded_prefix():
    """A prompt continued at pos0 > 0: the first 5 tokens decoded one step
    each, the next 10 prefilled from position 5 (the prefill's attention
    reads the decoded prefix from the cache); logits of the prefilled
    positions against forward_full over all 15 tokens."""
    import decode_persistent_megakernel_amd as mk
    cfg = 7
    o = mk.GraphOpts()
    o.use_mfma = 2
    ss = session(cfg, "random", opts=o, max_batch=16, max_seq=64)
    om = oracle_model(cfg, "random")
    toks = prompt_tokens(cfg, 15, 300)
    for p in range(5):
        ss.decode_step([toks[p]], [p], logits=False)
    nxt, lg = ss.prefill(toks[5:], seq=0, pos0=5)
    ref, _, _ = om.forward_full(toks)
    g = lg.double().cpu().numpy()
    for i in range(10):
        check_logits(g[i], ref[5 + i], f"prefill after prefix pos {5 + i}")
    ss.check()
    ss.close()


@pytest.mark.slow
def test_1b_prefill_prompt():
    """The workload's 39-token prompt on the Llama-3.2-1B shape as three
    prefill steps (16 + 16 + 7 columns, matrix-core bodies): logits at all 39
    positions and the caches against forward_full."""
    import decode_persistent_megakernel_amd as mk
    cfg = 1
    wl = workload.config(cfg)
    o = mk.GraphOpts()
    o.use_mfma = 2
    ss = session(cfg, "ones", opts=o, max_batch=16, max_seq=256)
    om = oracle_model(cfg, "ones")
    toks = [int(t) for t in workload.make_prompt(wl)[0]]
    nxt, lg = ss.prefill(toks)
    progress("[1b prefill] kernel done; oracle forward_full")
    ref, kref, vref = om.forward_full(toks)
    g = lg.double().cpu().numpy()
    for p in range(len(toks)):
        check_logits(g[p], ref[p], f"1b prefill pos {p}")
    n = len(toks)
    for name, dev, ref_kv in (("k", ss.k, kref), ("v", ss.v, vref)):
        got = dev[:, 0, :, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert kv_close(got, np.asarray(ref_kv), what=f"1b prefill {name} cache")
    ss.check()
    ss.close()


@pytest.mark.parametrize("use_mfma", [1, 2])
def test_prefill_to_the_last_position(use_mfma):
    """The cache filled to its end: a 60-token prompt prefilled into a
    64-position cache, then greedy decode steps at positions 60..63 (the last
    one the cache holds) in one mk_generate launch; their logits against
    forward_full over the 64 tokens (the oracle's greedy continuation is fed
    teacher-forced through stepwise decoding, so both sides see the same
    tokens), on the vector bodies and the matrix cores."""
    import decode_persistent_megakernel_amd as mk
    cfg = 7
    o = mk.GraphOpts()
    o.use_mfma = use_mfma
    ss = session(cfg, "random", opts=o, max_batch=16 if use_mfma == 2 else 4, max_seq=64)
    om = oracle_model(cfg, "random")
    toks = prompt_tokens(cfg, 60, 400)
    progress(f"[prefill to the end] use_mfma {use_mfma}")
    nxt, lg = ss.prefill(toks, seq=0, pos0=0)
    ref, _, _ = om.forward_full(toks)
    check_logits(lg[59].double().cpu().numpy(), ref[59], "prefill pos 59")
    # four steps at positions 60..63, each fed the oracle's greedy token
    seq = list(toks)
    for p in range(60, 64):
        t = int(np.argmax(ref[-1]))
        seq.append(t)
        _, g = ss.decode_step([t], [p])
        ref, _, _ = om.forward_full(seq)
        check_logits(g[0].double().cpu().numpy(), ref[-1], f"decode at position {p}")
    # position 64 is past the cache: reported, not written
    _, _ = ss.decode_step([0], [64], logits=False)
    with pytest.raises(mk.MKError):
        ss.check()
    ss.close()
