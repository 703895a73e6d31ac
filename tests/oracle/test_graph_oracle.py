"""Pins for the task-graph oracle.

* The event contract (MPK blog translation, "MPK compiler" section: one dependent and one triggering event per
  task, threshold = number of triggering tasks, round-robin queues).
* Static race check: every conflicting pair of buffer accesses is ordered by
  an event path, and the closing argmax follows every task (so the next step
  may reuse every buffer).
* Replay: executing the graph's tasks in random valid orders, with the split
  attention merged by log-sum-exp, equals the sequential decoder (this is
  where the split-K merge is pinned against unsplit attention).
"""
import dataclasses

import numpy as np
import pytest

import workload
from oracle import graph as G
from oracle.decoder import prefill_prompt
from tests.helpers import oracle_model


def tiny_desc(batch=1, max_seq=64, **kw):
    s = dataclasses.replace(workload.config(0).shape, **kw)
    return G.desc_from_shape(s, batch, max_seq), s


@pytest.mark.parametrize("opts", [G.Opts(), G.Opts(num_cus=8), G.Opts(num_cus=37, attn_chunks=5),
                                  G.Opts(num_cus=3, row_block=16, attn_chunks=1)])
@pytest.mark.parametrize("batch", [1, 3])
def test_structure_and_races(opts, batch):
    d, _ = tiny_desc(batch)
    gr = G.build(d, opts)
    G.check_structure(gr)
    assert G.race_check(gr) == []


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_structure_full_size(cfg):
    wl = workload.config(cfg)
    gr = G.build(G.desc_from_shape(wl.shape, wl.batch, wl.max_seq))
    G.check_structure(gr)
    n = {t.type for t in gr.tasks}
    # merge tasks exist only where attention is split over several chunks
    # (every full-size workload: 4 chunks of a 4096-position cache, 32 of the
    # long context, 8 on the batch-16 shape)
    assert gr.opts.attn_chunks > 1 and n == set(range(9))
    # every large operator spreads over all 256 compute units; the O
    # projection over half of them where its weights come to under 64 KiB
    # per unit (the 1B shape's 8 MiB on the vector bodies)
    small_o = (gr.opts.use_mfma == 1 and
               wl.shape.hidden * wl.shape.n_q_heads * wl.shape.head_dim * 2 < 256 * 65536)
    assert small_o == (cfg in (1, 3))
    for op in (G.QKV, G.OPROJ, G.GU, G.DOWN, G.LM):
        cus = {t.cu for t in gr.tasks if t.type == op and t.layer in (-1, 0)}
        assert len(cus) == (128 if op == G.OPROJ and small_o else 256), (op, len(cus))
    # on the matrix cores every QKV task is one whole 16-row block (no padded rows)
    if gr.opts.use_mfma == 2:
        assert all(t.row1 - t.row0 == G.MFMA_ROWS for t in gr.tasks if t.type == G.QKV)


def test_attention_placement_spreads_sequences():
    """The attention operator's rounds over the units are skewed by the chunk
    count: on the batch-16 8B shape (16 sequences x 8 kv groups x 8 chunks =
    1024 tasks over 256 units) plain round-robin would give each unit the same
    sequence in all four rounds (1.73x the mean load on the busiest unit for
    the seeded ragged context lengths); the skewed rule gives each unit four
    different sequences, and the busiest unit streams at most 1.3x the mean
    (1.25x)."""
    wl = workload.config(4)
    gr = G.build(G.desc_from_shape(wl.shape, wl.batch, wl.max_seq))
    N, Nc = gr.opts.num_cus, gr.opts.attn_chunks
    att = [t for t in gr.tasks if t.type == G.ATT and t.layer == 0]
    assert len(att) == 4 * N
    for i, t in enumerate(att):
        assert t.cu == (i + (i // N) * Nc) % N
    seqs = [set() for _ in range(N)]
    for t in att:
        seqs[t.cu].add(t.b)
    assert all(len(s) == 4 for s in seqs)
    lens = workload.kv_lengths(wl)
    load = np.zeros(N)
    for t in att:
        n = int(lens[t.b]) + 1
        load[t.cu] += (t.chunk + 1) * n // Nc - t.chunk * n // Nc
    assert load.max() <= 1.3 * load.mean()


@pytest.mark.parametrize("batch", [1, 3])
def test_single_chunk_attention_counts_the_merged_event(batch):
    """With one chunk per (sequence, kv group) the attention tasks are the
    merge: no COMB tasks and no per-chunk events, each attention task counts
    the layer's merged event (threshold Hkv * B, the number of attention tasks
    of the layer), and the O projection waits for that event."""
    d, _ = tiny_desc(batch)
    gr = G.build(d, G.Opts(num_cus=8, attn_chunks=1))
    split = G.build(d, G.Opts(num_cus=8, attn_chunks=2))
    assert not any(t.type == G.COMB for t in gr.tasks)
    # per layer: Hkv * B per-chunk events and as many COMB tasks fewer
    L, Hkv = d.n_layers, d.n_kv_heads
    assert len(split.events) - len(gr.events) == L * Hkv * batch
    for l in range(L):
        att = [t for t in gr.tasks if t.type == G.ATT and t.layer == l]
        o = [t for t in gr.tasks if t.type == G.OPROJ and t.layer == l]
        assert len(att) == Hkv * batch and len({t.trig for t in att}) == 1
        assert gr.events[att[0].trig].threshold == len(att)
        assert all(t.dep == att[0].trig for t in o)
    # a plant in the oracle's graph: one attention task counts the wrong event
    # (its output is then no longer ordered before the O projection)
    t0 = next(t for t in gr.tasks if t.type == G.ATT and t.layer == 0)
    t0.trig = next(t.trig for t in gr.tasks if t.type == G.QKV and t.layer == 1)
    assert any(buf == "attn" for _, _, buf in G.race_check(gr))


def test_race_check_catches_a_missing_edge():
    d, _ = tiny_desc()
    gr = G.build(d, G.Opts(num_cus=4))
    # plant a mistake in the oracle's graph: O-projection waits for the QKV
    # event of group 0 instead of the merged attention
    e_qkv0 = next(t.trig for t in gr.tasks if t.type == G.QKV)
    for t in gr.tasks:
        if t.type == G.OPROJ and t.layer == 0:
            t.dep = e_qkv0
    assert any(buf in ("x", "attn") for _, _, buf in G.race_check(gr))


def test_split_rows():
    assert G.split_rows(12, 3, 4) == [(0, 4), (4, 8), (8, 12)]
    assert G.split_rows(10, 2, 4) == [(0, 4), (4, 10)]
    assert G.split_rows(128256, 256, 4)[-1] == (127752, 128256)
    for rows, t, rb in [(688, 172, 4), (768, 32, 16), (5, 2, 4), (1024, 7, 16)]:
        r = G.split_rows(rows, t, rb)
        assert r[0][0] == 0 and r[-1][1] == rows
        assert all(a[1] == b[0] for a, b in zip(r, r[1:]))
        assert all(x[0] % rb == 0 and x[1] > x[0] for x in r)


@pytest.mark.parametrize("opts,seed", [(G.Opts(num_cus=8), 0), (G.Opts(num_cus=16, attn_chunks=3), 1),
                                       (G.Opts(num_cus=5, attn_chunks=7, row_block=16), 2)])
def test_replay_equals_sequential(opts, seed):
    wl = workload.config(0)
    d, s = tiny_desc(1, wl.max_seq)
    gr = G.build(d, opts)
    om = oracle_model(0, "random")
    prompt = workload.make_prompt(wl)
    st_a, st_b = om.new_state(1, wl.max_seq), om.new_state(1, wl.max_seq)
    prefill_prompt(om, st_a, prompt)
    prefill_prompt(om, st_b, prompt)
    rng = np.random.default_rng(seed)
    tok, p = int(prompt[0, -1]), prompt.shape[1] - 1
    for _ in range(3):
        ref = om.decode_step(st_a, [tok], [p])
        lg, nxt = G.replay(gr, om, st_b, [tok], [p], rng)
        assert np.allclose(lg, ref, rtol=0, atol=1e-12)
        assert int(nxt[0]) == int(np.argmax(ref[0]))
        assert np.array_equal(st_a.kcache, st_b.kcache) and np.array_equal(st_a.vcache, st_b.vcache)
        tok, p = int(nxt[0]), p + 1


def test_replay_batch_ragged_positions():
    wl = workload.config(0)
    d, s = tiny_desc(2, 32)
    gr = G.build(d, G.Opts(num_cus=6, attn_chunks=4))
    om = oracle_model(0, "random")
    st_a, st_b = om.new_state(2, 32), om.new_state(2, 32)
    rng = np.random.default_rng(3)
    toks = workload.make_prompt(wl)[0]
    for p in range(5):                      # sequence 1 is 3 positions behind
        tk, ps = [int(toks[p]), int(toks[(p + 3) % 8])], [p + 3, p]
        ref = om.decode_step(st_a, tk, ps)
        lg, nxt = G.replay(gr, om, st_b, tk, ps, rng)
        assert np.allclose(lg, ref, rtol=0, atol=1e-12)
        assert list(nxt) == [int(np.argmax(r)) for r in ref]


def test_chunk_ranges_cover_and_last_owns_newest():
    for n in (1, 2, 7, 64, 1000):
        for nc in (1, 3, 32):
            rs = [G.chunk_range(n, c, nc) for c in range(nc)]
            assert rs[0][0] == 0 and rs[-1][1] == n
            assert all(a[1] == b[0] for a, b in zip(rs, rs[1:]))
            assert rs[-1][0] <= n - 1 < rs[-1][1]


def test_serialize_layout():
    d, _ = tiny_desc()
    gr = G.build(d, G.Opts(num_cus=4))
    raw = G.serialize(gr)
    nt, ne = len(gr.tasks), len(gr.events)
    assert raw[:8] == b"MKGRAPH1"
    assert raw[8:12] == (5).to_bytes(4, "little")     # version 5: single-chunk attention merges itself
    assert len(raw) == 8 + 4 + 40 + 8 + 4 + 36 + 8 + nt * 40 + ne * 12 + 4 * 4 + nt * 4
