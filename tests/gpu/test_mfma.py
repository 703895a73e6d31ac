"""GPU parity of the matrix-core bodies (graph option use_mfma = 2): the
matvec tasks run as v_mfma_f32_16x16x32_bf16 on bf16 hi/lo splits of the
activations, up to 16 sequences per launch.

Bar: the logits bar of the decode target against the float64 oracle (the
teacher-forced tiny cases also far inside it, < 1e-3: hi + lo carries each
activation to about 2^-15 relative, fp32 sums; what reaches the logits is
mostly the KV-cache entries that this moves across a bf16 rounding boundary,
a 2^-9 relative step each); the megakernel and the per-operator launches
bit-identical; mk_generate equal to stepwise decoding.
"""
import numpy as np
import pytest

import workload
from tests.gpu.test_parity import check_logits, kv_close, session
from tests.helpers import oracle_model, progress

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def mf_opts(**kw):
    import decode_persistent_megakernel_amd as mk
    o = mk.GraphOpts()
    o.use_mfma = 2
    for k, v in kw.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("cfg", [7, 5])
def test_mfma_teacher_forced_logits(cfg):
    """One sequence through the matrix-core bodies (15 of the 16 MFMA rows are
    padding): config 7 (head dim 64, two query heads per kv head) and config 5
    (head dim 128, four per kv head, hidden 512)."""
    wl = workload.config(cfg)
    ss = session(cfg, "random", opts=mf_opts(), max_batch=1)
    assert ss.opts.use_mfma == 2
    om = oracle_model(cfg, "random")
    prompt = workload.make_prompt(wl)[0]
    st = om.new_state(1, wl.max_seq)
    worst = 0.0
    for p, t in enumerate(prompt):
        nxt, lg = ss.decode_step([int(t)], [p])
        ref = om.decode_step(st, [int(t)], [p])[0]
        g = lg[0].double().cpu().numpy()
        e, _ = check_logits(g, ref, f"cfg {cfg} pos {p}")
        worst = max(worst, e)
        assert int(nxt[0]) == int(np.argmax(g))
    assert worst < 1e-3
    P = len(prompt)
    for name, dev_cache, ref_cache in (("k", ss.k, st.kcache), ("v", ss.v, st.vcache)):
        kg = dev_cache[:, 0, :, :P].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert kv_close(kg, ref_cache[:, 0, :, :P], what=f"mfma cfg {cfg} {name} cache")
    ss.check()
    ss.close()


def test_mfma_batch16_vs_oracle():
    """Sixteen sequences in one launch (config 7 selects the matrix-core
    bodies by itself): ragged positions, batch 16 and batch 13 calls, every
    sequence's logits against the oracle; megakernel and per-operator launches
    bit-identical (logits and caches); mk_generate equal to stepwise decoding."""
    wl = workload.config(7)
    a = session(7, "random", max_seq=40)
    b = session(7, "random", max_seq=40)
    assert a.batch_per_launch == 16 and a.opts.use_mfma == 2
    om = oracle_model(7, "random")
    st = om.new_state(16, 40)
    toks = workload.make_prompt(wl)
    for k in range(5):
        nb = 13 if k == 3 else 16
        tk = [int(toks[s, k]) for s in range(nb)]
        ps = [k + (s % 5) for s in range(nb)]
        na, la = a.decode_step(tk, ps, mode=0)
        nb_, lb = b.decode_step(tk, ps, mode=1)
        assert torch.equal(la, lb) and torch.equal(na, nb_), k
        ref = om.decode_step(st, tk, ps)
        g = la.double().cpu().numpy()
        for s in range(nb):
            check_logits(g[s], ref[s], f"step {k} seq {s}")
            assert int(na[s]) == int(np.argmax(g[s]))
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    t0 = [int(toks[s, 5]) for s in range(16)]
    p0 = [5 + (s % 5) for s in range(16)]
    out = a.generate(t0, p0, 4)
    tk = list(t0)
    for k in range(4):
        nxt, _ = b.decode_step(tk, [p + k for p in p0], mode=1)
        tk = [int(x) for x in nxt.cpu().tolist()]
        assert tk == out[k].cpu().tolist(), k
    a.check()
    b.check()
    a.close()
    b.close()


@pytest.mark.parametrize("knobs", [dict(num_cus=64, o_tasks=5, gu_tasks=7, d_tasks=3, lm_tasks=9, row_block=4),
                                   dict(num_cus=37, qkv_tasks_per_group=3, o_tasks=37, gu_tasks=50, d_tasks=11,
                                        lm_tasks=5, attn_chunks=3),
                                   dict(num_cus=256, row_block=16, attn_chunks=7),
                                   dict(num_cus=16, o_tasks=3, gu_tasks=4, d_tasks=2, lm_tasks=2)])
def test_mfma_graph_options(knobs):
    """Task splits that give the matrix-core bodies several row blocks per
    task, a last row block with fewer than 16 rows, and stream-wave pieces that
    start and end inside row blocks; four sequences at ragged positions. The
    last case gives pieces of several passes over many row blocks (LM: 32 row
    blocks per task, 32 items per wave), where the activation column of an
    item wraps around the row block many times within one piece."""
    wl = workload.config(7)
    ss = session(7, "random", opts=mf_opts(**knobs), max_batch=4, max_seq=40)
    om = oracle_model(7, "random")
    st = om.new_state(4, 40)
    toks = workload.make_prompt(wl)
    for k in range(4):
        tk = [int(toks[s, k]) for s in range(4)]
        ps = [k + 2 * s for s in range(4)]
        nxt, lg = ss.decode_step(tk, ps)
        ref = om.decode_step(st, tk, ps)
        g = lg.double().cpu().numpy()
        for s in range(4):
            check_logits(g[s], ref[s], f"{knobs} step {k} seq {s}")
    progress(f"[mfma options] {knobs}: {ss.n_tasks} tasks")
    ss.check()
    ss.close()


def test_mfma_batch_above_one_launch():
    """max_batch 21 on the matrix cores: a launch takes 16 sequences, so a
    call of 21 runs as groups of 16 and 5 (the second group's KV rows start at
    sequence 16). Ragged positions; every sequence's logits against the oracle;
    megakernel and per-operator launches bit-identical; mk_generate over the
    groups equal to stepwise decoding."""
    wl = workload.config(7)
    a = session(7, "random", opts=mf_opts(), max_batch=21, max_seq=40)
    b = session(7, "random", opts=mf_opts(), max_batch=21, max_seq=40)
    assert a.batch_per_launch == 16
    om = oracle_model(7, "random")
    st = om.new_state(21, 40)
    toks = workload.make_prompt(wl)
    for k in range(3):
        tk = [int(toks[s % 16, k]) for s in range(21)]
        ps = [k + (s % 7) for s in range(21)]
        na, la = a.decode_step(tk, ps, mode=0)
        nb_, lb = b.decode_step(tk, ps, mode=1)
        assert torch.equal(la, lb) and torch.equal(na, nb_), k
        ref = om.decode_step(st, tk, ps)
        g = la.double().cpu().numpy()
        for s in range(21):
            check_logits(g[s], ref[s], f"step {k} seq {s}")
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    t0 = [int(toks[s % 16, 3]) for s in range(21)]
    p0 = [3 + (s % 7) for s in range(21)]
    out = a.generate(t0, p0, 3)
    tk = list(t0)
    for k in range(3):
        nxt, _ = b.decode_step(tk, [p + k for p in p0], mode=1)
        tk = [int(x) for x in nxt.cpu().tolist()]
        assert tk == out[k].cpu().tolist(), k
    a.check()
    b.check()
    a.close()
    b.close()
