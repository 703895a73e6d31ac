"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar (from the decode target): teacher-forced logits within max-abs 3e-2 AND
rel-L2 1e-2 per step and sequence; bit-exact greedy token ids over the tiny
config's 16 steps; the megakernel and the per-operator-launch baseline
bit-identical (same task bodies, same per-element order); bit-exact graph
bytes (checked on the CPU in tests/test_abi.py).
"""
import json
import os

import numpy as np
import pytest

import workload
from oracle import bf16
from tests.helpers import oracle_model, progress, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.dirname(__file__)), "golden", "tiny_greedy.json")
MAX_ABS, REL_L2 = 3e-2, 1e-2
# Logits when the oracle attends over the very cache entries the kernel wrote
# (copied from the device): what is left is fp32 against fp64 accumulation.
SHARED_REL_L2 = 1e-4
# Fraction of layer-0 KV-cache entries allowed to differ by one rounding
# (kv_close); 1.5e-4 was observed on the 1B shape's prompt.
KV_LAYER0_FRAC = 1e-3


def session(cfg, gains="ones", opts=None, max_batch=None, max_seq=None, shape=None, w=None, kv=None):
    import decode_persistent_megakernel_amd.session as S
    wl = workload.config(cfg)
    if w is None:
        _, w = weights(cfg, gains)
    progress(f"[session] cfg={cfg} gains={gains} opts={opts and tuple(getattr(opts, f[0]) for f in opts._fields_)}")
    return S.Session(shape or wl.shape, w, max_batch or wl.batch, max_seq or wl.max_seq, opts, kv=kv)


def check_logits(gpu: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(gpu - ref)
    rel = np.linalg.norm(gpu - ref) / np.linalg.norm(ref)
    progress(f"[{what}] max-abs {err.max():.3e} rel-L2 {rel:.3e}")
    assert err.max() <= MAX_ABS and rel <= REL_L2, (what, err.max(), rel)
    return err.max(), rel


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (7 stored mantissa bits): 2^(e-7) for
    |x| in [2^e, 2^(e+1)); the smallest normal's spacing below it."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def kv_close(got_u16, ref_u16, what="kv", layer0_frac=KV_LAYER0_FRAC):
    """bf16 caches [L][...] written by the kernel against the oracle's.

    Layer 0's inputs are identical on both sides (the embedding row), so its
    entries may differ only by one rounding: |got - ref| at most one bf16 ulp
    of the larger magnitude plus 1e-3 of the tensor's rms (RoPE's rotation can
    leave a small remainder of cancellation whose fp32 and fp64 values round
    differently), in fewer than layer0_frac of the entries. Later layers see
    inputs that already differ by the earlier layers' rounding (each side
    attends over its own cache), so their entries are held to the logits' bar
    instead: per layer, rel-L2 <= REL_L2. Fractions and errors are printed."""
    g = bf16.decode(np.asarray(got_u16, dtype=np.uint16))
    r = bf16.decode(np.asarray(ref_u16, dtype=np.uint16))
    g0, r0 = g[0], r[0]
    rms = float(np.sqrt(np.mean(r0 * r0))) if r0.size else 0.0
    tol = bf16_ulp(np.maximum(np.abs(g0), np.abs(r0))) + 1e-3 * rms
    d = np.abs(g0 - r0)
    f0 = float((d > 0).mean()) if d.size else 0.0
    ok0 = bool(np.all(d <= tol)) and f0 < layer0_frac
    rel = [float(np.linalg.norm(g[l] - r[l]) / max(np.linalg.norm(r[l]), 1e-30)) for l in range(1, g.shape[0])]
    worst = max(rel) if rel else 0.0
    progress(f"[{what}] layer 0: differing entries {f0:.2e} (limit {layer0_frac:.0e}); "
             f"later layers: largest rel-L2 {worst:.2e} (limit {REL_L2:.0e}); {d.size} entries per layer")
    if not ok0:
        i = np.unravel_index(int(np.argmax(d - tol)), d.shape)
        print(f"kv mismatch in layer 0 at {i}: got {g0[i]!r} ref {r0[i]!r} tol {tol[i]!r}")
    return ok0 and worst <= REL_L2


def prefill_and_compare(ss, om, prompt, mode=0, cmp_every=True):
    """Teacher-forced: feed each prompt token on GPU and oracle; compare logits."""
    st = om.new_state(1, ss.max_seq)
    worst = 0.0
    for p, t in enumerate(prompt):
        nxt, lg = ss.decode_step([int(t)], [p], mode=mode)
        ref = om.decode_step(st, [int(t)], [p])[0]
        if cmp_every or p == len(prompt) - 1:
            g = lg[0].double().cpu().numpy()
            e, _ = check_logits(g, ref, f"pos {p}")
            worst = max(worst, e)
            assert int(nxt[0]) == int(np.argmax(g))
    return st, worst


@pytest.mark.parametrize("cfg,gains", [(0, "ones"), (0, "random"), (5, "random"), (6, "random")])
def test_tiny_teacher_forced_logits(cfg, gains):
    """Config 0 (head dim 64, two query heads per kv head, untied) and config 5
    (head dim 128, four query heads per kv head, untied): the head widths and
    group sizes of the full-size shapes, at a size the oracle runs in seconds.
    Config 6 is config 0 with per-head RMSNorm of queries and keys before
    RoPE, with random gains (so a kernel that skipped or misplaced the norm,
    or read the wrong head's gains, would miss the bar by orders)."""
    wl = workload.config(cfg)
    ss = session(cfg, gains)
    om = oracle_model(cfg, gains)
    prompt = workload.make_prompt(wl)[0]
    st, worst = prefill_and_compare(ss, om, prompt)
    assert worst < 1e-4          # fp32 accumulation; far inside the bar
    # KV cache written by the kernel == the oracle's bf16 cache, up to the
    # rounding of an fp32 computation: one bf16 step where fp32 and fp64
    # straddle a rounding boundary, plus the fp32 absolute error where the
    # entry is a small result of cancellation (RoPE's rotation); rare.
    P = len(prompt)
    for name, dev_cache, ref_cache in (("k", ss.k, st.kcache), ("v", ss.v, st.vcache)):
        kg = dev_cache[:, 0, :, :P].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        ko = ref_cache[:, 0, :, :P]
        assert kv_close(kg, ko, what=f"cfg {cfg} {name} cache")
    ss.check()
    ss.close()


@pytest.mark.parametrize("gains", ["ones", "random"])
def test_tiny_greedy_bit_exact(gains):
    ref = json.load(open(GOLDEN))[gains]
    wl = workload.config(0)
    ss = session(0, gains)
    prompt = np.array(ref["prompt"])
    for p in range(len(prompt) - 1):
        ss.decode_step([int(prompt[p])], [p], logits=False)
    out = ss.generate([int(prompt[-1])], [len(prompt) - 1], wl.steps)
    toks = out[:, 0].cpu().tolist()
    print("[greedy]", toks, flush=True)
    assert toks == ref["tokens"]
    ss.check()
    ss.close()


@pytest.mark.parametrize("cfg", [0, 6])
def test_tiny_megakernel_equals_oplaunch(cfg):
    wl = workload.config(cfg)
    a = session(cfg, "random")
    b = session(cfg, "random")
    prompt = workload.make_prompt(wl)[0]
    for p, t in enumerate(prompt):
        na, la = a.decode_step([int(t)], [p], mode=0)
        nb, lb = b.decode_step([int(t)], [p], mode=1)
        assert torch.equal(la, lb) and torch.equal(na, nb), p
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    a.close()
    b.close()


def test_qknorm_greedy_vs_oracle():
    """Greedy decode of the q/k-norm config: the tokens the kernel picks over
    its 16 steps are the oracle's argmax at every step where the oracle's two
    best logits are apart by more than 1e-3, ten times the largest logit error
    the teacher-forced test allows these tiny shapes (at a closer near-tie
    either choice is correct; the comparison stops there, as the sequences may
    then part)."""
    wl = workload.config(6)
    ss = session(6, "random")
    om = oracle_model(6, "random")
    prompt = workload.make_prompt(wl)[0]
    for p in range(len(prompt) - 1):
        ss.decode_step([int(prompt[p])], [p], logits=False)
    out = ss.generate([int(prompt[-1])], [len(prompt) - 1], wl.steps)
    toks = out[:, 0].cpu().tolist()
    st = om.new_state(1, wl.max_seq)
    for p in range(len(prompt) - 1):
        om.decode_step(st, [int(prompt[p])], [p])
    tok, compared = int(prompt[-1]), 0
    for i in range(wl.steps):
        ref = om.decode_step(st, [tok], [len(prompt) - 1 + i])[0]
        top = np.sort(ref)[-2:]
        if top[1] - top[0] <= 1e-3:
            break
        assert toks[i] == int(np.argmax(ref)), (i, toks[i], int(np.argmax(ref)))
        tok, compared = toks[i], compared + 1
    progress(f"[qknorm greedy] {toks}; {compared} of {wl.steps} steps compared")
    assert compared == wl.steps       # the seeded case has no near-tie (smallest gap 1.6e-3)
    ss.check()
    ss.close()


@pytest.mark.parametrize("knobs", [(8, 0, 0, 0, 0, 0, 1, 0), (37, 3, 5, 7, 9, 11, 5, 0), (256, 0, 0, 0, 0, 0, 64, 16),
                                   (64, 1, 1, 1, 1, 1, 2, 4), (100, 0, 0, 0, 0, 0, 3, 8)])
def test_tiny_graph_options(knobs):
    import decode_persistent_megakernel_amd as mk
    wl = workload.config(0)
    ss = session(0, "random", mk.GraphOpts(*knobs))
    om = oracle_model(0, "random")
    prefill_and_compare(ss, om, workload.make_prompt(wl)[0], cmp_every=False)
    ss.check()
    ss.close()


def test_tiny_batch_ragged_positions():
    """max_batch 3 graph; sequences at different positions; batch 2 and 3 calls."""
    wl = workload.config(0)
    ss = session(0, "random", max_batch=3, max_seq=40)
    om = oracle_model(0, "random")
    st = om.new_state(3, 40)
    toks = workload.make_prompt(wl)[0]
    for k in range(6):
        tk = [int(toks[k]), int(toks[(k + 3) % 8]), int(toks[(k + 5) % 8])]
        ps = [k + 4, k, 2 * k]
        nb = 2 if k % 2 else 3
        # batch 2 calls leave sequence 2 unfed (its cache keeps zeros there on
        # both sides)
        nxt, lg = ss.decode_step(tk[:nb], ps[:nb])
        ref = om.decode_step(st, tk[:nb], ps[:nb])
        g = lg.double().cpu().numpy()
        for b in range(nb):
            check_logits(g[b], ref[b], f"step {k} seq {b}")
    ss.check()
    ss.close()


def test_tiny_generate_matches_stepwise():
    """mk_generate (all steps in one launch) == repeated mk_decode_step."""
    wl = workload.config(0)
    a = session(0, "random")
    b = session(0, "random")
    prompt = workload.make_prompt(wl)[0]
    for p in range(len(prompt) - 1):
        a.decode_step([int(prompt[p])], [p])
        b.decode_step([int(prompt[p])], [p])
    P = len(prompt)
    out = a.generate([int(prompt[-1])], [P - 1], 12, last_logits=True)
    tok = int(prompt[-1])
    for k in range(12):
        nxt, lg = b.decode_step([tok], [P - 1 + k])
        tok = int(nxt[0])
        assert tok == int(out[k, 0])
    assert torch.equal(a.logits[0], b.logits[0])
    a.close()
    b.close()


def test_instrumented_variant_matches():
    """With a profile buffer and wait counters set, the persistent launch runs
    the instrumented kernel variant: tokens and logits equal the plain
    variant's, every task of every step has ordered timestamps, and the wait
    counters are filled."""
    import decode_persistent_megakernel_amd as mk
    wl = workload.config(0)
    a = session(0, "random")
    b = session(0, "random")
    prompt = workload.make_prompt(wl)[0]
    for p in range(len(prompt) - 1):
        a.decode_step([int(prompt[p])], [p], logits=False)
        b.decode_step([int(prompt[p])], [p], logits=False)
    P, K = len(prompt), 6
    _, _, n_tasks, _, _, _ = mk.mk_model_info(b.model)
    prof = torch.zeros(K * n_tasks * 12, dtype=torch.int64, device="cuda")
    waits = torch.zeros(b.num_cus * 6 * 16, dtype=torch.int64, device="cuda")
    mk.mk_set_profile_buffer(b.model, prof, prof.numel() * 8)
    mk.mk_set_wait_counters(b.model, waits, waits.numel() * 8)
    oa = a.generate([int(prompt[-1])], [P - 1], K, last_logits=True)
    ob = b.generate([int(prompt[-1])], [P - 1], K, last_logits=True)
    a.check()
    b.check()
    assert torch.equal(oa, ob)
    assert torch.equal(a.logits[0], b.logits[0])
    r = prof.view(K, n_tasks, 12).cpu().numpy().astype(np.int64)
    # event seen <= staged <= computed <= signalled, all set
    assert (r[:, :, 0] > 0).all() and (r[:, :, 3] > 0).all()
    assert (r[:, :, 1] >= r[:, :, 0]).all() and (r[:, :, 2] >= r[:, :, 1]).all() and (r[:, :, 3] >= r[:, :, 2]).all()
    assert int(waits.sum()) > 0
    mk.mk_set_profile_buffer(b.model, None, 0)
    mk.mk_set_wait_counters(b.model, None, 0)
    a.close()
    b.close()


def test_device_errors_reported():
    import decode_persistent_megakernel_amd as mk
    wl = workload.config(0)
    ss = session(0)
    ss.decode_step([wl.shape.vocab + 5], [0])
    with pytest.raises(mk.MKError) as e:
        ss.check()
    assert e.value.code == mk.MK_EDEVICE
    ss.decode_step([1], [wl.max_seq])
    with pytest.raises(mk.MKError) as e:
        ss.check()
    assert e.value.code == mk.MK_EDEVICE
    ss.decode_step([1], [0])
    ss.check()                      # clean again
    ss.close()


def test_watchdog_recovers_from_dropped_signal():
    """A task that never signals: dependents wait until the watchdog, every wave
    leaves the kernel, mk_check reports MK_ETIMEOUT, and the next calls run
    correctly after the counter reset."""
    import decode_persistent_megakernel_amd as mk
    wl = workload.config(0)
    ss = session(0, "random")
    om = oracle_model(0, "random")
    mk.mk_set_watchdog_ms(ss.model, 50)
    qkv0 = 1                          # task 1 = first QKV task of layer 0
    mk.mk_debug_drop_signal(ss.model, qkv0)
    ss.decode_step([3], [0])
    with pytest.raises(mk.MKError) as e:
        ss.check()
    assert e.value.code == mk.MK_ETIMEOUT
    mk.mk_debug_drop_signal(ss.model, -1)
    mk.mk_set_watchdog_ms(ss.model, 0)
    prefill_and_compare(ss, om, workload.make_prompt(wl)[0], cmp_every=False)
    ss.check()
    ss.close()


def dev_cache_u16(t, layers_b, n):
    """Positions 0..n-1 of a device bf16 cache [L][B][Hkv][S][D] for sequence b
    as uint16 bit patterns [L][Hkv][n][D] (no arithmetic)."""
    return t[:, layers_b, :, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def shared_cache_state(om, ss, b, n, max_seq):
    """An oracle state whose cache positions 0..n-1 are the device's own bf16
    entries of sequence b."""
    st = om.new_state(1, max_seq)
    st.kcache[:, 0, :, :n] = dev_cache_u16(ss.k, b, n)
    st.vcache[:, 0, :, :n] = dev_cache_u16(ss.v, b, n)
    return st


def full_size_sampled(cfg: int, prefix: int, what: str):
    """A full-size shape in the launch configuration the benchmark times
    (default graph, megakernel): the first `prefix` prompt tokens fed one step
    each, logits at the last of them checked against the oracle's no-cache
    forward, then two decode steps checked against the oracle twice: with the
    oracle's own cache (the bar), and with the oracle attending over the
    device's own cache entries (copied after the step, the ones it wrote
    included), where only fp32 against fp64 accumulation is left
    (SHARED_REL_L2). The device cache is
    also compared entry by entry with the oracle's."""
    wl = workload.config(cfg)
    ss = session(cfg)
    om = oracle_model(cfg, cache=False)
    prompt = workload.make_prompt(wl)[0][:prefix]
    P = len(prompt)
    for p in range(P - 1):
        ss.decode_step([int(prompt[p])], [p], logits=False)
    full, ks, vs = om.forward_full(prompt)
    nxt, lg = ss.decode_step([int(prompt[-1])], [P - 1])
    check_logits(lg[0].double().cpu().numpy(), full[P - 1], f"{what} last prompt position")
    assert kv_close(dev_cache_u16(ss.k, 0, P), ks, what=f"{what} k cache")
    assert kv_close(dev_cache_u16(ss.v, 0, P), vs, what=f"{what} v cache")
    # oracle state = the forward's cache
    st = om.new_state(1, P + 2)
    st.kcache[:, 0, :, :P] = ks
    st.vcache[:, 0, :, :P] = vs
    tok = int(np.argmax(full[P - 1]))
    assert int(nxt[0]) == tok
    for k in range(2):
        ref = om.decode_step(st, [tok], [P + k])[0]
        nxt, lg = ss.decode_step([tok], [P + k])
        g = lg[0].double().cpu().numpy()
        check_logits(g, ref, f"{what} decode step {k}")
        # the device's cache, the entries this step wrote included
        shared = shared_cache_state(om, ss, 0, P + k + 1, P + k + 1)
        ref_s = om.decode_step(shared, [tok], [P + k], kv_given=True)[0]
        _, rel = check_logits(g, ref_s, f"{what} decode step {k}, shared cache")
        assert rel <= SHARED_REL_L2, (what, k, rel)
        tok = int(np.argmax(ref))
        assert int(nxt[0]) == tok
    ss.check()
    ss.close()


@pytest.mark.slow
def test_1b_full_size_sampled():
    """Llama-3.2-1B shape, the whole 39-token prompt."""
    full_size_sampled(1, 39, "1B")


@pytest.mark.slow
def test_8b_full_size_sampled():
    """Llama-3-8B shape (hidden 4096, head dim 128, untied LM head, the
    largest LDS staging of the vector bodies): the first 8 prompt tokens."""
    full_size_sampled(2, 8, "8B")


@pytest.mark.slow
def test_1b_generate_one_launch_vs_oracle():
    """The benchmark's configuration end to end: the Llama-3.2-1B shape, the
    39-token prompt, then 16 greedy steps inside ONE persistent launch
    (mk_generate). Token ids bit-exact against the oracle's greedy decoding
    (the oracle's smallest top-2 margin over these steps is printed: a flip
    needs an error that large), the launch's last-step logits within the bar,
    and the cache it wrote close to the oracle's."""
    from oracle.decoder import greedy
    wl = workload.config(1)
    n = 16
    ss = session(1)
    om = oracle_model(1, cache=False)
    prompt = workload.make_prompt(wl)[0]
    P = len(prompt)
    for p in range(P - 1):
        ss.decode_step([int(prompt[p])], [p], logits=False)
    out = ss.generate([int(prompt[-1])], [P - 1], n, last_logits=True)
    got = out[:, 0].cpu().tolist()
    last = ss.logits[0].double().cpu().numpy()
    # oracle: the prompt's cache from the no-cache forward, then n greedy steps
    _, ks, vs = om.forward_full(prompt[:-1])
    st = om.new_state(1, P + n)
    st.kcache[:, 0, :, :P - 1] = ks
    st.vcache[:, 0, :, :P - 1] = vs
    progress("[1B generate] device launch done; oracle greedy running")
    toks, margins, logits = greedy(om, st, [int(prompt[-1])], [P - 1], n, keep_logits=True)
    print(f"[1B generate] gpu {got}\n[1B generate] ref {toks[:, 0].tolist()}\n"
          f"[1B generate] smallest oracle top-2 margin {margins.min():.4f}", flush=True)
    assert got == toks[:, 0].tolist()
    check_logits(last, logits[-1][0], "1B one launch, last step")
    n_pos = P - 1 + n
    assert kv_close(dev_cache_u16(ss.k, 0, n_pos), st.kcache[:, 0, :, :n_pos], what="1B generate k cache")
    assert kv_close(dev_cache_u16(ss.v, 0, n_pos), st.vcache[:, 0, :, :n_pos], what="1B generate v cache")
    ss.check()
    ss.close()


@pytest.mark.slow
def test_1b_generate_long_launch_equals_stepwise():
    """The cross-step machinery of one long persistent launch at the benchmark's
    shape (copy-ahead across steps, staging-slot flips, epoch thresholds): 64
    greedy steps in one mk_generate equal 64 per-operator steps fed the same
    tokens, token for token, with bit-identical last-step logits."""
    from decode_persistent_megakernel_amd import MK_MODE_OPLAUNCH
    wl = workload.config(1)
    n = 64
    ss = session(1)
    prompt = workload.make_prompt(wl)[0]
    P = len(prompt)
    for p in range(P - 1):
        ss.decode_step([int(prompt[p])], [p], logits=False)
    out = ss.generate([int(prompt[-1])], [P - 1], n, last_logits=True)
    lg_mk = ss.logits[0].clone()
    toks = out[:, 0].cpu().tolist()
    tok = int(prompt[-1])
    for k in range(n):
        nxt, lg = ss.decode_step([tok], [P - 1 + k], mode=MK_MODE_OPLAUNCH, logits=(k == n - 1))
        assert int(nxt[0]) == toks[k], k
        tok = toks[k]
    assert torch.equal(lg[0], lg_mk)
    ss.check()
    ss.close()


@pytest.mark.slow
def test_long_context_sampled():
    """Llama-3.2-1B shape with 32768 KV positions prefilled (synthetic bf16
    N(0,1), read as already rotated): two decode steps from position 32768,
    logits and greedy token against the oracle over the same cache."""
    import torch
    wl = workload.config(3)
    L0 = int(workload.kv_lengths(wl)[0])
    kc, vc = workload.make_prefill(wl)
    ss = session(3, kv=(kc, vc))
    om = oracle_model(3, cache=False)
    st = om.new_state(1, wl.max_seq)
    st.kcache[:, 0] = kc[:, 0].contiguous().view(torch.int16).numpy().view(np.uint16)
    st.vcache[:, 0] = vc[:, 0].contiguous().view(torch.int16).numpy().view(np.uint16)
    del kc, vc
    tok = int(workload.make_prompt(wl)[0][0])
    for k in range(2):
        ref = om.decode_step(st, [tok], [L0 + k])[0]
        nxt, lg = ss.decode_step([tok], [L0 + k])
        check_logits(lg[0].double().cpu().numpy(), ref, f"long context step {k}")
        tok = int(np.argmax(ref))
        assert int(nxt[0]) == tok
    ss.check()
    ss.close()


def test_tiny_batch16_in_groups():
    """max_batch 16 on the tiny shape: a launch stages at most four sequences,
    so batch 16 and batch 13 calls run in groups. Ragged positions; logits of
    every sequence against the oracle; megakernel and per-operator launches
    bit-identical (logits and caches); mk_generate over the groups equal to
    step-by-step decoding."""
    wl = workload.config(0)
    a = session(0, "random", max_batch=16, max_seq=40)
    b = session(0, "random", max_batch=16, max_seq=40)
    assert 1 <= a.batch_per_launch < 16
    om = oracle_model(0, "random")
    st = om.new_state(16, 40)
    toks = workload.make_prompt(wl)[0]
    for k in range(5):
        nb = 13 if k == 3 else 16
        tk = [int(toks[(k + 3 * s) % len(toks)]) for s in range(nb)]
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
    # continue all 16 sequences: one mk_generate call against stepwise steps
    t0 = [int(toks[s % len(toks)]) for s in range(16)]
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


@pytest.mark.slow
def test_8b_batch16_sampled():
    """The batch workload at full size: Llama-3-8B shape, 16 sequences with
    prefilled caches of seeded lengths in 512..8192. Two decode steps for all
    16 sequences, every sequence checked against one batched oracle step:
    step 0 over the same prefilled cache (the bar), step 1 with the oracle
    attending over the device's own cache entries, the ones the step wrote
    included (SHARED_REL_L2), greedy tokens at both; mk_generate over the same two steps equal to them."""
    import torch
    wl = workload.config(4)
    lens = [int(x) for x in workload.kv_lengths(wl)]
    kc, vc = workload.make_prefill(wl)
    progress("[batch16] prefilled caches generated")
    ss = session(4, kv=(kc, vc))
    progress(f"[batch16] lens {lens} sequences per launch {ss.batch_per_launch} ring {ss.ring_slots}")
    om = oracle_model(4, cache=False)
    B = wl.batch
    S1 = max(lens) + 2
    st = om.new_state(B, S1)
    st.kcache[:] = kc[:, :, :, :S1].contiguous().view(torch.int16).numpy().view(np.uint16)
    st.vcache[:] = vc[:, :, :, :S1].contiguous().view(torch.int16).numpy().view(np.uint16)
    del kc, vc
    tok0 = [int(t) for t in workload.make_prompt(wl)[:, 0]]
    tk = list(tok0)
    steps = []
    for k in range(2):
        pos = [n + k for n in lens]
        nxt, lg = ss.decode_step(tk, pos)
        g = lg.double().cpu().numpy()
        nxt = [int(x) for x in nxt.cpu().tolist()]
        if k == 1:  # the device's own entries at every position the step reads (this step's included)
            for b in range(B):
                n = lens[b] + 2
                st.kcache[:, b, :, :n] = dev_cache_u16(ss.k, b, n)
                st.vcache[:, b, :, :n] = dev_cache_u16(ss.v, b, n)
        progress(f"[batch16] device step {k} done; oracle step {k} (16 sequences) running")
        ref = om.decode_step(st, tk, pos, kv_given=(k == 1))
        for b in range(B):
            _, rel = check_logits(g[b], ref[b], f"batch16 seq {b} (len {lens[b]}) step {k}")
            if k == 1:
                assert rel <= SHARED_REL_L2, (b, rel)
            assert nxt[b] == int(np.argmax(ref[b])), b
        steps.append(nxt)
        tk = nxt
    ss.check()
    # the same two steps in one mk_generate call (positions rewritten with the same values)
    out = ss.generate(tok0, lens, 2)
    assert out.cpu().tolist() == steps
    ss.check()
    ss.close()
