"""mk_generate_noalloc (launch scratch in the library's static workspace)
against mk_generate (the model's own workspace): the same kernels on the same
inputs, so tokens, final logits and the KV-cache entries written must be
bit-identical. Two calls in a row, the second with fewer sequences and steps;
the model's own entry points still agree afterwards; a second model of another
shape then reuses the same workspace; a model whose launch scratch exceeds the
workspace is refused with MK_EINVAL before anything is launched."""
import dataclasses

import pytest

import workload
from tests.helpers import progress, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _session(shape, w, max_batch, max_seq):
    import decode_persistent_megakernel_amd.session as S
    return S.Session(shape, w, max_batch, max_seq)


def _same(a, b, n_seq, what):
    assert torch.equal(a.logits[:n_seq], b.logits[:n_seq]), f"{what}: final logits differ"
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v), f"{what}: KV caches differ"


def test_noalloc_equals_generate_two_calls():
    wl = workload.config(0)
    _, w = weights(0, "random")
    a = _session(wl.shape, w, 4, wl.max_seq)
    b = _session(wl.shape, w, 4, wl.max_seq)
    prompt = [int(t) for t in workload.make_prompt(wl)[0]]
    P = len(prompt)
    # three sequences with different contexts: sequence j reads the prompt
    # rotated by j
    for p in range(P):
        toks = [prompt[(p + j) % P] for j in range(3)]
        for ss in (a, b):
            ss.decode_step(toks, [p] * 3, logits=False)
    torch.cuda.synchronize()
    progress("[noalloc] call 1: 3 sequences x 8 steps")
    t1 = [prompt[-1], prompt[0], prompt[1]]
    oa = a.generate(t1, [P] * 3, 8, last_logits=True)
    ob = b.generate(t1, [P] * 3, 8, last_logits=True, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob), (oa.cpu().tolist(), ob.cpu().tolist())
    _same(a, b, 3, "call 1")
    b.check()
    progress("[noalloc] call 2: 1 sequence x 3 steps")
    t2 = [int(oa[-1, 0])]
    oa = a.generate(t2, [P + 8], 3, last_logits=True)
    ob = b.generate(t2, [P + 8], 3, last_logits=True, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob), (oa.cpu().tolist(), ob.cpu().tolist())
    _same(a, b, 1, "call 2")
    b.check()
    progress("[noalloc] the model's own workspace after the static calls")
    t3 = [int(oa[-1, 0])]
    oa = a.generate(t3, [P + 11], 2, last_logits=True)
    ob = b.generate(t3, [P + 11], 2, last_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    _same(a, b, 1, "mk_generate after mk_generate_noalloc")
    a.check()
    b.check()
    a.close()
    b.close()


def test_noalloc_second_model_shares_the_workspace():
    wl = workload.config(5)
    _, w = weights(5, "random")
    a = _session(wl.shape, w, 1, wl.max_seq)
    b = _session(wl.shape, w, 1, wl.max_seq)
    prompt = [int(t) for t in workload.make_prompt(wl)[0]]
    for p, t in enumerate(prompt[:-1]):
        for ss in (a, b):
            ss.decode_step([t], [p], logits=False)
    progress("[noalloc] head-dim-128 model: 1 sequence x 6 steps")
    oa = a.generate([prompt[-1]], [len(prompt) - 1], 6, last_logits=True)
    ob = b.generate([prompt[-1]], [len(prompt) - 1], 6, last_logits=True, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    _same(a, b, 1, "head-dim-128 model")
    b.check()
    a.close()
    b.close()


def test_noalloc_refuses_a_model_beyond_the_workspace():
    import decode_persistent_megakernel_amd as mk
    wl0 = workload.config(0)
    # 352 tiny layers with one attention chunk (6 events per layer: 2 kv
    # groups' QKV, merged attention, O, gate/up, down), plus 3: 2115 events of
    # 8 KiB counters each, just over 16 MiB
    wl = dataclasses.replace(wl0, shape=dataclasses.replace(wl0.shape, n_layers=352))
    w = workload.make_weights(wl, gains="ones")
    ss = _session(wl.shape, w, 1, wl.max_seq)
    out = torch.full((2, 1), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(mk.MKError) as e:
        ss.generate([1], [0], 2, out=out, noalloc=True)
    assert e.value.code == mk.MK_EINVAL and "static workspace holds" in str(e.value), str(e.value)
    progress(f"[noalloc] refused: {e.value}")
    torch.cuda.synchronize()
    assert int((out != -7).sum()) == 0           # nothing was launched
    ss.check()
    ss.close()
