"""C-ABI checks that need no GPU: libmk.so loads, exports every entry point
include/mk.h declares, its host compiler produces the graph oracle's canonical
bytes exactly, and argument errors come back as the documented codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_persistent_megakernel_amd as mk
import workload
from oracle import graph as G

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mk.h")


def declared_symbols():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = mk.lib()
    names = declared_symbols()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n


def c_bytes(desc, opts=None):
    g = mk.mk_build_task_graph(desc, opts)
    try:
        return mk.mk_graph_serialize(g)
    finally:
        mk.mk_free_graph(g)


@pytest.mark.parametrize("cfg", range(len(workload.CONFIGS)))
def test_graph_bytes_equal_oracle_default(cfg):
    wl = workload.config(cfg)
    b = c_bytes(mk.desc_from_shape(wl.shape, wl.batch, wl.max_seq))
    assert b == G.serialize(G.build(G.desc_from_shape(wl.shape, wl.batch, wl.max_seq)))


def test_graph_bytes_equal_oracle_knob_sweep():
    rng = np.random.default_rng(11)
    shapes = [workload.config(i).shape for i in range(3)]
    for it in range(60):
        s = shapes[it % 3]
        B = int(rng.choice([1, 2, 3, 16]))
        S = int(rng.integers(1, 5000))
        knobs = [int(rng.choice([0, int(rng.integers(1, 400))])) for _ in range(9)]
        knobs[7] = int(rng.choice([0, 1, 4, 16, 7]))
        knobs[8] = int(rng.choice([0, 1, 2]))
        o = mk.GraphOpts(*knobs)
        b = c_bytes(mk.desc_from_shape(s, B, S), o)
        ref = G.serialize(G.build(G.desc_from_shape(s, B, S), G.Opts(*knobs)))
        assert b == ref, (it, knobs, B, S)


def test_resolved_opts_match_oracle():
    wl = workload.config(1)
    g = mk.mk_build_task_graph(mk.desc_from_shape(wl.shape, 1, wl.max_seq))
    nt, ne, o = mk.mk_graph_info(g)
    mk.mk_free_graph(g)
    r = G.resolve(G.desc_from_shape(wl.shape, 1, wl.max_seq), G.Opts())
    fields = ("num_cus", "qkv_tasks_per_group", "o_tasks", "gu_tasks", "d_tasks", "lm_tasks",
              "attn_chunks", "row_block", "use_mfma")
    assert tuple(getattr(o, f) for f in fields) == tuple(getattr(r, f) for f in fields)
    assert r.use_mfma == 1                       # one sequence: the vector bodies


def test_use_mfma_default_and_range():
    wl = workload.config(4)                      # 16 sequences: the matrix-core bodies
    g = mk.mk_build_task_graph(mk.desc_from_shape(wl.shape, wl.batch, 256))
    assert mk.mk_graph_info(g)[2].use_mfma == 2
    mk.mk_free_graph(g)
    with pytest.raises(mk.MKError):
        mk.mk_build_task_graph(mk.desc_from_shape(wl.shape, 1, 64), mk.GraphOpts(*([0] * 8 + [3])))


@pytest.mark.parametrize("field,val", [("n_q_heads", 5), ("head_dim", 60), ("hidden", 0), ("ffn", 690),
                                       ("max_batch", 0)])
def test_bad_desc_is_einval(field, val):
    wl = workload.config(0)
    d = mk.desc_from_shape(wl.shape, 1, 64)
    setattr(d, field, val)
    with pytest.raises(mk.MKError) as e:
        mk.mk_build_task_graph(d)
    assert e.value.code == mk.MK_EINVAL and mk.mk_last_error()


def test_negative_option_is_einval():
    wl = workload.config(0)
    with pytest.raises(mk.MKError) as e:
        mk.mk_build_task_graph(mk.desc_from_shape(wl.shape, 1, 64), mk.GraphOpts(-1))
    assert e.value.code == mk.MK_EINVAL


def test_serialize_small_buffer_and_nulls():
    L = mk.lib()
    wl = workload.config(0)
    g = mk.mk_build_task_graph(mk.desc_from_shape(wl.shape, 1, 64))
    n = ctypes.c_size_t()
    buf = ctypes.create_string_buffer(10)
    assert L.mk_graph_serialize(g, buf, 10, ctypes.byref(n)) == mk.MK_EINVAL
    assert n.value > 10
    assert L.mk_graph_serialize(None, buf, 10, ctypes.byref(n)) == mk.MK_EINVAL
    assert L.mk_graph_info(None, None, None, None) == mk.MK_EINVAL
    m = ctypes.c_void_p()
    assert L.mk_load_weights(g, None, None, ctypes.byref(m)) == mk.MK_EINVAL
    assert L.mk_decode_step(None, None, None, 1, None, None, 0, None) == mk.MK_EINVAL
    assert L.mk_generate(None, None, None, 1, 1, None, None, None) == mk.MK_EINVAL
    assert L.mk_generate_noalloc(None, None, None, 1, 1, None, None, None) == mk.MK_EINVAL
    assert L.mk_prefill(None, None, 1, 0, 0, None, None, None) == mk.MK_EINVAL
    assert b"NULL model" in L.mk_last_error()
    assert L.mk_check(None, None) == mk.MK_EINVAL
    mk.mk_free_graph(g)


def test_bad_qk_norm_is_einval():
    wl = workload.config(0)
    d = mk.desc_from_shape(wl.shape, 1, 64)
    d.qk_norm = 2
    with pytest.raises(mk.MKError) as e:
        mk.mk_build_task_graph(d)
    assert e.value.code == mk.MK_EINVAL
