"""Python binding of libmk, the MI355X persistent decode megakernel.

Argument marshalling only: every step of the decode path runs in the HIP
library (``libmk.so``, built in-tree by ``build.py``). The functions carry the
C ABI's names (``include/mk.h`` documents each one); they take plain integers
for device pointers and streams, or torch tensors / streams where noted, and
raise ``MKError`` for a non-zero status. Importing this module does not load
the library; the first call does, and fails loudly if it was not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

__all__ = [
    "MKError", "ModelDesc", "GraphOpts", "lib", "lib_path",
    "mk_build_task_graph", "mk_graph_serialize", "mk_graph_info", "mk_free_graph",
    "mk_load_weights", "mk_decode_step", "mk_generate", "mk_check", "mk_set_watchdog_ms",
    "mk_set_profile_buffer", "mk_set_wait_counters", "mk_debug_drop_signal", "mk_model_info", "mk_free_model", "mk_last_error",
    "MK_MODE_MEGAKERNEL", "MK_MODE_OPLAUNCH", "STATUS_NAMES",
]

MK_OK, MK_EINVAL, MK_ENOMEM, MK_EHIP, MK_ETIMEOUT, MK_EUNSUPPORTED, MK_EDEVICE = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "MK_OK", -1: "MK_EINVAL", -2: "MK_ENOMEM", -3: "MK_EHIP", -4: "MK_ETIMEOUT",
                -5: "MK_EUNSUPPORTED", -6: "MK_EDEVICE"}
MK_MODE_MEGAKERNEL, MK_MODE_OPLAUNCH = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmk.so")


class MKError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
        "tied_embeddings", "max_batch", "max_seq")] + [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                                                       ("qk_norm", ctypes.c_int32)]


class GraphOpts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_cus", "qkv_tasks_per_group", "o_tasks", "gu_tasks", "d_tasks", "lm_tasks",
        "attn_chunks", "row_block", "use_mfma")]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "g_attn", "g_mlp",
                                               "q_norm", "k_norm")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("g_final", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libmk.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: run `python -m decode_persistent_megakernel_amd.build` "
                          "(or __graft_entry__.build()) first; there is no fallback path")
    try:
        import torch  # noqa: F401  -- loads the HIP runtime libmk binds to
    except ImportError:
        pass
    L = ctypes.CDLL(lib_path, mode=ctypes.RTLD_GLOBAL)
    vp, i32, u64p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)
    sig = {
        "mk_build_task_graph": [ctypes.POINTER(ModelDesc), ctypes.POINTER(GraphOpts), ctypes.POINTER(vp)],
        "mk_graph_serialize": [vp, ctypes.c_char_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)],
        "mk_graph_info": [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(GraphOpts)],
        "mk_load_weights": [vp, ctypes.POINTER(Weights), vp, ctypes.POINTER(vp)],
        "mk_decode_step": [vp, vp, vp, i32, vp, vp, i32, vp],
        "mk_generate": [vp, vp, vp, i32, i32, vp, vp, vp],
        "mk_generate_noalloc": [vp, vp, vp, i32, i32, vp, vp, vp],
        "mk_prefill": [vp, vp, i32, i32, i32, vp, vp, vp],
        "mk_check": [vp, vp],
        "mk_set_watchdog_ms": [vp, i32],
        "mk_debug_drop_signal": [vp, i32],
        "mk_set_profile_buffer": [vp, vp, ctypes.c_size_t],
        "mk_set_wait_counters": [vp, vp, ctypes.c_size_t],
        "mk_model_info": [vp, u64p, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32),
                          ctypes.POINTER(i32), ctypes.POINTER(i32)],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name in ("mk_free_graph", "mk_free_model"):
        getattr(L, name).argtypes = [vp]
        getattr(L, name).restype = None
    L.mk_last_error.argtypes = []
    L.mk_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def mk_last_error() -> str:
    return lib().mk_last_error().decode()


def _ok(rc: int) -> None:
    if rc != MK_OK:
        raise MKError(rc, mk_last_error())


def _ptr(x) -> int:
    """Device pointer of a torch tensor, or an int passed through."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def desc_from_shape(shape, max_batch: int, max_seq: int) -> ModelDesc:
    return ModelDesc(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                     shape.ffn, shape.vocab, int(shape.tied), max_batch, max_seq,
                     float(shape.rms_eps), float(shape.rope_theta), int(getattr(shape, "qk_norm", False)))


def mk_build_task_graph(desc: ModelDesc, opts: Optional[GraphOpts] = None) -> int:
    g = ctypes.c_void_p()
    _ok(lib().mk_build_task_graph(ctypes.byref(desc), ctypes.byref(opts) if opts else None, ctypes.byref(g)))
    return g.value


def mk_graph_serialize(graph: int) -> bytes:
    n = ctypes.c_size_t()
    _ok(lib().mk_graph_serialize(graph, None, 0, ctypes.byref(n)))
    buf = ctypes.create_string_buffer(n.value)
    _ok(lib().mk_graph_serialize(graph, buf, n.value, ctypes.byref(n)))
    return buf.raw[: n.value]


def mk_graph_info(graph: int):
    nt, ne, o = ctypes.c_int32(), ctypes.c_int32(), GraphOpts()
    _ok(lib().mk_graph_info(graph, ctypes.byref(nt), ctypes.byref(ne), ctypes.byref(o)))
    return nt.value, ne.value, o


def mk_free_graph(graph: int) -> None:
    lib().mk_free_graph(graph)


def mk_load_weights(graph: int, w: Dict[str, object], k_cache, v_cache, n_layers: int, stream=None) -> int:
    """``w`` maps the names embed, lm_head (absent or None when tied), g_final
    and l{i}.wq ... l{i}.g_mlp (and l{i}.q_norm, l{i}.k_norm for a qk_norm
    model) to device bf16 tensors (or int pointers)."""
    layers = (LayerWeights * n_layers)()
    for l in range(n_layers):
        for f in ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "g_attn", "g_mlp", "q_norm", "k_norm"):
            setattr(layers[l], f, _ptr(w.get(f"l{l}.{f}")))
    ws = Weights(_ptr(w["embed"]), _ptr(w.get("lm_head")), _ptr(w["g_final"]),
                 ctypes.cast(layers, ctypes.POINTER(LayerWeights)), _ptr(k_cache), _ptr(v_cache))
    m = ctypes.c_void_p()
    _ok(lib().mk_load_weights(graph, ctypes.byref(ws), _stream(stream), ctypes.byref(m)))
    return m.value


def mk_decode_step(model: int, tokens, pos, batch: int, logits, next_tokens,
                   mode: int = MK_MODE_MEGAKERNEL, stream=None) -> None:
    _ok(lib().mk_decode_step(model, _ptr(tokens), _ptr(pos), batch, _ptr(logits), _ptr(next_tokens),
                             mode, _stream(stream)))


def mk_generate(model: int, tokens0, pos0, batch: int, n_steps: int, out_tokens, last_logits=None,
                stream=None) -> None:
    _ok(lib().mk_generate(model, _ptr(tokens0), _ptr(pos0), batch, n_steps, _ptr(out_tokens),
                          _ptr(last_logits), _stream(stream)))


def mk_generate_noalloc(model: int, tokens0, pos0, batch: int, n_steps: int, out_tokens, last_logits=None,
                        stream=None) -> None:
    _ok(lib().mk_generate_noalloc(model, _ptr(tokens0), _ptr(pos0), batch, n_steps, _ptr(out_tokens),
                                  _ptr(last_logits), _stream(stream)))


def mk_prefill(model: int, tokens, n_tokens: int, seq: int, pos0: int, logits, next_tokens, stream=None) -> None:
    _ok(lib().mk_prefill(model, _ptr(tokens), n_tokens, seq, pos0, _ptr(logits), _ptr(next_tokens),
                         _stream(stream)))


def mk_check(model: int, stream=None) -> None:
    _ok(lib().mk_check(model, _stream(stream)))


def mk_set_watchdog_ms(model: int, ms: int) -> None:
    _ok(lib().mk_set_watchdog_ms(model, ms))


def mk_debug_drop_signal(model: int, task_id: int) -> None:
    _ok(lib().mk_debug_drop_signal(model, task_id))


def mk_set_profile_buffer(model: int, buf, nbytes: int) -> None:
    _ok(lib().mk_set_profile_buffer(model, _ptr(buf), nbytes))


def mk_set_wait_counters(model: int, buf, nbytes: int) -> None:
    _ok(lib().mk_set_wait_counters(model, _ptr(buf), nbytes))


def mk_model_info(model: int):
    """(packed weight bytes, CUs, tasks per step, ring slots per stream wave, LDS bytes,
    sequences per launch)."""
    b, n, t, r, l, g = (ctypes.c_uint64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(),
                        ctypes.c_int32())
    _ok(lib().mk_model_info(model, ctypes.byref(b), ctypes.byref(n), ctypes.byref(t), ctypes.byref(r),
                            ctypes.byref(l), ctypes.byref(g)))
    return b.value, n.value, t.value, r.value, l.value, g.value


def mk_free_model(model: int) -> None:
    lib().mk_free_model(model)
