"""Device-memory plumbing around the C ABI: holds the torch tensors a model
needs (weights, KV cache, token/position buffers) and calls the mk_* entry
points. No decode arithmetic happens here."""
from __future__ import annotations

from typing import Dict, Optional

from . import (GraphOpts, MK_MODE_MEGAKERNEL, desc_from_shape, mk_build_task_graph, mk_check,
               mk_decode_step, mk_free_graph, mk_free_model, mk_generate, mk_generate_noalloc, mk_graph_info,
               mk_prefill,
               mk_graph_serialize, mk_load_weights, mk_model_info)


class Session:
    """One model on the current device.

    ``weights``: name -> CPU or device bf16 tensor (HF layout), names as in
    ``mk_load_weights``. ``kv``: optional (k, v) bf16 tensors
    ``[L][max_batch][Hkv][max_seq][D]`` to start from (copied to the device).
    """

    def __init__(self, shape, weights: Dict[str, object], max_batch: int, max_seq: int,
                 opts: Optional[GraphOpts] = None, kv=None, keep_weights: bool = False):
        import torch
        self.torch = torch
        self.model = 0
        self.graph = 0
        self.shape = shape
        self.max_batch, self.max_seq = max_batch, max_seq
        dev = torch.device("cuda", torch.cuda.current_device())
        self.desc = desc_from_shape(shape, max_batch, max_seq)
        self.graph = mk_build_task_graph(self.desc, opts)
        self.n_tasks, self.n_events, self.opts = mk_graph_info(self.graph)
        w = {k: (v if v.is_cuda else v.to(dev, non_blocking=False)).contiguous()
             for k, v in weights.items() if v is not None}
        kvshape = (shape.n_layers, max_batch, shape.n_kv_heads, max_seq, shape.head_dim)
        if kv is None or kv[0] is None:
            self.k = torch.zeros(kvshape, dtype=torch.bfloat16, device=dev)
            self.v = torch.zeros(kvshape, dtype=torch.bfloat16, device=dev)
        else:
            self.k = kv[0].to(dev).contiguous()
            self.v = kv[1].to(dev).contiguous()
            assert tuple(self.k.shape) == kvshape
        self.model = mk_load_weights(self.graph, w, self.k, self.v, shape.n_layers)
        self.weights = w if keep_weights else None
        (self.packed_bytes, self.num_cus, _, self.ring_slots, self.lds_bytes,
         self.batch_per_launch) = mk_model_info(self.model)
        self.tok = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        self.next = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        self.logits = torch.zeros(max_batch, shape.vocab, dtype=torch.float32, device=dev)

    def graph_bytes(self) -> bytes:
        return mk_graph_serialize(self.graph)

    def set_inputs(self, tokens, pos):
        b = len(tokens)
        self.tok[:b].copy_(self.torch.as_tensor(list(tokens), dtype=self.torch.int32))
        self.pos[:b].copy_(self.torch.as_tensor(list(pos), dtype=self.torch.int32))
        return b

    def decode_step(self, tokens, pos, mode: int = MK_MODE_MEGAKERNEL, logits: bool = True):
        """Feed tokens at positions; returns (next tokens tensor, logits tensor)."""
        b = self.set_inputs(tokens, pos)
        mk_decode_step(self.model, self.tok, self.pos, b, self.logits if logits else None, self.next, mode)
        return self.next[:b], self.logits[:b]

    def generate(self, tokens0, pos0, n_steps: int, out=None, last_logits: bool = False, noalloc: bool = False):
        """n_steps greedy steps in one launch; ``noalloc`` calls the entry point
        whose launch scratch is the library's static workspace."""
        b = self.set_inputs(tokens0, pos0)
        if out is None:
            out = self.torch.zeros((n_steps, b), dtype=self.torch.int32, device=self.tok.device)
        fn = mk_generate_noalloc if noalloc else mk_generate
        fn(self.model, self.tok, self.pos, b, n_steps, out, self.logits if last_logits else None)
        return out

    def prefill(self, tokens, seq: int = 0, pos0: int = 0, logits: bool = True):
        """Prompt tokens of sequence ``seq`` at positions pos0.. as columns of
        one graph step per launch group; returns (next tokens, logits [n, V])."""
        n = len(tokens)
        t = self.torch.as_tensor(list(tokens), dtype=self.torch.int32, device=self.tok.device)
        nxt = self.torch.zeros(n, dtype=self.torch.int32, device=self.tok.device)
        lg = self.torch.zeros((n, self.shape.vocab), dtype=self.torch.float32, device=self.tok.device) if logits else None
        mk_prefill(self.model, t, n, seq, pos0, lg, nxt)
        return nxt, lg

    def check(self):
        mk_check(self.model)

    def close(self):
        if self.model:
            self.torch.cuda.synchronize()
            mk_free_model(self.model)
            self.model = 0
        if self.graph:
            mk_free_graph(self.graph)
            self.graph = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
