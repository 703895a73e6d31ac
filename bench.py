"""Decode benchmark: per-token latency and HBM roofline fraction of the
persistent decode megakernel on one MI355X.

Workload (default): the Llama-3.2-1B-shaped decoder at batch 1, seeded random
bf16 weights, a 39-token prompt consumed untimed, then K greedy decode steps
inside ONE persistent launch (mk_generate), timed with HIP events on the
launch stream. W untimed warm-up steps run first as one persistent launch of
their own from the same start (it writes the same cache positions with the
same values the timed launch writes again), so the timed launch is a warm
kernel. Also timed, for context: the same steps with one launch per operator
(the baseline built from the same task bodies), and the CPU oracle on a
bounded sample.

Correctness of the timed launch: the per-operator leg replays its first steps
feeding the timed launch's own tokens, and every next token it computes must
equal the token the timed launch chose at that step (the two paths are
bit-identical by construction); any difference exits with status 3 before the
JSON line is printed.

Prints one JSON line (rank 0). `--gpus N` with N > 1 exits: the library runs
on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X published HBM3E bandwidth


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(shape, positions) -> int:
    """Bytes one decode step must move: every weight once (matrices, norm
    gains, one embedding row per sequence, the LM head), the KV cache of
    positions 0..p for each sequence (K and V, bf16; the entry at p is the one
    written this step)."""
    H, D, F, V, L = shape.hidden, shape.head_dim, shape.ffn, shape.vocab, shape.n_layers
    Hq, Hkv = shape.n_q_heads, shape.n_kv_heads
    per_layer = (Hq * D * H + 2 * Hkv * D * H + H * Hq * D + 2 * F * H + H * F + 2 * H) * 2
    w = L * per_layer + V * H * 2 + H * 2 + len(positions) * H * 2
    kv_per_pos = L * Hkv * D * 2 * 2
    return w + sum((p + 1) * kv_per_pos for p in positions)


# the sources whose hash keys a traffic record: the kernels and the host code
# that builds the graph they run and lays out its data
KERNEL_SOURCES = [os.path.join(ROOT, "decode_persistent_megakernel_amd", "csrc", f)
                  for f in ("kernels.hip", "pipeline.h", "mfma.h", "device.h", "graph.cpp", "graph.h", "api.cpp")]


def recorded_traffic(kernel: str, workload_name: str, steps: int, batch: int):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy of known size), if recorded for this
    kernel variant, workload, batch and step count with the kernel sources as
    they are now; else None. The record holds one entry per measured step
    count."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_b{batch}_hbm_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    if (rec.get("kernel_source_sha256") != h.hexdigest() or rec.get("workload") != workload_name
            or rec.get("batch") != batch):
        return None
    per_steps = rec.get("traffic_bytes_per_launch_by_steps", {})
    v = per_steps.get(str(steps))
    return int(v) if v is not None else None


def prefill_timing(wl, weights, prompt, ss):
    """The prompt through mk_prefill on a matrix-core model of the same weights
    (16 columns per graph step), against the same prompt as one-token
    megakernel launches on the benchmark's model; each timed after one
    untimed run, with HIP events on the launch stream. The prefill's tokens
    are checked against the one-token launches' (same greedy choice at every
    position)."""
    import torch
    import decode_persistent_megakernel_amd as mk
    from decode_persistent_megakernel_amd import MK_MODE_MEGAKERNEL, mk_decode_step
    from decode_persistent_megakernel_amd.session import Session
    P = len(prompt)
    o = mk.GraphOpts()
    o.use_mfma = 2
    pf = Session(wl.shape, weights, 16, P + 8, o)
    stream = torch.cuda.current_stream()
    toks = [int(t) for t in prompt]
    pf.prefill(toks)  # untimed
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    nxt, _ = pf.prefill(toks, logits=False)
    e1.record(stream)
    torch.cuda.synchronize()
    pf.check()
    us_pre = e0.elapsed_time(e1) * 1e3
    steps = (P + pf.batch_per_launch - 1) // pf.batch_per_launch
    pf.close()
    tok = torch.as_tensor(toks, dtype=torch.int32, device="cuda")
    pos = torch.arange(P, dtype=torch.int32, device="cuda")
    out = torch.zeros(P, dtype=torch.int32, device="cuda")
    for rep in range(2):  # the first run untimed
        torch.cuda.synchronize()
        e0.record(stream)
        for p in range(P):
            mk_decode_step(ss.model, tok[p:p + 1], pos[p:p + 1], 1, None, out[p:p + 1], MK_MODE_MEGAKERNEL)
        e1.record(stream)
        torch.cuda.synchronize()
    ss.check()
    us_step = e0.elapsed_time(e1) * 1e3
    agree = int((nxt == out).sum())
    return {"tokens": P, "us": round(us_pre, 1), "us_per_token": round(us_pre / P, 2), "graph_steps": steps,
            "stepwise_us": round(us_step, 1), "greedy_tokens_equal_stepwise": agree}


def cpu_baseline(wl, weights, seconds: float = 15.0):
    """The float64 oracle as it stands, timed on the host cores: single decode
    steps of the same shape at the prompt's last position (empty cache prefix),
    repeated until about `seconds` have elapsed (at least one step)."""
    import numpy as np
    import torch
    from oracle.decoder import Model
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    u16 = {k: v.contiguous().view(torch.int16).numpy().view(np.uint16) for k, v in weights.items()}
    m = Model(wl.shape, u16, cache=False)
    P = wl.prompt_len or 1
    st = m.new_state(1, P + 8)
    n, t0 = 0, time.perf_counter()
    while True:
        m.decode_step(st, [1 + n], [P - 1 + n])
        n += 1
        if time.perf_counter() - t0 > seconds or n >= 8:
            break
    dt = time.perf_counter() - t0
    return {"value": dt / n * 1e6, "unit": "us/token", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} float64 oracle decode steps of the {wl.name} config at positions "
                      f"{P - 1}..{P - 2 + n} (empty cache prefix), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index (1: Llama-3.2-1B shape)")
    ap.add_argument("--oplaunch-steps", type=int, default=32, help="steps timed for the per-operator baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-prefill timing")
    ap.add_argument("--use-mfma", type=int, default=0, choices=(0, 1, 2),
                    help="matvec bodies of the timed model (graph option use_mfma; 0: the default choice)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times, then sum the same MIB MiB 3 times (a plain "
                         "copy and a read-only pass of known size, to scale hardware byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is a design, not built", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        # a read-only pass of the same size (a reduction: loads only), to check
        # the read counter's factor on a path with no stores
        for _ in range(3):
            float(src.sum())
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": n, "read_bytes_per_reduction": n}), flush=True)
        return
    import workload
    from decode_persistent_megakernel_amd import MK_MODE_OPLAUNCH
    from decode_persistent_megakernel_amd.session import Session

    wl = workload.config(args.config)
    if wl.batch != 1 and wl.kv_prefill == "none":
        raise SystemExit(f"bench.py: the {wl.name} workload (batch {wl.batch} with a prompt) is not supported")
    torch.cuda.set_device(0)
    t = time.time()
    w = workload.make_weights(wl)
    kv = workload.make_prefill(wl)
    log(f"weights generated in {time.time() - t:.1f}s")
    import decode_persistent_megakernel_amd as mkp
    gopts = mkp.GraphOpts()
    gopts.use_mfma = args.use_mfma
    ss = Session(wl.shape, w, wl.batch, wl.max_seq, gopts, kv=kv)
    kv = None
    log(f"model loaded: {ss.n_tasks} tasks, {ss.num_cus} CUs, packed weights {ss.packed_bytes / 1e9:.3f} GB, "
        f"register ring {ss.ring_slots} items per stream wave, LDS {ss.lds_bytes} B, {ss.batch_per_launch} sequence(s) per launch")
    B = wl.batch
    K, W = args.steps, args.warmup
    if wl.kv_prefill == "none":
        prompt = workload.make_prompt(wl)[0]
        P = len(prompt)
        for p in range(P - 1):
            ss.decode_step([int(prompt[p])], [p], mode=MK_MODE_OPLAUNCH, logits=False)
        tok0, pos0 = [int(prompt[-1])], [P - 1]
    else:  # the cache holds positions 0 .. len_b - 1 of sequence b; decoding starts after them
        tok0 = [int(x) for x in workload.make_prompt(wl)[:, 0]]
        pos0 = [int(x) for x in workload.kv_lengths(wl)]
    if max(pos0) + max(K, W) > wl.max_seq:
        raise SystemExit("steps exceed max_seq")
    torch.cuda.synchronize()
    ss.check()
    log("prompt prefilled")

    stream = torch.cuda.current_stream()
    out = torch.zeros((max(K, 1), B), dtype=torch.int32, device="cuda")
    from decode_persistent_megakernel_amd import mk_decode_step, mk_generate
    ss.set_inputs(tok0, pos0)  # device token / position buffers, filled before any timing
    if W > 0:  # warm-up: one untimed persistent launch from the same start
        wout = torch.zeros((W, B), dtype=torch.int32, device="cuda")
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        mk_generate(ss.model, ss.tok, ss.pos, B, W, wout)
        w1.record(stream)
        torch.cuda.synchronize()
        ss.check()
        log(f"warm-up launch: {W} steps in {w0.elapsed_time(w1):.3f} ms")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    mk_generate(ss.model, ss.tok, ss.pos, B, K, out[:K])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ss.check()
    ms = e0.elapsed_time(e1)
    if W > 0 and K == W:
        assert torch.equal(wout, out[:K]), "the warm-up and timed launches chose different tokens"
    us_tok = ms * 1e3 / K
    bytes_launch = sum(algorithmic_bytes(wl.shape, [p + k for p in pos0]) for k in range(K))
    achieved = bytes_launch / (ms * 1e-3) / 1e9
    log(f"megakernel: {K} steps in {ms:.3f} ms (wall {wall * 1e3:.1f} ms): {us_tok:.2f} us/step, "
        f"{achieved:.1f} GB/s algorithmic")

    # per-operator-launch baseline (same task bodies), a shorter run that
    # replays the timed launch's steps: step k feeds the token the timed launch
    # fed, and its next token must equal the one the timed launch chose
    Kb = min(args.oplaunch_steps, K)
    toks_b = out[:Kb].cpu().tolist()
    tok_in = torch.as_tensor([tok0] + toks_b[:Kb - 1], dtype=torch.int32, device="cuda")
    pos_in = torch.as_tensor([[p + k for p in pos0] for k in range(Kb)], dtype=torch.int32, device="cuda")
    chk = torch.full((Kb, B), -1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for k in range(Kb):
        mk_decode_step(ss.model, tok_in[k], pos_in[k], B, None, chk[k], MK_MODE_OPLAUNCH)
    b1.record(stream)
    torch.cuda.synchronize()
    ss.check()
    us_b = b0.elapsed_time(b1) * 1e3 / Kb
    log(f"per-operator launches: {us_b:.2f} us/step over {Kb} steps")
    bad = (chk != out[:Kb]).nonzero().cpu().tolist()
    if bad:
        k, b_ = bad[0]
        log(f"MISMATCH: the timed launch chose token {toks_b[k][b_]} at step {k} (sequence {b_}), the per-operator "
            f"replay {int(chk[k, b_])}; {len(bad)} differing entries")
        ss.close()
        sys.exit(3)
    log(f"timed launch checked: {Kb} steps x {B} sequence(s) equal the per-operator replay")

    pre = None
    if wl.kv_prefill == "none" and not args.no_prefill:
        pre = prefill_timing(wl, w, prompt, ss)
        log(f"prefill of the {pre['tokens']}-token prompt: {pre['us']:.1f} us as {pre['graph_steps']} graph steps "
            f"(matrix-core bodies), {pre['stepwise_us']:.1f} us as {pre['tokens']} one-token launches")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, w, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.0f} us/token on {cpu['cores']} threads")

    kernel = "mk_persistent_b16" if ss.opts.use_mfma == 2 else f"mk_persistent_b{min(B, ss.batch_per_launch)}"
    per = "token at batch 1" if B == 1 else f"step at batch {B}"
    rec = {
        "metric": f"decode \u00b5s/{per} + achieved HBM GB/s as % of roofline",
        "value": round(us_tok, 3), "unit": "\u00b5s/token" if B == 1 else "\u00b5s/step", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms / K, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "global_batch": B, "seq_len": max(pos0) + K,
                   "prompt": P if wl.kv_prefill == "none" else 1,
                   "kv_prefilled": 0 if wl.kv_prefill == "none" else (pos0[0] if B == 1 else pos0),
                   "decode_steps": K, "sequences_per_launch": min(B, ss.batch_per_launch),
                   "parallelism": "none (1 GPU)"},
        "achieved_gbs": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(kernel, wl.name, K, B),
                     "kernel": kernel, "launch_ms": round(ms, 4),
                     "bytes_per_launch": bytes_launch},
        "oplaunch_baseline_us_per_step": round(us_b, 3),
        "timed_launch_checked_steps": Kb,
        "cpu_baseline": cpu,
        "prefill": pre,
    }
    if B > 1:
        rec["us_per_sequence_token"] = round(us_tok / B, 3)
    ss.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
