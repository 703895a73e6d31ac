"""Task-graph oracle: the fine-grained task graph of one decode step, written
from its specification (test infrastructure only).

Semantics taken from the pages (MPK blog translation, "MPK compiler" section
and Figure 2; "MPK runtime" section and Figure 3):

* a task is one unit of work placed on one compute unit;
* an event is a synchronisation point; every task has exactly one dependent
  (incoming) event and exactly one triggering (outgoing) event;
* a finishing task increments its triggering event's counter; when the counter
  reaches the event's threshold (the number of tasks that trigger it) the event
  is active and every task depending on it may start;
* tasks are spread over the compute units round-robin (MPK summary: simple
  round-robin placement); the attention operator's further rounds over the
  units are skewed by its chunk count, so that one unit's chunks come from
  different sequences (a step beyond plain round-robin, which the MPK blog
  translation's closing paragraph and the MPK summary list as future work).

The operator order of one step is the pages' wiring (MPK walk-through section
3.3.1): embed, then per layer [RMSNorm+QKV, attention, O-proj+residual,
RMSNorm+gate/up, down+residual], final RMSNorm+LM head, argmax. Attention is
split over position chunks and merged by a reduction task (Hazy summary:
attention as "matmul + reduction"); with a single chunk the attention task
normalises its own result and counts the merged event itself, so the graph
has no reduction tasks (see ``merge_mode``).

The layout of the task list, the event list, the partition rules and the
canonical byte format below are this project's specification; the C++ host
compiler implements the same specification independently and the tests
compare the two byte for byte.

This module also provides ``replay`` (run the task graph with the oracle's own
arithmetic in random valid orders and compare with the sequential decoder) and
``race_check`` (every pair of tasks whose buffer accesses conflict is ordered by
an event path).
"""
from __future__ import annotations

import dataclasses
import hashlib
import struct
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import bf16
from .decoder import Model, State, rmsnorm, rope, silu

# task types
EMB, QKV, ATT, COMB, OPROJ, GU, DOWN, LM, ARGMAX = range(9)
TYPE_NAMES = ["EMB", "QKV", "ATT", "COMB", "O", "GU", "D", "LM", "ARGMAX"]
# most sequences one launch decodes (the graph spec's group size)
GROUP_COLS = 4
MFMA_COLS = 16
MFMA_ROWS = 16   # rows of one matrix-core row block

MAGIC = b"MKGRAPH1"
VERSION = 5
# where a layer's attention chunks are merged
MERGE_IN_ATT, MERGE_TASKS = range(2)


@dataclasses.dataclass(frozen=True)
class Desc:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    tied: int
    max_batch: int
    max_seq: int
    rms_eps: float
    rope_theta: float
    qk_norm: int = 0


@dataclasses.dataclass(frozen=True)
class Opts:
    num_cus: int = 0
    qkv_tasks_per_group: int = 0
    o_tasks: int = 0
    gu_tasks: int = 0
    d_tasks: int = 0
    lm_tasks: int = 0
    attn_chunks: int = 0
    row_block: int = 0
    use_mfma: int = 0


@dataclasses.dataclass
class Task:
    type: int
    layer: int = -1
    b: int = -1
    g: int = -1
    chunk: int = -1
    row0: int = -1
    row1: int = -1
    dep: int = -1
    trig: int = -1
    cu: int = -1


@dataclasses.dataclass
class Event:
    threshold: int = 0
    first_dependent: int = -1
    n_dependents: int = 0


@dataclasses.dataclass
class Graph:
    desc: Desc
    opts: Opts            # resolved (no zeros)
    tasks: List[Task]
    events: List[Event]
    queues: List[List[int]]


def desc_from_shape(shape, max_batch: int, max_seq: int) -> Desc:
    return Desc(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                shape.head_dim, shape.ffn, shape.vocab, int(shape.tied), max_batch,
                max_seq, float(shape.rms_eps), float(shape.rope_theta),
                int(getattr(shape, "qk_norm", False)))


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _mfma_shape(d: Desc) -> bool:
    return all(k % 64 == 0 and k >= 256 for k in (d.hidden, d.n_q_heads * d.head_dim, d.ffn))


def resolve(d: Desc, o: Opts) -> Opts:
    """Fill every zero option with its default (a pure function of the shape)."""
    n = o.num_cus or 256
    rb = o.row_block or 4
    G = d.n_q_heads // d.n_kv_heads
    grp_rows = (G + 2) * d.head_dim

    def cap(req: int, rows: int) -> int:
        return max(1, min(req, _ceil_div(rows, rb)))

    # sequences decode in groups of at most GROUP_COLS per launch: chunks are
    # sized so that one group's attention tasks cover the compute units
    chunks = o.attn_chunks or max(1, min(n // (min(d.max_batch, GROUP_COLS) * d.n_kv_heads),
                                         max(1, d.max_seq // 1024)))
    # matvec bodies (1 vector ALU, 2 matrix cores): the matrix cores when a
    # launch would hold more sequences than the vector bodies stage and every
    # K dimension is a multiple of 64, at least 256
    use_mfma = o.use_mfma or (2 if min(d.max_batch, MFMA_COLS) > GROUP_COLS and _mfma_shape(d) else 1)
    # O projection on the vector bodies: half the units when its weights would
    # give each of n tasks less than 64 KiB
    o_def = n
    if use_mfma == 1 and d.hidden * d.n_q_heads * d.head_dim * 2 < n * 65536:
        o_def = _ceil_div(n, 2)
    # QKV on the matrix cores: at least one task per 16-row block of a group
    # (a task's rows are padded to whole blocks)
    qkv_def = _ceil_div(n, d.n_kv_heads)
    if use_mfma == 2:
        qkv_def = max(qkv_def, _ceil_div(grp_rows, MFMA_ROWS))
    return Opts(
        num_cus=n,
        qkv_tasks_per_group=cap(o.qkv_tasks_per_group or qkv_def, grp_rows),
        o_tasks=cap(o.o_tasks or o_def, d.hidden),
        gu_tasks=cap(o.gu_tasks or n, d.ffn),
        d_tasks=cap(o.d_tasks or n, d.hidden),
        attn_chunks=chunks,
        row_block=rb,
        use_mfma=use_mfma,
        # LM head: the matrix-core bodies' tasks default to 8 row blocks of 16
        lm_tasks=cap(o.lm_tasks or (max(n, _ceil_div(d.vocab, 128)) if use_mfma == 2 else n), d.vocab),
    )


def split_rows(rows: int, tasks: int, rb: int) -> List[Tuple[int, int]]:
    """Balanced split of ``rows`` into ``tasks`` ranges made of whole blocks of
    ``rb`` rows (only the final range may end in a partial block)."""
    nb = _ceil_div(rows, rb)
    out = []
    for t in range(tasks):
        b0, b1 = (t * nb) // tasks, ((t + 1) * nb) // tasks
        out.append((b0 * rb, min(rows, b1 * rb)))
    return out


def merge_mode(d: Desc, o: Opts) -> int:
    """Where the attention chunks of a layer are merged (``o`` resolved): in
    the attention task itself when there is one chunk, else by one merge
    (COMB) task per (kv group, sequence)."""
    return MERGE_IN_ATT if o.attn_chunks == 1 else MERGE_TASKS


def build(d: Desc, opts: Opts = Opts()) -> Graph:
    o = resolve(d, opts)
    B, L, Hkv = d.max_batch, d.n_layers, d.n_kv_heads
    G = d.n_q_heads // Hkv
    Nc = o.attn_chunks
    tasks: List[Task] = []
    events: List[Event] = []

    def new_event(thr: int) -> int:
        events.append(Event(threshold=thr))
        return len(events) - 1

    # events, in creation order
    e_tok = new_event(B)
    e_emb = new_event(B)
    e_qkv, e_att, e_comb, e_o, e_gu, e_d = [], [], [], [], [], []
    # one chunk per (sequence, kv group): the attention task merges its own
    # result, so there are no per-chunk events and no COMB tasks, and the
    # attention tasks count the merged event directly
    fold = merge_mode(d, o) == MERGE_IN_ATT
    for l in range(L):
        e_qkv.append([new_event(o.qkv_tasks_per_group) for g in range(Hkv)])
        if not fold:
            e_att.append([[new_event(Nc) for b in range(B)] for g in range(Hkv)])
        e_comb.append(new_event(Hkv * B))
        e_o.append(new_event(o.o_tasks))
        e_gu.append(new_event(o.gu_tasks))
        e_d.append(new_event(o.d_tasks))
    e_lm = new_event(o.lm_tasks)

    def op(new: List[Task], skew: int = 0):
        # round-robin within the operator; each further round over the units
        # starts `skew` units on (attention: the chunk count, so that a unit's
        # chunks come from different sequences)
        for i, t in enumerate(new):
            t.cu = (i + (i // o.num_cus) * skew) % o.num_cus
        tasks.extend(new)

    op([Task(EMB, b=b, dep=e_tok, trig=e_emb) for b in range(B)])
    for l in range(L):
        dep = e_emb if l == 0 else e_d[l - 1]
        grp_rows = (G + 2) * d.head_dim
        op([Task(QKV, layer=l, g=g, row0=r0, row1=r1, dep=dep, trig=e_qkv[l][g])
            for g in range(Hkv)
            for r0, r1 in split_rows(grp_rows, o.qkv_tasks_per_group, o.row_block)])
        op([Task(ATT, layer=l, g=g, b=b, chunk=c, dep=e_qkv[l][g],
                 trig=e_comb[l] if fold else e_att[l][g][b])
            for g in range(Hkv) for b in range(B) for c in range(Nc)], skew=Nc)
        if not fold:
            op([Task(COMB, layer=l, g=g, b=b, dep=e_att[l][g][b], trig=e_comb[l])
                for g in range(Hkv) for b in range(B)])
        op([Task(OPROJ, layer=l, row0=r0, row1=r1, dep=e_comb[l], trig=e_o[l])
            for r0, r1 in split_rows(d.hidden, o.o_tasks, o.row_block)])
        op([Task(GU, layer=l, row0=r0, row1=r1, dep=e_o[l], trig=e_gu[l])
            for r0, r1 in split_rows(d.ffn, o.gu_tasks, o.row_block)])
        op([Task(DOWN, layer=l, row0=r0, row1=r1, dep=e_gu[l], trig=e_d[l])
            for r0, r1 in split_rows(d.hidden, o.d_tasks, o.row_block)])
    op([Task(LM, row0=r0, row1=r1, dep=e_d[L - 1], trig=e_lm)
        for r0, r1 in split_rows(d.vocab, o.lm_tasks, o.row_block)])
    op([Task(ARGMAX, b=b, dep=e_lm, trig=e_tok) for b in range(B)])

    for i, t in enumerate(tasks):
        ev = events[t.dep]
        if ev.n_dependents == 0:
            ev.first_dependent = i
        ev.n_dependents += 1
    queues: List[List[int]] = [[] for _ in range(o.num_cus)]
    for i, t in enumerate(tasks):
        queues[t.cu].append(i)
    return Graph(d, o, tasks, events, queues)


# ----------------------------------------------------------------------------
# canonical bytes
# ----------------------------------------------------------------------------

def serialize(gr: Graph) -> bytes:
    d, o = gr.desc, gr.opts
    out = bytearray(MAGIC)
    out += struct.pack("<I", VERSION)
    out += struct.pack("<10i", d.n_layers, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim,
                       d.ffn, d.vocab, d.tied, d.max_batch, d.max_seq)
    out += struct.pack("<2f", d.rms_eps, d.rope_theta)
    out += struct.pack("<i", d.qk_norm)
    out += struct.pack("<9i", o.num_cus, o.qkv_tasks_per_group, o.o_tasks, o.gu_tasks,
                       o.d_tasks, o.lm_tasks, o.attn_chunks, o.row_block, o.use_mfma)
    out += struct.pack("<2i", len(gr.tasks), len(gr.events))
    for t in gr.tasks:
        out += struct.pack("<10i", t.type, t.layer, t.b, t.g, t.chunk, t.row0, t.row1,
                           t.dep, t.trig, t.cu)
    for e in gr.events:
        out += struct.pack("<3i", e.threshold, e.first_dependent, e.n_dependents)
    for q in gr.queues:
        out += struct.pack("<i", len(q))
        out += struct.pack(f"<{len(q)}i", *q)
    return bytes(out)


def sha256(gr: Graph) -> str:
    return hashlib.sha256(serialize(gr)).hexdigest()


# ----------------------------------------------------------------------------
# structural checks
# ----------------------------------------------------------------------------

def check_structure(gr: Graph) -> None:
    """Raise AssertionError unless the graph keeps the event contract of the MPK blog
    translation's "MPK compiler" section (one dependent and one triggering
    event per task, threshold = number of triggering tasks)."""
    n = len(gr.tasks)
    producers = [0] * len(gr.events)
    for t in gr.tasks:
        assert 0 <= t.dep < len(gr.events) and 0 <= t.trig < len(gr.events)
        producers[t.trig] += 1
    for e, ev in enumerate(gr.events):
        assert ev.threshold == producers[e], (e, ev.threshold, producers[e])
        assert ev.n_dependents >= 1
        for i in range(ev.first_dependent, ev.first_dependent + ev.n_dependents):
            assert gr.tasks[i].dep == e
    assert sum(ev.n_dependents for ev in gr.events) == n
    seen = sorted(i for q in gr.queues for i in q)
    assert seen == list(range(n))
    for c, q in enumerate(gr.queues):
        assert q == sorted(q)
        assert all(gr.tasks[i].cu == c for i in q)
    # acyclic within a step: every dependency (other than the step-start token
    # event) is produced only by tasks earlier in global order
    last_producer = [-1] * len(gr.events)
    for j, u in enumerate(gr.tasks):
        last_producer[u.trig] = j
    for i, t in enumerate(gr.tasks):
        if t.type != EMB:
            assert last_producer[t.dep] < i, (i, t)


def descendants(gr: Graph) -> List[int]:
    """Bitset (Python int) of the tasks ordered after each task within a step
    by an event path. The step-start edge (token event -> embed) is left out."""
    n = len(gr.tasks)
    dependents: List[List[int]] = [[] for _ in gr.events]
    for j, u in enumerate(gr.tasks):          # from the tasks' own dep fields
        dependents[u.dep].append(j)
    desc_task = [0] * n
    for i in range(n - 1, -1, -1):
        t = gr.tasks[i]
        acc = 0
        if t.type != ARGMAX:                   # the token event closes the step
            for j in dependents[t.trig]:
                if j > i:
                    acc |= (1 << j) | desc_task[j]
        desc_task[i] = acc
    return desc_task


# ----------------------------------------------------------------------------
# access sets and the static race check
# ----------------------------------------------------------------------------

def accesses(gr: Graph, i: int) -> List[Tuple[str, str, int, int]]:
    """(mode, buffer, lo, hi) intervals that task ``i`` reads ("r") or writes
    ("w") within one step. Buffers are flattened row-major; the KV cache is
    split into the entry at the current position ("kvcur") and the older
    entries ("kvpast"), which no task of the step writes."""
    d, o = gr.desc, gr.opts
    t = gr.tasks[i]
    B, H, Hkv, D = d.max_batch, d.hidden, d.n_kv_heads, d.head_dim
    G = d.n_q_heads // Hkv
    GR = (G + 2) * D
    Nc = o.attn_chunks
    acc: List[Tuple[str, str, int, int]] = []
    if t.type == EMB:
        acc += [("r", "tok", t.b, t.b + 1), ("w", "x", t.b * H, (t.b + 1) * H)]
    elif t.type == QKV:
        acc += [("r", "x", 0, B * H)]
        for b in range(B):
            base = (b * Hkv + t.g) * GR
            acc.append(("w", "qkv", base + t.row0, base + t.row1))
    elif t.type == ATT:
        base = (t.b * Hkv + t.g) * GR
        kvb = (t.layer * B + t.b) * Hkv + t.g
        acc += [("r", "qkv", base, base + GR), ("r", "kvpast", kvb, kvb + 1)]
        if t.chunk == Nc - 1:
            acc += [("w", "kvcur", kvb, kvb + 1), ("r", "kvcur", kvb, kvb + 1)]
        if merge_mode(d, o) == MERGE_IN_ATT:     # merged in the task itself
            a = t.b * d.n_q_heads * D + t.g * G * D
            acc.append(("w", "attn", a, a + G * D))
        else:
            for h in range(t.g * G, (t.g + 1) * G):
                p = ((t.b * d.n_q_heads + h) * Nc + t.chunk)
                acc.append(("w", "part", p, p + 1))
    elif t.type == COMB:
        for h in range(t.g * G, (t.g + 1) * G):
            p = (t.b * d.n_q_heads + h) * Nc
            acc.append(("r", "part", p, p + Nc))
        a = t.b * d.n_q_heads * D + t.g * G * D
        acc.append(("w", "attn", a, a + G * D))
    elif t.type == OPROJ:
        acc.append(("r", "attn", 0, B * d.n_q_heads * D))
        for b in range(B):
            acc += [("r", "x", b * H + t.row0, b * H + t.row1),
                    ("w", "x", b * H + t.row0, b * H + t.row1)]
    elif t.type == GU:
        acc.append(("r", "x", 0, B * H))
        for b in range(B):
            acc.append(("w", "mlp", b * d.ffn + t.row0, b * d.ffn + t.row1))
    elif t.type == DOWN:
        acc.append(("r", "mlp", 0, B * d.ffn))
        for b in range(B):
            acc += [("r", "x", b * H + t.row0, b * H + t.row1),
                    ("w", "x", b * H + t.row0, b * H + t.row1)]
    elif t.type == LM:
        k = i - gr.events[t.dep].first_dependent       # LM task ordinal
        acc.append(("r", "x", 0, B * H))
        for b in range(B):
            acc += [("w", "logits", b * d.vocab + t.row0, b * d.vocab + t.row1),
                    ("w", "lmpart", b * o.lm_tasks + k, b * o.lm_tasks + k + 1)]
    elif t.type == ARGMAX:
        acc += [("r", "lmpart", t.b * o.lm_tasks, (t.b + 1) * o.lm_tasks),
                ("w", "tok", t.b, t.b + 1)]
    return acc


def race_check(gr: Graph) -> List[Tuple[int, int, str]]:
    """Return every pair of tasks with conflicting accesses (same buffer,
    overlapping intervals, at least one write) that no event path orders, and
    every task that the closing argmax does not follow (cross-step order)."""
    desc = descendants(gr)
    n = len(gr.tasks)
    by_buf: Dict[str, List[Tuple[int, str, int, int]]] = {}
    for i in range(n):
        for mode, buf, lo, hi in accesses(gr, i):
            by_buf.setdefault(buf, []).append((i, mode, lo, hi))
    bad: List[Tuple[int, int, str]] = []
    for buf, lst in by_buf.items():
        lst.sort(key=lambda a: a[2])
        for x in range(len(lst)):
            i, mi, lo, hi = lst[x]
            for y in range(x + 1, len(lst)):
                j, mj, lo2, hi2 = lst[y]
                if lo2 >= hi:
                    break
                if i == j or (mi == "r" and mj == "r"):
                    continue
                if not ((desc[i] >> j) & 1 or (desc[j] >> i) & 1):
                    bad.append((min(i, j), max(i, j), buf))
    argmax_ids = [i for i, t in enumerate(gr.tasks) if t.type == ARGMAX]
    for i in range(n):
        if gr.tasks[i].type == ARGMAX:
            continue
        for a in argmax_ids:
            if not (desc[i] >> a) & 1:
                bad.append((i, a, "step-order"))
    return sorted(set(bad))


# ----------------------------------------------------------------------------
# replay: execute the graph with the oracle's arithmetic in a random valid order
# ----------------------------------------------------------------------------

def chunk_range(length: int, chunk: int, n_chunks: int) -> Tuple[int, int]:
    """Positions ``[lo, hi)`` of attention chunk ``chunk`` over ``length``
    positions: a balanced contiguous split; the final chunk holds the newest
    position."""
    return (chunk * length) // n_chunks, ((chunk + 1) * length) // n_chunks


def replay(gr: Graph, m: Model, st: State, tokens: Sequence[int], pos: Sequence[int],
           rng: Optional[np.random.Generator] = None):
    """Run one step of the task graph: repeatedly pick a random task whose
    dependent event is active, execute it, and count its triggering event.
    Returns float64 logits ``[B, V]`` and the next tokens ``[B]``."""
    d, o = gr.desc, gr.opts
    s = m.s
    B = len(tokens)
    assert B == d.max_batch
    H, Hq, Hkv, D, F, V = d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn, d.vocab
    G = Hq // Hkv
    GR = (G + 2) * D
    Nc = o.attn_chunks
    mode = merge_mode(d, o)
    x = np.zeros((B, H))
    qkv = np.zeros((B, Hkv, GR))
    pm = np.full((B, Hq, Nc), -np.inf)
    pl = np.zeros((B, Hq, Nc))
    pa = np.zeros((B, Hq, Nc, D))
    attn = np.zeros((B, Hq * D))
    mlp = np.zeros((B, F))
    logits = np.zeros((B, V))
    lmv = np.full((B, o.lm_tasks), -np.inf)
    lmi = np.zeros((B, o.lm_tasks), dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    rng = rng or np.random.default_rng(0)

    def wqkv(l: int, g: int) -> np.ndarray:
        return np.concatenate([m.W(f"l{l}.wq")[g * G * D:(g + 1) * G * D],
                               m.W(f"l{l}.wk")[g * D:(g + 1) * D],
                               m.W(f"l{l}.wv")[g * D:(g + 1) * D]])

    def merge(b: int, g: int):
        # softmax over the union of the chunks: rescale each chunk's sums by
        # exp(m_c - M), M the largest chunk maximum
        for j in range(G):
            h = g * G + j
            M = np.max(pm[b, h])
            wts = np.exp(pm[b, h] - M)
            attn[b, h * D:(h + 1) * D] = (wts @ pa[b, h]) / (wts @ pl[b, h])

    def run(i: int, t: Task):
        if t.type == EMB:
            x[t.b] = m.embed_row(tokens[t.b])
        elif t.type == QKV:
            ga = bf16.decode(m.w[f"l{t.layer}.g_attn"])
            w = wqkv(t.layer, t.g)[t.row0:t.row1]
            for b in range(B):
                qkv[b, t.g, t.row0:t.row1] = w @ rmsnorm(x[b], ga, s.rms_eps)
        elif t.type == ATT:
            b, g, l = t.b, t.g, t.layer
            p = int(pos[b])
            lo, hi = chunk_range(p + 1, t.chunk, Nc)
            q = rope(qkv[b, g, :G * D].reshape(G, D), p, s.rope_theta)
            knew = bf16.encode(rope(qkv[b, g, G * D:G * D + D], p, s.rope_theta))
            vnew = bf16.encode(qkv[b, g, G * D + D:])
            if t.chunk == Nc - 1:
                st.kcache[l, b, g, p] = knew
                st.vcache[l, b, g, p] = vnew
            kk = bf16.decode(st.kcache[l, b, g, lo:hi]).copy()
            vv = bf16.decode(st.vcache[l, b, g, lo:hi]).copy()
            if lo <= p < hi:                     # newest entry, as just rounded
                kk[p - lo] = bf16.decode(knew)
                vv[p - lo] = bf16.decode(vnew)
            for j in range(G):
                h = g * G + j
                if hi <= lo:
                    pm[b, h, t.chunk], pl[b, h, t.chunk], pa[b, h, t.chunk] = -np.inf, 0.0, 0.0
                    continue
                sc = kk @ q[j] / np.sqrt(float(D))
                mx = np.max(sc)
                e = np.exp(sc - mx)
                pm[b, h, t.chunk], pl[b, h, t.chunk], pa[b, h, t.chunk] = mx, e.sum(), e @ vv
            if mode == MERGE_IN_ATT:             # the only chunk: merge here
                merge(b, g)
        elif t.type == COMB:
            merge(t.b, t.g)
        elif t.type == OPROJ:
            w = m.W(f"l{t.layer}.wo")[t.row0:t.row1]
            x[:, t.row0:t.row1] += attn @ w.T
        elif t.type == GU:
            gm = bf16.decode(m.w[f"l{t.layer}.g_mlp"])
            wg = m.W(f"l{t.layer}.wg")[t.row0:t.row1]
            wu = m.W(f"l{t.layer}.wu")[t.row0:t.row1]
            for b in range(B):
                h2 = rmsnorm(x[b], gm, s.rms_eps)
                mlp[b, t.row0:t.row1] = silu(wg @ h2) * (wu @ h2)
        elif t.type == DOWN:
            w = m.W(f"l{t.layer}.wd")[t.row0:t.row1]
            x[:, t.row0:t.row1] += mlp @ w.T
        elif t.type == LM:
            k = i - gr.events[t.dep].first_dependent
            gf = bf16.decode(m.w["g_final"])
            w = m.W("lm_head")[t.row0:t.row1]
            for b in range(B):
                lg = w @ rmsnorm(x[b], gf, s.rms_eps)
                logits[b, t.row0:t.row1] = lg
                j = int(np.argmax(lg))
                lmv[b, k], lmi[b, k] = lg[j], t.row0 + j
        elif t.type == ARGMAX:
            k = int(np.argmax(lmv[t.b]))          # first maximal partial = lowest row
            nxt[t.b] = lmi[t.b, k]

    counter = [0] * len(gr.events)
    counter[gr.tasks[0].dep] = gr.events[gr.tasks[0].dep].threshold   # step start
    done = [False] * len(gr.tasks)
    pending = set(range(len(gr.tasks)))
    while pending:
        ready = sorted(i for i in pending
                       if counter[gr.tasks[i].dep] >= gr.events[gr.tasks[i].dep].threshold)
        assert ready, "task graph deadlocked"
        i = ready[int(rng.integers(len(ready)))]
        run(i, gr.tasks[i])
        pending.discard(i)
        done[i] = True
        t = gr.tasks[i]
        if t.type != ARGMAX:
            counter[t.trig] += 1
    return logits, nxt
