// Host compiler: operator list of one decode step -> tasks, events with
// thresholds, round-robin per-compute-unit queues, canonical bytes.
//
// The operator order is the pages' wiring of one step (MPK walk-through
// section 3.3.1, build_mirage_graph; Hazy megakernel summary, fused
// instruction list). The partition, event and byte-format rules are this
// project's own specification, written out in this file (defaults in the
// resolve step, tasks and events in creation order, bytes in serialize);
// oracle/graph.py implements the same specification separately and the
// tests compare bytes.
#include "graph.h"

#include <algorithm>
#include <cstring>

namespace mk {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Builder {
  Graph* g;
  int32_t new_event(int32_t threshold) {
    g->events.push_back(Event{threshold, -1, 0});
    return static_cast<int32_t>(g->events.size()) - 1;
  }
  // Appends one operator's tasks, placing its i-th task on unit
  // (i + floor(i / N) * skew) mod N: round-robin, each further round over the
  // N units starting `skew` units on. The attention operator passes its chunk
  // count, so that a unit's chunks come from different sequences (whose
  // lengths, and so chunk costs, differ) instead of all from one.
  void add_op(std::vector<Task>&& op, int32_t skew = 0) {
    const int64_t n = g->opts.num_cus;
    const int32_t begin = static_cast<int32_t>(g->tasks.size());
    for (size_t i = 0; i < op.size(); ++i) {
      op[i].cu = static_cast<int32_t>((int64_t(i) + int64_t(i) / n * skew) % n);
      g->tasks.push_back(op[i]);
    }
    g->ops.emplace_back(begin, static_cast<int32_t>(g->tasks.size()));
  }
};

Task blank(int32_t type) { return Task{type, -1, -1, -1, -1, -1, -1, -1, -1, -1}; }

// rows -> T ranges made of whole blocks of rb rows (balanced over blocks).
std::vector<std::pair<int32_t, int32_t>> row_split(int32_t rows, int32_t T, int32_t rb) {
  std::vector<std::pair<int32_t, int32_t>> r;
  const int64_t nb = cdiv(rows, rb);
  for (int64_t t = 0; t < T; ++t) {
    const int64_t b0 = t * nb / T, b1 = (t + 1) * nb / T;
    r.emplace_back(static_cast<int32_t>(b0 * rb), static_cast<int32_t>(std::min<int64_t>(rows, b1 * rb)));
  }
  return r;
}

}  // namespace

int build_graph(const mk_model_desc& d, const mk_graph_opts* in, Graph* out, std::string* err) {
  auto fail = [&](const char* m) { *err = m; return MK_EINVAL; };
  if (d.n_layers < 1 || d.hidden < 1 || d.n_q_heads < 1 || d.n_kv_heads < 1 || d.head_dim < 2 ||
      d.ffn < 1 || d.vocab < 1 || d.max_batch < 1 || d.max_seq < 1)
    return fail("mk_model_desc: every size must be positive");
  if (d.n_q_heads % d.n_kv_heads) return fail("n_q_heads must be a multiple of n_kv_heads");
  if (d.head_dim % 8) return fail("head_dim must be a multiple of 8");
  if (d.hidden % 8 || d.ffn % 8) return fail("hidden and ffn must be multiples of 8");
  if (!(d.rms_eps >= 0.f) || !(d.rope_theta > 0.f)) return fail("rms_eps >= 0 and rope_theta > 0 required");
  if (d.qk_norm != 0 && d.qk_norm != 1) return fail("qk_norm must be 0 or 1");
  mk_graph_opts o{};
  if (in) o = *in;
  if (o.num_cus < 0 || o.qkv_tasks_per_group < 0 || o.o_tasks < 0 || o.gu_tasks < 0 || o.d_tasks < 0 ||
      o.lm_tasks < 0 || o.attn_chunks < 0 || o.row_block < 0)
    return fail("mk_graph_opts: negative option");
  if (o.use_mfma > 2) return fail("mk_graph_opts: use_mfma must be 0, 1 or 2");

  const int32_t N = o.num_cus ? o.num_cus : 256;
  const int32_t rb = o.row_block ? o.row_block : 4;
  const int32_t Hkv = d.n_kv_heads, G = d.n_q_heads / d.n_kv_heads, B = d.max_batch;
  const int32_t grp_rows = (G + 2) * d.head_dim;
  auto cap = [&](int32_t req, int32_t rows) {
    return static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(req, cdiv(rows, rb))));
  };
  mk_graph_opts r{};
  r.num_cus = N;
  r.row_block = rb;
  r.gu_tasks = cap(o.gu_tasks ? o.gu_tasks : N, d.ffn);
  r.d_tasks = cap(o.d_tasks ? o.d_tasks : N, d.hidden);
  r.attn_chunks = o.attn_chunks
                      ? o.attn_chunks
                      : std::max(1, std::min(N / (std::min(B, kGroupCols) * Hkv), std::max(1, d.max_seq / 1024)));
  const int32_t Nc = r.attn_chunks;
  {  // the matrix-core bodies take K dimensions that are multiples of 64, at least 256
    auto mf_ok = [](int64_t k) { return k % 64 == 0 && k >= 256; };
    const bool shape_ok = mf_ok(d.hidden) && mf_ok(int64_t(d.n_q_heads) * d.head_dim) && mf_ok(d.ffn);
    r.use_mfma = o.use_mfma ? o.use_mfma : (std::min(B, kMfmaCols) > kGroupCols && shape_ok ? 2 : 1);
  }
  // QKV on the matrix cores: at least one task per 16-row block of a group. A
  // task's rows are padded to whole blocks, and a padded row streams at the
  // same per-unit cost (batch-16 8B shape: 24-row tasks padded to 32, 8.29
  // ms per step; one 16-row block per task, 8.06).
  {
    int64_t q = cdiv(N, Hkv);
    if (r.use_mfma == 2) q = std::max<int64_t>(q, cdiv(grp_rows, kMfmaRowBlock));
    r.qkv_tasks_per_group = cap(o.qkv_tasks_per_group ? o.qkv_tasks_per_group : int32_t(q), grp_rows);
  }
  // O projection on the vector bodies: half the units when its weights would
  // give each of N tasks less than 64 KiB. The units without an O task start
  // streaming the gate/up weights that much sooner (measured: 1B shape 878 ->
  // 866 us/token, 8B shape, 128 KiB per task at N, slower with half).
  {
    const bool small_o = int64_t(d.hidden) * d.n_q_heads * d.head_dim * 2 < int64_t(N) * 65536;
    r.o_tasks = cap(o.o_tasks ? o.o_tasks : (r.use_mfma == 1 && small_o ? int32_t(cdiv(N, 2)) : N), d.hidden);
  }
  // LM head: the matrix-core bodies' tasks default to 8 row blocks (128 rows),
  // so that a stream wave keeps all of a task's row blocks in registers
  r.lm_tasks = cap(o.lm_tasks ? o.lm_tasks : (r.use_mfma == 2 ? std::max<int32_t>(N, int32_t(cdiv(d.vocab, 128))) : N),
                   d.vocab);

  Graph& g = *out;
  g = Graph{};
  g.desc = d;
  g.opts = r;
  Builder bld{&g};

  // events in creation order
  const int32_t e_tok = bld.new_event(B);
  const int32_t e_emb = bld.new_event(B);
  const int32_t L = d.n_layers;
  // With one chunk per (sequence, kv group) each attention task merges its
  // own result: no per-chunk events, no COMB tasks, and the attention tasks
  // count the layer's merged event directly (one hand-off fewer per layer).
  const bool fold = Nc == 1;
  std::vector<int32_t> e_qkv(size_t(L) * Hkv), e_att(fold ? 0 : size_t(L) * Hkv * B), e_comb(L), e_o(L), e_gu(L),
      e_d(L);
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t gi = 0; gi < Hkv; ++gi) e_qkv[size_t(l) * Hkv + gi] = bld.new_event(r.qkv_tasks_per_group);
    if (!fold)
      for (int32_t gi = 0; gi < Hkv; ++gi)
        for (int32_t b = 0; b < B; ++b) e_att[(size_t(l) * Hkv + gi) * B + b] = bld.new_event(Nc);
    e_comb[l] = bld.new_event(Hkv * B);
    e_o[l] = bld.new_event(r.o_tasks);
    e_gu[l] = bld.new_event(r.gu_tasks);
    e_d[l] = bld.new_event(r.d_tasks);
  }
  const int32_t e_lm = bld.new_event(r.lm_tasks);

  {  // embedding
    std::vector<Task> op;
    for (int32_t b = 0; b < B; ++b) {
      Task t = blank(T_EMB);
      t.b = b; t.dep = e_tok; t.trig = e_emb;
      op.push_back(t);
    }
    bld.add_op(std::move(op));
  }
  for (int32_t l = 0; l < L; ++l) {
    const int32_t dep_in = l == 0 ? e_emb : e_d[l - 1];
    {
      std::vector<Task> op;
      const auto split = row_split(grp_rows, r.qkv_tasks_per_group, rb);
      for (int32_t gi = 0; gi < Hkv; ++gi)
        for (const auto& rr : split) {
          Task t = blank(T_QKV);
          t.layer = l; t.g = gi; t.row0 = rr.first; t.row1 = rr.second;
          t.dep = dep_in; t.trig = e_qkv[size_t(l) * Hkv + gi];
          op.push_back(t);
        }
      bld.add_op(std::move(op));
    }
    {
      std::vector<Task> op;
      for (int32_t gi = 0; gi < Hkv; ++gi)
        for (int32_t b = 0; b < B; ++b)
          for (int32_t c = 0; c < Nc; ++c) {
            Task t = blank(T_ATT);
            t.layer = l; t.g = gi; t.b = b; t.chunk = c;
            t.dep = e_qkv[size_t(l) * Hkv + gi];
            t.trig = fold ? e_comb[l] : e_att[(size_t(l) * Hkv + gi) * B + b];
            op.push_back(t);
          }
      bld.add_op(std::move(op), Nc);
    }
    if (!fold) {
      std::vector<Task> op;
      for (int32_t gi = 0; gi < Hkv; ++gi)
        for (int32_t b = 0; b < B; ++b) {
          Task t = blank(T_COMB);
          t.layer = l; t.g = gi; t.b = b;
          t.dep = e_att[(size_t(l) * Hkv + gi) * B + b]; t.trig = e_comb[l];
          op.push_back(t);
        }
      bld.add_op(std::move(op));
    }
    struct RowOp { int32_t type, rows, tasks, dep, trig; };
    const RowOp row_ops[3] = {{T_O, d.hidden, r.o_tasks, e_comb[l], e_o[l]},
                              {T_GU, d.ffn, r.gu_tasks, e_o[l], e_gu[l]},
                              {T_D, d.hidden, r.d_tasks, e_gu[l], e_d[l]}};
    for (const RowOp& ro : row_ops) {
      std::vector<Task> op;
      for (const auto& rr : row_split(ro.rows, ro.tasks, rb)) {
        Task t = blank(ro.type);
        t.layer = l; t.row0 = rr.first; t.row1 = rr.second; t.dep = ro.dep; t.trig = ro.trig;
        op.push_back(t);
      }
      bld.add_op(std::move(op));
    }
  }
  {
    std::vector<Task> op;
    for (const auto& rr : row_split(d.vocab, r.lm_tasks, rb)) {
      Task t = blank(T_LM);
      t.row0 = rr.first; t.row1 = rr.second; t.dep = e_d[L - 1]; t.trig = e_lm;
      op.push_back(t);
    }
    bld.add_op(std::move(op));
  }
  {
    std::vector<Task> op;
    for (int32_t b = 0; b < B; ++b) {
      Task t = blank(T_ARGMAX);
      t.b = b; t.dep = e_lm; t.trig = e_tok;
      op.push_back(t);
    }
    bld.add_op(std::move(op));
  }

  for (size_t i = 0; i < g.tasks.size(); ++i) {
    Event& ev = g.events[g.tasks[i].dep];
    if (ev.n_dependents == 0) ev.first_dependent = static_cast<int32_t>(i);
    ++ev.n_dependents;
  }
  g.queues.assign(N, {});
  for (size_t i = 0; i < g.tasks.size(); ++i) g.queues[g.tasks[i].cu].push_back(static_cast<int32_t>(i));
  return MK_OK;
}

namespace {
struct Writer {
  std::vector<uint8_t> b;
  void u32(uint32_t v) { for (int i = 0; i < 4; ++i) b.push_back(uint8_t(v >> (8 * i))); }
  void i32(int32_t v) { u32(static_cast<uint32_t>(v)); }
  void f32(float v) { uint32_t u; std::memcpy(&u, &v, 4); u32(u); }
};
}  // namespace

std::vector<uint8_t> serialize(const Graph& g) {
  Writer w;
  const char magic[8] = {'M', 'K', 'G', 'R', 'A', 'P', 'H', '1'};
  w.b.insert(w.b.end(), magic, magic + 8);
  w.u32(5);  // version 5: qk_norm in the desc, use_mfma in the options, skewed attention placement,
            // single-chunk attention merged in its own task
  const mk_model_desc& d = g.desc;
  for (int32_t v : {d.n_layers, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn, d.vocab,
                    d.tied_embeddings, d.max_batch, d.max_seq})
    w.i32(v);
  w.f32(d.rms_eps);
  w.f32(d.rope_theta);
  w.i32(d.qk_norm);
  const mk_graph_opts& o = g.opts;
  for (int32_t v : {o.num_cus, o.qkv_tasks_per_group, o.o_tasks, o.gu_tasks, o.d_tasks, o.lm_tasks,
                    o.attn_chunks, o.row_block, o.use_mfma})
    w.i32(v);
  w.i32(static_cast<int32_t>(g.tasks.size()));
  w.i32(static_cast<int32_t>(g.events.size()));
  for (const Task& t : g.tasks)
    for (int32_t v : {t.type, t.layer, t.b, t.g, t.chunk, t.row0, t.row1, t.dep, t.trig, t.cu}) w.i32(v);
  for (const Event& e : g.events)
    for (int32_t v : {e.threshold, e.first_dependent, e.n_dependents}) w.i32(v);
  for (const auto& q : g.queues) {
    w.i32(static_cast<int32_t>(q.size()));
    for (int32_t id : q) w.i32(id);
  }
  return w.b;
}

}  // namespace mk
