// C ABI of libmk: graph building, model load (weight packing), decode calls.
// The declarations and their contracts are in include/mk.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "device.h"
#include "graph.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return MK_EHIP;
}

#define HIP_TRY(expr, what)                   \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

static_assert(mk::kMaxCols == mk::kGroupCols, "the graph's group size is the launch's column capacity");
static_assert(mk::kMfmaCols == 16, "the matrix-core bodies' M dimension");

// The launch scratch of a model, in the order mk_generate_noalloc lays it out:
// the event counters and the abort flag first (cleared at every call), then
// the activations, attention partials, LM partials and the token buffer.
enum { kWsCounters, kWsAbort, kWsX, kWsQkv, kWsPartMl, kWsPartAcc, kWsAttn, kWsMlp, kWsLmVal, kWsLmIdx, kWsTok, kWsSsq,
       kWsN };

struct mk_model {
  mk::Graph g;
  int device = 0;
  int lds_bytes = 0;
  int ncap = 1;       // sequences one launch stages (a call with more runs them in groups)
  bool mfma = false;  // matrix-core bodies (graph option use_mfma = 2)
  int max_batch = 1;  // sequences the KV caches hold
  uint64_t packed_bytes = 0;
  uint32_t epoch = 0;
  uint32_t max_threshold = 1;
  bool need_reset = false;
  uint64_t timeout_ticks = 200000000ull;  // 2 s at 100 MHz
  uint64_t* profile = nullptr;
  int32_t drop_task = -1;
  size_t profile_bytes = 0;
  uint64_t* waits = nullptr;
  mk::Params base{};                      // everything but the per-call fields
  // 4-byte words of the buffers one launch uses as scratch, in the order of
  // kWs* below (what mk_generate_noalloc lays out in its static workspace)
  size_t ws_words[kWsN] = {};
  std::vector<void*> allocs;              // device buffers owned by the model

  ~mk_model() {
    for (void* p : allocs) (void)hipFree(p);
  }
  template <class T>
  int alloc(T** p, size_t count, const char* what) {
    void* q = nullptr;
    if (count == 0) count = 1;
    hipError_t e = hipMalloc(&q, count * sizeof(T));
    if (e != hipSuccess) return fail(MK_ENOMEM, std::string("hipMalloc failed for ") + what);
    allocs.push_back(q);
    *p = static_cast<T*>(q);
    return MK_OK;
  }
};

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }

int mk_build_task_graph(const mk_model_desc* desc, const mk_graph_opts* opts, mk_graph** out) {
  if (!desc || !out) return fail(MK_EINVAL, "mk_build_task_graph: NULL argument");
  mk_graph* g = new (std::nothrow) mk_graph;
  if (!g) return fail(MK_ENOMEM, "mk_build_task_graph: out of host memory");
  std::string err;
  int rc = mk::build_graph(*desc, opts, &g->g, &err);
  if (rc != MK_OK) {
    delete g;
    return fail(rc, "mk_build_task_graph: " + err);
  }
  *out = g;
  return MK_OK;
}

int mk_graph_serialize(const mk_graph* g, uint8_t* buf, size_t cap, size_t* len) {
  if (!g || !len) return fail(MK_EINVAL, "mk_graph_serialize: NULL argument");
  const std::vector<uint8_t> b = mk::serialize(g->g);
  *len = b.size();
  if (!buf) return cap == 0 ? MK_OK : fail(MK_EINVAL, "mk_graph_serialize: NULL buffer");
  if (cap < b.size()) return fail(MK_EINVAL, "mk_graph_serialize: buffer too small");
  std::memcpy(buf, b.data(), b.size());
  return MK_OK;
}

int mk_graph_info(const mk_graph* g, int32_t* n_tasks, int32_t* n_events, mk_graph_opts* resolved) {
  if (!g) return fail(MK_EINVAL, "mk_graph_info: NULL graph");
  if (n_tasks) *n_tasks = static_cast<int32_t>(g->g.tasks.size());
  if (n_events) *n_events = static_cast<int32_t>(g->g.events.size());
  if (resolved) *resolved = g->g.opts;
  return MK_OK;
}

void mk_free_graph(mk_graph* g) { delete g; }

// Load `gsrc` (whose per-sequence tasks cover gsrc.desc.max_batch sequences)
// for KV caches that hold cache_batch sequences.
static int load_model(const mk::Graph& gsrc, int32_t cache_batch, const mk_weights* w, void* stream, mk_model** out) {
  using namespace mk;
  const mk_model_desc& d = gsrc.desc;
  if (!d.tied_embeddings && !w->lm_head) return fail(MK_EINVAL, "mk_load_weights: lm_head is NULL but not tied");
  for (int l = 0; l < d.n_layers; ++l) {
    const mk_layer_weights& L = w->layers[l];
    if (!L.wq || !L.wk || !L.wv || !L.wo || !L.wg || !L.wu || !L.wd || !L.g_attn || !L.g_mlp)
      return fail(MK_EINVAL, "mk_load_weights: NULL layer weight");
    if (d.qk_norm && (!L.q_norm || !L.k_norm))
      return fail(MK_EINVAL, "mk_load_weights: qk_norm model with a NULL q_norm or k_norm");
  }
  const int G = d.n_q_heads / d.n_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);

  mk_model* m = new (std::nothrow) mk_model;
  if (!m) return fail(MK_ENOMEM, "mk_load_weights: out of host memory");
  struct Guard {
    mk_model*& m;
    ~Guard() { delete m; }
  } guard{m};
  m->g = gsrc;
  m->max_batch = cache_batch;
  const Graph& g = m->g;
  HIP_TRY(hipGetDevice(&m->device), "hipGetDevice");
  // set-up of mk_generate_noalloc's static workspace on this device (once per device)
  HIP_TRY(noalloc_scratch_init(m->device), "hipGetSymbolAddress(static workspace)");
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, m->device), "hipGetDeviceProperties");

  // --- task descriptors and packed-weight offsets ---------------------------
  // column blocks per row block, rounded up to even (zero weights pad K): a
  // streamed item is two units of one row block
  const bool mf = g.opts.use_mfma == 2;
  m->mfma = mf;
  if (mf && (d.hidden % kMfmaItemCols || (int64_t(d.n_q_heads) * d.head_dim) % kMfmaItemCols || d.ffn % kMfmaItemCols ||
             std::min({d.hidden, d.n_q_heads * d.head_dim, d.ffn}) < 4 * kMfmaItemCols))
    return fail(MK_EUNSUPPORTED,
                "mk_load_weights: the matrix-core bodies need hidden, q width and ffn multiples of 64, at least 256");
  // vector bodies: 128-column blocks, rounded up to an even count; matrix-core
  // bodies: 32-column blocks (K is a multiple of 64)
  const int kb_h = mf ? d.hidden / 32 : static_cast<int>(cdiv(d.hidden, 2 * kUnitCols) * 2);
  const int kb_qd = mf ? d.n_q_heads * d.head_dim / 32
                       : static_cast<int>(cdiv(int64_t(d.n_q_heads) * d.head_dim, 2 * kUnitCols) * 2);
  const int kb_f = mf ? d.ffn / 32 : static_cast<int>(cdiv(d.ffn, 2 * kUnitCols) * 2);
  int wave_tiles = 1;
  std::vector<DevTask> dt(g.tasks.size());
  std::vector<int32_t> walk(g.tasks.size(), 0);  // units the stream waves walk (column-major: 8 row blocks)
  std::vector<PackJob> jobs;
  uint64_t off = 0;
  int max_vrows = 4, wave_vrows = 4, max_res = 4;
  std::vector<int32_t> ordinal_in_op(g.tasks.size());
  for (const auto& op : g.ops)
    for (int32_t i = op.first; i < op.second; ++i) ordinal_in_op[i] = i - op.first;
  for (size_t i = 0; i < g.tasks.size(); ++i) {
    const Task& t = g.tasks[i];
    DevTask& x = dt[i];
    x = DevTask{t.type, t.layer, t.b, t.g, t.chunk, t.row0, t.row1, t.dep, t.trig, ordinal_in_op[i], 0, 0, 0, 0, 0};
    int K = 0, KB = 0;
    switch (t.type) {
      case T_QKV: case T_GU: case T_LM: K = d.hidden; KB = kb_h; break;
      case T_O: K = d.n_q_heads * d.head_dim; KB = kb_qd; break;
      case T_D: K = d.ffn; KB = kb_f; break;
      default: break;
    }
    if (KB == 0) continue;
    const int nrb = static_cast<int>(cdiv(t.row1 - t.row0, kUnitRows));
    const int n_vrb = mf ? static_cast<int>(cdiv(t.row1 - t.row0, t.type == T_GU ? kMfmaRows / 2 : kMfmaRows))
                         : t.type == T_GU ? 2 * nrb : nrb;
    x.n_units = n_vrb * KB;
    x.kb = KB;
    x.kdim = K;
    x.w_off = static_cast<int64_t>(off);
    x.cm = mf && n_vrb >= 3 && n_vrb <= 8 ? n_vrb : 0;
    walk[i] = x.cm ? 8 * KB : x.n_units;
    max_vrows = std::max(max_vrows, n_vrb * kUnitRows);
    if (t.type == T_O || t.type == T_D) max_res = std::max(max_res, t.row1 - t.row0);
    if (x.cm) wave_tiles = std::max(wave_tiles, x.cm);  // column-major: every wave touches every row block
    else {  // rows of the row blocks each stream wave's piece touches (its partial sums)
      const int items = x.n_units / 2;
      for (int w = 0; w < kStreams; ++w) {
        // the stream waves' cut of the items (the kernels' piece()): weighted
        // on the vector bodies, equal quarters on the matrix cores
        static const int64_t cum[kStreams + 1] = {0, 67, 134, 195, 256};
        const int i0 = mf ? int(int64_t(items) * w / kStreams) : int((int64_t(items) * cum[w]) >> 8);
        const int i1 = mf ? int(int64_t(items) * (w + 1) / kStreams) : int((int64_t(items) * cum[w + 1]) >> 8);
        if (i1 <= i0) continue;
        const int touched = (2 * i1 - 1) / KB - (2 * i0) / KB + 1;
        wave_vrows = std::max(wave_vrows, touched * kUnitRows);
        wave_tiles = std::max(wave_tiles, touched);
      }
    }
    jobs.push_back(PackJob{x.w_off, t.type, t.layer, t.g, t.row0, t.row1, K, KB, n_vrb, x.cm});
    off += uint64_t(x.n_units) * kUnitBytes;
  }
  m->packed_bytes = off;

  // --- stream records: the stream tasks of every queue, with staging slots --
  std::vector<StreamRec> srec;
  std::vector<int32_t> sptr(1, 0);
  int srec_max = 0;
  for (const auto& q : g.queues) {
    if (q.size() > 65535) return fail(MK_EUNSUPPORTED, "mk_load_weights: a queue holds more than 65535 tasks");
    int nsmall = 0;
    const size_t first = srec.size();
    for (size_t qp = 0; qp < q.size(); ++qp) {
      const DevTask& x = dt[q[qp]];
      // staging slot as the kernel assigns it: 3 down-projection (overlays the
      // others), 2 merge, else the small slots alternately
      const int slot = x.type == T_D ? 3 : x.type == T_COMB ? 2 : (nsmall++ & 1);
      const bool stream = x.type == T_QKV || x.type == T_ATT || x.type == T_O || x.type == T_GU ||
                          x.type == T_D || x.type == T_LM;
      if (!stream) continue;
      if (x.b > 1023 || x.g > 65535 || x.layer > 65535 || x.chunk > 65535)
        return fail(MK_EUNSUPPORTED, "mk_load_weights: task field out of the stream record's range");
      StreamRec r{};
      r.tsbg = uint32_t(x.type) | uint32_t(slot) << 4 | uint32_t(x.b) << 6 | uint32_t(x.g) << 16;
      r.lc = x.type == T_ATT ? uint32_t(x.layer) | uint32_t(x.chunk) << 16
                             : (uint32_t(x.layer) & 0xffffu) | uint32_t(x.cm) << 16;
      r.n_units = walk[q[qp]];
      r.kq = uint32_t(x.kb) | uint32_t(qp) << 16;
      r.w_off = x.w_off;
      r.id = q[qp];
      srec.push_back(r);
    }
    for (size_t j = first; j < srec.size(); ++j) srec[j].flip = nsmall & 1;
    srec_max = std::max(srec_max, static_cast<int>(srec.size()) - sptr.back());
    sptr.push_back(static_cast<int32_t>(srec.size()));
  }

  // --- LDS budget -------------------------------------------------------------
  const int D = d.head_dim;
  if (d.max_batch > kMaxBatch)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: max_batch above " + std::to_string(kMaxBatch));
  if (G > kMaxG) return fail(MK_EUNSUPPORTED, "mk_load_weights: more than 4 query heads per kv head");
  if (D != 64 && D != 128) return fail(MK_EUNSUPPORTED, "mk_load_weights: head_dim must be 64 or 128");
  if (d.hidden > 4096) return fail(MK_EUNSUPPORTED, "mk_load_weights: hidden above 4096");
  if (!mf && std::max({kb_h, kb_qd, kb_f}) > 254)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: a K dimension above 32512");
  if (mf && std::max({kb_h, kb_qd, kb_f}) > 65535)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: a K dimension above 2^21");
  if (int64_t(g.opts.attn_chunks) * (int64_t(d.max_seq) + 1) >= (int64_t(1) << 32))
    return fail(MK_EUNSUPPORTED, "mk_load_weights: attn_chunks * (max_seq + 1) must stay below 2^32");
  if (d.hidden % 4 || (d.n_q_heads * d.head_dim) % 4 || d.ffn % 4)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: hidden, q width and ffn must be multiples of 4");
  // LDS: control words, two small staging slots, the merge slot (attention
  // merges), three partial-sum areas, then the stream records. A
  // down-projection input overlays the two small slots and the merge slot (the
  // kernel stages it only once every earlier task has retired). Staged copies
  // move whole 1 KiB pieces, so every region is rounded up to 256 floats where
  // a copy lands. (The stream waves' weight rings live in registers.)
  auto r256 = [](int64_t n) { return (n + 255) / 256 * 256; };
  // The sequences one launch stages (ncap): as many as fit the LDS; a call
  // with more sequences runs them in groups of ncap (sequences are
  // independent).
  int ncap = std::min<int>(d.max_batch, mf ? kMfmaCols : kMaxCols);
  const int kp = static_cast<int>(r256(std::max(d.hidden, d.n_q_heads * D)));
  const int kp_big = static_cast<int>(r256(d.ffn));
  int nlm_tasks = 0;
  for (const Task& t : g.tasks) nlm_tasks += t.type == T_LM;
  const int64_t Ncx = g.opts.attn_chunks;
  const int res_stride = (max_res + 3) & ~3;
  const size_t lds_max = 160 * 1024;
  int64_t small_floats = 0, big_floats = 0, part_floats = 0;
  size_t fixed = 0;
  for (; ncap >= 1; --ncap) {
    // matrix-core bodies: the gains of a normalised input (bf16) or the
    // residual rows of all kMfmaCols sequences; vector bodies: the staged
    // inputs and residual rows of ncap sequences
    const int64_t need_mv = mf ? std::max(r256(d.hidden / 2), int64_t(kMfmaCols) * res_stride)
                               : int64_t(ncap) * kp + int64_t(ncap) * res_stride;
    // attention: raw q|k|v, rotated q, new k and v, their bf16 bits, k and v of
    // position p - 1, the scaled rotated q, then the stream waves' partials (acc[wave][head][D],
    // then (m, l) per wave and head)
    const int64_t need_att = r256(int64_t(G + 2) * D) + int64_t(G) * D + 2 * D + D + 2 * D + int64_t(G) * D +
                             int64_t(kStreams) * G * (D + 2);
    const int64_t need_arg = r256(nlm_tasks) * 2;
    const int64_t need_emb = r256(d.hidden / 2 + 1);
    const int64_t need_mv_big = mf ? int64_t(kMfmaCols) * res_stride : int64_t(ncap) * kp_big + int64_t(ncap) * res_stride;
    const int64_t need_comb = r256(int64_t(G) * Ncx * 2) + r256(int64_t(G) * Ncx * D);
    small_floats = (32 + std::max({need_mv, need_att, need_arg, need_emb}) + 3) & ~int64_t(3);
    // the merge slot follows the two small ones; the down-projection input
    // overlays all three, so the merge slot holds what it needs beyond them
    big_floats = (std::max(32 + need_comb, 32 + need_mv_big - 2 * small_floats) + 3) & ~int64_t(3);
    part_floats = mf ? int64_t(kStreams) * wave_tiles * 256 : (int64_t(kStreams) * ncap * wave_vrows + 3) & ~int64_t(3);
    // a prefill step's attention stages its earlier columns' keys and values
    // (and their scores) in the partial-sum area of its slot
    part_floats = std::max<int64_t>(part_floats, (int64_t(ncap - 1) * 2 * D + kMaxG * kPrefillMax + 3) & ~int64_t(3));
    fixed = kCtlBytes + size_t(4) * size_t(2 * small_floats + big_floats + 3 * part_floats) +
            size_t(srec_max) * sizeof(StreamRec);
    if (fixed <= lds_max || mf) break;  // (the matrix-core bodies stage no per-sequence inputs)
  }
  if (mf && fixed > lds_max)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: the matrix-core bodies need " + std::to_string(fixed) +
                                     " bytes of LDS, more than the 160 KiB a workgroup has");
  if (ncap < 1)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: staging one sequence needs " + std::to_string(fixed) +
                                     " bytes of LDS, more than the 160 KiB a workgroup has");
  m->ncap = ncap;
  const size_t lds = fixed;
  m->lds_bytes = static_cast<int>(lds);
  HIP_TRY(set_lds_limit(m->lds_bytes), "hipFuncSetAttribute(max dynamic LDS)");
  int per_cu = 0;
  HIP_TRY(persistent_occupancy(m->lds_bytes, &per_cu), "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (int64_t(per_cu) * prop.multiProcessorCount < g.opts.num_cus)
    return fail(MK_EUNSUPPORTED, "mk_load_weights: num_cus=" + std::to_string(g.opts.num_cus) +
                                     " workgroups cannot be co-resident (" + std::to_string(prop.multiProcessorCount) +
                                     " CUs x " + std::to_string(per_cu) + ")");

  // --- device buffers -----------------------------------------------------------
  Params& P = m->base;
  P = Params{};
  const int64_t H = d.hidden, V = d.vocab, L = d.n_layers, B = d.max_batch, S = d.max_seq;
  const int64_t Hq = d.n_q_heads, Hkv = d.n_kv_heads, F = d.ffn;
  int nlm = 0;
  for (const Task& t : g.tasks) nlm += t.type == T_LM;
  DevTask* d_tasks;
  StreamRec* d_srec;
  int32_t *d_qptr, *d_qids, *d_sptr;
  uint32_t *d_thr, *d_cnt;
  int rc;
  if ((rc = m->alloc(&d_tasks, dt.size(), "tasks")) || (rc = m->alloc(&d_qptr, g.queues.size() + 1, "queues")) ||
      (rc = m->alloc(&d_qids, g.tasks.size(), "queue ids")) || (rc = m->alloc(&d_thr, g.events.size(), "thresholds")) ||
      (rc = m->alloc(&d_cnt, g.events.size() * kEventWords, "counters")) ||
      (rc = m->alloc(&d_srec, std::max<size_t>(srec.size(), 1), "stream records")) ||
      (rc = m->alloc(&d_sptr, sptr.size(), "stream record offsets")))
    return rc;
  std::vector<int32_t> qptr(1, 0), qids;
  for (const auto& q : g.queues) {
    qids.insert(qids.end(), q.begin(), q.end());
    qptr.push_back(static_cast<int32_t>(qids.size()));
  }
  std::vector<uint32_t> thr(g.events.size());
  for (size_t e = 0; e < g.events.size(); ++e) {
    thr[e] = static_cast<uint32_t>(g.events[e].threshold);
    m->max_threshold = std::max(m->max_threshold, thr[e]);
  }
  HIP_TRY(hipMemcpy(d_tasks, dt.data(), dt.size() * sizeof(DevTask), hipMemcpyHostToDevice), "copy tasks");
  HIP_TRY(hipMemcpy(d_qptr, qptr.data(), qptr.size() * 4, hipMemcpyHostToDevice), "copy queue offsets");
  if (!srec.empty())
    HIP_TRY(hipMemcpy(d_srec, srec.data(), srec.size() * sizeof(StreamRec), hipMemcpyHostToDevice), "copy stream records");
  HIP_TRY(hipMemcpy(d_sptr, sptr.data(), sptr.size() * 4, hipMemcpyHostToDevice), "copy stream record offsets");
  HIP_TRY(hipMemcpy(d_qids, qids.data(), qids.size() * 4, hipMemcpyHostToDevice), "copy queues");
  HIP_TRY(hipMemcpy(d_thr, thr.data(), thr.size() * 4, hipMemcpyHostToDevice), "copy thresholds");
  HIP_TRY(hipMemset(d_cnt, 0, thr.size() * 4 * kEventWords), "clear counters");

  uint8_t *d_wpack, *d_zeros;
  uint16_t *d_embed, *d_gains;
  float2* d_rope;
  if ((rc = m->alloc(&d_wpack, m->packed_bytes, "packed weights")) || (rc = m->alloc(&d_embed, V * H + 512, "embedding")) ||
      (rc = m->alloc(&d_gains, (2 * L + 1) * H + 2 * L * D + 512, "norm gains")) || (rc = m->alloc(&d_rope, S * (D / 2), "rope table")) ||
      (rc = m->alloc(&d_zeros, size_t(kZeroBlocks) * 2 * kUnitBytes, "zero blocks")))
    return rc;
  HIP_TRY(hipMemset(d_zeros, 0, size_t(kZeroBlocks) * 2 * kUnitBytes), "clear zero blocks");
  HIP_TRY(hipMemcpyAsync(d_embed, w->embed, V * H * 2, hipMemcpyDeviceToDevice, s), "copy embedding");
  for (int l = 0; l < L; ++l) {
    HIP_TRY(hipMemcpyAsync(d_gains + (2 * l) * H, w->layers[l].g_attn, H * 2, hipMemcpyDeviceToDevice, s), "copy gain");
    HIP_TRY(hipMemcpyAsync(d_gains + (2 * l + 1) * H, w->layers[l].g_mlp, H * 2, hipMemcpyDeviceToDevice, s), "copy gain");
  }
  HIP_TRY(hipMemcpyAsync(d_gains + 2 * L * H, w->g_final, H * 2, hipMemcpyDeviceToDevice, s), "copy gain");
  if (d.qk_norm)  // per-head q/k gains [L][2][D] after the hidden-size gains
    for (int l = 0; l < L; ++l) {
      uint16_t* dst = d_gains + (2 * L + 1) * H + 2 * l * D;
      HIP_TRY(hipMemcpyAsync(dst, w->layers[l].q_norm, D * 2, hipMemcpyDeviceToDevice, s), "copy q norm gain");
      HIP_TRY(hipMemcpyAsync(dst + D, w->layers[l].k_norm, D * 2, hipMemcpyDeviceToDevice, s), "copy k norm gain");
    }
  {  // RoPE: angle p * theta^(-2j/D) in double, cos/sin rounded to float
    std::vector<float2> cs(size_t(S) * (D / 2));
    for (int64_t p = 0; p < S; ++p)
      for (int64_t j = 0; j < D / 2; ++j) {
        const double a = double(p) * std::pow(double(d.rope_theta), -2.0 * double(j) / double(D));
        cs[p * (D / 2) + j] = float2{float(std::cos(a)), float(std::sin(a))};
      }
    HIP_TRY(hipMemcpy(d_rope, cs.data(), cs.size() * sizeof(float2), hipMemcpyHostToDevice), "copy rope table");
  }
  {  // pack weights
    std::vector<PackSrc> srcs(L + 1);
    for (int l = 0; l < L; ++l) {
      const mk_layer_weights& Lw = w->layers[l];
      srcs[l] = PackSrc{{static_cast<const uint16_t*>(Lw.wq), static_cast<const uint16_t*>(Lw.wk),
                         static_cast<const uint16_t*>(Lw.wv), static_cast<const uint16_t*>(Lw.wo),
                         static_cast<const uint16_t*>(Lw.wg), static_cast<const uint16_t*>(Lw.wu),
                         static_cast<const uint16_t*>(Lw.wd)}};
    }
    srcs[L] = PackSrc{{static_cast<const uint16_t*>(d.tied_embeddings ? w->embed : w->lm_head)}};
    PackJob* d_jobs;
    PackSrc* d_srcs;
    void *pj = nullptr, *ps = nullptr;
    HIP_TRY(hipMalloc(&pj, jobs.size() * sizeof(PackJob)), "hipMalloc pack jobs");
    d_jobs = static_cast<PackJob*>(pj);
    hipError_t e = hipMalloc(&ps, srcs.size() * sizeof(PackSrc));
    if (e != hipSuccess) { (void)hipFree(pj); return hip_fail(e, "hipMalloc pack sources"); }
    d_srcs = static_cast<PackSrc*>(ps);
    e = hipMemcpy(d_jobs, jobs.data(), jobs.size() * sizeof(PackJob), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(d_srcs, srcs.data(), srcs.size() * sizeof(PackSrc), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = launch_pack(d_jobs, static_cast<int>(jobs.size()), d_srcs, d_wpack, G, d.head_dim, d.n_layers, mf, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)hipFree(pj);
    (void)hipFree(ps);
    if (e != hipSuccess) return hip_fail(e, "weight packing");
  }

  float *d_x, *d_qkv, *d_pml, *d_pacc, *d_attn, *d_mlp, *d_lmv, *d_ssq;
  int32_t *d_lmi, *d_tok, *d_status, *d_abort;
  const int64_t Nc = g.opts.attn_chunks;
  int n_ss_o = 0, n_ss_d = 0;  // tasks of the O and D projections (each writes one sum-of-squares part)
  for (const Task& t : g.tasks) {
    if (t.type == T_O && t.layer == 0) ++n_ss_o;
    if (t.type == T_D && t.layer == 0) ++n_ss_d;
  }
  const int64_t ssq_floats = mf ? int64_t(std::max({n_ss_o, n_ss_d, 1})) * kMfmaCols + 256 : 1;
  const int64_t slack = 4096;  // floats read past the end by 1 KiB-granular copies
  if ((rc = m->alloc(&d_x, B * H + slack, "x")) || (rc = m->alloc(&d_qkv, B * Hkv * (G + 2) * D + slack, "qkv")) ||
      (rc = m->alloc(&d_pml, B * Hq * Nc * 2 + slack, "attention partials")) ||
      (rc = m->alloc(&d_pacc, B * Hq * Nc * D + slack, "attention partials")) ||
      (rc = m->alloc(&d_attn, B * Hq * D + slack, "attn")) || (rc = m->alloc(&d_mlp, B * F + slack, "mlp")) ||
      (rc = m->alloc(&d_lmv, B * nlm + slack, "lm partials")) || (rc = m->alloc(&d_lmi, B * nlm + slack, "lm partials")) ||
      (rc = m->alloc(&d_tok, B + 64, "tokens")) || (rc = m->alloc(&d_ssq, ssq_floats, "sums of squares")) ||
      (rc = m->alloc(&d_status, 1, "status")) || (rc = m->alloc(&d_abort, 1, "abort flag")))
    return rc;
  {
    const size_t w[kWsN] = {g.events.size() * kEventWords, 1, size_t(B * H + slack),
                            size_t(B * Hkv * (G + 2) * D + slack), size_t(B * Hq * Nc * 2 + slack),
                            size_t(B * Hq * Nc * D + slack), size_t(B * Hq * D + slack), size_t(B * F + slack),
                            size_t(B * nlm + slack), size_t(B * nlm + slack), size_t(B + 64), size_t(ssq_floats)};
    std::copy(w, w + kWsN, m->ws_words);
  }
  HIP_TRY(hipMemset(d_status, 0, 4), "clear status");
  HIP_TRY(hipMemset(d_abort, 0, 4), "clear abort flag");
  HIP_TRY(hipMemset(d_tok, 0, B * 4), "clear tokens");
  HIP_TRY(hipStreamSynchronize(s), "load synchronisation");

  P.tasks = d_tasks;
  P.queue_ptr = d_qptr;
  P.queue_ids = d_qids;
  P.srecs = d_srec;
  P.srec_ptr = d_sptr;
  P.srec_max = srec_max;
  P.thresholds = d_thr;
  P.counters = d_cnt;
  P.n_tasks = static_cast<int32_t>(g.tasks.size());
  P.L = d.n_layers; P.H = d.hidden; P.Hq = d.n_q_heads; P.Hkv = d.n_kv_heads; P.D = d.head_dim; P.F = d.ffn;
  P.V = d.vocab; P.G = G; P.B = cache_batch; P.S = d.max_seq; P.Nc = g.opts.attn_chunks; P.n_lm = nlm;
  P.eps = d.rms_eps;
  P.qk_norm = d.qk_norm;
  P.small_floats = static_cast<int32_t>(small_floats);
  P.big_floats = static_cast<int32_t>(big_floats);
  P.kp_big = kp_big;
  P.part_floats = static_cast<int32_t>(part_floats);
  P.attn_scale = static_cast<float>(1.0 / std::sqrt(double(d.head_dim)));
  P.kp = kp;
  P.wave_vrows = wave_vrows;
  P.wave_tiles = wave_tiles;
  P.n_ss_o = n_ss_o;
  P.n_ss_d = n_ss_d;
  P.res_stride = res_stride;
  P.ncap = ncap;
  P.wpack = d_wpack;
  P.zeros = d_zeros;
  P.embed = d_embed;
  P.gains = d_gains;
  P.kcache = static_cast<uint16_t*>(w->k_cache);
  P.vcache = static_cast<uint16_t*>(w->v_cache);
  P.rope_cs = d_rope;
  P.x = d_x; P.qkv = d_qkv; P.part_ml = d_pml; P.part_acc = d_pacc; P.attn = d_attn; P.mlp = d_mlp;
  P.lm_val = d_lmv; P.lm_idx = d_lmi; P.tok_cur = d_tok; P.status = d_status; P.abort_flag = d_abort;
  P.ssq = d_ssq;
  *out = m;
  m = nullptr;  // ownership passes to the caller
  return MK_OK;
}

int mk_load_weights(const mk_graph* gr, const mk_weights* w, void* stream, mk_model** out) {
  if (!gr || !w || !out || !w->layers || !w->embed || !w->g_final || !w->k_cache || !w->v_cache)
    return fail(MK_EINVAL, "mk_load_weights: NULL argument");
  const mk_model_desc& d = gr->g.desc;
  // One launch decodes a group of at most kGroupCols sequences (fewer when the
  // LDS stages fewer). A model whose batch exceeds its group runs, on every
  // group, the graph of a desc with the group's size and the same options, so
  // that a launch holds no tasks of sequences outside its group.
  int32_t group = std::min<int32_t>(d.max_batch, gr->g.opts.use_mfma == 2 ? mk::kMfmaCols : mk::kGroupCols);
  mk_graph_opts opts = gr->g.opts;
  for (;;) {
    mk::Graph g1;
    const mk::Graph* src = &gr->g;
    if (group < d.max_batch) {
      mk_model_desc d1 = d;
      d1.max_batch = group;
      std::string err;
      const int brc = mk::build_graph(d1, &opts, &g1, &err);
      if (brc != MK_OK) return fail(brc, "mk_load_weights: group graph: " + err);
      src = &g1;
    }
    const int rc = load_model(*src, d.max_batch, w, stream, out);
    if (rc != MK_OK || (*out)->ncap == group) return rc;
    // the LDS stages fewer sequences than the graph holds: rebuild for that many
    group = (*out)->ncap;
    mk_free_model(*out);
    *out = nullptr;
  }
}

static int check_call(mk_model* m, const int32_t* tok, const int32_t* pos, int32_t batch, const void* outp) {
  if (!m) return fail(MK_EINVAL, "NULL model");
  if (!tok || !pos || !outp) return fail(MK_EINVAL, "NULL token, position or output pointer");
  if (batch < 1 || batch > m->max_batch)
    return fail(MK_EINVAL, "batch must be in 1..max_batch (" + std::to_string(m->max_batch) + ")");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != m->device)
    return fail(MK_EINVAL, "the current HIP device is not the model's device");
  return MK_OK;
}

static int prepare_epoch(mk_model* m, int32_t n_steps, hipStream_t s) {
  const uint64_t top = (uint64_t(m->epoch) + uint64_t(n_steps) + 1) * m->max_threshold;
  if (m->need_reset || top >= (1ull << 31)) {
    HIP_TRY(hipMemsetAsync(m->base.counters, 0, m->g.events.size() * 4 * mk::kEventWords, s), "reset counters");
    HIP_TRY(hipMemsetAsync(m->base.abort_flag, 0, 4, s), "reset abort flag");
    m->epoch = 0;
    m->need_reset = false;
  }
  return MK_OK;
}

// The per-call fields for the group of sequences [b0, b0 + nb) of a call with
// `batch` sequences: its tokens, positions, outputs and KV cache rows.
static mk::Params group_params(const mk_model* m, const int32_t* tok, const int32_t* pos, int32_t batch, int32_t b0,
                               int32_t nb, int32_t n_steps, int32_t* out_tokens, float* logits) {
  mk::Params P = m->base;
  const size_t seq_kv = size_t(P.Hkv) * size_t(P.S) * size_t(P.D);  // one sequence's rows of a layer
  P.tokens_in = tok + b0;
  P.pos_in = pos + b0;
  P.out_tokens = out_tokens + b0;
  P.out_stride = batch;
  P.logits_out = logits ? logits + size_t(b0) * size_t(P.V) : nullptr;
  P.kcache = m->base.kcache + size_t(b0) * seq_kv;
  P.vcache = m->base.vcache + size_t(b0) * seq_kv;
  P.batch = nb;
  P.n_steps = n_steps;
  P.timeout_ticks = m->timeout_ticks;
  return P;
}

// One persistent launch per group of at most ncap sequences, in order on the
// stream (sequences never interact, so the groups may run one after another).
static int run_megakernel(mk_model* m, const int32_t* tok, const int32_t* pos, int32_t batch, int32_t n_steps,
                          int32_t* out_tokens, float* logits, hipStream_t s) {
  for (int32_t b0 = 0; b0 < batch; b0 += m->ncap) {
    int rc = prepare_epoch(m, n_steps, s);
    if (rc) return rc;
    mk::Params P = group_params(m, tok, pos, batch, b0, std::min(m->ncap, batch - b0), n_steps, out_tokens, logits);
    P.epoch0 = m->epoch;
    P.use_events = 1;
    P.drop_task = m->drop_task;
    P.profile = (m->profile && m->profile_bytes >= size_t(n_steps) * m->g.tasks.size() * mk::kProfWords * 8) ? m->profile : nullptr;
    P.waits = m->waits;
    HIP_TRY(mk::launch_persistent(P, m->g.opts.num_cus, m->lds_bytes, m->mfma, s),
            "hipLaunchCooperativeKernel(mk_persistent)");
    m->epoch += static_cast<uint32_t>(n_steps);
  }
  return MK_OK;
}

int mk_decode_step(mk_model* m, const int32_t* d_tokens, const int32_t* d_pos, int32_t batch, float* d_logits,
                   int32_t* d_next, int32_t mode, void* stream) {
  int rc = check_call(m, d_tokens, d_pos, batch, d_next);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == MK_MODE_MEGAKERNEL) return run_megakernel(m, d_tokens, d_pos, batch, 1, d_next, d_logits, s);
  if (mode != MK_MODE_OPLAUNCH) return fail(MK_EINVAL, "mk_decode_step: unknown mode");
  for (int32_t b0 = 0; b0 < batch; b0 += m->ncap) {
    mk::Params P = group_params(m, d_tokens, d_pos, batch, b0, std::min(m->ncap, batch - b0), 1, d_next, d_logits);
    P.epoch0 = 0;
    P.use_events = 0;
    P.drop_task = -1;
    for (const auto& op : m->g.ops)
      HIP_TRY(mk::launch_op(P, op.first, op.second - op.first, m->lds_bytes, m->mfma, s), "hipLaunchKernel(mk_oplaunch)");
  }
  return MK_OK;
}

int mk_generate(mk_model* m, const int32_t* d_tokens0, const int32_t* d_pos0, int32_t batch, int32_t n_steps,
                int32_t* d_out_tokens, float* d_last_logits, void* stream) {
  int rc = check_call(m, d_tokens0, d_pos0, batch, d_out_tokens);
  if (rc) return rc;
  if (n_steps < 1) return fail(MK_EINVAL, "mk_generate: n_steps must be >= 1");
  return run_megakernel(m, d_tokens0, d_pos0, batch, n_steps, d_out_tokens, d_last_logits,
                        static_cast<hipStream_t>(stream));
}

int mk_generate_noalloc(mk_model* m, const int32_t* d_tokens0, const int32_t* d_pos0, int32_t batch,
                        int32_t n_steps, int32_t* d_out_tokens, float* d_last_logits, void* stream) {
  int rc = check_call(m, d_tokens0, d_pos0, batch, d_out_tokens);
  if (rc) return rc;
  if (n_steps < 1) return fail(MK_EINVAL, "mk_generate_noalloc: n_steps must be >= 1");
  if ((uint64_t(n_steps) + 1) * m->max_threshold >= (1ull << 31))
    return fail(MK_EINVAL, "mk_generate_noalloc: n_steps too large for the event counters");
  uint8_t* base = static_cast<uint8_t*>(mk::noalloc_scratch(m->device));
  if (!base) return fail(MK_EHIP, "mk_generate_noalloc: the static workspace was not resolved on this device");
  size_t off[kWsN], total = 0;
  for (int i = 0; i < kWsN; ++i) {
    off[i] = total;
    total += (m->ws_words[i] * 4 + 255) / 256 * 256;
  }
  if (total > MK_NOALLOC_SCRATCH_BYTES)
    return fail(MK_EINVAL, "mk_generate_noalloc: one launch of this model needs " + std::to_string(total) +
                               " bytes of scratch; the static workspace holds " +
                               std::to_string(size_t(MK_NOALLOC_SCRATCH_BYTES)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t b0 = 0; b0 < batch; b0 += m->ncap) {
    // counters and abort flag sit at the front: every launch starts them at 0
    HIP_TRY(mk::launch_fill_zero(reinterpret_cast<uint32_t*>(base), off[kWsX] / 4, s), "hipLaunchKernel(mk_fill_zero)");
    mk::Params P = group_params(m, d_tokens0, d_pos0, batch, b0, std::min(m->ncap, batch - b0), n_steps,
                                d_out_tokens, d_last_logits);
    P.counters = reinterpret_cast<uint32_t*>(base + off[kWsCounters]);
    P.abort_flag = reinterpret_cast<int32_t*>(base + off[kWsAbort]);
    P.x = reinterpret_cast<float*>(base + off[kWsX]);
    P.qkv = reinterpret_cast<float*>(base + off[kWsQkv]);
    P.part_ml = reinterpret_cast<float*>(base + off[kWsPartMl]);
    P.part_acc = reinterpret_cast<float*>(base + off[kWsPartAcc]);
    P.attn = reinterpret_cast<float*>(base + off[kWsAttn]);
    P.mlp = reinterpret_cast<float*>(base + off[kWsMlp]);
    P.lm_val = reinterpret_cast<float*>(base + off[kWsLmVal]);
    P.lm_idx = reinterpret_cast<int32_t*>(base + off[kWsLmIdx]);
    P.tok_cur = reinterpret_cast<int32_t*>(base + off[kWsTok]);
    P.ssq = reinterpret_cast<float*>(base + off[kWsSsq]);
    P.epoch0 = 0;
    P.use_events = 1;
    P.drop_task = m->drop_task;
    P.profile = (m->profile && m->profile_bytes >= size_t(n_steps) * m->g.tasks.size() * mk::kProfWords * 8) ? m->profile : nullptr;
    P.waits = m->waits;
    HIP_TRY(mk::launch_persistent(P, m->g.opts.num_cus, m->lds_bytes, m->mfma, s),
            "hipLaunchCooperativeKernel(mk_persistent)");
  }
  return MK_OK;
}

int mk_prefill(mk_model* m, const int32_t* d_tokens, int32_t n_tokens, int32_t seq, int32_t pos0, float* d_logits,
               int32_t* d_next, void* stream) {
  if (!m) return fail(MK_EINVAL, "mk_prefill: NULL model");
  if (!d_tokens || !d_next) return fail(MK_EINVAL, "mk_prefill: NULL token or output pointer");
  if (n_tokens < 1 || seq < 0 || seq >= m->max_batch || pos0 < 0 || int64_t(pos0) + n_tokens > m->base.S)
    return fail(MK_EINVAL, "mk_prefill: need n_tokens >= 1, 0 <= seq < max_batch and pos0 + n_tokens <= max_seq");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != m->device)
    return fail(MK_EINVAL, "the current HIP device is not the model's device");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t seq_kv = size_t(m->base.Hkv) * size_t(m->base.S) * size_t(m->base.D);
  for (int32_t c0 = 0; c0 < n_tokens; c0 += m->ncap) {
    const int32_t nb = std::min(m->ncap, n_tokens - c0);
    int rc = prepare_epoch(m, 1, s);
    if (rc) return rc;
    mk::Params P = m->base;
    P.tokens_in = d_tokens + c0;
    P.pos_in = d_tokens + c0;  // (positions come from pre_p0)
    P.out_tokens = d_next + c0;
    P.out_stride = nb;
    P.logits_out = d_logits ? d_logits + size_t(c0) * size_t(P.V) : nullptr;
    P.kcache = m->base.kcache + size_t(seq) * seq_kv;
    P.vcache = m->base.vcache + size_t(seq) * seq_kv;
    P.batch = nb;
    P.n_steps = 1;
    P.prefill = 1;
    P.pre_p0 = pos0 + c0;
    P.timeout_ticks = m->timeout_ticks;
    P.epoch0 = m->epoch;
    P.use_events = 1;
    P.drop_task = m->drop_task;
    P.profile = nullptr;
    P.waits = m->waits;
    HIP_TRY(mk::launch_persistent(P, m->g.opts.num_cus, m->lds_bytes, m->mfma, s),
            "hipLaunchCooperativeKernel(mk_persistent)");
    m->epoch += 1;
  }
  return MK_OK;
}

int mk_check(mk_model* m, void* stream) {
  if (!m) return fail(MK_EINVAL, "mk_check: NULL model");
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
  int32_t st = 0;
  HIP_TRY(hipMemcpy(&st, m->base.status, 4, hipMemcpyDeviceToHost), "read status");
  if (st == 0) return MK_OK;
  HIP_TRY(hipMemset(m->base.status, 0, 4), "clear status");
  if (st & mk::kStatusTimeout) {
    m->need_reset = true;
    return fail(MK_ETIMEOUT, "device watchdog expired; counters are reset on the next call");
  }
  return fail(MK_EDEVICE, std::string("device argument error:") + ((st & mk::kStatusBadToken) ? " token>=vocab" : "") +
                              ((st & mk::kStatusBadPos) ? " position>=max_seq" : ""));
}

int mk_set_watchdog_ms(mk_model* m, int32_t ms) {
  if (!m || ms < 0) return fail(MK_EINVAL, "mk_set_watchdog_ms: bad argument");
  m->timeout_ticks = uint64_t(ms ? ms : 2000) * 100000ull;
  return MK_OK;
}

int mk_debug_drop_signal(mk_model* m, int32_t task_id) {
  if (!m || task_id < -1 || task_id >= static_cast<int32_t>(m->g.tasks.size()))
    return fail(MK_EINVAL, "mk_debug_drop_signal: bad argument");
  m->drop_task = task_id;
  return MK_OK;
}

int mk_set_profile_buffer(mk_model* m, void* d_buf, size_t bytes) {
  if (!m) return fail(MK_EINVAL, "mk_set_profile_buffer: NULL model");
  if (d_buf && bytes < m->g.tasks.size() * mk::kProfWords * 8) return fail(MK_EINVAL, "mk_set_profile_buffer: buffer too small");
  m->profile = static_cast<uint64_t*>(d_buf);
  m->profile_bytes = d_buf ? bytes : 0;
  return MK_OK;
}

int mk_set_wait_counters(mk_model* m, void* d_buf, size_t bytes) {
  if (!m) return fail(MK_EINVAL, "mk_set_wait_counters: NULL model");
  if (d_buf && bytes < size_t(m->g.opts.num_cus) * mk::kWaves * mk::kWaitWords * 8)
    return fail(MK_EINVAL, "mk_set_wait_counters: buffer too small");
  m->waits = static_cast<uint64_t*>(d_buf);
  return MK_OK;
}

int mk_model_info(const mk_model* m, uint64_t* packed_weight_bytes, int32_t* num_cus, int32_t* n_tasks,
                  int32_t* ring_slots, int32_t* lds_bytes, int32_t* batch_per_launch) {
  if (!m) return fail(MK_EINVAL, "mk_model_info: NULL model");
  if (batch_per_launch) *batch_per_launch = m->ncap;
  if (packed_weight_bytes) *packed_weight_bytes = m->packed_bytes;
  if (num_cus) *num_cus = m->g.opts.num_cus;
  if (n_tasks) *n_tasks = static_cast<int32_t>(m->g.tasks.size());
  if (ring_slots) *ring_slots = mk::kRing;
  if (lds_bytes) *lds_bytes = m->lds_bytes;
  return MK_OK;
}

void mk_free_model(mk_model* m) { delete m; }

}  // extern "C"
