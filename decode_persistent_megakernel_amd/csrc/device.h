// Device-side descriptors shared by the runtime's host and device code
// (internal to libmk).
#pragma once

#include <cstdint>

namespace mk {

// Weights are streamed in 1 KiB "units": 64 lanes x 16 bytes. A unit covers a
// block of 4 consecutive rows and 128 consecutive columns: lane 16*j + i holds
// columns [4i, 4i+4) and [64+4i, 64+4i+4) of row j of the block (8 bf16
// values), so that the 16 lanes of a row read their activations as two
// contiguous 256-byte runs of LDS (no bank conflicts). A matvec task's
// weights are its units in (row block, column block) order, stored
// contiguously in the packed buffer; gate/up tasks alternate a gate row block
// and the up row block of the same rows.
constexpr int kUnitBytes = 1024;
constexpr int kUnitCols = 128;
constexpr int kUnitRows = 4;

// The matrix-core bodies (launches of up to kMfmaCols sequences) stream the
// same 1 KiB units in another arrangement: a unit covers 16 rows and 32
// consecutive columns, lane 16*j + i holding columns [8j, 8j+8) of row i, which
// is the B operand of one v_mfma_f32_16x16x32_bf16 (the 16 rows are its N
// dimension, the sequences its M dimension). A row block is 16 rows (gate/up:
// 8 gate rows then the 8 up rows of the same outputs); an item is the units of
// column blocks 2j and 2j+1 of one row block; a task's items are stored in
// (row block, column pair) order, or, for a task of 3 to 8 row blocks, in
// (column pair, row block) order (column-major: a stream wave then reads each
// column pair's activations once for all the task's row blocks).
constexpr int kMfmaRows = 16;
constexpr int kMfmaItemCols = 64;

// Workgroup layout: wave 0 stages task inputs (and polls events), wave 1
// retires tasks (epilogue, stores, signals); then kStreams stream waves, each
// loading its piece of every streamed task into a ring of registers and
// computing on it.
constexpr int kCtlWaves = 2;
constexpr int kStreams = 4;
constexpr int kThreads = 64 * (kCtlWaves + kStreams);
#ifndef MK_RING
#define MK_RING 8
#endif
constexpr int kRing = MK_RING;  // 2 KiB items each stream wave keeps in flight (in registers)
constexpr int kZeroBlocks = 256;  // 2 KiB zero blocks, one per compute unit (index taken modulo)
constexpr int kMaxCols = 4;    // sequences a matvec task handles (vector bodies; the
                               // matrix-core bodies handle kMfmaCols, graph.h)
constexpr int kMaxBatch = 256; // sequences a model holds (larger calls run in groups of at most kMaxCols)
constexpr int kMaxG = 4;       // query heads per kv head
constexpr int kPrefillMax = 16;  // columns of a prefill step (the matrix-core bodies' width)
constexpr int kStripes = 64;   // event counter stripes: one per lane of the polling wave
constexpr int kEventWords = kStripes * 32;  // each stripe in its own 128-byte line
constexpr int kCtlBytes = 1024;             // control words (see kernels)
constexpr int kWaves = kThreads / 64;
constexpr int kWaitWords = 16;              // per-wave wait counters (mk_set_wait_counters)
constexpr int kProfWords = 12;              // uint64 words per task in the profile buffer

// status word bits (device)
constexpr int32_t kStatusBadToken = 1;
constexpr int32_t kStatusBadPos = 2;
constexpr int32_t kStatusTimeout = 4;

struct DevTask {
  int32_t type, layer, b, g, chunk, row0, row1;
  int32_t dep, trig;
  int32_t ordinal;   // index of the task within its operator
  int32_t n_units;   // weight units of a matvec task (0 otherwise)
  int32_t kb;        // column blocks of a matvec task
  int32_t kdim;      // K of a matvec task
  int32_t cm;        // matrix-core bodies: row blocks of a task stored column-major (3..8), 0: row-block-major
  int64_t w_off;     // byte offset of the task's units in the packed weights
};

// A streamed task (weight or KV units) as the stream waves walk it: one per
// such task of a workgroup's queue, in queue order, held in LDS.
struct StreamRec {
  uint32_t tsbg;     // type | slot << 4 | b << 6 | g << 16  (staging slot in the first step:
                     // 0, 1 small, 2 big)
  uint32_t lc;       // layer | chunk << 16 (attention); layer | column-major row blocks << 16 (matvec)
  int32_t n_units;   // weight units (matvec; column-major: 8 items per column pair, the missing row
                     // blocks read as zeros)
  uint32_t kq;       // column blocks | queue position << 16
  int64_t w_off;     // packed weight offset (matvec)
  int32_t flip;      // 1: the small slots swap from one step to the next (odd count per step)
  int32_t id;        // global task id
};
static_assert(sizeof(StreamRec) == 32, "stream records are two 16-byte words");

struct Params {
  // graph
  const DevTask* tasks;
  const int32_t* queue_ptr;   // [num_cus + 1]
  const int32_t* queue_ids;
  const StreamRec* srecs;     // stream records of all queues
  const int32_t* srec_ptr;    // [num_cus + 1]
  int32_t srec_max;           // most records of one queue (LDS holds them)
  const uint32_t* thresholds;
  uint32_t* counters;         // [n_events][kEventWords]
  int32_t n_tasks;
  // shape
  int32_t L, H, Hq, Hkv, D, F, V, G, B, S, Nc, n_lm;
  float eps;
  float attn_scale;
  int32_t qk_norm;      // per-head q/k RMSNorm before RoPE (gains after the hidden-size ones)
  int32_t kp;           // staged floats per column in the small slots (K rounded up to 256)
  int32_t kp_big;       // staged floats per column in the big slot (FFN rounded up to 256)
  int32_t wave_vrows;   // partial-sum rows per (stream wave, column): the row blocks its piece touches
  int32_t res_stride;   // staged residual rows per column (projection tasks)
  int32_t ncap;         // staged columns: the most sequences one launch handles (<= kMaxCols)
  int32_t small_floats; // LDS staging slot size (two small slots)
  int32_t big_floats;   // LDS staging slot size for down-projection and merge tasks
  int32_t part_floats;  // LDS partial-sum area per slot
  int32_t wave_tiles;   // matrix-core bodies: 16x16 partial tiles per stream wave (row blocks its piece touches)
  int32_t n_ss_o, n_ss_d;  // matrix-core bodies: sum-of-squares partials the O and D projections write
  // model data
  const uint8_t* wpack;
  const uint8_t* zeros;       // [kZeroBlocks][2 KiB] of zeros: the loads that fill a stream block up
  const uint16_t* embed;      // [V][H] bf16 (library copy)
  const uint16_t* gains;      // [L][2][H], [H] final, then [L][2][D] q/k head gains, bf16
  uint16_t* kcache;           // [L][B][Hkv][S][D] bf16 (caller-owned)
  uint16_t* vcache;
  const float2* rope_cs;      // [S][D/2] (cos, sin)
  // workspace (fp32 activations; every buffer has 16 KiB of slack at the end)
  float* x;                   // [B][H]
  float* qkv;                 // [B][Hkv][(G+2)D]
  float* part_ml;             // [B][Hq][Nc][2]
  float* part_acc;            // [B][Hq][Nc][D]
  float* attn;                // [B][Hq*D]
  float* mlp;                 // [B][F]
  float* ssq;                 // matrix-core bodies: [task][16] sums of squares of the rows of x a
                              // projection task (or the embedding, at index 0) wrote
  float* lm_val;              // [B][n_lm]
  int32_t* lm_idx;            // [B][n_lm]
  int32_t* tok_cur;           // [B]
  int32_t* status;
  int32_t* abort_flag;
  // call
  const int32_t* tokens_in;   // [batch]
  const int32_t* pos_in;      // [batch]
  int32_t* out_tokens;        // [n_steps][out_stride]
  int32_t out_stride;         // sequences between consecutive steps' rows of out_tokens
  float* logits_out;          // [batch][V] or null (written at the last step)
  int32_t batch;
  int32_t n_steps;
  int32_t prefill;            // 1: the columns are the consecutive positions pre_p0 + b of one sequence (its
                              //    cache rows are the call's, kcache / vcache point at them), one step
  int32_t pre_p0;             // prefill: position of column 0
  uint32_t epoch0;
  int32_t use_events;         // 0: single-task workgroups ordered by the stream
  uint64_t timeout_ticks;     // 100 MHz constant clock
  uint64_t* profile;          // null or [n_steps][n_tasks][kProfWords]
  int32_t drop_task;          // fault injection: this task never signals (-1: off)
  uint64_t* waits;            // null or [grid][kWaves][kWaitWords] wait-time counters
};

// One matvec task to repack: rows [row0, row1) of its logical matrix (the
// kv group's [q; k; v] rows for QKV), K columns, KB column blocks, n_vrb
// streamed row blocks.
struct PackJob {
  int64_t dst_off;
  int32_t type, layer, g, row0, row1, K, KB, n_vrb;
  int32_t cm;  // matrix-core arrangement stored column-major (items (column pair, row block)), 0: row-block-major
};
// (the matrix-core arrangement: KB units of 32 columns per row block, n_vrb row blocks)

// Source matrices per layer: wq wk wv wo wg wu wd; entry [L].p[0] is the LM head.
struct PackSrc {
  const uint16_t* p[7];
};

}  // namespace mk
