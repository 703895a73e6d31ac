// Device-side descriptors shared by the runtime's host and device code
// (internal to libmk).
#pragma once

#include <cstdint>

namespace mk {

// Weights are streamed in 1 KiB "units": 64 lanes x 16 bytes. A unit covers a
// block of 4 consecutive rows and 128 consecutive columns: lane 16*j + i holds
// columns [8i, 8i+8) of row j of the block (8 bf16 values). A matvec task's
// weights are its units in (row block, column block) order, stored
// contiguously in the packed buffer; gate/up tasks alternate a gate row block
// and the up row block of the same rows.
constexpr int kUnitBytes = 1024;
constexpr int kUnitCols = 128;
constexpr int kUnitRows = 4;

constexpr int kThreads = 256;  // workgroup size: 4 wave64
constexpr int kWaves = kThreads / 64;
constexpr int kMaxCols = 4;    // sequences a matvec task handles (VALU path)
constexpr int kAttTile = 256;  // positions per attention tile

// status word bits (device)
constexpr int32_t kStatusBadToken = 1;
constexpr int32_t kStatusBadPos = 2;
constexpr int32_t kStatusTimeout = 4;

struct DevTask {
  int32_t type, layer, b, g, chunk, row0, row1;
  int32_t dep, trig;
  int32_t ordinal;   // index of the task within its operator
  int32_t n_units;   // weight units of a matvec task (0 otherwise)
  int32_t n_vrb;     // row blocks streamed (gate/up count both)
  int64_t w_off;     // byte offset of the task's units in the packed weights
};

struct Params {
  // graph
  const DevTask* tasks;
  const int32_t* queue_ptr;   // [num_cus + 1]
  const int32_t* queue_ids;
  const uint32_t* thresholds;
  uint32_t* counters;
  int32_t n_tasks;
  // shape
  int32_t L, H, Hq, Hkv, D, F, V, G, B, S, Nc, n_lm;
  int32_t kb_h, kb_qd, kb_f;  // column blocks of 128 for K = H, Hq*D, F
  float eps;
  float attn_scale;
  int32_t kp;           // staged floats per column (max padded K)
  int32_t vrow_stride;  // partial-sum rows per wave and column
  int32_t ncap;         // staged columns = min(max_batch, kMaxCols)
  // model data
  const uint8_t* wpack;
  const uint16_t* embed;      // [V][H] bf16 (library copy)
  const uint16_t* gains;      // [L][2][H] then [H] final, bf16
  uint16_t* kcache;           // [L][B][Hkv][S][D] bf16 (caller-owned)
  uint16_t* vcache;
  const float2* rope_cs;      // [S][D/2] (cos, sin)
  // workspace (fp32 activations)
  float* x;                   // [B][H]
  float* qkv;                 // [B][Hkv][(G+2)D]
  float* part_ml;             // [B][Hq][Nc][2]
  float* part_acc;            // [B][Hq][Nc][D]
  float* attn;                // [B][Hq*D]
  float* mlp;                 // [B][F]
  float* lm_val;              // [B][n_lm]
  int32_t* lm_idx;            // [B][n_lm]
  int32_t* tok_cur;           // [B]
  int32_t* status;
  int32_t* abort_flag;
  // call
  const int32_t* tokens_in;   // [batch]
  const int32_t* pos_in;      // [batch]
  int32_t* out_tokens;        // [n_steps][batch]
  float* logits_out;          // [batch][V] or null (written at the last step)
  int32_t batch;
  int32_t n_steps;
  uint32_t epoch0;
  uint64_t timeout_ticks;     // 100 MHz constant clock
  uint64_t* profile;          // null or [n_steps][n_tasks][4]
  int32_t drop_task;          // fault injection: this task never signals (-1: off)
};

// One matvec task to repack: rows [row0, row1) of its logical matrix (the
// kv group's [q; k; v] rows for QKV), K columns, KB column blocks, n_vrb
// streamed row blocks.
struct PackJob {
  int64_t dst_off;
  int32_t type, layer, g, row0, row1, K, KB, n_vrb;
};

// Source matrices per layer: wq wk wv wo wg wu wd; entry [L].p[0] is the LM head.
struct PackSrc {
  const uint16_t* p[7];
};

}  // namespace mk
