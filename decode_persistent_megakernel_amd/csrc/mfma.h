// Stream waves of the matrix-core bodies (launches of up to 16 sequences;
// included by kernels.hip after pipeline.h; internal to libmk).
//
// The walk over pieces and blocks and the register weight ring are those of
// the vector bodies (pipeline.h); the units are in the matrix-core arrangement
// (device.h). Beside the weight ring runs an activation ring of XR = RING / 2
// items: the A operand of an item, this lane's sequence (lane & 15) and eight
// columns (8 (lane >> 4) of each of the item's two 32-column units), read as
// four 16-byte loads straight from the activation rows in global memory. The
// activation loads run XR items ahead of the compute cursor and stay inside
// the task being computed (its activations exist once it is staged): at a
// task's first block the wave loads the first XR items' activations and waits
// for them. Every slot issues the same loads (four activation, two weight;
// padding loads read this compute unit's zero block), so the compiler's wait
// before each item is one exact count.
//
// An item's activations are multiplied by the staged gains (RMS-normalised
// inputs) and split into two bf16 parts, hi = the value with its low 16 bits
// cleared (exact) and lo = the rest truncated to bf16, so that hi + lo carries
// 16 significant bits; each part multiplies each weight unit in one
// v_mfma_f32_16x16x32_bf16 into the 16 x 16 (sequences x rows) sums of the row
// block, four accumulator registers per lane. At the end of a row block's
// columns in the piece, the sums go to the wave's partial tile in LDS, rows
// major ([row][sequence]); the retirer adds the waves' tiles of each row block
// in wave order and applies the RMS factor and the epilogue.

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// The activation side of the matvec task being computed.
struct XPiece {
  rsrc_t rx;       // activation rows of the call's sequences, K floats each (past the batch: zeros)
  uint32_t lx;     // this lane's byte offset in them: sequence lane & 15, columns 8 (lane >> 4)
  int KB2;         // column pairs (64 columns) per row block
  int col0;        // column pair of the piece's first item
  int n;           // items of the piece
  uint32_t gl;     // LDS byte address of this lane's gains at column pair 0 (or of the ones)
  uint32_t gstep;  // LDS bytes per column pair (0: the ones)
};

__device__ __forceinline__ XPiece make_xpiece(const Params& P, const Ctx& cx, int s, const StreamRec& R, int slot,
                                              int type) {
  XPiece xp;
  const int lane = cx.lane;
  const int K = type == T_O ? P.Hq * P.D : type == T_D ? P.F : P.H;
  const float* src = type == T_O ? P.attn : type == T_D ? P.mlp : P.x;
  xp.rx = make_rsrc(src, (uint32_t)P.batch * (uint32_t)K * 4u);
  xp.lx = ((uint32_t)(lane & 15) * (uint32_t)K + 8u * (uint32_t)(lane >> 4)) * 4u;
  xp.KB2 = K / kMfmaItemCols;
  const int items = (int)rfl((uint32_t)R.n_units) / 2;
  int i0, i1;
  piece<false>(items, s, i0, i1);
  xp.n = i1 - i0;
  xp.col0 = i0 % xp.KB2;
  const bool normed = is_normed(type);
  xp.gl = normed ? lds_addr(slot_ptr(cx, slot) + kHdr) + (uint32_t)(lane >> 4) * 16u : lds_addr(&cx.ctl[kOnesCtl]);
  xp.gstep = normed ? (uint32_t)kMfmaItemCols * 2u : 0u;
  return xp;
}

// Activation loads of column pair c into one ring slot (zeros when !real).
__device__ __forceinline__ void load_x(const Params& P, const Ctx& cx, const XPiece& xp, int c, bool real,
                                       u32x4 (&x)[4]) {
  const rsrc_t z = make_rsrc(P.zeros + (size_t)rfl((uint32_t)cx.cu & (kZeroBlocks - 1)) * 2 * kUnitBytes, 2 * kUnitBytes);
  const rsrc_t r = real ? xp.rx : z;
  const uint32_t vo = real ? xp.lx : (uint32_t)cx.lane * 16u;
  const uint32_t so = real ? (uint32_t)c * (uint32_t)(kMfmaItemCols * 4) : 0u;
  x[0] = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kAuxCoherent);
  x[1] = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 16u, so, kAuxCoherent);
  x[2] = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 128u, so, kAuxCoherent);
  x[3] = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 144u, so, kAuxCoherent);
}

// x * gain split into bf16 hi and lo parts (8 values: two 16-byte words of
// activations, one of bf16 gains).
__device__ __forceinline__ void split8(const u32x4 a, const u32x4 b, const u32x4 g, bf16x8& hi, bf16x8& lo) {
  const float v[8] = {__uint_as_float(a.x) * bf2f(g.x & 0xffffu), __uint_as_float(a.y) * bf2f(g.x >> 16),
                      __uint_as_float(a.z) * bf2f(g.y & 0xffffu), __uint_as_float(a.w) * bf2f(g.y >> 16),
                      __uint_as_float(b.x) * bf2f(g.z & 0xffffu), __uint_as_float(b.y) * bf2f(g.z >> 16),
                      __uint_as_float(b.z) * bf2f(g.w & 0xffffu), __uint_as_float(b.w) * bf2f(g.w >> 16)};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h0 = __float_as_uint(v[2 * e]) & 0xffff0000u, h1 = __float_as_uint(v[2 * e + 1]) & 0xffff0000u;
    const uint32_t l0 = __float_as_uint(v[2 * e] - __uint_as_float(h0));
    const uint32_t l1 = __float_as_uint(v[2 * e + 1] - __uint_as_float(h1));
    h[e] = (h0 >> 16) | h1;
    l[e] = (l0 >> 16) | (l1 & 0xffff0000u);
  }
  u32x4 hv = {h[0], h[1], h[2], h[3]}, lv = {l[0], l[1], l[2], l[3]};
  hi = __builtin_bit_cast(bf16x8, hv);
  lo = __builtin_bit_cast(bf16x8, lv);
}

__device__ __forceinline__ u32x4 lds_ld16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)addr);
}

// The matrix-core walk: wave s's piece of record r. Row-block-major records
// are cut into items as on the vector bodies (make_piece); a column-major
// record (lc >> 16 = its row blocks, 3..8) is cut by column pairs, 8 items
// per column pair (item j of a column is row block j; those past the task's
// row blocks read zeros).
struct PieceM {
  Piece pc;
  int cm;  // row blocks of a column-major record, 0: row-block-major
};
__device__ __forceinline__ PieceM make_piece_m(const Params& P, const Ctx& cx, int s, int r) {
  PieceM m;
  m.pc = make_piece<false>(P, cx, s, r);
  m.cm = 0;
  const StreamRec R = cx.recs[r];
  if ((rfl(R.tsbg) & 15) == T_ATT) return m;
  const int cm = (int)(rfl(R.lc) >> 16);
  if (cm == 0) return m;
  const int ncol = (int)rfl((uint32_t)R.n_units) / 16;  // column pairs (8 items, 16 units each)
  int c0, c1;
  piece<false>(ncol, s, c0, c1);
  const int64_t woff =
      (int64_t)(((uint64_t)rfl((uint32_t)((uint64_t)R.w_off >> 32)) << 32) | rfl((uint32_t)R.w_off));
  m.pc.n = 8 * (c1 - c0);
  m.pc.ra = m.pc.rb = make_rsrc(P.wpack + woff + (int64_t)c0 * cm * kItemBytes,
                                (uint32_t)(c1 - c0) * (uint32_t)cm * (uint32_t)kItemBytes);
  m.cm = cm;
  return m;
}

// Loads of piece item i into one ring slot: row-block-major as load_item;
// column-major item i is row block i & 7 of column pair i >> 3, stored at
// (i >> 3) * cm + (i & 7) (zeros past the task's row blocks).
__device__ __forceinline__ void load_item_m(const Params& P, const Ctx& cx, const PieceM& m, int i, bool real, u32x4& a,
                                            u32x4& b) {
  const bool cmr = m.cm != 0;
  const int it = cmr ? (i >> 3) * m.cm + (i & 7) : i;
  load_item(P, cx, m.pc, it, real && (!cmr || (i & 7) < m.cm), a, b);
}

struct WalkM {
  int r, step, t;
  PieceM pm;
};
template <int RING>
__device__ __forceinline__ Blk next_block_m(const Params& P, const Ctx& cx, int s, WalkM& W) {
  Blk B;
  B.i0 = 0;
  B.n = 0;
  if (W.t >= W.pm.pc.n) {
    for (;;) {
      if (++W.r >= cx.nrec) {
        W.r = 0;
        ++W.step;
      }
      if (W.step >= P.n_steps || cx.nrec == 0) {
        B.r = W.r;
        B.step = W.step;
        B.flags = kEnd;
        W.pm.pc.n = 0;
        W.t = 0;
        return B;
      }
      W.pm = make_piece_m(P, cx, s, W.r);
      W.t = 0;
      if (W.pm.pc.n > 0) break;
    }
  }
  B.r = W.r;
  B.step = W.step;
  B.i0 = W.t;
  B.n = min(RING, W.pm.pc.n - W.t);
  B.flags = (W.t == 0 ? kFirst : 0) | (W.t + B.n == W.pm.pc.n ? kLast : 0);
  W.t += B.n;
  return B;
}

// Compute state of the matvec task being computed.
struct CompM {
  int r, step;      // stream record and step
  int slot, type;   // staging slot; type -1: none
  int rb, kc, rb0;  // row block and column pair of the next item, first row block of the piece
  bool pend;        // sums of an unfinished row block are held
  bool any;
  float* tiles;     // this wave's partial tiles (LDS)
  XPiece xp;
  int cm, col, c1;  // column-major: row blocks, next column pair, end of this wave's column pairs
  int natt;
  int layer, b, g;  // attention
  int lo, end, u0;
};

__device__ __forceinline__ void tile_flush(f32x4& acc, float* tiles, int t, int lane) {
  *reinterpret_cast<float4*>(tiles + t * 256 + (lane & 15) * 16 + 4 * (lane >> 4)) =
      make_float4(acc[0], acc[1], acc[2], acc[3]);
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
}

// One item: weight units w0, w1 (column blocks 2c, 2c + 1 of row block rb)
// against the activations x of column pair c.
__device__ __forceinline__ void mf_item(CompM& C, f32x4& acc, const u32x4 w0, const u32x4 w1, const u32x4 (&x)[4],
                                        int lane) {
  const uint32_t ga = C.xp.gl + (uint32_t)C.kc * C.xp.gstep;
  const u32x4 g0 = lds_ld16(ga), g1 = lds_ld16(ga + C.xp.gstep / 2u);
  bf16x8 h0, l0, h1, l1;
  split8(x[0], x[1], g0, h0, l0);
  split8(x[2], x[3], g1, h1, l1);
  const bf16x8 b0 = __builtin_bit_cast(bf16x8, w0), b1 = __builtin_bit_cast(bf16x8, w1);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, b0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l0, b0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, b1, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l1, b1, acc, 0, 0, 0);
  C.pend = true;
  if (++C.kc == C.xp.KB2) {
    tile_flush(acc, C.tiles, C.rb - C.rb0, lane);
    C.kc = 0;
    ++C.rb;
    C.pend = false;
  }
}

template <bool PROF>
__device__ __forceinline__ bool comp_start_m(const Params& P, const Ctx& cx, int s, CompM& C, f32x4& acc, AttState& S,
                                             Waits& wt, bool prof) {
  const int lane = cx.lane;
  const StreamRec R = cx.recs[C.r];
  const uint32_t tsbg = rfl(R.tsbg), kq = rfl(R.kq);
  C.type = tsbg & 15;
  C.slot = (tsbg >> 4) & 3;
  if (C.slot < 2) C.slot ^= (int)rfl((uint32_t)R.flip) & C.step;
  {
    const uint64_t s0 = waits_now(wt);
    if (!spin_ctl(P, cx, C_STAGED, C.step * (cx.q1 - cx.q0) + (int)(kq >> 16) + 1)) return false;
    waits_add(wt, 2, s0);
  }
  if (prof) prof_words(cx, C.slot, s)[0] = rfl((uint32_t)wall_clock64());
  if (C.type == T_ATT) {
    C.tiles = att_part_ptr(P, cx, C.slot);
    const int* ih = reinterpret_cast<const int*>(slot_ptr(cx, C.slot));
    const int flags = lds_ld(&ih[H_FLAGS]);
    C.lo = lds_ld(&ih[H_LO]);
    C.end = lds_ld(&ih[H_END]);
    const int lpp = P.D / 8, ppi = 64 / lpp;
    const int nb = (flags & 1) && C.end > C.lo ? (C.end - C.lo + ppi - 1) / ppi : 0;
    int j1;
    piece<false>(nb, s, C.u0, j1);
    C.natt = j1 - C.u0;
    const uint32_t lc = rfl(R.lc);
    C.layer = lc & 0xffff;
    C.b = (tsbg >> 6) & 1023;
    C.g = tsbg >> 16;
    S.qs = att_qs_ptr(P, cx, C.slot) + (lane % lpp) * 8;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      S.m[h] = -INFINITY;
      S.l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) S.acc[h][e] = 0.f;
    }
  } else {
    C.tiles = part_ptr(cx, C.slot) + (size_t)s * P.wave_tiles * 256;
    C.xp = make_xpiece(P, cx, s, R, C.slot, C.type);
    C.cm = (int)(rfl(R.lc) >> 16);
    if (C.cm) {  // column-major: this wave's column pairs, all the task's row blocks
      int c0, c1;
      piece<false>(C.xp.KB2, s, c0, c1);
      C.col = c0;
      C.c1 = c1;
      C.rb0 = 0;
      C.rb = C.cm;
      C.pend = false;
    } else {
      const int items = (int)rfl((uint32_t)R.n_units) / 2;
      int i0, i1;
      piece<false>(items, s, i0, i1);
      C.rb = i0 / C.xp.KB2;
      C.rb0 = C.rb;
      C.kc = C.xp.col0;
      C.pend = false;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  C.any = false;
  return true;
}

__device__ __forceinline__ void comp_finish_m(const Params& P, const Ctx& cx, int s, CompM& C, f32x4& acc, AttState& S,
                                              bool prof, uint32_t t_first) {
  if (C.type == T_ATT) {
    att_finish(P, S, C.tiles, s, cx.lane, !C.any);
  } else if (C.cm) {  // column-major: every row block of the task (the tiles are written at its last pass)
    int* pr = piece_words(cx, C.slot, s);
    pr[0] = 0;
    pr[1] = C.any ? C.cm - 1 : -1;
  } else {
    if (C.pend) tile_flush(acc, C.tiles, C.rb - C.rb0, cx.lane);
    int* pr = piece_words(cx, C.slot, s);
    pr[0] = C.rb0;
    pr[1] = !C.any ? C.rb0 - 1 : (C.pend ? C.rb : C.rb - 1);
  }
  if (prof) {
    uint32_t* pw = prof_words(cx, C.slot, s);
    pw[1] = t_first;
    pw[2] = rfl((uint32_t)wall_clock64());
  }
  lds_add_lane0(&cx.ctl[C_DONE + ctl_slot(C.slot)], 1);
  C.type = -1;
}

// The attention-task path of the vector bodies, on this compute state, with
// each head's scaled query in registers for the whole task (the activation
// ring is not live here; measured on the batch-16 8B workload: 8.80 -> 8.29 ms
// per step against reading the queries from LDS per KV block).
template <int AR>
__device__ __forceinline__ void att_run_m(const Params& P, const Ctx& cx, CompM& C, AttState& S, const Piece& pc,
                                          u32x4 (&ka)[AR], u32x4 (&kv)[AR]) {
  Comp A;
  A.lo = C.lo;
  A.end = C.end;
  A.u0 = C.u0;
  att_run<AR>(P, cx, A, S, pc, ka, kv);

  C.any = A.any;
}

// KV items an attention task keeps in flight on the matrix-core stream waves
// (fewer than the vector bodies' kAttRing: 6 and 8 spill registers and
// measured slower)
#ifndef MK_ATT_RING_M
#define MK_ATT_RING_M 4
#endif
constexpr int kAttRingM = MK_ATT_RING_M;
#ifndef MK_RING_M
#define MK_RING_M 8
#endif
#ifndef MK_XRING_M
#define MK_XRING_M 4
#endif
template <int RING, int XR, bool PROF>
__device__ __forceinline__ void run_stream_m16(const Params& P0, const Ctx& cx, int s) {
  static_assert(RING % XR == 0, "blocks start at a multiple of the activation ring");
  const Params& P = P0;
  const int lane = cx.lane;
  const bool prof = PROF && P.profile != nullptr;
  Waits wt;
  waits_init<PROF>(P, cx, wt);

  WalkM W;
  W.r = -1;
  W.step = 0;
  W.t = 0;
  W.pm = make_piece_m(P, cx, s, 0);
  W.pm.pc.n = 0;

  CompM C;
  C.r = -1;
  C.step = 0;
  C.type = -1;
  C.slot = 0;
  C.any = false;
  C.xp.n = 0;
  C.xp.KB2 = 4;
  C.xp.col0 = 0;
  C.cm = 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint32_t t_first = 0;

  u32x4 ra[RING], rb[RING];
  u32x4 xa[XR][4];

  // the first block's weights
  static_assert(RING == 8, "a column-major block is one column pair of 8 row blocks");
  Blk cur = next_block_m<RING>(P, cx, s, W);
#pragma unroll
  for (int j = 0; j < RING; ++j) {
    load_item_m(P, cx, W.pm, cur.i0 + j, j < cur.n, ra[j], rb[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  bool fin = false;
  // One iteration per task change: the task-change code (one copy, outside
  // the unrolled pass), then the passes over the blocks of the new piece. The
  // activation ring lives only inside the pass loop (reloaded at every task
  // start), so no register of it is held across the task-change code; the
  // weight ring's loads run on across it.
  for (;;) {
    {
      const Params& P = fresh_params();
      for (;;) {
        if (fin) {
          AttState S0;
          comp_finish_m(P, cx, s, C, acc, S0, prof, t_first);
          fin = false;
        }
        int r = C.r + 1, st = C.step;
        if (r >= cx.nrec) {
          r = 0;
          ++st;
        }
        if (st >= P.n_steps || cx.nrec == 0) break;
        const bool at = r == cur.r && st == cur.step;
        C.r = r;
        C.step = st;
        if (!at && (rfl(cx.recs[r].tsbg) & 15) == T_ATT) {
          // an attention task: its first KV blocks load while it is staged
          AttState S;
          u32x4 ka[kAttRingM], kv[kAttRingM];
          const Piece kpc = kv_piece_of<false>(P, cx, s, r, st);
          att_prefetch(P, cx, kpc, ka, kv);
          if (!comp_start_m<PROF>(P, cx, s, C, acc, S, wt, prof)) return;
          const uint32_t t_att = prof ? rfl((uint32_t)wall_clock64()) : 0u;
          att_run_m(P, cx, C, S, kpc, ka, kv);
          comp_finish_m(P, cx, s, C, acc, S, prof, t_att);
          continue;
        }
        AttState S1;
        if (!comp_start_m<PROF>(P, cx, s, C, acc, S1, wt, prof)) return;
        t_first = 0;
        if (at) break;
        fin = true;  // a matvec piece without items for this wave
      }
    }
    if (cur.flags & kEnd) break;
    if (C.cm) {
      // column-major task: per pass one column pair of 8 row blocks; the
      // activations of a column pair are read once, split into hi/lo once,
      // and the next column pair's are read at the start of the pass (as far
      // ahead as the weights)
      const Params& P = fresh_params();
      load_x(P, cx, C.xp, C.col, C.col < C.c1, xa[0]);
      f32x4 acc8[8];  // the sums of each row block of the task
#pragma unroll
      for (int r = 0; r < 8; ++r) acc8[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      wait_all();
      for (;;) {
        cur.n = (int)rfl((uint32_t)cur.n);
        cur.flags = (int)rfl((uint32_t)cur.flags);
        cur.i0 = (int)rfl((uint32_t)cur.i0);
        asm volatile("" : "+s"(cur.n), "+s"(cur.flags), "+s"(cur.i0));
        const Params& P = fresh_params();
        if (prof && t_first == 0) t_first = rfl((uint32_t)wall_clock64());
        waits_count(wt, 3, cur.n);
        const Blk nxt = next_block_m<RING>(P, cx, s, W);
        asm volatile("" : : "v"(xa[0][0]), "v"(xa[0][1]), "v"(xa[0][2]), "v"(xa[0][3]));
        bf16x8 h0, l0, h1, l1;
        {
          const uint32_t ga = C.xp.gl + (uint32_t)C.col * C.xp.gstep;
          const u32x4 g0 = lds_ld16(ga), g1 = lds_ld16(ga + C.xp.gstep / 2u);
          split8(xa[0][0], xa[0][1], g0, h0, l0);
          split8(xa[0][2], xa[0][3], g1, h1, l1);
        }
        load_x(P, cx, C.xp, C.col + 1, C.col + 1 < C.c1, xa[1]);
        C.any = true;
#pragma unroll
        for (int j = 0; j < RING; ++j) {
          asm volatile("" : : "v"(ra[j]), "v"(rb[j]));
          if (j < C.cm) {
            const bf16x8 b0 = __builtin_bit_cast(bf16x8, ra[j]), b1 = __builtin_bit_cast(bf16x8, rb[j]);
            acc8[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, b0, acc8[j], 0, 0, 0);
            acc8[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l0, b0, acc8[j], 0, 0, 0);
            acc8[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, b1, acc8[j], 0, 0, 0);
            acc8[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l1, b1, acc8[j], 0, 0, 0);
          }
          load_item_m(P, cx, W.pm, nxt.i0 + j, j < nxt.n, ra[j], rb[j]);
          __builtin_amdgcn_sched_barrier(0);
        }
        ++C.col;
        const bool last = (cur.flags & kLast) != 0;
        cur = nxt;
        if (last) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) xa[0][e] = xa[1][e];
      }
      // the sums of every row block of the task
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < C.cm) tile_flush(acc8[r], C.tiles, r, lane);
      fin = true;
      continue;
    }
    {
      // the task's activations exist now: its first XR items' (column pairs
      // col0, col0 + 1, ... modulo KB2)
      const Params& P = fresh_params();
      int xc = C.xp.col0;
#pragma unroll
      for (int j = 0; j < XR; ++j) {
        load_x(P, cx, C.xp, xc, j < C.xp.n, xa[j]);
        xc = xc + 1 == C.xp.KB2 ? 0 : xc + 1;
      }
      wait_all();
    }
    for (;;) {
      cur.n = (int)rfl((uint32_t)cur.n);
      cur.flags = (int)rfl((uint32_t)cur.flags);
      cur.i0 = (int)rfl((uint32_t)cur.i0);
      asm volatile("" : "+s"(cur.n), "+s"(cur.flags), "+s"(cur.i0));  // opaque: no peeled first pass
      const Params& P = fresh_params();
      if (prof && t_first == 0) t_first = rfl((uint32_t)wall_clock64());
      waits_count(wt, 3, cur.n);
      const Blk nxt = next_block_m<RING>(P, cx, s, W);
      // column pair of piece item cur.i0 + XR, advanced one item per slot
      int xc = (int)rfl((uint32_t)((C.xp.col0 + cur.i0 + XR) % C.xp.KB2));
#pragma unroll
      for (int j = 0; j < RING; ++j) {
        asm volatile("" : : "v"(ra[j]), "v"(rb[j]), "v"(xa[j % XR][0]), "v"(xa[j % XR][1]), "v"(xa[j % XR][2]),
                     "v"(xa[j % XR][3]));
        if (j < cur.n) {
          C.any = true;
          mf_item(C, acc, ra[j], rb[j], xa[j % XR], lane);
        }
        // activations XR items on, within this piece
        const int t = cur.i0 + j + XR;
        load_x(P, cx, C.xp, xc, t < C.xp.n, xa[j % XR]);
        xc = xc + 1 == C.xp.KB2 ? 0 : xc + 1;
        load_item_m(P, cx, W.pm, nxt.i0 + j, j < nxt.n, ra[j], rb[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool last = (cur.flags & kLast) != 0;
      cur = nxt;
      if (last) break;
    }
    fin = true;
  }
  wait_all();
  waits_put(P, cx, wt);
}
