// Stream waves of the persistent decode megakernel (included by kernels.hip;
// internal to libmk).
//
// Every streamed task (a matvec over packed weight units, or attention over a
// chunk of the KV cache) is cut into kStreams contiguous pieces, one per
// stream wave. A piece is a run of 2 KiB items: two weight units of one row
// block (column blocks 2j and 2j+1; the packing makes the number of column
// blocks even), or the K block and the V block of one group of positions.
//
// A stream wave loads its weight items straight into registers. A ring of
// RING items (two 16-byte loads per lane each) stays in flight, and the loads
// run ahead across task and event boundaries, so weights keep arriving while
// the workgroup waits on an event. The ring is one fully unrolled pass over
// its RING register slots: at slot s the wave computes on the item the slot
// holds, then refills the slot with the item RING places further on. Every
// pass issues exactly two loads per slot, in slot order, so the compiler's
// wait before each use is the exact count: the loads of the RING - 1 younger
// items stay in flight. (Measured on one MI355X: about 7 TB/s over 256
// compute units with four such waves each, against 5.7 TB/s for four waves
// copying into LDS rings.)
//
// Matvec pieces are walked in blocks of RING items; the last block of a piece
// is filled up with loads of a zero block. Task changes therefore fall between
// passes: one copy of the task-change code, outside the unrolled pass. The
// block loaded in one pass is computed in the next.
//
// Attention pieces are not in the ring: when the compute cursor reaches an
// attention task, the wave runs it in the task-change path with a ring of its
// own (kAttRing items) over the chunk's KV entries, while the weight ring's
// loads stay in flight. The task has been staged, so its step is open; the
// streamed positions are below p - 1 (the stager supplies p - 1 and p), and
// those were appended two or more steps back: every task of a step waits,
// through its events, for the whole step before.

constexpr int kItemBytes = 2 * kUnitBytes;

__device__ __forceinline__ uint32_t rfl(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// [a0, a1): piece s of n things cut into kStreams contiguous pieces. The
// vector bodies (W) give stream waves 0 and 1 (waves 2 and 3, a SIMD each)
// 67/256 of the things each and stream waves 2 and 3 (waves 4 and 5, which
// share their SIMDs with the stager and the retirer) 61/256 each: measured on
// the 1B shape, equal quarters left waves 4 and 5 finishing 0.1-0.4 us after
// the others on every matvec (879.5 -> 868.4 us/token with the weighted cut).
// The matrix-core bodies keep equal quarters (the weighted cut measured
// slower there). The host computes the same cut (api.cpp).
template <bool W = true>
__device__ __forceinline__ void piece(int n, int s, int& a0, int& a1) {
  if constexpr (W) {
    const uint32_t c0 = s == 0 ? 0u : s == 1 ? 67u : s == 2 ? 134u : 195u;
    const uint32_t c1 = s == 0 ? 67u : s == 1 ? 134u : s == 2 ? 195u : 256u;
    a0 = (int)(((uint32_t)n * c0) >> 8);
    a1 = (int)(((uint32_t)n * c1) >> 8);
  } else {
    a0 = (int)((uint32_t)n * (uint32_t)s / kStreams);
    a1 = (int)((uint32_t)n * (uint32_t)(s + 1) / kStreams);
  }
}

// ---------------------------------------------------------------------------
// pieces and blocks
// ---------------------------------------------------------------------------

// Wave s's piece of one stream record at one step: its item count and where
// item i lives. Both kinds are read through buffer resources: weights from
// one resource (the item's two units are 1 KiB apart), attention from the K
// rows and the V rows of its (layer, sequence, kv group).
struct Piece {
  int n;                 // items
  bool kv;
  rsrc_t ra, rb;         // resources of an item's first and second unit
  int kpos, ppi, last;   // attention: this lane's position in item 0; positions per item; last streamed position
  uint32_t lane_off;     // this lane's byte offset within a unit (weights) or a position's row (attention)
};

__device__ __forceinline__ rsrc_t zero_rsrc(const Params& P, const Ctx& cx) {
  return make_rsrc(P.zeros + (size_t)rfl((uint32_t)cx.cu & (kZeroBlocks - 1)) * 2 * kUnitBytes, 2 * kUnitBytes);
}

// Wave s's piece of a matvec record (an attention record has no ring items).
template <bool W = true>
__device__ __forceinline__ Piece make_piece(const Params& P, const Ctx& cx, int s, int r) {
  Piece pc;
  pc.n = 0;
  pc.kv = false;
  pc.ra = pc.rb = zero_rsrc(P, cx);
  pc.kpos = 0;
  pc.ppi = 1;
  pc.last = 0;
  pc.lane_off = (uint32_t)cx.lane * 16u;
  const StreamRec R = cx.recs[r];
  const uint32_t tsbg = rfl(R.tsbg);
  if ((tsbg & 15) == T_ATT) return pc;
  const int items = (int)rfl((uint32_t)R.n_units) / 2;
  int i0, i1;
  piece<W>(items, s, i0, i1);
  pc.n = i1 - i0;
  const int64_t woff =
      (int64_t)(((uint64_t)rfl((uint32_t)((uint64_t)R.w_off >> 32)) << 32) | rfl((uint32_t)R.w_off));
  pc.ra = pc.rb = make_rsrc(P.wpack + woff + (int64_t)i0 * kItemBytes, (uint32_t)pc.n * (uint32_t)kItemBytes);
  return pc;
}

// Wave s's piece of attention task (layer, b, g, chunk) for a sequence at
// position p: `n` blocks of ppi positions from lo + u0 * ppi, the last
// streamed position `last`.
__device__ __forceinline__ Piece make_kv_piece(const Params& P, const Ctx& cx, int layer, int b, int g, int lo, int end,
                                               int u0, int n) {
  Piece pc;
  const int lpp = P.D / 8;
  pc.n = n;
  pc.kv = true;
  pc.ppi = 64 / lpp;
  pc.kpos = lo + u0 * pc.ppi + cx.lane / lpp;
  pc.last = end - 1;
  pc.lane_off = (uint32_t)(cx.lane % lpp) * 16u;
  const size_t row = (((size_t)layer * P.B + b) * P.Hkv + g) * (size_t)P.S * P.D;
  pc.ra = make_rsrc(P.kcache + row, (uint32_t)P.S * (uint32_t)P.D * 2u);
  pc.rb = make_rsrc(P.vcache + row, (uint32_t)P.S * (uint32_t)P.D * 2u);
  return pc;
}

// The same piece computed from an attention record and the call's positions,
// before the task is staged (the staged header gives the same bounds).
template <bool W = true>
__device__ __forceinline__ Piece kv_piece_of(const Params& P, const Ctx& cx, int s, int r, int step) {
  const StreamRec R = cx.recs[r];
  const uint32_t tsbg = rfl(R.tsbg), lc = rfl(R.lc);
  const int b = (tsbg >> 6) & 1023, g = tsbg >> 16, layer = lc & 0xffff, chunk = lc >> 16;
  const int pos = b < P.batch ? call_pos(P, b, step) : -1;
  int lo = 0, end = 0, j0 = 0, j1 = 0;
  if (pos >= 0 && pos < P.S) {
    att_stream_range(P, chunk, pos, lo, end);
    const int ppi = 64 / (P.D / 8);
    piece<W>(end > lo ? (end - lo + ppi - 1) / ppi : 0, s, j0, j1);
  }
  return make_kv_piece(P, cx, layer, b < P.batch ? kv_row_b(P, b) : 0, g, lo, end, j0, j1 - j0);
}

// A block: up to RING consecutive items of one piece.
struct Blk {
  int r, step;  // stream record and step
  int n;        // real items (0: a null block, nothing to compute)
  int i0;       // its first item's index in the piece
  int flags;    // kFirst, kLast, kEnd
};
enum { kFirst = 1, kLast = 2, kEnd = 4 };

// The walk over this wave's pieces, in queue order, step by step (empty
// pieces skipped).
struct Walk {
  int r, step, t;  // current piece, next item in it
  Piece pc;
};

// Loads of item i of piece pc into one ring slot (a zero item when !real):
// always the same two non-temporal loads (every byte is read once per step);
// only the resources and offsets differ, selected without a branch, so the
// compiler sees one instruction sequence per slot. Zero items read this
// compute unit's own 2 KiB of zeros (they stay in its L2).
//
// KV entries need no device-coherent load: within a launch an entry is read
// only in steps after the one that appended it (the streamed positions are
// below p - 1), each position's row fills whole 128-byte lines of its own, so
// no cache can hold a line of it from before the append; and kernel
// boundaries write back and invalidate the caches.
__device__ __forceinline__ void load_item(const Params& P, const Ctx& cx, const Piece& pc, int i, bool real, u32x4& a,
                                          u32x4& b) {
  const rsrc_t z = make_rsrc(P.zeros + (size_t)rfl((uint32_t)cx.cu & (kZeroBlocks - 1)) * 2 * kUnitBytes, 2 * kUnitBytes);
  const bool kv = real && pc.kv;
  const uint32_t koff = (uint32_t)min(pc.kpos + i * pc.ppi, pc.last) * (uint32_t)P.D * 2u + pc.lane_off;
  const uint32_t woff = (uint32_t)i * (uint32_t)kItemBytes + pc.lane_off;
  const uint32_t offa = kv ? koff : real ? woff : (uint32_t)cx.lane * 16u;
  const uint32_t offb = kv ? koff : offa + kUnitBytes;
  const rsrc_t ra = real ? pc.ra : z;
  const rsrc_t rb = real ? pc.rb : z;
  a = __builtin_amdgcn_raw_buffer_load_b128(ra, offa, 0, kAuxStream);
  b = __builtin_amdgcn_raw_buffer_load_b128(rb, offb, 0, kAuxStream);
}

// The next block of the walk over this wave's matvec pieces (kEnd past the
// last step).
template <int RING>
__device__ __forceinline__ Blk next_block(const Params& P, const Ctx& cx, int s, Walk& W) {
  Blk B;
  B.i0 = 0;
  B.n = 0;
  if (W.t >= W.pc.n) {
    for (;;) {
      if (++W.r >= cx.nrec) {
        W.r = 0;
        ++W.step;
      }
      if (W.step >= P.n_steps || cx.nrec == 0) {
        B.r = W.r;
        B.step = W.step;
        B.flags = kEnd;
        W.pc.n = 0;
        W.t = 0;
        return B;
      }
      W.pc = make_piece(P, cx, s, W.r);
      W.t = 0;
      if (W.pc.n > 0) break;
    }
  }
  B.r = W.r;
  B.step = W.step;
  B.i0 = W.t;
  B.n = min(RING, W.pc.n - W.t);
  B.flags = (W.t == 0 ? kFirst : 0) | (W.t + B.n == W.pc.n ? kLast : 0);
  W.t += B.n;
  return B;
}

// ---------------------------------------------------------------------------
// compute
// ---------------------------------------------------------------------------

struct Comp {
  int r, step;     // stream record and step of the task being computed
  int slot, type;  // staging slot; type -1: none
  int rb, kb, KB;  // matvec: row block and column block of the next item, column blocks
  int rb0;         // matvec: first row block of this wave's piece (its partial sums start there)
  bool pend;       // matvec: sums of an unfinished row block are held
  bool any;        // the piece has items
  int lo, end, u0; // attention: streamed positions [lo, end) of the chunk, first block of this wave
  int natt;        // attention: blocks of this wave
  int layer, b, g; // attention: the task's layer, sequence and kv group
  float* part;     // partial sums (LDS)
  const float* hin;
  int kp;
};

template <int NC>
struct Acc {
  float a[NC];
};

// Dot product of 8 bf16 weights (packed in w) with 8 activations.
__device__ __forceinline__ float dot8(const u32x4 w, const float4 x, const float4 y) {
  float a = __uint_as_float(w.x << 16) * x.x;
  a = fmaf(__uint_as_float(w.x & 0xffff0000u), x.y, a);
  a = fmaf(__uint_as_float(w.y << 16), x.z, a);
  a = fmaf(__uint_as_float(w.y & 0xffff0000u), x.w, a);
  float b = __uint_as_float(w.z << 16) * y.x;
  b = fmaf(__uint_as_float(w.z & 0xffff0000u), y.y, b);
  b = fmaf(__uint_as_float(w.w << 16), y.z, b);
  b = fmaf(__uint_as_float(w.w & 0xffff0000u), y.w, b);
  return a + b;
}

// The row sums of row block rb (counted from the piece's first), reduced over
// the 16 lanes of each row, as this wave's partial sums. Every lane of row j
// holds the sum and all of them store it to row j's word (no lane-dependent
// branch).
template <int NC>
__device__ __forceinline__ void mv_flush(Acc<NC>& A, float* pout, int cs, int rb) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    pout[c * cs + rb * 4] = sum16(A.a[c]);
    A.a[c] = 0.f;
  }
}

// Attention state of one wave over its piece: for G query heads, this lane's 8
// dims of the output accumulator, and the running maximum and denominator of
// this lane's position group (the lanes that share a position). The groups are
// merged once, at the end of the piece. The scaled queries are read from the
// staging slot (qs, this lane's 8 dims at de).
struct AttState {
  float acc[kMaxG][8], m[kMaxG], l[kMaxG];
  const float* qs;
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reduce over the position groups of a wave (lanes equal modulo lpp, which is
// 8 or 16; l16: lpp is 16): max or sum.
template <bool MAX>
__device__ __forceinline__ float across_groups(float v, bool l16) {
  float lo, hi;
  xpair<8>(v, lo, hi);
  v = l16 ? v : (MAX ? fmaxf(lo, hi) : lo + hi);
  xpair<16>(v, lo, hi);
  v = MAX ? fmaxf(lo, hi) : lo + hi;
  xpair<32>(v, lo, hi);
  return MAX ? fmaxf(lo, hi) : lo + hi;
}

// Two items (position blocks) of attention: for each of the G heads, the
// scores of this lane's two positions, then one online-softmax update of its
// group's running maximum, denominator and weighted values for both (one
// rescale per pair of items). Scores are in base-2 units (the queries carry
// scale * log2(e)), so the exponentials are the hardware's exp2. The heads'
// dot products and lane-group sums are computed side by side, so the
// cross-lane steps of different heads overlap. q: this lane's 8 dims of each
// head's scaled query, read from the staging slot once per task (load_q) and
// held in registers.
__device__ __forceinline__ void load_q(const Params& P, const AttState& S, float (&q)[kMaxG][8]) {
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    const float4 a = h < P.G ? ld_f4(S.qs + h * P.D) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 b = h < P.G ? ld_f4(S.qs + h * P.D + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[h][0] = a.x; q[h][1] = a.y; q[h][2] = a.z; q[h][3] = a.w;
    q[h][4] = b.x; q[h][5] = b.y; q[h][6] = b.z; q[h][7] = b.w;
  }
}
__device__ __forceinline__ void att_pair(const Params& P, AttState& S, const float (&q)[kMaxG][8], const u32x4 k0,
                                         const u32x4 v0, const u32x4 k1, const u32x4 v1, bool valid0, bool valid1,
                                         bool l16) {
  float kf0[8], kf1[8];
  unpack8(k0, kf0);
  unpack8(k1, kf1);
  float s0[kMaxG], s1[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      d0 = fmaf(q[h][e], kf0[e], d0);
      d1 = fmaf(q[h][e], kf1[e], d1);
    }
    s0[h] = d0;
    s1[h] = d1;
  }
  // sums over the lanes of a position group, all heads at each step
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) { s0[h] += dpp<kDppSwap1>(s0[h]); s1[h] += dpp<kDppSwap1>(s1[h]); }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) { s0[h] += dpp<kDppSwap2>(s0[h]); s1[h] += dpp<kDppSwap2>(s1[h]); }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) { s0[h] += dpp<kDppHalfMirror>(s0[h]); s1[h] += dpp<kDppHalfMirror>(s1[h]); }
  if (l16) {
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) { s0[h] += dpp<kDppMirror>(s0[h]); s1[h] += dpp<kDppMirror>(s1[h]); }
  }
  float vf0[8], vf1[8];
  unpack8(v0, vf0);
  unpack8(v1, vf1);
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < P.G) {
      const float a = valid0 ? s0[h] : -INFINITY, b = valid1 ? s1[h] : -INFINITY;
      const float mn = fmaxf(S.m[h], fmaxf(a, b));
      const float al = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(S.m[h] - mn);
      const float p0 = valid0 ? __builtin_amdgcn_exp2f(a - mn) : 0.f;
      const float p1 = valid1 ? __builtin_amdgcn_exp2f(b - mn) : 0.f;
      S.l[h] = fmaf(S.l[h], al, p0 + p1);
#pragma unroll
      for (int e = 0; e < 8; ++e) S.acc[h][e] = fmaf(p1, vf1[e], fmaf(p0, vf0[e], S.acc[h][e] * al));
      S.m[h] = mn;
    }
  }
}

// End of a wave's attention piece: merge the position groups (with M the
// largest group maximum, each group's denominator and values scaled by
// 2^(m_g - M) and added over the groups) and store this wave's partial: acc[D]
// of each head (at [wave][head]), then (m, l) of each head (at [wave][head]
// after all the accumulators), m in natural-log units. A piece without items
// stores m = -inf, l = 0 and zeros.
__device__ __forceinline__ void att_finish(const Params& P, AttState& S, float* part, int s, int lane, bool empty) {
  const bool l16 = P.D == 128;
  const int D = P.D, G = P.G, de = (lane % (l16 ? 16 : 8)) * 8;
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      float M = -INFINITY, l = 0.f;
      if (!empty) {
        M = across_groups<true>(S.m[h], l16);
        const float f = S.m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S.m[h] - M);
        l = across_groups<false>(S.l[h] * f, l16);
#pragma unroll
        for (int e = 0; e < 8; ++e) S.acc[h][e] = across_groups<false>(S.acc[h][e] * f, l16);
      }
      // every lane holds the sums of its dims (and the wave's m, l): lanes with
      // equal dims store equal values to the same words
      float* dst = part + (size_t)(s * G + h) * D;
      *reinterpret_cast<float4*>(dst + de) = make_float4(S.acc[h][0], S.acc[h][1], S.acc[h][2], S.acc[h][3]);
      *reinterpret_cast<float4*>(dst + de + 4) = make_float4(S.acc[h][4], S.acc[h][5], S.acc[h][6], S.acc[h][7]);
      float* ml = part + (size_t)kStreams * G * D + (s * G + h) * 2;
      ml[0] = M * kLn2;
      ml[1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// stream wave
// ---------------------------------------------------------------------------

// Start computing record r at `step`: wait for its staging, then set up the
// matvec cursor or the attention state.
template <int NC, bool PROF>
__device__ __forceinline__ bool comp_start(const Params& P, const Ctx& cx, int s, Comp& C, Acc<NC>& A, AttState& S,
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
  C.hin = slot_ptr(cx, C.slot) + kHdr;
  if (C.type == T_ATT) {
    C.part = att_part_ptr(P, cx, C.slot);
    const int* ih = reinterpret_cast<const int*>(slot_ptr(cx, C.slot));
    const int flags = lds_ld(&ih[H_FLAGS]);
    C.lo = lds_ld(&ih[H_LO]);
    C.end = lds_ld(&ih[H_END]);
    const int lpp = P.D / 8, ppi = 64 / lpp;
    const int nb = (flags & 1) && C.end > C.lo ? (C.end - C.lo + ppi - 1) / ppi : 0;
    int j1;
    piece(nb, s, C.u0, j1);
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
    C.part = part_ptr(cx, C.slot) + (size_t)s * P.ncap * P.wave_vrows + (lane >> 4);
    const int items = (int)rfl((uint32_t)R.n_units) / 2;
    int i0, i1;
    piece(items, s, i0, i1);
    C.KB = kq & 0xffff;
    C.rb = (2 * i0) / C.KB;
    C.rb0 = C.rb;
    C.kb = 2 * i0 - C.rb * C.KB;
    C.pend = false;
    C.kp = slot_kp(P, C.slot);
#pragma unroll
    for (int c = 0; c < NC; ++c) A.a[c] = 0.f;
  }
  C.any = false;
  return true;
}

// Finish the task being computed: store this wave's partials (and the row
// blocks they cover) and count the wave done.
template <int NC>
__device__ __forceinline__ void comp_finish(const Params& P, const Ctx& cx, int s, Comp& C, Acc<NC>& A, AttState& S,
                                            bool prof, uint32_t t_first) {
  if (C.type == T_ATT) {
    att_finish(P, S, C.part, s, cx.lane, !C.any);
  } else {
    if (C.pend) mv_flush<NC>(A, C.part, P.wave_vrows, C.rb - C.rb0);
    // the row blocks this piece touched (b < a: none), for the retirer's sums
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

// One matvec item (weight units w0, w1 = column blocks kb, kb + 1 of row block
// rb) against the staged activations of NC columns.
template <int NC>
__device__ __forceinline__ void mv_item(const Params& P, Comp& C, Acc<NC>& A, const u32x4 w0, const u32x4 w1,
                                        int icol) {
  const float* h = C.hin + icol * 4 + C.kb * kUnitCols;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float* hc = h + c * C.kp;
    A.a[c] += dot8(w0, ld_f4(hc), ld_f4(hc + 64)) + dot8(w1, ld_f4(hc + kUnitCols), ld_f4(hc + kUnitCols + 64));
  }
  C.kb += 2;
  C.pend = true;
  if (C.kb == C.KB) {
    mv_flush<NC>(A, C.part, P.wave_vrows, C.rb - C.rb0);
    C.kb = 0;
    ++C.rb;
    C.pend = false;
  }
}

// An attention task's piece: the chunk's streamed KV blocks of this wave,
// through a ring of kAttRing register slots (the same unrolled pass as the
// weight ring: compute the slot's block, then refill the slot). The first
// kAttRing blocks are loaded before the task is staged (att_prefetch): the
// step is open by then, since this compute unit's previous task was staged.
#ifndef MK_ATT_RING
#define MK_ATT_RING 8
#endif
constexpr int kAttRing = MK_ATT_RING;
template <int AR>
__device__ __forceinline__ void att_prefetch(const Params& P, const Ctx& cx, const Piece& pc, u32x4 (&ka)[AR],
                                             u32x4 (&kv)[AR]) {
#pragma unroll
  for (int j = 0; j < AR; ++j) {
    load_item(P, cx, pc, j, j < pc.n, ka[j], kv[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
}
template <int AR>
__device__ __forceinline__ void att_run(const Params& P, const Ctx& cx, Comp& C, AttState& S, const Piece& pc,
                                        u32x4 (&ka)[AR], u32x4 (&kv)[AR]) {
  static_assert(AR % 2 == 0, "attention items are computed in pairs");
  const int lane = cx.lane, lpp = P.D / 8, ppi = 64 / lpp;
  const bool l16 = lpp == 16;
  // this lane's 8 dims of each head's scaled query, for the whole task
  float q[kMaxG][8];
  load_q(P, S, q);
  int cn = min(AR, pc.n), cbase = 0, base = AR;  // blocks computed in this pass, their first; next to load
  for (;;) {
    cn = (int)rfl((uint32_t)cn);
    asm volatile("" : "+s"(cn));  // opaque: no peeled first pass
    const int ln = min(AR, max(0, pc.n - base));
#pragma unroll
    for (int j = 0; j < AR; j += 2) {
      asm volatile("" : : "v"(ka[j]), "v"(kv[j]), "v"(ka[j + 1]), "v"(kv[j + 1]));
      if (j < cn) {
        const int pos0 = C.lo + (C.u0 + cbase + j) * ppi + lane / lpp;
        att_pair(P, S, q, ka[j], kv[j], ka[j + 1], kv[j + 1], pos0 < C.end, j + 1 < cn && pos0 + ppi < C.end,
                       l16);
      }
      load_item(P, cx, pc, base + j, j < ln, ka[j], kv[j]);
      load_item(P, cx, pc, base + j + 1, j + 1 < ln, ka[j + 1], kv[j + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ln == 0) break;
    cbase = base;
    cn = ln;
    base += AR;
  }
  // The last pass's zero loads are left in flight: waiting for them here would
  // also wait for every older load, the weight ring's included, and the task
  // is done without them (the compiler waits before their registers are
  // reused).
  C.any = pc.n > 0;
}

template <int RING, int NC, bool PROF>
__device__ __forceinline__ void run_stream(const Params& P0, const Ctx& cx, int s) {
  const Params& P = P0;
  const int lane = cx.lane, icol = lane & 15;
  const bool prof = PROF && P.profile != nullptr;
  Waits wt;  // j2: task not staged; j3: items
  waits_init<PROF>(P, cx, wt);

  Walk W;
  W.r = -1;
  W.step = 0;
  W.t = 0;
  W.pc = make_piece(P, cx, s, 0);
  W.pc.n = 0;

  Comp C;
  C.r = -1;
  C.step = 0;
  C.type = -1;
  C.slot = 0;
  C.any = false;
  Acc<NC> A;
#pragma unroll
  for (int c = 0; c < NC; ++c) A.a[c] = 0.f;
  AttState S;
  uint32_t t_first = 0;

  u32x4 ra[RING], rb[RING];
#pragma unroll
  for (int j = 0; j < RING; ++j) ra[j] = rb[j] = u32x4{0u, 0u, 0u, 0u};

  bool fin = false;  // the task being computed has had all its items: finish it
  Blk cur;           // the block the ring holds, computed in this pass (none in the first pass)
  cur.r = 0;
  cur.step = 0;
  cur.n = 0;
  cur.i0 = 0;
  cur.flags = 0;
  for (;;) {
    cur.n = (int)rfl((uint32_t)cur.n);
    cur.flags = (int)rfl((uint32_t)cur.flags);
    asm volatile("" : "+s"(cur.n), "+s"(cur.flags));  // opaque: no peeled first pass (it would load in another order)
    const Params& P = fresh_params();
    if (fin || (cur.flags & (kFirst | kEnd))) {
      // The compute cursor's task changes, all here (one copy of the code):
      // finish the task whose items are done; walk the records up to this
      // block's piece (and start it) or to the end. Records on the way have no
      // ring items for this wave: attention tasks run here, matvec pieces
      // without items are started and finished at once (the retirer waits for
      // every stream wave on every stream task).
      for (;;) {
        if (fin) {
          comp_finish<NC>(P, cx, s, C, A, S, prof, t_first);
          fin = false;
        }
        if (C.type >= 0) break;
        int r = C.r + 1, st = C.step;
        if (r >= cx.nrec) {
          r = 0;
          ++st;
        }
        if (st >= P.n_steps || cx.nrec == 0) break;
        const bool at = r == cur.r && st == cur.step;
        C.r = r;
        C.step = st;
        // an attention task: its first KV blocks load while it is staged
        const bool att = !at && (rfl(cx.recs[r].tsbg) & 15) == T_ATT;
        Piece kpc;
        u32x4 ka[kAttRing], kv[kAttRing];
        if (att) {
          kpc = kv_piece_of(P, cx, s, r, st);
          att_prefetch(P, cx, kpc, ka, kv);
        }
        if (!comp_start<NC, PROF>(P, cx, s, C, A, S, wt, prof)) return;
        t_first = 0;
        if (at) break;
        if (att) {
          if (prof) t_first = rfl((uint32_t)wall_clock64());
          att_run(P, cx, C, S, kpc, ka, kv);
        }
        fin = true;
      }
      if (cur.flags & kEnd) break;
    }
    if (prof && t_first == 0 && cur.n > 0) t_first = rfl((uint32_t)wall_clock64());
    waits_count(wt, 3, cur.n);
    // the block to load in this pass
    const Blk nxt = next_block<RING>(P, cx, s, W);
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      // every slot's item is waited for at its position, computed or not (a
      // padding item): its registers are then free, and no later write to them
      // has to wait for a load still in flight
      asm volatile("" : : "v"(ra[j]), "v"(rb[j]));
      if (j < cur.n) {
        C.any = true;
        mv_item<NC>(P, C, A, ra[j], rb[j], icol);
      }
      load_item(P, cx, W.pc, nxt.i0 + j, j < nxt.n, ra[j], rb[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (cur.flags & kLast) fin = true;
    cur = nxt;
  }
  wait_all();
  waits_put(P, cx, wt);
}
