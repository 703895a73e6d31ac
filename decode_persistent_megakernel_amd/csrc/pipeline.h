// Stream waves of the persistent decode megakernel (included by kernels.hip;
// internal to libmk).
//
// Every streamed task (a matvec over packed weight units, or attention over a
// chunk of the KV cache) is cut into kStreams contiguous pieces, one per
// stream wave. A piece is a run of 2 KiB items: two weight units of one row
// block (column blocks 2j and 2j+1; the packing makes the number of column
// blocks even), or the K block and the V block of one group of positions.
//
// A stream wave feeds itself: it copies its items from HBM straight into a
// private LDS ring of DEPTH slots (LDS DMA), DEPTH items ahead of the one it
// computes, running ahead across task boundaries so weights keep arriving
// while the workgroup waits on an event. Copies complete in issue order, so
// "item k has landed" is a wait for the vector-memory counter to drop to twice
// the number of younger items; the wave issues no other vector-memory
// operation while it streams. The copies are inline assembly: the compiler
// then leaves the wave's own LDS reads alone (it would otherwise wait for
// every copy in flight before each of them, not knowing which LDS bytes a copy
// writes).
//
// The wave is one loop over items with two cursors over the same task list:
// the copy cursor (ahead) and the compute cursor. Each cursor's task change is
// a single, rarely taken path and the per-item work is straight-line code, so
// the role stays small in the instruction cache and light on registers.
//
// Attention items of a step read KV entries appended in earlier steps, so
// they are copied only after the stager has passed the step's first
// dependency (C_STEPOK); weight items never wait for anything but a free slot.

// ---------------------------------------------------------------------------
// copies
// ---------------------------------------------------------------------------

// 1 KiB per wave: lane l copies 16 bytes from its own address src into LDS
// byte address lds + 16*l (lds is wave-uniform; it goes in M0, which this
// wave's code uses for nothing else). nt: streamed once; sc1: device-coherent.
__device__ __forceinline__ void copy_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void copy_sc1(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1" : : "v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

__device__ __forceinline__ u32x4 ld_u32x4(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N): vmcnt bits [3:0] and [15:14], expcnt/lgkmcnt at max
  constexpr int imm = (N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Wait until the item with `younger` items issued after it has landed: at most
// 2*younger copies may still be in flight. Counts below the steady state
// round down (a longer wait, never a shorter one).
template <int DEPTH>
__device__ __forceinline__ void wait_item(int younger) {
  cbar();
  if (younger >= DEPTH - 1) wait_vmcnt<2 * (DEPTH - 1)>();
  else if (younger >= DEPTH - 2) wait_vmcnt<2 * (DEPTH - 2)>();
  else if (younger >= DEPTH / 2) wait_vmcnt<2 * (DEPTH / 2)>();
  else if (younger >= 2) wait_vmcnt<4>();
  else if (younger == 1) wait_vmcnt<2>();
  else wait_vmcnt<0>();
  cbar();
}

__device__ __forceinline__ uint32_t rfl(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// [a0, a1): piece s of n things cut into kStreams nearly equal contiguous pieces
__device__ __forceinline__ void piece(int n, int s, int& a0, int& a1) {
  a0 = (int)((uint32_t)n * (uint32_t)s / kStreams);
  a1 = (int)((uint32_t)n * (uint32_t)(s + 1) / kStreams);
}

constexpr int kItemBytes = 2 * kUnitBytes;

// ---------------------------------------------------------------------------
// the copy cursor
// ---------------------------------------------------------------------------

struct Fetch {
  int r, step;        // stream record and step of the task being copied
  int t, n;           // next item of this wave in the task, and its item count
  bool kv, done;
  int pos0, last;     // attention: this lane's position in the piece's first block; last cached position
  int ppi;            // attention: positions per item
  const uint8_t* src; // matvec: this lane's 16 bytes of the next item; attention: the (layer, b, g) K rows
  int issued;         // items copied so far (all tasks)
  uint32_t soff;      // ring byte offset of the slot of item `issued`
};

// Ring slots are visited in order: the next slot's byte offset.
template <int DEPTH>
__device__ __forceinline__ uint32_t next_slot_off(uint32_t off) {
  off += kItemBytes;
  return off == (uint32_t)DEPTH * kItemBytes ? 0u : off;
}

// Move to the next task (in queue order, across steps) that has items for
// wave s. A matvec piece is whole items; an attention piece is a run of
// position blocks of the chunk's cached positions [lo, end).
__device__ __forceinline__ void fetch_next_task(const Params& P, const Ctx& cx, int s, Fetch& F) {
  F.t = 0;
  F.n = 0;
  for (;;) {
    if (++F.r >= cx.nrec) {
      F.r = 0;
      ++F.step;
    }
    if (F.step >= P.n_steps || cx.nrec == 0) {
      F.done = true;
      return;
    }
    const StreamRec R = cx.recs[F.r];
    const uint32_t tsbg = rfl(R.tsbg);
    F.kv = (tsbg & 15) == T_ATT;
    if (F.kv) {
      const int b = (tsbg >> 6) & 1023;
      if (b >= P.batch) continue;
      const int pos = ld_uniform(P.pos_in, b) + F.step;
      if (pos < 0 || pos >= P.S) continue;
      const uint32_t lc = rfl(R.lc);
      const int layer = lc & 0xffff, chunk = lc >> 16, g = tsbg >> 16;
      const int64_t len = (int64_t)pos + 1;
      const int lo = chunk_bound(chunk, len, P.Nc);
      const int end = min(chunk_bound(chunk + 1, len, P.Nc), pos);
      const int lpp = P.D / 8;
      F.ppi = 64 / lpp;
      const int nb = end > lo ? (end - lo + F.ppi - 1) / F.ppi : 0;
      int j0, j1;
      piece(nb, s, j0, j1);
      F.n = j1 - j0;
      F.pos0 = lo + j0 * F.ppi + cx.lane / lpp;
      F.last = end - 1;
      F.src = reinterpret_cast<const uint8_t*>(P.kcache + (((size_t)layer * P.B + b) * P.Hkv + g) * (size_t)P.S * P.D) +
              (cx.lane % lpp) * 16;
    } else {
      const int items = (int)rfl((uint32_t)R.n_units) / 2;
      int i0, i1;
      piece(items, s, i0, i1);
      F.n = i1 - i0;
      const int64_t woff =
          (int64_t)(((uint64_t)rfl((uint32_t)((uint64_t)R.w_off >> 32)) << 32) | rfl((uint32_t)R.w_off));
      F.src = P.wpack + woff + (int64_t)i0 * kItemBytes + cx.lane * 16;
    }
    if (F.n > 0) return;
  }
}

// Copy items until `limit` have been issued, the task sequence ends, or the
// next item is a KV block of a step the stager has not opened yet.
template <int DEPTH>
__device__ __forceinline__ void fetch_upto(const Params& P, const Ctx& cx, int s, Fetch& F, int limit,
                                           uint32_t ring) {
  while (F.issued < limit) {
    if (F.t == F.n) {
      fetch_next_task(P, cx, s, F);
      if (F.done) return;
    }
    const uint32_t dst = ring + F.soff;
    if (!F.kv) {
      copy_nt(F.src, dst);
      copy_nt(F.src + kUnitBytes, dst + kUnitBytes);
      F.src += kItemBytes;
    } else {
      if (F.t == 0 && lds_ld(&cx.ctl[C_STEPOK]) < F.step + 1) return;
      const int pos = min(F.pos0 + F.t * F.ppi, F.last);
      const uint8_t* kb = F.src + (size_t)pos * P.D * 2;
      copy_sc1(kb, dst);
      copy_sc1(kb + (reinterpret_cast<const uint8_t*>(P.vcache) - reinterpret_cast<const uint8_t*>(P.kcache)),
               dst + kUnitBytes);
    }
    ++F.issued;
    ++F.t;
    F.soff = next_slot_off<DEPTH>(F.soff);
  }
}

// ---------------------------------------------------------------------------
// compute
// ---------------------------------------------------------------------------

struct Comp {
  int r, step;     // stream record and step of the task being computed
  int slot, type;  // type -1: none
  int left;        // items of this wave left in the task
  int rb, kb, KB;  // matvec: row block and column block of the next item, column blocks
  int rb0;         // matvec: first row block of this wave's piece (its partial sums start there)
  int k0;          // items consumed before the task (profile)
  bool pend;       // matvec: sums of an unfinished row block are held
  int t, lo, end;  // attention: next block, cached positions [lo, end) of the chunk
  int u0;          // attention: first block of this wave
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 to_f4(const f32x4 v) { return make_float4(v.x, v.y, v.z, v.w); }

// One column's LDS operands of two items at once: both items' weight units and
// the activations of their column blocks, all twelve reads issued before one
// wait (inside the block, so no read is in flight when it ends). w: the items'
// slots (this lane's 16 bytes); ha, hb: the column blocks' activations (this
// lane's first float).
__device__ __forceinline__ void lds_two_items(uint32_t i0, uint32_t i1, uint32_t ha, uint32_t hb, u32x4 (&w)[4],
                                              f32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %13\n\t"
      "ds_read_b128 %3, %13 offset:1024\n\t"
      "ds_read_b128 %4, %14\n\t"
      "ds_read_b128 %5, %14 offset:256\n\t"
      "ds_read_b128 %6, %14 offset:512\n\t"
      "ds_read_b128 %7, %14 offset:768\n\t"
      "ds_read_b128 %8, %15\n\t"
      "ds_read_b128 %9, %15 offset:256\n\t"
      "ds_read_b128 %10, %15 offset:512\n\t"
      "ds_read_b128 %11, %15 offset:768\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
        "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(i0), "v"(i1), "v"(ha), "v"(hb)
      : "memory");
}

// The same for one item: its two weight units and its column blocks' activations.
__device__ __forceinline__ void lds_one_item(uint32_t i0, uint32_t ha, u32x4 (&w)[2], f32x4 (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:1024\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:256\n\t"
      "ds_read_b128 %4, %7 offset:512\n\t"
      "ds_read_b128 %5, %7 offset:768\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(i0), "v"(ha)
      : "memory");
}

// The row sums of row block rb (counted from the piece's first), reduced over
// the 16 lanes of each row, as this wave's partial sums. Every lane of row j holds the sum and all of them
// store it to row j's word: no lane-dependent branch in the stream loop (a
// divergent branch there would make the loop's own control divergent).
template <int NC>
__device__ __forceinline__ void mv_flush(Acc<NC>& A, float* pout, int cs, int rb, int icol) {
  (void)icol;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    pout[c * cs + rb * 4] = sum16(A.a[c]);
    A.a[c] = 0.f;
  }
}

// Attention state of one wave over its piece: G query heads, this lane's 8
// dims of the query and of the output accumulator, and the running maximum and
// denominator of this lane's position group (the lanes that share a
// position). The groups are merged once, at the end of the piece.
struct AttState {
  float q[kMaxG][8], acc[kMaxG][8], m[kMaxG], l[kMaxG];
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reduce over the position groups of a wave (lanes equal modulo lpp, which is
// 8 or 16; l16: lpp is 16): max or sum. One code path for both head widths
// keeps the kernel small.
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

// Sum over the lpp lanes of a position group.
__device__ __forceinline__ float in_group(float v, bool l16) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  const float w = v + dpp<kDppMirror>(v);
  return l16 ? w : v;
}

// One item (position block) of attention: for each of the G heads, the score
// of this lane's position, and the online-softmax update of its group's
// running maximum, denominator and weighted values. Scores are in base-2 units
// (the queries carry scale * log2(e)), so the exponentials are the hardware's
// exp2.
__device__ __forceinline__ void att_item(const Params& P, AttState& S, const u32x4 wk, const u32x4 wv, bool valid,
                                         bool l16) {
  float kf[8], vf[8];
  unpack8(wk, kf);
  unpack8(wv, vf);
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < P.G) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(S.q[h][e], kf[e], d);
      const float sc = valid ? in_group(d, l16) : -INFINITY;
      const float mn = fmaxf(S.m[h], sc);
      const float al = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(S.m[h] - mn);
      const float pe = valid ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
      S.l[h] = fmaf(S.l[h], al, pe);
#pragma unroll
      for (int e = 0; e < 8; ++e) S.acc[h][e] = fmaf(pe, vf[e], S.acc[h][e] * al);
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

// Items of a matvec piece, two at a time while both have been copied,
// refilling the ring from the same copy task; returns to the caller (which
// owns the slow paths) when the compute task ends, the next item is not copied
// yet, or the copy cursor reaches the end of its task. koff: ring byte offset
// of item k's slot.
template <int DEPTH, int NC>
__device__ __forceinline__ void matvec_run(const Params& P, Comp& C, Fetch& F, int& k, uint32_t& koff,
                                           uint32_t ring, const uint8_t* rp, const float* hin, int kp, float* pout,
                                           int icol, Acc<NC>& A, uint32_t& t_first, bool prof) {
  const int KB = C.KB;
  const float* h = hin + icol * 4;
  if (prof && t_first == 0 && F.issued > k) {
    wait_item<DEPTH>(F.issued - k - 1);
    t_first = rfl((uint32_t)wall_clock64());
  }
  for (;;) {
    const int ready = F.issued - k;
    if (ready >= 2 && C.left >= 2) {
      wait_item<DEPTH>(ready - 2);
      const uint32_t k1off = next_slot_off<DEPTH>(koff);
      const uint8_t* i0 = rp + koff;
      const uint8_t* i1 = rp + k1off;
      const int kb1 = C.kb + 2 == KB ? 0 : C.kb + 2;
      float d0[NC], d1[NC];
      if constexpr (NC == 1) {
        u32x4 w[4];
        f32x4 a[8];
        lds_two_items(lds_addr(i0), lds_addr(i1), lds_addr(h + C.kb * kUnitCols), lds_addr(h + kb1 * kUnitCols), w, a);
        d0[0] = dot8(w[0], to_f4(a[0]), to_f4(a[1])) + dot8(w[1], to_f4(a[2]), to_f4(a[3]));
        d1[0] = dot8(w[2], to_f4(a[4]), to_f4(a[5])) + dot8(w[3], to_f4(a[6]), to_f4(a[7]));
      } else {
        const u32x4 w0 = ld_u32x4(i0), w1 = ld_u32x4(i0 + kUnitBytes);
        const u32x4 w2 = ld_u32x4(i1), w3 = ld_u32x4(i1 + kUnitBytes);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float* ha = h + c * kp + C.kb * kUnitCols;
          const float* hb = h + c * kp + kb1 * kUnitCols;
          d0[c] = dot8(w0, ld_f4(ha), ld_f4(ha + 64)) + dot8(w1, ld_f4(ha + kUnitCols), ld_f4(ha + kUnitCols + 64));
          d1[c] = dot8(w2, ld_f4(hb), ld_f4(hb + 64)) + dot8(w3, ld_f4(hb + kUnitCols), ld_f4(hb + kUnitCols + 64));
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) A.a[c] += d0[c];
      C.kb += 2;
      if (C.kb == KB) {
        mv_flush<NC>(A, pout, P.wave_vrows, C.rb - C.rb0, icol);
        C.kb = 0;
        ++C.rb;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) A.a[c] += d1[c];
      C.kb += 2;
      C.pend = true;
      if (C.kb == KB) {
        mv_flush<NC>(A, pout, P.wave_vrows, C.rb - C.rb0, icol);
        C.kb = 0;
        ++C.rb;
        C.pend = false;
      }
      k += 2;
      koff = next_slot_off<DEPTH>(k1off);
      C.left -= 2;
      // steady state: the two slots just read take the copy task's next two items
      if (!F.kv && F.t + 2 <= F.n && F.issued + 2 <= k + DEPTH) {
        const uint32_t d0s = ring + F.soff;
        const uint32_t s1 = next_slot_off<DEPTH>(F.soff);
        const uint32_t d1s = ring + s1;
        copy_nt(F.src, d0s);
        copy_nt(F.src + kUnitBytes, d0s + kUnitBytes);
        copy_nt(F.src + kItemBytes, d1s);
        copy_nt(F.src + kItemBytes + kUnitBytes, d1s + kUnitBytes);
        F.src += 2 * kItemBytes;
        F.issued += 2;
        F.t += 2;
        F.soff = next_slot_off<DEPTH>(s1);
        continue;
      }
    } else if (ready >= 1 && C.left >= 1) {
      wait_item<DEPTH>(ready - 1);
      const uint8_t* i0 = rp + koff;
      if constexpr (NC == 1) {
        u32x4 w[2];
        f32x4 a[4];
        lds_one_item(lds_addr(i0), lds_addr(h + C.kb * kUnitCols), w, a);
        A.a[0] += dot8(w[0], to_f4(a[0]), to_f4(a[1])) + dot8(w[1], to_f4(a[2]), to_f4(a[3]));
      } else {
        const u32x4 w0 = ld_u32x4(i0), w1 = ld_u32x4(i0 + kUnitBytes);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float* ha = h + c * kp + C.kb * kUnitCols;
          A.a[c] += dot8(w0, ld_f4(ha), ld_f4(ha + 64)) + dot8(w1, ld_f4(ha + kUnitCols), ld_f4(ha + kUnitCols + 64));
        }
      }
      C.kb += 2;
      C.pend = true;
      if (C.kb == KB) {
        mv_flush<NC>(A, pout, P.wave_vrows, C.rb - C.rb0, icol);
        C.kb = 0;
        ++C.rb;
        C.pend = false;
      }
      k += 1;
      koff = next_slot_off<DEPTH>(koff);
      C.left -= 1;
    } else {
      return;
    }
    // refill the read slots from the current copy task (weights only)
    if (F.kv) return;
    while (F.issued < k + DEPTH && F.t < F.n) {
      const uint32_t dst = ring + F.soff;
      copy_nt(F.src, dst);
      copy_nt(F.src + kUnitBytes, dst + kUnitBytes);
      F.src += kItemBytes;
      ++F.issued;
      ++F.t;
      F.soff = next_slot_off<DEPTH>(F.soff);
    }
    if (C.left == 0 || F.issued < k + DEPTH) return;
  }
}

// ---------------------------------------------------------------------------
// stream wave
// ---------------------------------------------------------------------------

template <int DEPTH, int NC, bool PROF>
__device__ __forceinline__ void run_stream(const Params& P0, const Ctx& cx, int s) {
  const Params& P = P0;
  const int lane = cx.lane, jrow = lane >> 4, icol = lane & 15;
  const uint32_t ring = lds_addr(cx.ring) + (uint32_t)s * DEPTH * kItemBytes;
  const uint8_t* rp = cx.ring + (size_t)s * DEPTH * kItemBytes + lane * 16;  // this lane's bytes of slot 0
  const bool prof = PROF && P.profile != nullptr;
  const int lpp = P.D / 8, ppi = 64 / lpp;
  Waits wt;  // j0: KV step not open; j2: task not staged; j3: items
  waits_init<PROF>(P, cx, wt);

  Fetch F;
  F.r = -1;
  F.step = 0;
  F.t = F.n = 0;
  F.issued = 0;
  F.done = false;

  Comp C;
  C.r = -1;
  C.step = 0;
  C.left = 0;
  C.type = -1;
  C.slot = 0;
  int k = 0;  // items consumed
  const float* hin = nullptr;
  float* part = nullptr;
  int kp = 0;
  Acc<NC> A;
  AttState S;
  uint32_t t_first = 0;
  uint32_t koff = 0;  // ring byte offset of item k's slot
  F.soff = 0;

  for (;;) {
    const Params& P = fresh_params();
    // refill every slot whose item has been read
    wait_lgkm();
    fetch_upto<DEPTH>(P, cx, s, F, k + DEPTH, ring);

    if (C.left == 0) {
      // ---- the compute cursor's task change: finish the task, start the next
      if (C.type >= 0) {
        if (C.type == T_ATT) {
          att_finish(P, S, part, s, lane, C.t == 0);
        } else {
          if (C.pend) mv_flush<NC>(A, part + (size_t)s * P.ncap * P.wave_vrows + jrow, P.wave_vrows, C.rb - C.rb0, icol);
          // the row blocks this piece touched (b < a: none), for the retirer's sums
          int* pr = piece_words(cx, C.slot, s);
          pr[0] = C.rb0;
          pr[1] = C.k0 == k ? C.rb0 - 1 : (C.pend ? C.rb : C.rb - 1);
        }
        if (prof) {
          uint32_t* pw = prof_words(cx, C.slot, s);
          pw[1] = t_first;
          pw[2] = rfl((uint32_t)wall_clock64());
        }
        lds_add_lane0(&cx.ctl[C_DONE + ctl_slot(C.slot)], 1);
        C.type = -1;
      }
      if (++C.r >= cx.nrec) {
        C.r = 0;
        ++C.step;
      }
      if (C.step >= P.n_steps || cx.nrec == 0) break;
      const StreamRec R = cx.recs[C.r];
      const uint32_t tsbg = rfl(R.tsbg), kq = rfl(R.kq);
      C.type = tsbg & 15;
      C.slot = (tsbg >> 4) & 3;
      if (C.slot < 2) C.slot ^= (int)rfl((uint32_t)R.flip) & C.step;
      {
        const uint64_t s0 = waits_now(wt);
        if (!spin_ctl(P, cx, C_STAGED, C.step * (cx.q1 - cx.q0) + (int)(kq >> 16) + 1)) return;
        waits_add(wt, 2, s0);
      }
      t_first = 0;
      C.k0 = k;
      if (prof) prof_words(cx, C.slot, s)[0] = rfl((uint32_t)wall_clock64());
      hin = slot_ptr(cx, C.slot) + kHdr;
      part = C.type == T_ATT ? att_part_ptr(P, cx, C.slot) : part_ptr(cx, C.slot);
      if (C.type == T_ATT) {
        const int* ih = reinterpret_cast<const int*>(slot_ptr(cx, C.slot));
        const int flags = lds_ld(&ih[H_FLAGS]);
        C.lo = lds_ld(&ih[H_LO]);
        C.end = lds_ld(&ih[H_END]);
        const int nb = (flags & 1) && C.end > C.lo ? (C.end - C.lo + ppi - 1) / ppi : 0;
        int j1;
        piece(nb, s, C.u0, j1);
        C.left = j1 - C.u0;
        C.t = 0;
        const float* q = hin + att_raw_floats(P);
        const int de = (lane % lpp) * 8;
        const float qs = P.attn_scale * kLog2e;  // scores in base-2 units
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
          S.m[h] = -INFINITY;
          S.l[h] = 0.f;
          float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
          if (h < P.G) {
            x = ld_f4(q + h * P.D + de);
            y = ld_f4(q + h * P.D + de + 4);
          }
          S.q[h][0] = x.x * qs; S.q[h][1] = x.y * qs; S.q[h][2] = x.z * qs; S.q[h][3] = x.w * qs;
          S.q[h][4] = y.x * qs; S.q[h][5] = y.y * qs; S.q[h][6] = y.z * qs; S.q[h][7] = y.w * qs;
#pragma unroll
          for (int e = 0; e < 8; ++e) S.acc[h][e] = 0.f;
        }
      } else {
        const int items = (int)rfl((uint32_t)R.n_units) / 2;
        int i0, i1;
        piece(items, s, i0, i1);
        C.left = i1 - i0;
        C.KB = kq & 0xffff;
        C.rb = (2 * i0) / C.KB;
        C.rb0 = C.rb;
        C.kb = 2 * i0 - C.rb * C.KB;
        C.pend = false;
        kp = slot_kp(P, C.slot);
#pragma unroll
        for (int c = 0; c < NC; ++c) A.a[c] = 0.f;
      }
      waits_count(wt, 3, C.left);
      continue;  // the new task may have no items for this wave
    }

    // ---- item k
    if (F.issued <= k) {
      // not copied yet: a KV block of a step the stager has not opened
      const uint64_t s0 = waits_now(wt);
      if (!spin_ctl(P, cx, C_STEPOK, F.step + 1)) return;
      waits_add(wt, 0, s0);
      continue;
    }
    if (C.type == T_ATT) {
      wait_item<DEPTH>(F.issued - k - 1);
      if (prof && t_first == 0) t_first = rfl((uint32_t)wall_clock64());
      const uint8_t* it = rp + koff;
      const u32x4 w0 = ld_u32x4(it), w1 = ld_u32x4(it + kUnitBytes);
      const bool valid = C.lo + (C.u0 + C.t) * ppi + lane / lpp < C.end;
      att_item(P, S, w0, w1, valid, lpp == 16);
      ++C.t;
      ++k;
      koff = next_slot_off<DEPTH>(koff);
      --C.left;
    } else {
      matvec_run<DEPTH, NC>(P, C, F, k, koff, ring, rp, hin, kp, part + (size_t)s * P.ncap * P.wave_vrows + jrow,
                            icol, A, t_first, prof);
    }
  }
  wait_all();
  waits_put(P, cx, wt);
}
