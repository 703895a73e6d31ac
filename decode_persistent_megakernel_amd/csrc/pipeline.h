// Stream waves of the persistent decode megakernel (included by kernels.hip;
// internal to libmk).
//
// Every streamed task (a matvec over packed weight units, or attention over a
// chunk of the KV cache) is cut into kStreams contiguous pieces, one per
// stream wave: a matvec task's units (packed order: row block major, column
// block minor) in whole items of two units, an attention task's position
// blocks, one item each. An item is 2 KiB: two consecutive weight units, or
// the K block and the V block of one group of positions.
//
// A stream wave feeds itself: it copies its items from HBM straight into a
// private LDS ring of DEPTH slots (LDS DMA), DEPTH items ahead of the one it
// computes, running ahead across task boundaries so weights keep arriving
// while the workgroup waits on an event. Copies complete in issue order, so
// "item k has landed" is a wait for the vector-memory counter to drop to twice
// the number of younger items. The copies are issued as inline assembly: the
// compiler then leaves the wave's own LDS reads alone (it would otherwise wait
// for every copy in flight before each of them, not knowing which LDS bytes
// a copy writes) and schedules them freely; the explicit counter waits order
// every read after the copy that fills its slot.

// Attention items of a step read KV entries appended in earlier steps, so
// they are copied only after the stager has passed the step's first
// dependency (C_STEPOK); weight items never wait for anything but a free slot.

// ---------------------------------------------------------------------------
// copies for the stream waves
// ---------------------------------------------------------------------------

// 1 KiB per wave: lane l copies 16 bytes from its own address src into LDS
// byte address lds + 16*l (lds is wave-uniform; it goes in M0, which this
// wave's code uses for nothing else). nt: streamed once; sc1: device-coherent.
__device__ __forceinline__ void copy_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void copy_sc1(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1" : : "v"(src), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ u32x4 ld_u32x4(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// ---------------------------------------------------------------------------
// task walking
// ---------------------------------------------------------------------------

// Walks the stream tasks (those with weight or KV units) of this workgroup's
// queue, across steps, for stream wave s: the queue's stream records in LDS.
struct Walker {
  int step, r, i;    // r: record; i: global task counter of the task (all tasks)
  int slot, type, layer, b, g;
  int nu;            // matvec: units of wave s; attention: position blocks of wave s
  int n;             // items of wave s in the task (may be 0)
  int u0;            // matvec: first unit of wave s; attention: first position block
  int lo, end;       // attention: positions [lo, end) come from the cache
  int KB;            // matvec: column blocks
  int64_t woff;      // matvec: packed weight offset of the task
  bool done;
};

__device__ __forceinline__ void walker_init(Walker& w, const Ctx& cx) {
  w.step = 0;
  w.r = -1;
  w.i = 0;
  w.slot = 0;
  w.type = -1;
  w.layer = w.b = w.g = 0;
  w.nu = w.n = w.u0 = 0;
  w.lo = w.end = 0;
  w.KB = 1;
  w.woff = 0;
  w.done = false;
}

// [a0, a1): piece s of n things cut into kStreams nearly equal contiguous pieces
__device__ __forceinline__ void piece(int n, int s, int& a0, int& a1) {
  a0 = (int)((uint32_t)n * (uint32_t)s / kStreams);
  a1 = (int)((uint32_t)n * (uint32_t)(s + 1) / kStreams);
}

__device__ __forceinline__ uint32_t rfl(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void walker_next(const Params& P, Walker& w, const Ctx& cx, int s) {
  if (++w.r >= cx.nrec) {
    w.r = 0;
    ++w.step;
  }
  if (w.step >= P.n_steps || cx.nrec == 0) {
    w.done = true;
    return;
  }
  const StreamRec R = cx.recs[w.r];
  const uint32_t tsbg = rfl(R.tsbg), lc = rfl(R.lc), kq = rfl(R.kq);
  w.type = tsbg & 15;
  w.slot = (tsbg >> 4) & 3;
  if (w.slot < 2) w.slot ^= (int)rfl((uint32_t)R.flip) & w.step;
  w.b = (tsbg >> 6) & 1023;
  w.g = tsbg >> 16;
  w.layer = lc & 0xffff;
  const int chunk = lc >> 16;
  w.i = w.step * (cx.q1 - cx.q0) + (int)(kq >> 16);
  w.nu = 0;
  w.u0 = 0;
  if (w.type == T_ATT) {
    w.lo = w.end = 0;
    if (w.b < P.batch) {
      const int pos = ld_uniform(P.pos_in, w.b) + w.step;
      if (pos >= 0 && pos < P.S) {
        const int64_t len = (int64_t)pos + 1;
        w.lo = chunk_bound(chunk, len, P.Nc);
        w.end = min(chunk_bound(chunk + 1, len, P.Nc), pos);
        const int ppu = 512 / P.D;  // positions per unit
        const int npu = w.end > w.lo ? (w.end - w.lo + ppu - 1) / ppu : 0;
        int j1;
        piece(npu, s, w.u0, j1);
        w.nu = j1 - w.u0;
      }
    }
    w.n = w.nu;
  } else {
    const int U = (int)rfl((uint32_t)R.n_units);
    int i0, i1;
    piece((U + 1) / 2, s, i0, i1);
    w.u0 = 2 * i0;
    w.nu = max(min(2 * i1, U) - w.u0, 0);
    w.n = i1 - i0;
    w.KB = kq & 0xffff;
    w.woff = (int64_t)(((uint64_t)rfl((uint32_t)((uint64_t)R.w_off >> 32)) << 32) | rfl((uint32_t)R.w_off));
  }
}

// ---------------------------------------------------------------------------
// the copy side of a stream wave
// ---------------------------------------------------------------------------

constexpr int kItemBytes = 2 * kUnitBytes;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N): vmcnt bits [3:0] and [15:14], expcnt/lgkmcnt at max
  constexpr int imm = (N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}



struct Fetch {
  Walker w;            // the task of the next item to copy
  int t;               // its item within that task
  int issued;          // items copied so far
  bool kv;             // the task is attention (KV blocks), else a matvec
  const uint8_t* src;  // matvec: this lane's 16 bytes of the next item's first unit
};

__device__ __forceinline__ void fetch_next_task(const Params& P, const Ctx& cx, int s, Fetch& F) {
  do {
    walker_next(P, F.w, cx, s);
  } while (!F.w.done && F.w.n == 0);
  F.t = 0;
  F.kv = F.w.type == T_ATT;
  F.src = P.wpack + F.w.woff + (int64_t)F.w.u0 * kUnitBytes + cx.lane * 16;
}

// Ring of a stream wave: DEPTH (a power of two) slots of 2 KiB; item k sits in
// slot k % DEPTH. Byte address of item k (LDS) for the copies; pointer for reads.
template <int DEPTH>
__device__ __forceinline__ uint32_t ring_slot(uint32_t ring, int k) {
  return ring + (uint32_t)(k & (DEPTH - 1)) * kItemBytes;
}

// Copy items until `limit` have been issued, the task sequence ends, or the
// next item is a KV block of a step the stager has not opened yet. A matvec
// item is the next 2 KiB of the task's packed weights.
template <int DEPTH>
__device__ __forceinline__ void fetch_upto(const Params& P, const Ctx& cx, int s, Fetch& F, int limit,
                                           uint32_t ring) {
  while (F.issued < limit && !F.w.done) {
    const uint32_t dst = ring_slot<DEPTH>(ring, F.issued);
    if (!F.kv) {
      copy_nt(F.src, dst);
      // the second unit of a piece's last item may not exist: copy the first again
      copy_nt(2 * F.t + 1 < F.w.nu ? F.src + kUnitBytes : F.src, dst + kUnitBytes);
      F.src += kItemBytes;
    } else {
      if (F.t == 0 && lds_ld(&cx.ctl[C_STEPOK]) < F.w.step + 1) return;
      const int lane = cx.lane;
      const int D8 = P.D / 8, ppu = 64 / D8;
      const int pos = min(F.w.lo + (F.w.u0 + F.t) * ppu + lane / D8, F.w.end - 1);
      const size_t off =
          ((((size_t)F.w.layer * P.B + F.w.b) * P.Hkv + F.w.g) * (size_t)P.S + pos) * P.D + (lane % D8) * 8;
      copy_sc1(P.kcache + off, dst);
      copy_sc1(P.vcache + off, dst + kUnitBytes);
    }
    ++F.issued;
    if (++F.t == F.w.n) fetch_next_task(P, cx, s, F);
  }
}

// Wait until the oldest `n` not yet consumed items (from item k on) have
// landed. Steady state: DEPTH - n younger items in flight; fewer only at the
// end of the sequence or behind a KV step not yet open: then wait for all.
template <int DEPTH, int N>
__device__ __forceinline__ void wait_landed(const Fetch& F, int k) {
  cbar();
  if (F.issued - k == DEPTH) wait_vmcnt<2 * (DEPTH - N)>();
  else wait_vmcnt<0>();
  cbar();
}

// Make sure items k .. k+n-1 have been copied (waiting for a KV step to open
// if needed). false = leave the kernel.
template <int DEPTH>
__device__ __forceinline__ bool ensure_copied(const Params& P, const Ctx& cx, int s, Fetch& F, int k, int n,
                                              uint32_t ring, Waits& wt) {
  if (F.issued >= k + n) return true;
  const uint64_t s0 = waits_now(wt);
  while (F.issued < k + n) {
    if (!spin_ctl(P, cx, C_STEPOK, F.w.step + 1)) return false;
    fetch_upto<DEPTH>(P, cx, s, F, k + DEPTH, ring);
  }
  waits_add(wt, 0, s0);
  return true;
}

// Items before k have been read: refill their slots, up to item k + DEPTH - 1.
// In the steady state that is two whole items of the matvec task being
// copied: four copies of consecutive 1 KiB.
template <int DEPTH>
__device__ __forceinline__ void refill(const Params& P, const Ctx& cx, int s, Fetch& F, int k, uint32_t ring) {
  wait_lgkm();  // the reads of the slots being refilled have completed
  if (F.issued == k + DEPTH - 2 && !F.kv && F.t + 2 < F.w.n && 2 * F.t + 3 < F.w.nu) {
    const uint32_t d0 = ring_slot<DEPTH>(ring, F.issued), d1 = ring_slot<DEPTH>(ring, F.issued + 1);
    copy_nt(F.src, d0);
    copy_nt(F.src + kUnitBytes, d0 + kUnitBytes);
    copy_nt(F.src + 2 * kUnitBytes, d1);
    copy_nt(F.src + 3 * kUnitBytes, d1 + kUnitBytes);
    F.src += 2 * kItemBytes;
    F.issued += 2;
    F.t += 2;
  } else {
    fetch_upto<DEPTH>(P, cx, s, F, k + DEPTH, ring);
  }
}

// ---------------------------------------------------------------------------
// matvec
// ---------------------------------------------------------------------------

// the column block after b in a row block of KB
__device__ __forceinline__ int next_cb(int b, int KB) { return b + 1 == KB ? 0 : b + 1; }

// Running state of a matvec piece: NC row sums and the (row block, column
// block) of the next unit.
template <int NC>
struct MvState {
  float acc[NC];
  int rb, kb;
  bool pend;  // acc holds sums of an unfinished row block
};

// Reduce the row sums over the 16 lanes of each row and store them as this
// wave's partial sums of row block r (pout: this lane's row in column 0;
// cs: floats between columns).
template <int NC>
__device__ __forceinline__ void mv_flush(MvState<NC>& st, float* pout, int cs, int icol, int r) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float v = sum16(st.acc[c]);
    if (icol == 0) pout[(size_t)c * cs + r * 4] = v;
    st.acc[c] = 0.f;
  }
}

template <int NC>
__device__ __forceinline__ void mv_add(MvState<NC>& st, const float (&d)[NC], int KB, float* pout, int cs,
                                       int icol) {
#pragma unroll
  for (int c = 0; c < NC; ++c) st.acc[c] += d[c];
  if (st.kb == KB - 1) {
    mv_flush<NC>(st, pout, cs, icol, st.rb);
    st.kb = 0;
    ++st.rb;
    st.pend = false;
  } else {
    ++st.kb;
    st.pend = true;
  }
}

// Dot products of one unit's 8 weights (this lane) with NC activation columns
// (lane 16*jrow + icol: columns 4*icol.. and 64 + 4*icol.. of column block b).
template <int NC>
__device__ __forceinline__ void mv_unit(const u32x4 wv, const float* hl, int kp, int b, float (&d)[NC]) {
  float x[8];
  unpack8(wv, x);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float* q = hl + (size_t)c * kp + b * kUnitCols;
    const float4 h0 = ld_f4(q), h1 = ld_f4(q + 64);
    float a = x[0] * h0.x;
    a = fmaf(x[1], h0.y, a); a = fmaf(x[2], h0.z, a); a = fmaf(x[3], h0.w, a);
    a = fmaf(x[4], h1.x, a); a = fmaf(x[5], h1.y, a);
    a = fmaf(x[6], h1.z, a); a = fmaf(x[7], h1.w, a);
    d[c] = a;
  }
}

// Matvec piece of stream wave s with NC staged columns: each lane accumulates
// row jrow of a unit's row block over its 8 columns; a row block's sums are
// reduced over the 16 lanes of the row and stored as this wave's partial sums.
// Unit layout: lane 16*jrow + icol holds columns [4*icol, +4) and
// [64 + 4*icol, +4) of its row. Items go two at a time (four units).
template <int DEPTH, int NC>
__device__ __forceinline__ bool stream_matvec(const Params& P, const Ctx& cx, int s, const Walker& w, Fetch& F,
                                              int& k, uint32_t ring, Waits& wt, const float* hin, int kp,
                                              float* part) {
  const int lane = cx.lane;
  const int jrow = lane >> 4, icol = lane & 15;
  const int KB = w.KB;
  const float* hl = hin + icol * 4;
  float* pout = part + (size_t)s * P.ncap * P.vrow_stride + jrow;
  const int pcs = P.vrow_stride;
  const uint8_t* rp = reinterpret_cast<const uint8_t*>(cx.ring) - lds_addr(cx.ring) + lane * 16;  // LDS address -> pointer
  MvState<NC> st;
#pragma unroll
  for (int c = 0; c < NC; ++c) st.acc[c] = 0.f;
  st.rb = w.u0 / KB;
  st.kb = w.u0 - st.rb * KB;
  st.pend = false;
  int t = 0;
  for (; t + 1 < w.n && 2 * t + 3 < w.nu; t += 2) {
    if (!ensure_copied<DEPTH>(P, cx, s, F, k, 2, ring, wt)) return false;
    wait_landed<DEPTH, 2>(F, k);
    const uint8_t* i0 = rp + ring_slot<DEPTH>(ring, k);
    const uint8_t* i1 = rp + ring_slot<DEPTH>(ring, k + 1);
    const u32x4 w0 = ld_u32x4(i0), w1 = ld_u32x4(i0 + kUnitBytes);
    const u32x4 w2 = ld_u32x4(i1), w3 = ld_u32x4(i1 + kUnitBytes);
    const int b0 = st.kb, b1 = next_cb(b0, KB), b2 = next_cb(b1, KB), b3 = next_cb(b2, KB);
    float d[4][NC];
    mv_unit<NC>(w0, hl, kp, b0, d[0]);
    mv_unit<NC>(w1, hl, kp, b1, d[1]);
    mv_unit<NC>(w2, hl, kp, b2, d[2]);
    mv_unit<NC>(w3, hl, kp, b3, d[3]);
    k += 2;
    refill<DEPTH>(P, cx, s, F, k, ring);
    if (st.kb + 4 < KB) {  // the row block goes on past these four units
#pragma unroll
      for (int c = 0; c < NC; ++c) st.acc[c] += (d[0][c] + d[1][c]) + (d[2][c] + d[3][c]);
      st.kb += 4;
      st.pend = true;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) mv_add<NC>(st, d[u], KB, pout, pcs, icol);
    }
  }
  for (; t < w.n; ++t) {
    if (!ensure_copied<DEPTH>(P, cx, s, F, k, 1, ring, wt)) return false;
    wait_landed<DEPTH, 1>(F, k);
    const uint8_t* i0 = rp + ring_slot<DEPTH>(ring, k);
    const u32x4 w0 = ld_u32x4(i0), w1 = ld_u32x4(i0 + kUnitBytes);
    float d0[NC], d1[NC];
    mv_unit<NC>(w0, hl, kp, st.kb, d0);
    mv_unit<NC>(w1, hl, kp, next_cb(st.kb, KB), d1);
    k += 1;
    wait_lgkm();  // the item's slot has been read
    fetch_upto<DEPTH>(P, cx, s, F, k + DEPTH, ring);
    mv_add<NC>(st, d0, KB, pout, pcs, icol);
    if (2 * t + 1 < w.nu) mv_add<NC>(st, d1, KB, pout, pcs, icol);
  }
  if (st.pend) mv_flush<NC>(st, pout, pcs, icol, st.rb);
  return true;
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------

// One level of the merge of online-softmax states across lanes paired by xor
// O; both lanes of a pair merge the same ordered pair of states.
template <int O>
__device__ __forceinline__ void att_merge_step(int G, float (&mv)[kMaxG], float (&lv)[kMaxG],
                                               float (&av)[kMaxG][8]) {
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      float m1, m2, l1, l2;
      xpair<O>(mv[h], m1, m2);
      xpair<O>(lv[h], l1, l2);
      const float M = fmaxf(m1, m2);
      const float a1 = m1 == -INFINITY ? 0.f : expf(m1 - M);
      const float a2 = m2 == -INFINITY ? 0.f : expf(m2 - M);
      lv[h] = l1 * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x1, x2;
        xpair<O>(av[h][e], x1, x2);
        av[h][e] = x1 * a1 + x2 * a2;
      }
      mv[h] = M;
    }
  }
}

// Attention piece of stream wave s: lanes hold 8 dims of one position of a
// block (D/8 lanes per position); each position group keeps an online-softmax
// state per query head, merged across the wave at the end and stored as
// {acc[D], m, l} per head.
template <int DEPTH>
__device__ __forceinline__ bool stream_att(const Params& P, const Ctx& cx, int s, const Walker& w, Fetch& F,
                                           int& k, uint32_t ring, Waits& wt, const float* hin, float* part) {
  const int lane = cx.lane;
  const int D = P.D, lpp = D / 8, ppu = 64 / lpp;
  const int pg = lane / lpp, de = (lane % lpp) * 8;
  const int G = P.G;
  const float scale = P.attn_scale;
  const uint8_t* rp = reinterpret_cast<const uint8_t*>(cx.ring) - lds_addr(cx.ring) + lane * 16;
  float qv[kMaxG][8], av[kMaxG][8], mv[kMaxG], lv[kMaxG];
  const float* q = hin + att_raw_floats(P);
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    mv[h] = -INFINITY;
    lv[h] = 0.f;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
    if (h < G) {
      x = ld_f4(q + h * D + de);
      y = ld_f4(q + h * D + de + 4);
    }
    qv[h][0] = x.x; qv[h][1] = x.y; qv[h][2] = x.z; qv[h][3] = x.w;
    qv[h][4] = y.x; qv[h][5] = y.y; qv[h][6] = y.z; qv[h][7] = y.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) av[h][e] = 0.f;
  }
  for (int t = 0; t < w.n; ++t) {
    if (!ensure_copied<DEPTH>(P, cx, s, F, k, 1, ring, wt)) return false;
    wait_landed<DEPTH, 1>(F, k);
    const uint8_t* it = rp + ring_slot<DEPTH>(ring, k);
    const u32x4 wk = ld_u32x4(it), wv = ld_u32x4(it + kUnitBytes);
    k += 1;
    wait_lgkm();  // the item's slot has been read
    fetch_upto<DEPTH>(P, cx, s, F, k + DEPTH, ring);
    const bool valid = w.lo + (w.u0 + t) * ppu + pg < w.end;
    float kf[8], vf[8];
    unpack8(wk, kf);
    unpack8(wv, vf);
    // heads past G hold zero queries; their state is never stored
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[h][e], kf[e], d);
      d = group_sum(d, lpp);
      const float sc = valid ? d * scale : -INFINITY;
      const float mn = fmaxf(mv[h], sc);
      const float al = mn == -INFINITY ? 1.f : expf(mv[h] - mn);
      const float pe = sc == -INFINITY ? 0.f : expf(sc - mn);
      lv[h] = fmaf(lv[h], al, pe);
#pragma unroll
      for (int e = 0; e < 8; ++e) av[h][e] = fmaf(pe, vf[e], av[h][e] * al);
      mv[h] = mn;
    }
  }
  // merge the position groups of the wave (lanes with equal dims)
  if (lpp <= 1) att_merge_step<1>(G, mv, lv, av);
  if (lpp <= 2) att_merge_step<2>(G, mv, lv, av);
  if (lpp <= 4) att_merge_step<4>(G, mv, lv, av);
  if (lpp <= 8) att_merge_step<8>(G, mv, lv, av);
  if (lpp <= 16) att_merge_step<16>(G, mv, lv, av);
  if (lpp <= 32) att_merge_step<32>(G, mv, lv, av);
  const int stride = G * (D + 2);
  if (pg == 0) {
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float* dst = part + s * stride + h * (D + 2);
        *reinterpret_cast<float4*>(dst + de) = make_float4(av[h][0], av[h][1], av[h][2], av[h][3]);
        *reinterpret_cast<float4*>(dst + de + 4) = make_float4(av[h][4], av[h][5], av[h][6], av[h][7]);
        if (lane == 0) {
          dst[D] = mv[h];
          dst[D + 1] = lv[h];
        }
      }
    }
  }
  return true;
}

// ---------------------------------------------------------------------------
// stream wave
// ---------------------------------------------------------------------------

template <int DEPTH>
__device__ __forceinline__ void run_stream(const Params& P, const Ctx& cx, int s) {
  Waits wt;  // KV step not open, -, task staged, items
  waits_init(P, cx, wt);
  const uint32_t ring = lds_addr(cx.ring) + (uint32_t)s * DEPTH * kItemBytes;
  Fetch F;
  walker_init(F.w, cx);
  F.issued = 0;
  fetch_next_task(P, cx, s, F);
  fetch_upto<DEPTH>(P, cx, s, F, DEPTH, ring);
  int k = 0;  // items consumed
  Walker w;
  walker_init(w, cx);
  const int ncols = P.batch;
  for (;;) {
    {
      const uint64_t s0 = waits_now(wt);
      walker_next(P, w, cx, s);
      waits_add(wt, 7, s0);
    }
    if (w.done) break;
    {
      const uint64_t s0 = waits_now(wt);
      if (!spin_ctl(P, cx, C_STAGED, w.i + 1)) return;
      waits_add(wt, 2, s0);
    }
    const float* hin = slot_ptr(cx, w.slot) + kHdr;
    float* part = part_ptr(cx, w.slot);
    const uint64_t s1 = waits_now(wt);
    bool ok;
    if (w.type == T_ATT) {
      ok = stream_att<DEPTH>(P, cx, s, w, F, k, ring, wt, hin, part);
    } else {
      const int kp = slot_kp(P, w.slot);
      switch (ncols) {
        case 1: ok = stream_matvec<DEPTH, 1>(P, cx, s, w, F, k, ring, wt, hin, kp, part); break;
        case 2: ok = stream_matvec<DEPTH, 2>(P, cx, s, w, F, k, ring, wt, hin, kp, part); break;
        case 3: ok = stream_matvec<DEPTH, 3>(P, cx, s, w, F, k, ring, wt, hin, kp, part); break;
        default: ok = stream_matvec<DEPTH, 4>(P, cx, s, w, F, k, ring, wt, hin, kp, part); break;
      }
    }
    if (!ok) return;
    if (w.type == T_LM) waits_add(wt, 5, s1);
    else waits_add(wt, 8, s1);
    waits_count(wt, 3, w.n);
    const uint64_t s2 = waits_now(wt);
    lds_add(&cx.ctl[C_DONE + w.slot], 1);
    waits_add(wt, 9, s2);
  }
  wait_all();
  waits_put(P, cx, wt);
}
