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
// private LDS ring of D slots (LDS DMA), D items ahead of the one it computes,
// running ahead across task boundaries so weights keep arriving while the
// workgroup waits on an event. Copies complete in issue order, so "item k has
// landed" is a wait for the vector-memory counter to drop to twice the number
// of younger items. The wave's LDS reads and writes are written as inline
// assembly: the compiler cannot tell them apart from the LDS the copies are
// writing and would otherwise wait for every copy in flight before each of
// them. (Each asm block that loads waits for its own loads before it ends.)
//
// Attention items of a step read KV entries appended in earlier steps, so
// they are copied only after the stager has passed the step's first
// dependency (C_STEPOK); weight items never wait for anything but a free slot.

// ---------------------------------------------------------------------------
// LDS access for the stream waves (invisible to the compiler's memory model)
// ---------------------------------------------------------------------------

typedef float f32x4 __attribute__((ext_vector_type(4)));  // asm operand type of 16 bytes

__device__ __forceinline__ void lds_write_b32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b128(uint32_t addr, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add_raw(uint32_t addr, int v) {
  asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_read_2x128(uint32_t a, uint32_t b, f32x4& x, f32x4& y) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y)
      : "v"(a), "v"(b)
      : "memory");
}
// An item (two 1 KiB halves at `item` and item+1024) and, for NC columns, the
// activations of the item's two units (unit A at ha[c], unit B at hb[c]; each
// 4 floats at +0 and 4 floats at +256 bytes).
template <int NC>
struct ItemRegs {
  u32x4 w0, w1;
  f32x4 a[NC][2], b[NC][2];
};
__device__ __forceinline__ void lds_item(uint32_t item, const uint32_t (&ha)[1], const uint32_t (&hb)[1],
                                         ItemRegs<1>& r) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:1024\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:256\n\t"
      "ds_read_b128 %4, %8\n\t"
      "ds_read_b128 %5, %8 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.w0), "=&v"(r.w1), "=&v"(r.a[0][0]), "=&v"(r.a[0][1]), "=&v"(r.b[0][0]), "=&v"(r.b[0][1])
      : "v"(item), "v"(ha[0]), "v"(hb[0])
      : "memory");
}
__device__ __forceinline__ void lds_item(uint32_t item, const uint32_t (&ha)[2], const uint32_t (&hb)[2],
                                         ItemRegs<2>& r) {
  asm volatile(
      "ds_read_b128 %0, %10\n\t"
      "ds_read_b128 %1, %10 offset:1024\n\t"
      "ds_read_b128 %2, %11\n\t"
      "ds_read_b128 %3, %11 offset:256\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %12 offset:256\n\t"
      "ds_read_b128 %6, %13\n\t"
      "ds_read_b128 %7, %13 offset:256\n\t"
      "ds_read_b128 %8, %14\n\t"
      "ds_read_b128 %9, %14 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.w0), "=&v"(r.w1), "=&v"(r.a[0][0]), "=&v"(r.a[0][1]), "=&v"(r.b[0][0]), "=&v"(r.b[0][1]),
        "=&v"(r.a[1][0]), "=&v"(r.a[1][1]), "=&v"(r.b[1][0]), "=&v"(r.b[1][1])
      : "v"(item), "v"(ha[0]), "v"(hb[0]), "v"(ha[1]), "v"(hb[1])
      : "memory");
}
__device__ __forceinline__ void lds_item(uint32_t item, const uint32_t (&ha)[3], const uint32_t (&hb)[3],
                                         ItemRegs<3>& r) {
  asm volatile(
      "ds_read_b128 %0, %14\n\t"
      "ds_read_b128 %1, %14 offset:1024\n\t"
      "ds_read_b128 %2, %15\n\t"
      "ds_read_b128 %3, %15 offset:256\n\t"
      "ds_read_b128 %4, %16\n\t"
      "ds_read_b128 %5, %16 offset:256\n\t"
      "ds_read_b128 %6, %17\n\t"
      "ds_read_b128 %7, %17 offset:256\n\t"
      "ds_read_b128 %8, %18\n\t"
      "ds_read_b128 %9, %18 offset:256\n\t"
      "ds_read_b128 %10, %19\n\t"
      "ds_read_b128 %11, %19 offset:256\n\t"
      "ds_read_b128 %12, %20\n\t"
      "ds_read_b128 %13, %20 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.w0), "=&v"(r.w1), "=&v"(r.a[0][0]), "=&v"(r.a[0][1]), "=&v"(r.b[0][0]), "=&v"(r.b[0][1]),
        "=&v"(r.a[1][0]), "=&v"(r.a[1][1]), "=&v"(r.b[1][0]), "=&v"(r.b[1][1]), "=&v"(r.a[2][0]),
        "=&v"(r.a[2][1]), "=&v"(r.b[2][0]), "=&v"(r.b[2][1])
      : "v"(item), "v"(ha[0]), "v"(hb[0]), "v"(ha[1]), "v"(hb[1]), "v"(ha[2]), "v"(hb[2])
      : "memory");
}
__device__ __forceinline__ void lds_item(uint32_t item, const uint32_t (&ha)[4], const uint32_t (&hb)[4],
                                         ItemRegs<4>& r) {
  asm volatile(
      "ds_read_b128 %0, %18\n\t"
      "ds_read_b128 %1, %18 offset:1024\n\t"
      "ds_read_b128 %2, %19\n\t"
      "ds_read_b128 %3, %19 offset:256\n\t"
      "ds_read_b128 %4, %20\n\t"
      "ds_read_b128 %5, %20 offset:256\n\t"
      "ds_read_b128 %6, %21\n\t"
      "ds_read_b128 %7, %21 offset:256\n\t"
      "ds_read_b128 %8, %22\n\t"
      "ds_read_b128 %9, %22 offset:256\n\t"
      "ds_read_b128 %10, %23\n\t"
      "ds_read_b128 %11, %23 offset:256\n\t"
      "ds_read_b128 %12, %24\n\t"
      "ds_read_b128 %13, %24 offset:256\n\t"
      "ds_read_b128 %14, %25\n\t"
      "ds_read_b128 %15, %25 offset:256\n\t"
      "ds_read_b128 %16, %26\n\t"
      "ds_read_b128 %17, %26 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.w0), "=&v"(r.w1), "=&v"(r.a[0][0]), "=&v"(r.a[0][1]), "=&v"(r.b[0][0]), "=&v"(r.b[0][1]),
        "=&v"(r.a[1][0]), "=&v"(r.a[1][1]), "=&v"(r.b[1][0]), "=&v"(r.b[1][1]), "=&v"(r.a[2][0]),
        "=&v"(r.a[2][1]), "=&v"(r.b[2][0]), "=&v"(r.b[2][1]), "=&v"(r.a[3][0]), "=&v"(r.a[3][1]),
        "=&v"(r.b[3][0]), "=&v"(r.b[3][1])
      : "v"(item), "v"(ha[0]), "v"(hb[0]), "v"(ha[1]), "v"(hb[1]), "v"(ha[2]), "v"(hb[2]), "v"(ha[3]),
        "v"(hb[3])
      : "memory");
}
// Two items (in slots at i0 and i1) and, for NC columns, the activations of
// their four units u = 0..3 at h[u][c].
template <int NC>
struct Item2Regs {
  u32x4 w[4];
  f32x4 h[4][NC][2];
};
__device__ __forceinline__ void lds_item2(uint32_t i0, uint32_t i1, const uint32_t (&h)[4][1], Item2Regs<1>& r) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %13\n\t"
      "ds_read_b128 %3, %13 offset:1024\n\t"
      "ds_read_b128 %4, %14\n\t"
      "ds_read_b128 %5, %14 offset:256\n\t"
      "ds_read_b128 %6, %15\n\t"
      "ds_read_b128 %7, %15 offset:256\n\t"
      "ds_read_b128 %8, %16\n\t"
      "ds_read_b128 %9, %16 offset:256\n\t"
      "ds_read_b128 %10, %17\n\t"
      "ds_read_b128 %11, %17 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.w[0]), "=&v"(r.w[1]), "=&v"(r.w[2]), "=&v"(r.w[3]), "=&v"(r.h[0][0][0]), "=&v"(r.h[0][0][1]),
        "=&v"(r.h[1][0][0]), "=&v"(r.h[1][0][1]), "=&v"(r.h[2][0][0]), "=&v"(r.h[2][0][1]), "=&v"(r.h[3][0][0]),
        "=&v"(r.h[3][0][1])
      : "v"(i0), "v"(i1), "v"(h[0][0]), "v"(h[1][0]), "v"(h[2][0]), "v"(h[3][0])
      : "memory");
}
__device__ __forceinline__ void lds_item2(uint32_t i0, uint32_t i1, const uint32_t (&h)[4][2], Item2Regs<2>& r) {
  asm volatile(
      "ds_read_b128 %0, %20\n\t"
      "ds_read_b128 %1, %20 offset:1024\n\t"
      "ds_read_b128 %2, %21\n\t"
      "ds_read_b128 %3, %21 offset:1024\n\t"
      "ds_read_b128 %4, %22\n\t"
      "ds_read_b128 %5, %22 offset:256\n\t"
      "ds_read_b128 %6, %23\n\t"
      "ds_read_b128 %7, %23 offset:256\n\t"
      "ds_read_b128 %8, %24\n\t"
      "ds_read_b128 %9, %24 offset:256\n\t"
      "ds_read_b128 %10, %25\n\t"
      "ds_read_b128 %11, %25 offset:256\n\t"
      "ds_read_b128 %12, %26\n\t"
      "ds_read_b128 %13, %26 offset:256\n\t"
      "ds_read_b128 %14, %27\n\t"
      "ds_read_b128 %15, %27 offset:256\n\t"
      "ds_read_b128 %16, %28\n\t"
      "ds_read_b128 %17, %28 offset:256\n\t"
      "ds_read_b128 %18, %29\n\t"
      "ds_read_b128 %19, %29 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.w[0]), "=&v"(r.w[1]), "=&v"(r.w[2]), "=&v"(r.w[3]), "=&v"(r.h[0][0][0]), "=&v"(r.h[0][0][1]),
        "=&v"(r.h[0][1][0]), "=&v"(r.h[0][1][1]), "=&v"(r.h[1][0][0]), "=&v"(r.h[1][0][1]), "=&v"(r.h[1][1][0]),
        "=&v"(r.h[1][1][1]), "=&v"(r.h[2][0][0]), "=&v"(r.h[2][0][1]), "=&v"(r.h[2][1][0]), "=&v"(r.h[2][1][1]),
        "=&v"(r.h[3][0][0]), "=&v"(r.h[3][0][1]), "=&v"(r.h[3][1][0]), "=&v"(r.h[3][1][1])
      : "v"(i0), "v"(i1), "v"(h[0][0]), "v"(h[0][1]), "v"(h[1][0]), "v"(h[1][1]), "v"(h[2][0]), "v"(h[2][1]),
        "v"(h[3][0]), "v"(h[3][1])
      : "memory");
}
__device__ __forceinline__ void lds_item_kv(uint32_t item, u32x4& k, u32x4& v) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k), "=&v"(v)
      : "v"(item)
      : "memory");
}

// Spin until ctl[word] >= v (asm reads; bounded by the watchdog).
__device__ __forceinline__ bool spin_raw(const Params& P, const Ctx& cx, int word, int v) {
  if (lds_ld_raw(&cx.ctl[word]) >= v) return true;
  const uint64_t t0 = wall_clock64();
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    if (lds_ld_raw(&cx.ctl[word]) >= v) return true;
    if (lds_ld_raw(&cx.ctl[C_ABORT])) return false;
    if (wall_clock64() - t0 > P.timeout_ticks) {
      raise_abort(P, cx, kStatusTimeout);
      return false;
    }
  }
}

// ---------------------------------------------------------------------------
// task walking
// ---------------------------------------------------------------------------

// Walks the stream tasks (those with weight or KV units) of this workgroup's
// queue, across steps, for stream wave s, keeping the slot assignment of every
// task.
struct Walker {
  int step, qi, i;   // i: global task counter of the current task (all tasks)
  int nsmall, slot;
  int id, type, layer, b, g;
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
  w.qi = cx.q0 - 1;
  w.i = -1;
  w.nsmall = 0;
  w.slot = 0;
  w.id = 0;
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

__device__ __forceinline__ void walker_next(const Params& P, Walker& w, const Ctx& cx, int s) {
  for (;;) {
    ++w.qi;
    ++w.i;
    if (w.qi >= cx.q1) {
      w.qi = cx.q0;
      ++w.step;
    }
    if (w.step >= P.n_steps || cx.q0 >= cx.q1) {
      w.done = true;
      return;
    }
    w.id = task_at(P, cx, w.qi);
    const DevTask T = ld_task(P, w.id);
    w.type = T.type;
    w.slot = next_slot(w.nsmall, w.type);
    if (!has_stream(w.type)) continue;
    w.layer = T.layer;
    w.b = T.b;
    w.g = T.g;
    w.nu = 0;
    w.u0 = 0;
    if (w.type == T_ATT) {
      w.lo = w.end = 0;
      if (w.b < P.batch) {
        const int pos = ld_uniform(P.pos_in, w.b) + w.step;
        if (pos >= 0 && pos < P.S) {
          const int64_t len = (int64_t)pos + 1;
          w.lo = chunk_bound(T.chunk, len, P.Nc);
          w.end = min(chunk_bound(T.chunk + 1, len, P.Nc), pos);
          const int ppu = 512 / P.D;  // positions per unit
          const int npu = w.end > w.lo ? (w.end - w.lo + ppu - 1) / ppu : 0;
          int j1;
          piece(npu, s, w.u0, j1);
          w.nu = j1 - w.u0;
        }
      }
      w.n = w.nu;
    } else {
      const int U = T.n_units;
      int i0, i1;
      piece((U + 1) / 2, s, i0, i1);
      w.u0 = 2 * i0;
      w.nu = max(min(2 * i1, U) - w.u0, 0);
      w.n = i1 - i0;
      w.KB = T.kb;
      w.woff = T.w_off;
    }
    return;
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
  int slot;            // ring slot of the next item
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

// Copy items until `limit` have been issued, the task sequence ends, or the
// next item is a KV block of a step the stager has not opened yet. A matvec
// item is the next 2 KiB of the task's packed weights.
template <int DEPTH>
__device__ __forceinline__ void fetch_upto(const Params& P, const Ctx& cx, int s, Fetch& F, int limit,
                                           uint8_t* ring) {
  while (F.issued < limit && !F.w.done) {
    uint8_t* dst = ring + F.slot * kItemBytes;
    if (!F.kv) {
      dma16<kAuxStream>(F.src, dst);
      // the second unit of a piece's last item may not exist: copy the first again
      dma16<kAuxStream>(2 * F.t + 1 < F.w.nu ? F.src + kUnitBytes : F.src, dst + kUnitBytes);
      F.src += kItemBytes;
    } else {
      if (F.t == 0 && lds_ld_raw(&cx.ctl[C_STEPOK]) < F.w.step + 1) return;
      const int lane = cx.lane;
      const int D8 = P.D / 8, ppu = 64 / D8;
      const int pos = min(F.w.lo + (F.w.u0 + F.t) * ppu + lane / D8, F.w.end - 1);
      const size_t off =
          ((((size_t)F.w.layer * P.B + F.w.b) * P.Hkv + F.w.g) * (size_t)P.S + pos) * P.D + (lane % D8) * 8;
      dma16<kAuxCoherent>(P.kcache + off, dst);
      dma16<kAuxCoherent>(P.vcache + off, dst + kUnitBytes);
    }
    ++F.issued;
    F.slot = F.slot + 1 == DEPTH ? 0 : F.slot + 1;
    if (++F.t == F.w.n) fetch_next_task(P, cx, s, F);
  }
}

// The consuming side: item k (a count over the wave's whole item sequence)
// is next; it sits in ring slot `slot`.
struct Feed {
  int k, slot;
  uint8_t* ring;
};

// Make sure item f.k has been copied (waiting for its step to open if needed)
// and has landed.
template <int DEPTH>
__device__ __forceinline__ bool feed_item(const Params& P, const Ctx& cx, int s, Fetch& F, Feed& f, Waits& wt) {
  if (F.issued <= f.k) {
    const uint64_t s0 = waits_now(wt);
    while (F.issued <= f.k) {
      if (!spin_raw(P, cx, C_STEPOK, F.w.step + 1)) return false;
      fetch_upto<DEPTH>(P, cx, s, F, f.k + DEPTH, f.ring);
    }
    waits_add(wt, 0, s0);
  }
  // Steady state: DEPTH - 1 younger items in flight. Fewer only at the end
  // of the sequence or behind a KV step not yet open: then wait for all.
  cbar();
  if (F.issued - f.k - 1 == DEPTH - 1) wait_vmcnt<2 * (DEPTH - 1)>();
  else wait_vmcnt<0>();
  cbar();
  return true;
}

// Items f.k and f.k+1 (both already copied) have landed.
template <int DEPTH>
__device__ __forceinline__ void feed_wait2(const Fetch& F, const Feed& f) {
  cbar();
  if (F.issued - f.k - 2 == DEPTH - 2) wait_vmcnt<2 * (DEPTH - 2)>();
  else wait_vmcnt<0>();
  cbar();
}

// Item f.k has been read into registers: its slot takes item k + DEPTH. In
// the steady state that is one copy, of the matvec task being copied.
template <int DEPTH>
__device__ __forceinline__ void feed_done(const Params& P, const Ctx& cx, int s, Fetch& F, Feed& f) {
  ++f.k;
  f.slot = f.slot + 1 == DEPTH ? 0 : f.slot + 1;
  if (F.issued == f.k + DEPTH - 1 && !F.kv && F.t + 1 < F.w.n) {
    uint8_t* dst = f.ring + F.slot * kItemBytes;
    dma16<kAuxStream>(F.src, dst);
    dma16<kAuxStream>(2 * F.t + 1 < F.w.nu ? F.src + kUnitBytes : F.src, dst + kUnitBytes);
    F.src += kItemBytes;
    ++F.issued;
    F.slot = F.slot + 1 == DEPTH ? 0 : F.slot + 1;
    ++F.t;
  } else {
    fetch_upto<DEPTH>(P, cx, s, F, f.k + DEPTH, f.ring);
  }
}

// ---------------------------------------------------------------------------
// arithmetic
// ---------------------------------------------------------------------------

// Running state of a matvec piece: NC row sums and the (row block, column
// block) of the next unit.
template <int NC>
struct MvState {
  float acc[NC];
  int rb, kb;
  bool pend;  // acc holds sums of an unfinished row block
};

// Reduce the row sums over the 16 lanes of each row and store them as this
// wave's partial sums of row block r (pout: LDS byte address of this lane's
// row in column 0; cs: byte stride between columns).
template <int NC>
__device__ __forceinline__ void mv_flush(MvState<NC>& st, uint32_t pout, uint32_t cs, int icol, int r) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float v = sum16(st.acc[c]);
    if (icol == 0) lds_write_b32(pout + c * cs + r * 16, v);
    st.acc[c] = 0.f;
  }
}

template <int NC>
__device__ __forceinline__ void mv_add(MvState<NC>& st, const float (&d)[NC], int KB, uint32_t pout, uint32_t cs,
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

template <int NC>
__device__ __forceinline__ void mv_dot(const u32x4 wv, const f32x4 (&h)[NC][2], float (&d)[NC]) {
  float x[8];
  unpack8(wv, x);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float a = x[0] * h[c][0].x;
    a = fmaf(x[1], h[c][0].y, a); a = fmaf(x[2], h[c][0].z, a); a = fmaf(x[3], h[c][0].w, a);
    a = fmaf(x[4], h[c][1].x, a); a = fmaf(x[5], h[c][1].y, a);
    a = fmaf(x[6], h[c][1].z, a); a = fmaf(x[7], h[c][1].w, a);
    d[c] = a;
  }
}

// Matvec piece of stream wave s with NC staged columns: each lane accumulates
// row jrow of a unit's row block over its 8 columns; a row block's sums are
// reduced over the 16 lanes of the row and stored as this wave's partial sums.
// Unit layout: lane 16*jrow + icol holds columns [4*icol, +4) and
// [64 + 4*icol, +4) of its row.
template <int DEPTH, int NC>
__device__ __forceinline__ bool stream_matvec(const Params& P, const Ctx& cx, int s, const Walker& w, Fetch& F,
                                              Feed& f, Waits& wt, const float* hin, int kp, float* part) {
  const int lane = cx.lane;
  const int jrow = lane >> 4, icol = lane & 15;
  const int KB = w.KB;
  const uint32_t hl = lds_addr(hin + icol * 4);
  const uint32_t cstride = (uint32_t)kp * 4;
  const uint32_t pout = lds_addr(part + (size_t)s * P.ncap * P.vrow_stride + jrow);
  const uint32_t pcs = (uint32_t)P.vrow_stride * 4;
  const uint32_t ring = lds_addr(f.ring) + lane * 16;
  MvState<NC> st;
#pragma unroll
  for (int c = 0; c < NC; ++c) st.acc[c] = 0.f;
  st.rb = w.u0 / KB;
  st.kb = w.u0 - st.rb * KB;
  st.pend = false;
  int t = 0;
  if constexpr (NC <= 2) {
    // two items (four units) at a time while both are copied and whole
    while (t + 1 < w.n && 2 * t + 3 < w.nu && F.issued >= f.k + 2) {
      feed_wait2<DEPTH>(F, f);
      uint32_t h[4][NC];
      int b = st.kb;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int c = 0; c < NC; ++c) h[u][c] = hl + c * cstride + b * (kUnitCols * 4);
        b = b + 1 == KB ? 0 : b + 1;
      }
      const int s1 = f.slot + 1 == DEPTH ? 0 : f.slot + 1;
      Item2Regs<NC> r;
      lds_item2(ring + f.slot * kItemBytes, ring + s1 * kItemBytes, h, r);
      feed_done<DEPTH>(P, cx, s, F, f);
      feed_done<DEPTH>(P, cx, s, F, f);
      float d[4][NC];
#pragma unroll
      for (int u = 0; u < 4; ++u) mv_dot<NC>(r.w[u], r.h[u], d[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) mv_add<NC>(st, d[u], KB, pout, pcs, icol);
      t += 2;
    }
  }
  for (; t < w.n; ++t) {
    if (!feed_item<DEPTH>(P, cx, s, F, f, wt)) return false;
    const int kb1 = st.kb + 1 == KB ? 0 : st.kb + 1;
    uint32_t ha[NC], hb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ha[c] = hl + c * cstride + st.kb * (kUnitCols * 4);
      hb[c] = hl + c * cstride + kb1 * (kUnitCols * 4);
    }
    ItemRegs<NC> r;
    lds_item(ring + f.slot * kItemBytes, ha, hb, r);
    feed_done<DEPTH>(P, cx, s, F, f);
    float d0[NC];
    mv_dot<NC>(r.w0, r.a, d0);
    mv_add<NC>(st, d0, KB, pout, pcs, icol);
    if (2 * t + 1 < w.nu) {
      float d1[NC];
      mv_dot<NC>(r.w1, r.b, d1);
      mv_add<NC>(st, d1, KB, pout, pcs, icol);
    }
  }
  if (st.pend) mv_flush<NC>(st, pout, pcs, icol, st.rb);
  return true;
}

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
                                           Feed& f, Waits& wt, const float* hin, float* part) {
  const int lane = cx.lane;
  const int D = P.D, lpp = D / 8, ppu = 64 / lpp;
  const int pg = lane / lpp, de = (lane % lpp) * 8;
  const int G = P.G;
  const float scale = P.attn_scale;
  const uint32_t ring = lds_addr(f.ring) + lane * 16;
  float qv[kMaxG][8], av[kMaxG][8], mv[kMaxG], lv[kMaxG];
  const float* q = hin + att_raw_floats(P);
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    mv[h] = -INFINITY;
    lv[h] = 0.f;
    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = x;
    if (h < G) lds_read_2x128(lds_addr(q + h * D + de), lds_addr(q + h * D + de + 4), x, y);
    qv[h][0] = x.x; qv[h][1] = x.y; qv[h][2] = x.z; qv[h][3] = x.w;
    qv[h][4] = y.x; qv[h][5] = y.y; qv[h][6] = y.z; qv[h][7] = y.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) av[h][e] = 0.f;
  }
  for (int t = 0; t < w.n; ++t) {
    if (!feed_item<DEPTH>(P, cx, s, F, f, wt)) return false;
    u32x4 wk, wv;
    lds_item_kv(ring + f.slot * kItemBytes, wk, wv);
    feed_done<DEPTH>(P, cx, s, F, f);
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
        const f32x4 lo = {av[h][0], av[h][1], av[h][2], av[h][3]};
        const f32x4 hi = {av[h][4], av[h][5], av[h][6], av[h][7]};
        lds_write_b128(lds_addr(dst + de), lo);
        lds_write_b128(lds_addr(dst + de + 4), hi);
        if (lane == 0) {
          lds_write_b32(lds_addr(dst + D), mv[h]);
          lds_write_b32(lds_addr(dst + D + 1), lv[h]);
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
  waits_init(P, wt);
  Feed f;
  f.k = 0;
  f.slot = 0;
  f.ring = cx.ring + (size_t)s * DEPTH * kItemBytes;
  Fetch F;
  walker_init(F.w, cx);
  F.issued = 0;
  F.slot = 0;
  fetch_next_task(P, cx, s, F);
  fetch_upto<DEPTH>(P, cx, s, F, DEPTH, f.ring);
  Walker w;
  walker_init(w, cx);
  const int ncols = P.batch;
  for (;;) {
    walker_next(P, w, cx, s);
    if (w.done) break;
    {
      const uint64_t s0 = waits_now(wt);
      if (!spin_raw(P, cx, C_STAGED, w.i + 1)) return;
      waits_add(wt, 2, s0);
    }
    const float* hin = slot_ptr(cx, w.slot) + kHdr;
    float* part = part_ptr(cx, w.slot);
    const uint64_t s1 = waits_now(wt);
    bool ok;
    if (w.type == T_ATT) {
      ok = stream_att<DEPTH>(P, cx, s, w, F, f, wt, hin, part);
    } else {
      const int kp = slot_kp(P, w.slot);
      switch (ncols) {
        case 1: ok = stream_matvec<DEPTH, 1>(P, cx, s, w, F, f, wt, hin, kp, part); break;
        case 2: ok = stream_matvec<DEPTH, 2>(P, cx, s, w, F, f, wt, hin, kp, part); break;
        case 3: ok = stream_matvec<DEPTH, 3>(P, cx, s, w, F, f, wt, hin, kp, part); break;
        default: ok = stream_matvec<DEPTH, 4>(P, cx, s, w, F, f, wt, hin, kp, part); break;
      }
    }
    if (!ok) return;
    if (w.type == T_LM) waits_add(wt, 5, s1);
    wt.c[3] += w.n;
    if (cx.lane == 0) lds_add_raw(lds_addr(&cx.ctl[C_DONE + w.slot]), 1);
  }
  wait_all();
  waits_put(P, cx, wt);
}
