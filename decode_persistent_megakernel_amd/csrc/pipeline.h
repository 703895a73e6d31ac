// Loader / compute wave pairs of the persistent decode megakernel (included
// by kernels.hip; internal to libmk).
//
// Pair p owns every kPairs-th piece of each streamed task: matvec units
// u = p, p+kPairs, ... and attention position blocks j = p, p+kPairs, ...
// Items of 2 KiB move through an LDS ring of ring_slots entries: a matvec item
// is two of the pair's units, an attention item is the K block and the V block
// of one group of positions. A stream task in which the pair has nothing still
// gets one (empty) item so that the compute wave checks in for it.
//
// The loader copies items straight from HBM into the ring (LDS DMA) and runs
// ahead across task boundaries; it never depends on activations, only on
// free ring slots (and, for KV blocks written in an earlier step, on the
// stager having passed that step's first dependency). The compute wave walks
// the same item sequence, so nothing but two counters crosses between them:
// items published (loader -> compute) and items consumed (compute -> loader),
// both updated in batches.

// Walks the stream tasks (those with weight or KV units) of this workgroup's
// queue, across steps, for pair p, keeping the slot assignment of every task.
struct Walker {
  int step, qi, i;   // i: global task counter of the current task (all tasks)
  int nsmall, slot;
  int id, type, layer, b, g;
  int nu;            // matvec: units of pair p; attention: position blocks of pair p
  int n;             // items of pair p in the task (>= 1; an empty task has one empty item)
  int lo, end;       // attention: positions [lo, end) come from the cache
  int kb0, KB;       // matvec: column blocks; unit p's column block
  int rb0;           // matvec: unit p's row block
  int64_t woff;      // matvec: packed weight offset
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
  w.nu = w.n = 0;
  w.lo = w.end = 0;
  w.kb0 = 0;
  w.KB = 1;
  w.rb0 = 0;
  w.woff = 0;
  w.done = false;
}

__device__ __forceinline__ void walker_next(const Params& P, Walker& w, const Ctx& cx, int p) {
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
    const DevTask T = P.tasks[w.id];
    w.type = T.type;
    w.slot = next_slot(w.nsmall, w.type);
    if (!has_stream(w.type)) continue;
    w.layer = T.layer;
    w.b = T.b;
    w.g = T.g;
    w.nu = 0;
    if (w.type == T_ATT) {
      w.lo = w.end = 0;
      if (w.b < P.batch) {
        const int pos = P.pos_in[w.b] + w.step;
        if (pos >= 0 && pos < P.S) {
          const int64_t len = (int64_t)pos + 1;
          w.lo = (int)((int64_t)T.chunk * len / P.Nc);
          w.end = min((int)((int64_t)(T.chunk + 1) * len / P.Nc), pos);
          const int ppu = 512 / P.D;  // positions per unit
          const int npu = w.end > w.lo ? (w.end - w.lo + ppu - 1) / ppu : 0;
          w.nu = npu > p ? (npu - p + kPairs - 1) / kPairs : 0;
        }
      }
      w.n = max(w.nu, 1);
    } else {
      const int U = T.n_units;
      w.nu = U > p ? (U - p + kPairs - 1) / kPairs : 0;
      w.n = max((w.nu + 1) / 2, 1);
      w.KB = T.kb;
      w.rb0 = p / w.KB;
      w.kb0 = p - w.rb0 * w.KB;
      w.woff = T.w_off;
    }
    return;
  }
}

// next (row block, column block) of a pair's matvec unit sequence
__device__ __forceinline__ void unit_advance(int& rb, int& kb, int KB) {
  kb += kPairs;
  while (kb >= KB) {
    kb -= KB;
    ++rb;
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N): vmcnt bits [3:0] and [15:14], expcnt/lgkmcnt at max
  constexpr int imm = (N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Wait until at most 2*n of this wave's copies are in flight (n items).
__device__ __forceinline__ void wait_items_inflight(int n) {
  cbar();
  switch (n) {
    case 8: wait_vmcnt<16>(); break;
    case 12: wait_vmcnt<24>(); break;
    case 16: wait_vmcnt<32>(); break;
    case 20: wait_vmcnt<40>(); break;
    default: wait_vmcnt<48>(); break;
  }
  cbar();
}

constexpr int kItemBytes = 2 * kUnitBytes;

__device__ __forceinline__ void run_loader(const Params& P, const Ctx& cx, int p) {
  const int lane = cx.lane;
  const int NR = P.ring_slots, NIF = P.ring_inflight;
  const int D = P.D, lpp = D / 8, ppu = 64 / lpp;
  const int pg = lane / lpp, de = (lane % lpp) * 8;
  int* pub = &cx.ctl[C_PUB + p];
  const int* cons = &cx.ctl[C_CONS + p];
  uint8_t* ring = cx.ring + (size_t)p * NR * kItemBytes;
  const uint8_t* dummy = P.wpack + lane * 16;

  Walker w;
  walker_init(w, cx);
  walker_next(P, w, cx, p);
  int t = 0;  // item within the task

  int k = 0, slot = 0, inflight = 0, published = 0, cons_c = 0;
  auto drain = [&]() {
    wait_all();
    lds_st_raw(pub, k);
    published = k;
    inflight = 0;
  };
  auto wait_for = [&](const int* word, int v) -> bool {
    drain();
    const uint64_t t0 = wall_clock64();
    while (lds_ld_raw(word) < v) {
      if (lds_ld_raw(&cx.ctl[C_ABORT])) return false;
      if (wall_clock64() - t0 > P.timeout_ticks) { raise_abort(P, cx, kStatusTimeout); return false; }
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };

  while (!w.done) {
    if (k - NR + 1 > cons_c) {
      cons_c = lds_ld_raw(cons);
      if (k - NR + 1 > cons_c) {
        if (!wait_for(cons, k - NR + 1)) return;
        cons_c = lds_ld_raw(cons);
      }
    }
    if (t == 0 && w.type == T_ATT && w.nu > 0 && lds_ld_raw(&cx.ctl[C_STEPOK]) < w.step + 1 &&
        !wait_for(&cx.ctl[C_STEPOK], w.step + 1))
      return;
    uint8_t* dst = ring + (size_t)slot * kItemBytes;
    if (w.type == T_ATT) {
      if (w.nu > 0) {
        const int j = p + t * kPairs;
        const int pos = min(w.lo + j * ppu + pg, w.end - 1);
        const size_t off = ((((size_t)w.layer * P.B + w.b) * P.Hkv + w.g) * (size_t)P.S + pos) * D + de;
        dma16<kAuxCoherent>(P.kcache + off, dst);
        dma16<kAuxCoherent>(P.vcache + off, dst + kUnitBytes);
      } else {
        dma16<0>(dummy, dst);
        dma16<0>(dummy, dst + kUnitBytes);
      }
    } else {
      const int u0 = 2 * t;  // pair-local unit index
      if (u0 < w.nu) {
        dma16<kAuxStream>(P.wpack + w.woff + (int64_t)(p + u0 * kPairs) * kUnitBytes + lane * 16, dst);
      } else {
        dma16<0>(dummy, dst);
      }
      if (u0 + 1 < w.nu) {
        dma16<kAuxStream>(P.wpack + w.woff + (int64_t)(p + (u0 + 1) * kPairs) * kUnitBytes + lane * 16,
                          dst + kUnitBytes);
      } else {
        dma16<0>(dummy, dst + kUnitBytes);
      }
    }
    ++k;
    if (++slot == NR) slot = 0;
    if (++inflight > NIF) {
      wait_items_inflight(NIF);
      inflight = NIF;
      if (k - NIF - published >= 2) {
        published = k - NIF;
        lds_st_raw(pub, published);
      }
    }
    if (++t == w.n) {
      walker_next(P, w, cx, p);
      t = 0;
    }
  }
  drain();
}

__device__ __forceinline__ void run_compute(const Params& P, const Ctx& cx, int p) {
  const int lane = cx.lane;
  const int NR = P.ring_slots;
  const int D = P.D, lpp = D / 8, ppu = 64 / lpp;
  const int pg = lane / lpp, de = (lane % lpp) * 8;  // attention: position in unit, first dim
  const int jrow = lane >> 4, icol = lane & 15;      // matvec: row in block, column group
  const int G = P.G, ncols = P.batch;
  const float scale = P.attn_scale;
  int* cons = &cx.ctl[C_CONS + p];
  const uint8_t* ring = cx.ring + (size_t)p * NR * kItemBytes;

  float acc[kMaxCols];
  float qv[kMaxG][8], av[kMaxG][8], mv[kMaxG], lv[kMaxG];
#pragma unroll
  for (int c = 0; c < kMaxCols; ++c) acc[c] = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    mv[h] = -INFINITY;
    lv[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { av[h][e] = 0.f; qv[h][e] = 0.f; }
  }
  int cur_rb = -1;
  const float* hin = cx.slots + kHdr;
  float* pbase = cx.parts;
  int kp = P.kp;

  auto flush = [&]() {
    if (cur_rb < 0) return;
#pragma unroll
    for (int c = 0; c < kMaxCols; ++c) {
      if (c < ncols) {
        float v = acc[c];
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 1, 64);
        if (icol == 0) pbase[((size_t)p * P.ncap + c) * P.vrow_stride + cur_rb * 4 + jrow] = v;
      }
      acc[c] = 0.f;
    }
  };
  auto matvec_unit = [&](const u32x4 wv, int rb, int kb) {
    if (rb != cur_rb) {
      flush();
      cur_rb = rb;
    }
    float f[8];
    unpack8(wv, f);
#pragma unroll
    for (int c = 0; c < kMaxCols; ++c) {
      if (c < ncols) {
        const float4* hp = reinterpret_cast<const float4*>(hin + (size_t)c * kp + kb * kUnitCols + icol * 8);
        const float4 h0 = hp[0], h1 = hp[1];
        float a = acc[c];
        a = fmaf(f[0], h0.x, a); a = fmaf(f[1], h0.y, a);
        a = fmaf(f[2], h0.z, a); a = fmaf(f[3], h0.w, a);
        a = fmaf(f[4], h1.x, a); a = fmaf(f[5], h1.y, a);
        a = fmaf(f[6], h1.z, a); a = fmaf(f[7], h1.w, a);
        acc[c] = a;
      }
    }
  };

  Walker w;
  walker_init(w, cx);
  int k = 0, slot = 0, pub_c = 0, released = 0;
  auto release = [&]() {
    if (released != k) {
      lds_st(cons, k);
      released = k;
    }
  };

  for (;;) {
    walker_next(P, w, cx, p);
    if (w.done) break;
    int rb = w.rb0, kb = w.kb0;
    for (int t = 0; t < w.n; ++t) {
      if (k >= pub_c) {
        release();
        if (!spin_ctl(P, cx, C_PUB + p, k + 1)) return;
        pub_c = lds_ld(&cx.ctl[C_PUB + p]);
      }
      const uint8_t* item = ring + (size_t)slot * kItemBytes + lane * 16;
      const u32x4 wa = *reinterpret_cast<const u32x4*>(item);
      const u32x4 wb = *reinterpret_cast<const u32x4*>(item + kUnitBytes);
      if (t == 0) {
        release();
        if (!spin_ctl(P, cx, C_STAGED, w.i + 1)) return;
        hin = slot_ptr(cx, w.slot) + kHdr;
        pbase = part_ptr(cx, w.slot);
        kp = slot_kp(P, w.slot);
        cur_rb = -1;
#pragma unroll
        for (int c = 0; c < kMaxCols; ++c) acc[c] = 0.f;
        if (w.type == T_ATT) {
          const float* q = hin + att_raw_floats(P);
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) {
            mv[h] = -INFINITY;
            lv[h] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              av[h][e] = 0.f;
              qv[h][e] = h < G ? q[h * D + de + e] : 0.f;
            }
          }
        }
      }
      if (w.type == T_ATT) {
        if (w.nu > 0) {
          const int j = p + t * kPairs;
          const bool valid = w.lo + j * ppu + pg < w.end;
          float kf[8], vf[8];
          unpack8(wa, kf);
          unpack8(wb, vf);
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) {
            if (h < G) {
              float d = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) d = fmaf(qv[h][e], kf[e], d);
              for (int o = 1; o < lpp; o <<= 1) d += __shfl_xor(d, o, 64);
              const float s = valid ? d * scale : -INFINITY;
              const float mn = fmaxf(mv[h], s);
              const float al = mn == -INFINITY ? 1.f : expf(mv[h] - mn);
              const float pe = s == -INFINITY ? 0.f : expf(s - mn);
              lv[h] = fmaf(lv[h], al, pe);
#pragma unroll
              for (int e = 0; e < 8; ++e) av[h][e] = fmaf(pe, vf[e], av[h][e] * al);
              mv[h] = mn;
            }
          }
        }
      } else if (2 * t < w.nu) {
        matvec_unit(wa, rb, kb);
        unit_advance(rb, kb, w.KB);
        if (2 * t + 1 < w.nu) {
          matvec_unit(wb, rb, kb);
          unit_advance(rb, kb, w.KB);
        }
      }
      ++k;
      if (++slot == NR) slot = 0;
      if (k - released >= 4) release();
      if (t == w.n - 1) {
        if (w.type == T_ATT) {
          // merge the position groups of the wave (lanes with equal dims)
          for (int o = lpp; o < 64; o <<= 1) {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
              if (h < G) {
                const float m2 = __shfl_xor(mv[h], o, 64), l2 = __shfl_xor(lv[h], o, 64);
                const float M = fmaxf(mv[h], m2);
                const float a1 = mv[h] == -INFINITY ? 0.f : expf(mv[h] - M);
                const float a2 = m2 == -INFINITY ? 0.f : expf(m2 - M);
                lv[h] = lv[h] * a1 + l2 * a2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const float o2 = __shfl_xor(av[h][e], o, 64);
                  av[h][e] = av[h][e] * a1 + o2 * a2;
                }
                mv[h] = M;
              }
            }
          }
          const int stride = G * (D + 2);
          if (pg == 0) {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
              if (h < G) {
                float* dst = pbase + p * stride + h * (D + 2);
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[de + e] = av[h][e];
                if (lane == 0) {
                  dst[D] = mv[h];
                  dst[D + 1] = lv[h];
                }
              }
            }
          }
        } else {
          flush();
        }
        lds_add(&cx.ctl[C_DONE + w.slot], 1);
      }
    }
  }
  release();
}
