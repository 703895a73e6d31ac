// gfx950 device code of the persistent decode megakernel (internal to libmk).
//
//  * task bodies: EMB, RMSNorm+QKV, split attention (RoPE + KV append), merge,
//    O-proj+residual, RMSNorm+gate/up+SiLU*up, down+residual, final
//    RMSNorm+LM head+partial argmax, argmax (Hazy megakernel summary: the fused
//    instruction list; MPK walk-through 3.3.1: the layer calls of one step);
//  * mk_persistent: one workgroup per compute unit walks its static task queue
//    for every step; a task waits until its dependent event's counter reaches
//    the threshold and then adds one to its triggering event (MPK blog
//    translation, "MPK runtime" section and Figure 3);
//  * mk_oplaunch: the same bodies, one launch per operator (the conventional
//    many-kernel engine the pages compare against);
//  * mk_pack: weight repacking into the streamed unit layout.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.h"
#include "graph.h"
#include "launch.h"

namespace mk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float f[8]) {
  f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
  f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
  f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ void set_status(const Params& P, int32_t bits) {
  __hip_atomic_fetch_or(P.status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Shared-memory layout of one workgroup (dynamic LDS, sized by the host).
struct Smem {
  float* in;     // [kMaxCols][Kp] staged input vector(s)
  float* part;   // [kWaves][kMaxCols][vrow_stride] matvec partial sums
  float* scal;   // 64 floats of scratch (norm scales, reductions)
  int* iscal;    // 64 ints of scratch
  float* att;    // attention scratch
  int kp;        // floats per staged column
  int vrow_stride;
  int ncap;      // staged columns (min(max_batch, kMaxCols))
};

// ---------------------------------------------------------------------------
// matvec engine: a wave streams its contiguous share of the task's units
// ---------------------------------------------------------------------------

// Each of the 4 waves takes units [U*w/4, U*(w+1)/4). Inside a unit, lane
// 16j+i multiplies its 8 weights of row j by the 8 staged inputs at the same
// columns; a row block's 16-lane partial sums are combined when the wave leaves
// the block and stored to part[wave][col][4*block + j].
__device__ void matvec_share(const Params& P, const DevTask& T, int KB, int ncols, const Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane >> 4, i = lane & 15;
  const int U = T.n_units;
  const int u0 = (U * wave) / kWaves, u1 = (U * (wave + 1)) / kWaves;
  if (u0 >= u1) return;
  const uint8_t* wb = P.wpack + T.w_off + lane * 16;
  float acc[kMaxCols];
#pragma unroll
  for (int c = 0; c < kMaxCols; ++c) acc[c] = 0.f;
  int vrb = u0 / KB, kb = u0 - vrb * KB;
  float* part = sm.part + (size_t)wave * sm.ncap * sm.vrow_stride;

  auto flush = [&](int blk) {
#pragma unroll
    for (int c = 0; c < kMaxCols; ++c) {
      if (c < ncols) {
        float v = acc[c];
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 1, 64);
        if (i == 0) part[c * sm.vrow_stride + blk * 4 + j] = v;
      }
      acc[c] = 0.f;
    }
  };

  constexpr int NB = 16;
  for (int u = u0; u < u1; u += NB) {
    u32x4 w[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (u + k < u1) w[k] = __builtin_nontemporal_load((const u32x4*)(wb + (size_t)(u + k) * kUnitBytes));
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (u + k < u1) {
        float f[8];
        unpack8(w[k], f);
#pragma unroll
        for (int c = 0; c < kMaxCols; ++c) {
          if (c < ncols) {
            const float4* hp = reinterpret_cast<const float4*>(sm.in + c * sm.kp + kb * kUnitCols + i * 8);
            const float4 h0 = hp[0], h1 = hp[1];
            float a = acc[c];
            a = fmaf(f[0], h0.x, a); a = fmaf(f[1], h0.y, a);
            a = fmaf(f[2], h0.z, a); a = fmaf(f[3], h0.w, a);
            a = fmaf(f[4], h1.x, a); a = fmaf(f[5], h1.y, a);
            a = fmaf(f[6], h1.z, a); a = fmaf(f[7], h1.w, a);
            acc[c] = a;
          }
        }
        if (++kb == KB) {
          flush(vrb);
          kb = 0;
          ++vrb;
        }
      }
    }
  }
  if (kb != 0) flush(vrb);
}

// Stage `ncols` input vectors of length K (row stride `stride`) into sm.in,
// optionally multiplied by a bf16 gain; zero-pad to Kp. When `norm`, also
// compute 1/sqrt(mean(x^2) + eps) per column into sm.scal[c].
__device__ void stage_input(const Params& P, const float* src, int stride, int K, int ncols,
                            const uint16_t* gain, bool norm, const Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int c = 0; c < ncols; ++c) {
    float ss = 0.f;
    for (int k = tid; k < sm.kp; k += kThreads) {
      float v = 0.f;
      if (k < K) {
        v = src[(size_t)c * stride + k];
        ss = fmaf(v, v, ss);
        if (gain) v *= bf2f(gain[k]);
      }
      sm.in[c * sm.kp + k] = v;
    }
    if (norm) {
      ss = wave_sum(ss);
      if (lane == 0) sm.scal[8 + c * kWaves + wave] = ss;
    }
  }
  __syncthreads();
  if (norm && tid < ncols) {
    float ss = 0.f;
    for (int w = 0; w < kWaves; ++w) ss += sm.scal[8 + tid * kWaves + w];
    sm.scal[tid] = 1.0f / sqrtf(ss / (float)K + P.eps);
  }
}

__device__ void zero_part(const Smem& sm) {
  const int n = kWaves * sm.ncap * sm.vrow_stride;
  for (int k = threadIdx.x; k < n; k += kThreads) sm.part[k] = 0.f;
}

__device__ __forceinline__ float part_sum(const Smem& sm, int c, int vrow) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += sm.part[((size_t)w * sm.ncap + c) * sm.vrow_stride + vrow];
  return s;
}

// ---------------------------------------------------------------------------
// task bodies (whole workgroup; every thread reaches every barrier)
// ---------------------------------------------------------------------------

__device__ void body_emb(const Params& P, const DevTask& T, int step) {
  const int b = T.b;
  if (b >= P.batch) return;
  int tok = step == 0 ? P.tokens_in[b] : P.tok_cur[b];
  if (tok < 0 || tok >= P.V) {
    if (threadIdx.x == 0) set_status(P, kStatusBadToken);
    tok = 0;
  }
  const uint16_t* row = P.embed + (size_t)tok * P.H;
  for (int k = threadIdx.x; k < P.H; k += kThreads) P.x[(size_t)b * P.H + k] = bf2f(row[k]);
}

// RMSNorm-fused matvecs (QKV, GU, LM) and plain ones with residual (O, D).
__device__ void body_matvec(const Params& P, const DevTask& T, int step, const Smem& sm) {
  const int ncols = P.batch;
  const int R = T.row1 - T.row0;
  int K, KB, stride;
  const float* src;
  const uint16_t* gain = nullptr;
  bool norm = false;
  switch (T.type) {
    case T_QKV: src = P.x; stride = P.H; K = P.H; KB = P.kb_h; gain = P.gains + (size_t)T.layer * 2 * P.H; norm = true; break;
    case T_GU: src = P.x; stride = P.H; K = P.H; KB = P.kb_h; gain = P.gains + ((size_t)T.layer * 2 + 1) * P.H; norm = true; break;
    case T_LM: src = P.x; stride = P.H; K = P.H; KB = P.kb_h; gain = P.gains + (size_t)P.L * 2 * P.H; norm = true; break;
    case T_O: src = P.attn; stride = P.Hq * P.D; K = P.Hq * P.D; KB = P.kb_qd; break;
    default: src = P.mlp; stride = P.F; K = P.F; KB = P.kb_f; break;  // T_D
  }
  zero_part(sm);
  stage_input(P, src, stride, K, ncols, gain, norm, sm);
  __syncthreads();
  matvec_share(P, T, KB, ncols, sm);
  __syncthreads();

  const int tid = threadIdx.x;
  if (T.type == T_QKV) {
    const int GR = (P.G + 2) * P.D;
    for (int idx = tid; idx < ncols * R; idx += kThreads) {
      const int c = idx / R, r = idx - c * R;
      P.qkv[((size_t)c * P.Hkv + T.g) * GR + T.row0 + r] = part_sum(sm, c, r) * sm.scal[c];
    }
  } else if (T.type == T_O || T.type == T_D) {
    for (int idx = tid; idx < ncols * R; idx += kThreads) {
      const int c = idx / R, r = idx - c * R;
      float* xp = P.x + (size_t)c * P.H + T.row0 + r;
      *xp = *xp + part_sum(sm, c, r);
    }
  } else if (T.type == T_GU) {
    for (int idx = tid; idx < ncols * R; idx += kThreads) {
      const int c = idx / R, r = idx - c * R;
      const int vr = 8 * (r >> 2) + (r & 3);
      const float gt = part_sum(sm, c, vr) * sm.scal[c];
      const float up = part_sum(sm, c, vr + 4) * sm.scal[c];
      P.mlp[(size_t)c * P.F + T.row0 + r] = gt / (1.0f + expf(-gt)) * up;
    }
  } else {  // T_LM: logits and this task's (max, lowest index) per column
    const bool last = step == P.n_steps - 1;
    const int lane = tid & 63, wave = tid >> 6;
    for (int c = 0; c < ncols; ++c) {
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int r = tid; r < R; r += kThreads) {
        const float v = part_sum(sm, c, r) * sm.scal[c];
        if (last && P.logits_out) P.logits_out[(size_t)c * P.V + T.row0 + r] = v;
        if (v > best || (v == best && T.row0 + r < bi)) { best = v; bi = T.row0 + r; }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
      }
      if (lane == 0) { sm.scal[40 + wave] = best; sm.iscal[40 + wave] = bi; }
      __syncthreads();
      if (tid == 0) {
        for (int w = 1; w < kWaves; ++w) {
          const float ov = sm.scal[40 + w];
          const int oi = sm.iscal[40 + w];
          if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
        }
        P.lm_val[(size_t)c * P.n_lm + T.ordinal] = best;
        P.lm_idx[(size_t)c * P.n_lm + T.ordinal] = bi;
      }
      __syncthreads();
    }
  }
}

// One attention chunk of one (kv group, sequence): rotate the group's query
// heads and the new key by the position, append K/V at the position (final
// chunk only), then softmax statistics and the value sum over the chunk's
// positions, tile by tile with a running maximum.
__device__ void body_att(const Params& P, const DevTask& T, int step, const Smem& sm) {
  const int b = T.b, g = T.g, G = P.G, D = P.D, Dh = P.D / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool active = b < P.batch;
  int p = active ? P.pos_in[b] + step : 0;
  const bool valid = active && p >= 0 && p < P.S;
  if (active && !valid && tid == 0) set_status(P, kStatusBadPos);
  if (!valid) p = 0;
  const int64_t len = (int64_t)p + 1;
  int lo = (int)((int64_t)T.chunk * len / P.Nc), hi = (int)((int64_t)(T.chunk + 1) * len / P.Nc);
  if (!valid) hi = lo;
  const bool owner = valid && T.chunk == P.Nc - 1;

  float* s_q = sm.att;                 // [G][D]
  float* s_k = s_q + G * D;            // [D]
  float* s_v = s_k + D;                // [D]
  float* s_m = s_v + D;                // [G]
  float* s_l = s_m + G;                // [G]
  float* s_sc = s_l + G;               // [G] scale of this tile
  float* s_p = s_sc + G;               // [G][kAttTile]

  const size_t kvrow = (((size_t)T.layer * P.B + b) * P.Hkv + g) * (size_t)P.S;
  const float* qsrc = P.qkv + ((size_t)b * P.Hkv + g) * (G + 2) * D;
  if (valid) {
    for (int idx = tid; idx < (G + 1) * Dh; idx += kThreads) {
      const int h = idx / Dh, jj = idx - h * Dh;
      const float* src = qsrc + h * D;  // h == G is the key
      const float a = src[jj], bb = src[jj + Dh];
      const float2 cs = P.rope_cs[(size_t)p * Dh + jj];
      const float r0 = a * cs.x - bb * cs.y, r1 = bb * cs.x + a * cs.y;
      if (h < G) {
        s_q[h * D + jj] = r0;
        s_q[h * D + jj + Dh] = r1;
      } else {
        const uint16_t k0 = f2bf(r0), k1 = f2bf(r1);
        s_k[jj] = bf2f(k0);
        s_k[jj + Dh] = bf2f(k1);
        if (owner) {
          P.kcache[(kvrow + p) * D + jj] = k0;
          P.kcache[(kvrow + p) * D + jj + Dh] = k1;
        }
      }
    }
    for (int d = tid; d < D; d += kThreads) {
      const uint16_t vb = f2bf(qsrc[(G + 1) * D + d]);
      s_v[d] = bf2f(vb);
      if (owner) P.vcache[(kvrow + p) * D + d] = vb;
    }
  }
  if (tid < G) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }
  __syncthreads();

  constexpr int kMaxPairs = 4;  // (head, dim) pairs per thread: G*D <= 1024
  float acc[kMaxPairs];
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k) acc[k] = 0.f;

  for (int t0 = lo; t0 < hi; t0 += kAttTile) {
    const int n = min(kAttTile, hi - t0);
    for (int t = tid; t < n; t += kThreads) {
      const int pos = t0 + t;
      float dot[8];
      for (int h = 0; h < G; ++h) dot[h] = 0.f;
      const uint16_t* krow = P.kcache + (kvrow + pos) * D;
      for (int d0 = 0; d0 < D; d0 += 8) {
        float kf[8];
        if (pos == p) {
          for (int e = 0; e < 8; ++e) kf[e] = s_k[d0 + e];
        } else {
          unpack8(*reinterpret_cast<const u32x4*>(krow + d0), kf);
        }
        for (int h = 0; h < G; ++h) {
          const float* q = s_q + h * D + d0;
          float a = dot[h];
          for (int e = 0; e < 8; ++e) a = fmaf(q[e], kf[e], a);
          dot[h] = a;
        }
      }
      for (int h = 0; h < G; ++h) s_p[h * kAttTile + t] = dot[h] * P.attn_scale;
    }
    __syncthreads();
    for (int h = wave; h < G; h += kWaves) {
      float mx = -INFINITY;
      for (int t = lane; t < n; t += 64) mx = fmaxf(mx, s_p[h * kAttTile + t]);
      mx = wave_max(mx);
      const float m_new = fmaxf(s_m[h], mx);
      float sum = 0.f;
      for (int t = lane; t < n; t += 64) {
        const float e = expf(s_p[h * kAttTile + t] - m_new);
        s_p[h * kAttTile + t] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float sc = expf(s_m[h] - m_new);
        s_l[h] = s_l[h] * sc + sum;
        s_m[h] = m_new;
        s_sc[h] = sc;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxPairs; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < G * D) {
        const int h = idx / D, d = idx - h * D;
        float a = acc[k] * s_sc[h];
        const float* pp = s_p + h * kAttTile;
        for (int t = 0; t < n; ++t) {
          const int pos = t0 + t;
          const float v = pos == p ? s_v[d] : bf2f(P.vcache[(kvrow + pos) * D + d]);
          a = fmaf(pp[t], v, a);
        }
        acc[k] = a;
      }
    }
    __syncthreads();
  }
  if (active) {
    for (int k = 0; k < kMaxPairs; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < G * D) {
        const int h = idx / D, d = idx - h * D;
        const size_t slot = ((size_t)b * P.Hq + g * G + h) * P.Nc + T.chunk;
        P.part_acc[slot * D + d] = acc[k];
        if (d == 0) {
          P.part_ml[slot * 2] = s_m[h];
          P.part_ml[slot * 2 + 1] = s_l[h];
        }
      }
    }
  }
}

// Merge the chunk partials of one (kv group, sequence): rescale each chunk by
// exp(m_c - max m) and divide the summed values by the summed weights.
__device__ void body_comb(const Params& P, const DevTask& T) {
  const int b = T.b;
  if (b >= P.batch) return;
  const int G = P.G, D = P.D;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    const int hq = T.g * G + h;
    const size_t base = ((size_t)b * P.Hq + hq) * P.Nc;
    float M = -INFINITY;
    for (int c = 0; c < P.Nc; ++c) M = fmaxf(M, P.part_ml[(base + c) * 2]);
    float num = 0.f, den = 0.f;
    for (int c = 0; c < P.Nc; ++c) {
      const float mc = P.part_ml[(base + c) * 2];
      if (mc == -INFINITY) continue;
      const float w = expf(mc - M);
      num = fmaf(w, P.part_acc[(base + c) * D + d], num);
      den = fmaf(w, P.part_ml[(base + c) * 2 + 1], den);
    }
    P.attn[(size_t)b * P.Hq * D + (size_t)hq * D + d] = den > 0.f ? num / den : 0.f;
  }
}

__device__ void body_argmax(const Params& P, const DevTask& T, int step, const Smem& sm) {
  const int b = T.b;
  if (b >= P.batch) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = tid; t < P.n_lm; t += kThreads) {
    const float v = P.lm_val[(size_t)b * P.n_lm + t];
    const int ix = P.lm_idx[(size_t)b * P.n_lm + t];
    if (v > best || (v == best && ix < bi)) { best = v; bi = ix; }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
  }
  if (lane == 0) { sm.scal[48 + wave] = best; sm.iscal[48 + wave] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) {
      const float ov = sm.scal[48 + w];
      const int oi = sm.iscal[48 + w];
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    if (bi < 0 || bi >= P.V) bi = 0;  // every logit was NaN
    P.out_tokens[(size_t)step * P.batch + b] = bi;
    P.tok_cur[b] = bi;
  }
}

__device__ void exec_task(const Params& P, const DevTask& T, int step, const Smem& sm) {
  switch (T.type) {
    case T_EMB: body_emb(P, T, step); break;
    case T_ATT: body_att(P, T, step, sm); break;
    case T_COMB: body_comb(P, T); break;
    case T_ARGMAX: body_argmax(P, T, step, sm); break;
    default: body_matvec(P, T, step, sm); break;
  }
}

// LDS carve-up: 64 float + 64 int scratch, staged inputs, matvec partials,
// attention scratch (sizes from Params; the host checks the total).
__device__ Smem carve(const Params& P, char* base) {
  Smem s;
  s.kp = P.kp;
  s.vrow_stride = P.vrow_stride;
  s.ncap = P.ncap;
  s.scal = reinterpret_cast<float*>(base);
  s.iscal = reinterpret_cast<int*>(base + 64 * 4);
  s.in = reinterpret_cast<float*>(base + 128 * 4);
  s.part = s.in + (size_t)P.ncap * P.kp;
  s.att = s.part + (size_t)kWaves * P.ncap * P.vrow_stride;
  return s;
}

// ---------------------------------------------------------------------------
// runtime: events
// ---------------------------------------------------------------------------

// Spin until counter[ev] >= need (acquire), bounded by the watchdog. Returns
// false when the kernel must stop (timeout here or elsewhere).
__device__ bool wait_event(const Params& P, int ev, uint32_t need) {
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const uint32_t v = __hip_atomic_load(&P.counters[ev], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int32_t)(v - need) >= 0) break;
    if (__hip_atomic_load(P.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    if (wall_clock64() - t0 > P.timeout_ticks) {
      set_status(P, kStatusTimeout);
      __hip_atomic_store(P.abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

extern "C" __global__ void __launch_bounds__(kThreads) mk_persistent(Params P) {
  extern __shared__ __align__(16) char smem_raw[];
  const Smem sm = carve(P, smem_raw);
  __shared__ int s_go;
  const int cu = blockIdx.x;
  const int q0 = P.queue_ptr[cu], q1 = P.queue_ptr[cu + 1];
  for (int step = 0; step < P.n_steps; ++step) {
    const uint32_t epoch = P.epoch0 + (uint32_t)step;
    for (int qi = q0; qi < q1; ++qi) {
      const int id = P.queue_ids[qi];
      const DevTask T = P.tasks[id];
      uint64_t t_ready = 0, t_start = 0;
      if (threadIdx.x == 0) {
        const uint32_t mult = T.type == T_EMB ? epoch : epoch + 1;
        s_go = wait_event(P, T.dep, P.thresholds[T.dep] * mult) ? 1 : 0;
        t_ready = wall_clock64();
      }
      __syncthreads();
      if (!s_go) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (threadIdx.x == 0) t_start = wall_clock64();
      exec_task(P, T, step, sm);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (threadIdx.x == 0) {
        if (id != P.drop_task)
          __hip_atomic_fetch_add(&P.counters[T.trig], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (P.profile) {
          uint64_t* rec = P.profile + ((size_t)step * P.n_tasks + id) * 4;
          rec[0] = (uint64_t)(uint32_t)id | ((uint64_t)cu << 32);
          rec[1] = t_ready;
          rec[2] = t_start;
          rec[3] = wall_clock64();
        }
      }
    }
  }
}

extern "C" __global__ void __launch_bounds__(kThreads) mk_oplaunch(Params P, int first) {
  extern __shared__ __align__(16) char smem_raw[];
  const Smem sm = carve(P, smem_raw);
  const DevTask T = P.tasks[first + blockIdx.x];
  exec_task(P, T, 0, sm);
}

// ---------------------------------------------------------------------------
// weight packing
// ---------------------------------------------------------------------------

extern "C" __global__ void __launch_bounds__(256) mk_pack(const PackJob* jobs, const PackSrc* src, uint8_t* dst,
                                                         int G, int D, int L) {
  const PackJob J = jobs[blockIdx.x];
  const int64_t lanes = (int64_t)J.n_vrb * J.KB * 64;
  const int R = J.row1 - J.row0;
  for (int64_t idx = threadIdx.x; idx < lanes; idx += blockDim.x) {
    const int64_t u = idx >> 6;
    const int lane = (int)(idx & 63);
    const int vrb = (int)(u / J.KB), kb = (int)(u - (int64_t)vrb * J.KB);
    const int j = lane >> 4, i = lane & 15;
    const int col = kb * kUnitCols + i * 8;
    int r;  // task-relative row
    const uint16_t* m = nullptr;
    int64_t row = 0;
    if (J.type == T_GU) {
      r = (vrb >> 1) * 4 + j;
      m = src[J.layer].p[(vrb & 1) ? 5 : 4];
      row = J.row0 + r;
    } else {
      r = vrb * 4 + j;
      const int ar = J.row0 + r;
      switch (J.type) {
        case T_QKV:
          if (ar < G * D) { m = src[J.layer].p[0]; row = (int64_t)J.g * G * D + ar; }
          else if (ar < (G + 1) * D) { m = src[J.layer].p[1]; row = (int64_t)J.g * D + ar - G * D; }
          else { m = src[J.layer].p[2]; row = (int64_t)J.g * D + ar - (G + 1) * D; }
          break;
        case T_O: m = src[J.layer].p[3]; row = ar; break;
        case T_D: m = src[J.layer].p[6]; row = ar; break;
        default: m = src[L].p[0]; row = ar; break;  // T_LM
      }
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && col < J.K) v = *reinterpret_cast<const u32x4*>(m + row * J.K + col);
    *reinterpret_cast<u32x4*>(dst + J.dst_off + u * kUnitBytes + lane * 16) = v;
  }
}

}  // namespace mk

// ---------------------------------------------------------------------------
// host-side launchers (called from api.cpp)
// ---------------------------------------------------------------------------
namespace mk {

hipError_t set_lds_limit(int bytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_persistent),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_oplaunch),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t persistent_occupancy(int lds, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, reinterpret_cast<const void*>(&mk_persistent),
                                                      kThreads, lds);
}

hipError_t launch_persistent(const Params& P, int grid, int lds, hipStream_t s) {
  Params p = P;
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&mk_persistent), dim3(grid), dim3(kThreads), args,
                                    lds, s);
}

hipError_t launch_op(const Params& P, int first, int count, int lds, hipStream_t s) {
  hipLaunchKernelGGL(mk_oplaunch, dim3(count), dim3(kThreads), lds, s, P, first);
  return hipGetLastError();
}

hipError_t launch_pack(const PackJob* jobs, int n_jobs, const PackSrc* src, uint8_t* dst, int G, int D, int L,
                       hipStream_t s) {
  hipLaunchKernelGGL(mk_pack, dim3(n_jobs), dim3(256), 0, s, jobs, src, dst, G, D, L);
  return hipGetLastError();
}

}  // namespace mk
