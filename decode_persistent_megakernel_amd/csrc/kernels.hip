// gfx950 device code of the persistent decode megakernel (internal to libmk).
//
// One workgroup per compute unit runs that unit's static task queue for every
// decode step (MPK blog translation, "MPK runtime" section and Figure 3: a
// worker per SM with its own queue; a task waits for its dependent event and
// counts its triggering event on completion). The workgroup is split by wave:
//
//  * wave 0, the stager: for each task in queue order it waits until the task's
//    dependent event reaches its threshold, then stages the task's inputs into
//    an LDS slot (RMSNorm statistics and gains applied on the way in, RoPE
//    applied to attention inputs);
//  * wave 1, the retirer: once a task's compute is done it runs the epilogue
//    (partial-sum reduction, residual add, SiLU*up, attention merge, argmax),
//    stores the results and adds one to the task's triggering event;
//  * kStreams stream waves: each loads its share of every task's weight (or
//    KV cache) units into a ring of registers and computes on them, loading
//    ahead across task boundaries so weights keep arriving while the
//    workgroup waits on an event (Hazy megakernel summary: the next
//    instruction's weights load early; MPK blog translation: loads of the
//    next layer overlap the current one).
//
// Cross-compute-unit data moves with device-coherent (sc1) loads and stores;
// a producer waits for its stores to complete before it counts the event, and
// a consumer reads the inputs only after it has seen the count, so no cache
// writeback or invalidate is needed. Event counters are split into 64 stripes
// (four producer CUs of one XCD per stripe) to spread the atomic traffic; a
// poll reads all of them with one load per lane.
//
// mk_oplaunch runs the same roles on a one-task queue per workgroup with no
// event waits: one launch per operator (the conventional many-kernel engine
// that the MPK blog translation's introduction and Figure 1 measure against). mk_pack repacks the weights into units.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>

#include "mk.h"
#include "device.h"
#include "graph.h"
#include "launch.h"

namespace mk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kAuxCoherent = 16;   // sc1
constexpr int kAuxStream = 2;      // nt
constexpr int kHdr = 32;           // floats of header at the start of a slot

// LDS control words (ints)
enum { C_STAGED = 0, C_RETIRED = 1, C_DONE = 2 /* 3 slots */, C_STEPOK = 5, C_ABORT = 6, kCtlWords = 64 };
// then the waves' wait counters (kWaitWords each), then the stream waves'
// per-task timestamps for the profile (3 slots x kStreams x {start, first item, end, -})
constexpr int kProfCtl = kCtlWords + kWaves * kWaitWords;
// then, per slot and stream wave, the row blocks its piece of the task touched
constexpr int kPieceCtl = kProfCtl + 3 * kStreams * 4;
static_assert((kPieceCtl + 3 * kStreams * 2) * 4 <= kCtlBytes, "control area");
// then eight bf16 ones (16 bytes): the gains of inputs that are not normalised
// (matrix-core bodies)
constexpr int kOnesCtl = 240;
static_assert(kOnesCtl >= kPieceCtl + 3 * kStreams * 2 && (kOnesCtl + 4) * 4 <= kCtlBytes, "control area");
// slot header fields (as int)
enum { H_P = 8, H_LO = 9, H_END = 10, H_FLAGS = 11, H_NIN = 12 };

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ void cbar() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }
// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt left at their maximum)
__device__ __forceinline__ void wait_lgkm() { cbar(); __builtin_amdgcn_s_waitcnt(0xC07F); cbar(); }
__device__ __forceinline__ void wait_all() { cbar(); __builtin_amdgcn_s_waitcnt(0); cbar(); }

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ void unpack8(const u32x4 w, float f[8]) {
  f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
  f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
  f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
}

// ---- cross-lane exchange without the LDS crossbar ---------------------------
// DPP lane moves inside rows of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppSwap1 = 0xB1;        // quad_perm [1,0,3,2]: lane i <- i^1
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2,3,0,1]: lane i <- i^2
constexpr int kDppRor8 = 0x128;        // row_ror:8: lane i <- i^8 within each 16
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within each 16

// For lanes paired by xor o, the two values ordered (lane with bit o clear,
// lane with bit o set): the same ordered pair in both lanes, so any function
// of it gives both lanes the same result. o = 16 and 32 use the permlane
// swaps (each returns exactly that pair); o = 4 goes through the crossbar.
template <int O>
__device__ __forceinline__ void xpair(float v, float& lo, float& hi) {
  if constexpr (O == 16 || O == 32) {
    const auto r = O == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    float p;
    if constexpr (O == 1) p = dpp<kDppSwap1>(v);
    else if constexpr (O == 2) p = dpp<kDppSwap2>(v);
    else if constexpr (O == 8) p = dpp<kDppRor8>(v);
    else p = __shfl_xor(v, O, 64);
    const bool upper = (threadIdx.x & O) != 0;
    lo = upper ? p : v;
    hi = upper ? v : p;
  }
}

// Sum over the 16 lanes of each row (every lane of the row gets it).
__device__ __forceinline__ float sum16(float v) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<kDppSwap1>(v));
  v = fmaxf(v, dpp<kDppSwap2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}
// Sum over aligned groups of n lanes (n a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n >= 2) v += dpp<kDppSwap1>(v);
  if (n >= 4) v += dpp<kDppSwap2>(v);
  if (n >= 8) v += dpp<kDppHalfMirror>(v);
  if (n >= 16) v += dpp<kDppMirror>(v);
  float lo, hi;
  if (n >= 32) { xpair<16>(v, lo, hi); v = lo + hi; }
  if (n >= 64) { xpair<32>(v, lo, hi); v = lo + hi; }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }
// Largest value and, among equal values, the smallest index, over the wave
// (every lane gets it).
template <int O>
__device__ __forceinline__ void argmax_step(float& best, int& bi) {
  float v1, v2, i1, i2;
  xpair<O>(best, v1, v2);
  xpair<O>(__int_as_float(bi), i1, i2);
  const int j1 = __float_as_int(i1), j2 = __float_as_int(i2);
  const bool take2 = v2 > v1 || (v2 == v1 && j2 < j1);
  best = take2 ? v2 : v1;
  bi = take2 ? j2 : j1;
}
__device__ __forceinline__ void wave_argmax(float& best, int& bi) {
  argmax_step<1>(best, bi);
  argmax_step<2>(best, bi);
  argmax_step<4>(best, bi);
  argmax_step<8>(best, bi);
  argmax_step<16>(best, bi);
  argmax_step<32>(best, bi);
}

// The kernel arguments read through a pointer the compiler cannot prove equal
// to any earlier one. Each role takes a fresh view at the top of its per-task
// loop, so the fields are loaded again there (scalar loads from the argument
// segment, which stays unchanged for the whole launch) instead of being held
// in scalar registers across the whole kernel, where they spilled to vector
// lanes. Only the kernels that run the roles (mk_persistent*, mk_oplaunch*)
// call this; each takes its Params as the first argument, which the HSA kernel
// ABI places at offset 0 of the argument segment.
__device__ __forceinline__ const Params& fresh_params() {
  using KP = const __attribute__((address_space(4))) Params*;
  KP p = (KP)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const Params*)p;
}

template <class T>
__device__ __forceinline__ T ld_coh(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_coh(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// 1 KiB per wave: lane l copies 16 bytes from its own address src into
// lds_dst + 16*l (lds_dst is wave-uniform).
template <int AUX>
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const gvoid*)src, (lvoid*)lds_dst, 16, 0, AUX);
}

// Control words are read as wave-uniform values (readfirstlane), so that
// every loop and branch on them is scalar control flow.
__device__ __forceinline__ int lds_ld(const int* p) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// lane 0 only; earlier LDS accesses of this wave complete first
__device__ __forceinline__ void lds_st(int* p, int v) {
  wait_lgkm();
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  wait_lgkm();
}
__device__ __forceinline__ void lds_add(int* p, int v) {
  wait_lgkm();
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  wait_lgkm();
}
// The same without a lane-dependent branch, for loops whose control must stay
// uniform: the add runs with only lane 0 enabled (exec set and restored inside
// the block), after this wave's earlier LDS accesses, and completes in it.
__device__ __forceinline__ void lds_add_lane0(int* p, int v) {
  uint64_t saved;
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "ds_add_u32 %1, %2\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p), "v"(v)
      : "memory");
}

// LDS word access for the loader waves. Their LDS DMA is tracked by vmcnt and
// the compiler would otherwise drain it before every LDS access; these blocks
// complete their own access (lgkmcnt) before they end.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ int lds_ld_raw(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void lds_st_raw(int* p, int v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

struct Ctx {
  int* ctl;
  float* slots;    // small0 | small1 | big
  float* parts;    // three partial-sum areas
  int small_floats, part_floats;
  StreamRec* recs; // this queue's stream records (LDS)
  int nrec;
  int cu;          // stripe / profile id
  int single;      // >= 0: the one task this workgroup runs (per-operator mode)
  int q0, q1;      // queue range
  int lane;
};

// Graph tables and call inputs are read-only while a kernel runs. Reading them
// through the constant address space with a wave-uniform index makes them
// scalar loads (lgkmcnt): a vector load would share vmcnt with a stream
// wave's in-flight weight loads, and waiting for it would drain them.
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const i32x4 ci32x4;
static_assert(sizeof(DevTask) == 64, "task descriptors are four 16-byte words");
__device__ __forceinline__ int ld_uniform(const int32_t* p, int idx) {
  return ((cint32*)p)[__builtin_amdgcn_readfirstlane(idx)];
}
__device__ __forceinline__ DevTask ld_task(const Params& P, int id) {
  ci32x4* src = (ci32x4*)P.tasks + 4 * __builtin_amdgcn_readfirstlane(id);
  i32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = src[i];
  DevTask T;
  __builtin_memcpy(&T, w, sizeof(T));
  return T;
}

__device__ __forceinline__ int task_at(const Params& P, const Ctx& cx, int qi) {
  return cx.single >= 0 ? cx.single : ld_uniform(P.queue_ids, qi);
}

// floor(c * len / Nc), the first position of attention chunk c of a sequence
// of len positions (c <= Nc <= 256 and len <= 2^22 keep the product in 32 bits).
__device__ __forceinline__ int chunk_bound(int c, int64_t len, int Nc) {
  return (int)((uint32_t)c * (uint32_t)len / (uint32_t)Nc);
}

// Position of column b at `step` (prefill: consecutive positions of one
// sequence from pre_p0), and the column's row index in the KV caches (prefill:
// every column is the one sequence whose rows kcache / vcache point at).
__device__ __forceinline__ int call_pos(const Params& P, int b, int step) {
  return P.prefill ? P.pre_p0 + b : ld_uniform(P.pos_in, b) + step;
}
__device__ __forceinline__ int kv_row_b(const Params& P, int b) { return P.prefill ? 0 : b; }

// Positions attention chunk c of a column at position p streams from the KV
// cache: decode, the chunk's share of [0, p + 1) below p - 1 (p - 1 and p are
// staged); prefill, the chunk's share of [0, pre_p0) (the positions of this
// call's columns up to p are staged from this step's projections).
__device__ __forceinline__ void att_stream_range(const Params& P, int chunk, int p, int& lo, int& end) {
  if (P.prefill) {
    lo = chunk_bound(chunk, P.pre_p0, P.Nc);
    end = chunk_bound(chunk + 1, P.pre_p0, P.Nc);
  } else {
    const int64_t len = (int64_t)p + 1;
    lo = chunk_bound(chunk, len, P.Nc);
    end = max(lo, min(chunk_bound(chunk + 1, len, P.Nc), p - 1));
  }
}

// Staging slots: two small ones (0, 1), the merge slot (2) and the
// down-projection slot (3), which overlays all three: [small 0][small 1][merge]
// in LDS, with the down-projection input starting at small 0. A task of slot 3
// is staged once every earlier task has retired, and every later task waits
// for it (its dependency event implies both); the other slots are disjoint.
// Slot 3 shares slot 2's control words, partial sums and profile words (merge
// tasks use none of them).
enum { kSlotMerge = 2, kSlotDown = 3 };
__device__ __forceinline__ int ctl_slot(int slot) { return slot == kSlotDown ? kSlotMerge : slot; }
// Staging slot of the next task: the small slots alternate over the whole walk
// of the queue (across steps). The stream waves' records carry the assignment
// of the first step and whether it flips from one step to the next.
__device__ __forceinline__ int next_slot(int& nsmall, int type) {
  if (type == T_D) return kSlotDown;
  if (type == T_COMB) return kSlotMerge;
  return (nsmall++) & 1;
}
__device__ __forceinline__ int slot_kp(const Params& P, int slot) { return slot == kSlotDown ? P.kp_big : P.kp; }
__device__ __forceinline__ float* slot_ptr(const Ctx& cx, int slot) {
  return slot == kSlotDown ? cx.slots : cx.slots + slot * cx.small_floats;
}
__device__ __forceinline__ float* part_ptr(const Ctx& cx, int slot) { return cx.parts + ctl_slot(slot) * cx.part_floats; }

__device__ __forceinline__ void raise_abort(const Params& P, const Ctx& cx, int32_t status_bits) {
  if (cx.lane == 0) {
    if (status_bits) __hip_atomic_fetch_or(P.status, status_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(P.abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&cx.ctl[C_ABORT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Spin until ctl[w] >= v. Bounded by the watchdog; false = leave the kernel.
__device__ __forceinline__ bool spin_ctl(const Params& P, const Ctx& cx, int w, int v) {
  if (lds_ld(&cx.ctl[w]) >= v) { cbar(); return true; }
  const uint64_t t0 = wall_clock64();
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    if (lds_ld(&cx.ctl[w]) >= v) break;
    if (lds_ld(&cx.ctl[C_ABORT])) return false;
    if (wall_clock64() - t0 > P.timeout_ticks) { raise_abort(P, cx, kStatusTimeout); return false; }
  }
  cbar();
  return true;
}

// Optional per-wave wait accounting (diagnostics): counters of 100 MHz ticks
// (or counts) kept in this wave's words of the LDS control area, so that they
// hold no registers; added into P.waits when the wave finishes.
__device__ __forceinline__ uint32_t rfl32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

struct Waits {
  uint32_t* c;  // kWaitWords words; word 4 holds the start time, then the lifetime
  bool on;
};
__device__ __forceinline__ uint32_t* waits_area(const Ctx& cx) {
  return reinterpret_cast<uint32_t*>(cx.ctl) + kCtlWords + (threadIdx.x >> 6) * kWaitWords;
}
template <bool PROF>
__device__ __forceinline__ void waits_init(const Params& P, const Ctx& cx, Waits& w) {
  w.on = PROF && P.waits != nullptr;
  w.c = waits_area(cx);
  if (w.on) w.c[4] = rfl32((uint32_t)wall_clock64());
}
__device__ __forceinline__ uint64_t waits_now(const Waits& w) { return w.on ? wall_clock64() : 0; }
// every lane reads and stores the same value (no lane-dependent branch)
__device__ __forceinline__ void waits_count(Waits& w, int j, uint32_t n) {
  if (w.on) {
    const uint32_t v = rfl32(w.c[j]) + n;
    wait_lgkm();
    w.c[j] = v;
  }
}
__device__ __forceinline__ void waits_add(Waits& w, int j, uint64_t since) {
  if (w.on) waits_count(w, j, (uint32_t)(wall_clock64() - since));
}
__device__ __forceinline__ void waits_put(const Params& P, const Ctx& cx, const Waits& w) {
  if (!w.on || cx.lane != 0) return;
  uint64_t* o = P.waits + ((size_t)cx.cu * kWaves + (threadIdx.x >> 6)) * kWaitWords;
  const uint32_t life = (uint32_t)wall_clock64() - w.c[4];
  for (int j = 0; j < kWaitWords; ++j)
    __hip_atomic_fetch_add(&o[j], (uint64_t)(j == 4 ? life : w.c[j]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t* prof_words(const Ctx& cx, int slot, int s) {
  return reinterpret_cast<uint32_t*>(cx.ctl) + kProfCtl + (ctl_slot(slot) * kStreams + s) * 4;
}

__device__ __forceinline__ int* piece_words(const Ctx& cx, int slot, int s) {
  return cx.ctl + kPieceCtl + (ctl_slot(slot) * kStreams + s) * 2;
}

__device__ __forceinline__ bool has_stream(int type) {
  return type == T_QKV || type == T_O || type == T_GU || type == T_D || type == T_LM || type == T_ATT;
}

// ---------------------------------------------------------------------------
// stager (wave 0)
// ---------------------------------------------------------------------------

// Wait until the striped counter of `ev` reaches `need` (coherent polling).
__device__ __forceinline__ bool wait_event(const Params& P, const Ctx& cx, int ev, uint32_t need) {
  const uint64_t t0 = wall_clock64();
  // each lane reads one stripe; the abort word is read in the same round trip
  static_assert(kStripes == 64, "one stripe per lane");
  const uint32_t* src = &P.counters[(size_t)ev * kEventWords + cx.lane * 32];
  for (;;) {
    uint32_t v = ld_coh(src);
    const uint32_t aborted = __builtin_amdgcn_readfirstlane(ld_coh(P.abort_flag));
    // sum over the wave (integer adds, any order)
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppSwap1, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppSwap2, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xF, 0xF, false);
    {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      v = r[0] + r[1];
    }
    {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      v = r[0] + r[1];
    }
    v = __builtin_amdgcn_readfirstlane(v);
    if ((int32_t)(v - need) >= 0) break;
    if (aborted || lds_ld(&cx.ctl[C_ABORT])) {
      if (cx.lane == 0) __hip_atomic_store(&cx.ctl[C_ABORT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
    if (wall_clock64() - t0 > P.timeout_ticks) { raise_abort(P, cx, kStatusTimeout); return false; }
    __builtin_amdgcn_s_sleep(1);
  }
  cbar();
  return true;
}

// DMA `n` floats (coherent) from global src into LDS dst (both 16-byte
// aligned), in whole 1 KiB pieces: up to 255 floats past n are read (every
// activation buffer has slack) and written (every LDS region is sized for it).
// (wait = false: the copy is left in flight, for a later copy's wait to cover)
__device__ __forceinline__ void stage_copy(const Ctx& cx, const float* src, float* dst, int n, bool wait = true) {
  const int nl = (n + 255) / 256;
  for (int t = 0; t < nl; ++t) dma16<kAuxCoherent>(src + t * 256 + cx.lane * 4, dst + t * 256);
  if (wait) wait_all();
}

// Work of a matvec task that does not depend on its event, done while the
// stager waits for it: clear the slot's partial sums and, for tasks whose
// input is RMS-normalised, load this lane's gains.
struct StagePre {
  uint2 g[16];  // bf16 gains of columns (lane + 64 t) * 4 .. +4 (hidden <= 4096)
};
__device__ __forceinline__ bool is_normed(int type) { return type == T_QKV || type == T_GU || type == T_LM; }

__device__ __forceinline__ void stage_matvec_pre(const Params& P, const Ctx& cx, const DevTask& T, int slot,
                                                 StagePre& pre) {
  const int lane = cx.lane;
  (void)slot;
  if (is_normed(T.type)) {
    const uint16_t* gain = P.gains + (T.type == T_LM ? (size_t)P.L * 2 * P.H
                                                     : ((size_t)T.layer * 2 + (T.type == T_GU)) * P.H);
    const int K = T.kdim;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int k0 = (lane + 64 * t) * 4;
      pre.g[t] = k0 < K ? *reinterpret_cast<const uint2*>(gain + k0) : make_uint2(0u, 0u);
    }
  }
}

// NC: sequences staged, the call's batch (each kernel variant runs one batch size)
template <int NC>
__device__ __forceinline__ void stage_matvec(const Params& P, const Ctx& cx, const DevTask& T, int slot,
                                             const StagePre& pre) {
  float* hdr = slot_ptr(cx, slot);
  const int kp = slot_kp(P, slot);
  float* in = hdr + kHdr;
  float* res = in + (size_t)P.ncap * kp;
  const int lane = cx.lane;
  constexpr int ncols = NC;
  const int K = T.kdim;
  if (is_normed(T.type)) {
    for (int c = 0; c < ncols; ++c) {
      const rsrc_t r = make_rsrc(P.x + (size_t)c * P.H, (uint32_t)P.H * 4);
      const int nl = (K + 255) / 256;  // <= 16 (H <= 4096)
      u32x4 buf[16];
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (t < nl) buf[t] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64 * t) * 16, 0, kAuxCoherent);
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        if (t < nl) {
          const int k0 = (lane + 64 * t) * 4;
          float4 v;
          v.x = __uint_as_float(buf[t].x); v.y = __uint_as_float(buf[t].y);
          v.z = __uint_as_float(buf[t].z); v.w = __uint_as_float(buf[t].w);
          if (k0 < K) {
            ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss); ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
            const uint2 gg = pre.g[t];
            v.x *= bf2f(gg.x & 0xffffu); v.y *= bf2f(gg.x >> 16); v.z *= bf2f(gg.y & 0xffffu); v.w *= bf2f(gg.y >> 16);
          } else {
            v = make_float4(0.f, 0.f, 0.f, 0.f);
          }
          *reinterpret_cast<float4*>(in + (size_t)c * kp + k0) = v;
        }
      }
      for (int k = nl * 256 + lane * 4; k < kp; k += 256)
        *reinterpret_cast<float4*>(in + (size_t)c * kp + k) = make_float4(0.f, 0.f, 0.f, 0.f);
      ss = wave_sum(ss);
      if (lane == 0) hdr[c] = 1.0f / sqrtf(ss / (float)K + P.eps);
    }
  } else {  // O (attention output) or D (SiLU*up), plus the residual rows
    const float* src = T.type == T_O ? P.attn : P.mlp;
    const int R = T.row1 - T.row0;
    // every column's input copy and residual rows in one round trip
    float rv[NC];
    const int nl = (K + 255) / 256;
#pragma unroll
    for (int c = 0; c < ncols; ++c) {
      rv[c] = 0.f;
      if (lane < R) rv[c] = ld_coh(P.x + (size_t)c * P.H + T.row0 + lane);
      for (int t = 0; t < nl; ++t) dma16<kAuxCoherent>(src + (size_t)c * K + t * 256 + lane * 4, in + (size_t)c * kp + t * 256);
    }
    wait_all();
#pragma unroll
    for (int c = 0; c < ncols; ++c) {
      for (int k = K + lane; k < kp; k += 64) in[(size_t)c * kp + k] = 0.f;
      if (lane < R) res[(size_t)c * P.res_stride + lane] = rv[c];
      for (int r = 64 + lane; r < R; r += 64) res[(size_t)c * P.res_stride + r] = ld_coh(P.x + (size_t)c * P.H + T.row0 + r);
    }
  }
}

// Matrix-core bodies (up to 16 sequences): the stream waves read the
// activations straight from global memory, so staging a matvec task leaves
// in the slot only what every wave shares: for an RMS-normalised input, the
// per-sequence factor 1/rms (header words 0..15, from the sums of squares the
// producing tasks wrote) and the gains [K] as bf16 after the header; for the
// O and down projections, the residual rows [16][res_stride].
__device__ __forceinline__ void stage_matvec_m16(const Params& P, const Ctx& cx, const DevTask& T, int slot) {
  float* hdr = slot_ptr(cx, slot);
  float* data = hdr + kHdr;
  const int lane = cx.lane;
  if (is_normed(T.type)) {
    // sums of squares: part t, sequences 4q..4q+3 in lane 4t' + q (fixed order:
    // each lane adds its parts in turn, then the lanes of one q are added in a
    // fixed butterfly)
    const int nparts = T.type == T_GU ? P.n_ss_o : (T.type == T_QKV && T.layer == 0 ? 1 : P.n_ss_d);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const rsrc_t r = make_rsrc(P.ssq, (uint32_t)nparts * kMfmaCols * 4);
    for (int t0 = 0; t0 < nparts; t0 += 256) {
      u32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)((t0 + 16 * i + (lane >> 2)) * kMfmaCols + (lane & 3) * 4) * 4u,
                                                    0, kAuxCoherent);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc.x += __uint_as_float(v[i].x); acc.y += __uint_as_float(v[i].y);
        acc.z += __uint_as_float(v[i].z); acc.w += __uint_as_float(v[i].w);
      }
    }
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) {
      acc.x += __shfl_xor(acc.x, o); acc.y += __shfl_xor(acc.y, o);
      acc.z += __shfl_xor(acc.z, o); acc.w += __shfl_xor(acc.w, o);
    }
    if (lane < 4) {
      const float inv_k = 1.0f / (float)T.kdim;
      hdr[lane * 4 + 0] = 1.0f / sqrtf(acc.x * inv_k + P.eps);
      hdr[lane * 4 + 1] = 1.0f / sqrtf(acc.y * inv_k + P.eps);
      hdr[lane * 4 + 2] = 1.0f / sqrtf(acc.z * inv_k + P.eps);
      hdr[lane * 4 + 3] = 1.0f / sqrtf(acc.w * inv_k + P.eps);
    }
    const uint16_t* gain = P.gains + (T.type == T_LM ? (size_t)P.L * 2 * P.H
                                                     : ((size_t)T.layer * 2 + (T.type == T_GU)) * P.H);
    const int nl = (T.kdim * 2 + 1023) / 1024;  // 1 KiB pieces (the gains buffer has slack)
    for (int t = 0; t < nl; ++t) dma16<0>(gain + t * 512 + lane * 8, data + t * 256);
    wait_all();
  } else {  // O, D: the residual rows of the call's sequences (eight loads in flight per lane)
    const int R = T.row1 - T.row0, total = P.batch * R;
    const rsrc_t rx = make_rsrc(P.x, (uint32_t)P.batch * (uint32_t)P.H * 4u);
    for (int q0 = 0; q0 < total; q0 += 512) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = q0 + 64 * i + lane, m = q / R, r = q - m * R;
        const uint32_t off = q < total ? (uint32_t)(m * P.H + T.row0 + r) * 4u : 0xfffffff0u;  // out of range: 0
        v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, kAuxCoherent));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = q0 + 64 * i + lane, m = q / R, r = q - m * R;
        if (q < total) data[(size_t)m * P.res_stride + r] = v[i];
      }
    }
  }
}

// Attention slot layout after the header: raw q|k|v of the kv group (rounded
// up to 256 floats), rotated queries [G][D], new key [D] and value [D] as
// bf16-rounded floats, their bf16 bits [2D], the key [D] and value [D] of
// position p - 1 read back from the cache, then the rotated queries again,
// scaled by log2(e)/sqrt(D) for the stream waves' base-2 scores [G][D].
__device__ __forceinline__ int att_raw_floats(const Params& P) { return ((P.G + 2) * P.D + 255) & ~255; }
__device__ __forceinline__ float* att_qs_ptr(const Params& P, const Ctx& cx, int slot) {
  return slot_ptr(cx, slot) + kHdr + att_raw_floats(P) + P.G * P.D + 2 * P.D + P.D + 2 * P.D;
}
// The stream waves' attention partials follow, in the same slot: acc[wave][head][D],
// then (m, l) of [wave][head].
__device__ __forceinline__ float* att_part_ptr(const Params& P, const Ctx& cx, int slot) {
  return att_qs_ptr(P, cx, slot) + P.G * P.D;
}

// Before the event wait: the RoPE (cos, sin) pair jj = lane of the position
// the task appends, which does not depend on the event (held in pre.g[0]).
__device__ __forceinline__ void stage_att_pre(const Params& P, const Ctx& cx, const DevTask& T, int step,
                                              StagePre& pre) {
  const int p = T.b < P.batch ? call_pos(P, T.b, step) : -1;
  float2 cs = make_float2(0.f, 0.f);
  if (p >= 0 && p < P.S && cx.lane < P.D / 2) cs = P.rope_cs[(size_t)p * (P.D / 2) + cx.lane];
  pre.g[0] = make_uint2(__float_as_uint(cs.x), __float_as_uint(cs.y));
}

// Prefill, the owner chunk of a column at position p: the keys and values of
// positions pre_p0 .. p - 1 (columns 0 .. n_in - 1 of this call, their
// projections from this step), each key RMS-normalised per head (qk_norm) and
// rotated at its own position, both rounded to bf16 as the cache stores them,
// into the slot's partial-sum area (idle during an attention task):
// [n_in][key D | value D] floats (n_in < ncap), then, from (ncap - 1) * 2D,
// the scores [kMaxG][kPrefillMax].
__device__ __forceinline__ float* prefill_kv_ptr(const Ctx& cx, int slot) { return part_ptr(cx, slot); }
__device__ __forceinline__ void stage_att_prefill(const Params& P, const Ctx& cx, const DevTask& T, int slot, int n_in) {
  const int G = P.G, D = P.D, Dh = D / 2, GR = (G + 2) * D;
  const int lane = cx.lane;
  float* dst = prefill_kv_ptr(cx, slot);
  const uint16_t* gk = P.gains + (size_t)(2 * P.L + 1) * P.H + (size_t)T.layer * 2 * D + D;
  // lane jj < Dh handles the rotation pair (jj, jj + Dh) of the key and the
  // value dims jj and jj + Dh; four columns' loads in flight at a time
  constexpr int kGrp = 4;
  for (int j0 = 0; j0 < n_in; j0 += kGrp) {
    float ka[kGrp], kb[kGrp], va[kGrp], vb[kGrp];
    float2 cs[kGrp];
#pragma unroll
    for (int i = 0; i < kGrp; ++i) {
      const int j = j0 + i;
      ka[i] = kb[i] = va[i] = vb[i] = 0.f;
      cs[i] = make_float2(1.f, 0.f);
      if (j < n_in && lane < Dh) {
        const float* src = P.qkv + ((size_t)j * P.Hkv + T.g) * GR;
        ka[i] = ld_coh(src + G * D + lane);
        kb[i] = ld_coh(src + G * D + lane + Dh);
        va[i] = ld_coh(src + (G + 1) * D + lane);
        vb[i] = ld_coh(src + (G + 1) * D + lane + Dh);
        cs[i] = P.rope_cs[(size_t)(P.pre_p0 + j) * Dh + lane];
      }
    }
#pragma unroll
    for (int i = 0; i < kGrp; ++i) {
      const int j = j0 + i;
      if (j < n_in) {
        float a = ka[i], b = kb[i];
        if (P.qk_norm) {
          const float f = 1.0f / sqrtf(wave_sum(a * a + b * b) / (float)D + P.eps);
          if (lane < Dh) {
            a *= f * bf2f(gk[lane]);
            b *= f * bf2f(gk[lane + Dh]);
          }
        }
        if (lane < Dh) {
          float* kd = dst + (size_t)j * 2 * D;
          kd[lane] = bf2f(f2bf(a * cs[i].x - b * cs[i].y));
          kd[lane + Dh] = bf2f(f2bf(b * cs[i].x + a * cs[i].y));
          kd[D + lane] = bf2f(f2bf(va[i]));
          kd[D + lane + Dh] = bf2f(f2bf(vb[i]));
        }
      }
    }
  }
}

__device__ __forceinline__ void stage_att(const Params& P, const Ctx& cx, const DevTask& T, int slot, int step,
                                          const StagePre& pre) {
  float* hdr = slot_ptr(cx, slot);
  int* ih = reinterpret_cast<int*>(hdr);
  float* raw = hdr + kHdr;
  const int G = P.G, D = P.D, Dh = D / 2, GR = (G + 2) * D;
  float* q = raw + att_raw_floats(P);
  float* kf = q + G * D;
  float* vf = kf + D;
  uint16_t* kvb = reinterpret_cast<uint16_t*>(vf + D);
  float* qs = att_qs_ptr(P, cx, slot);
  const float qscale = P.attn_scale * 1.4426950408889634f;  // scores in base-2 units
  const int lane = cx.lane;
  const bool active = T.b < P.batch;
  int p = active ? call_pos(P, T.b, step) : 0;
  const bool valid = active && p >= 0 && p < P.S;
  if (active && !valid && lane == 0) __hip_atomic_fetch_or(P.status, kStatusBadPos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!valid) p = 0;
  int lo, end;
  att_stream_range(P, T.chunk, p, lo, end);
  const int hi = chunk_bound(T.chunk + 1, (int64_t)p + 1, P.Nc);
  const bool owner = valid && T.chunk == P.Nc - 1;
  // decode: position p - 1 (appended by the previous step) is not streamed:
  // this task's dependency implies its append is complete, and the chunk that
  // holds it reads it here
  const bool prev = valid && !P.prefill && p >= 1 && lo <= p - 1 && p - 1 < hi;
  // prefill: the owner chunk also takes the positions pre_p0 .. p - 1 (this
  // call's earlier columns), staged below from this step's projections
  const int n_in = valid && owner && P.prefill ? p - P.pre_p0 : 0;
  if (lane == 0) {
    ih[H_P] = p;
    ih[H_LO] = lo;
    ih[H_END] = valid ? end : lo;
    ih[H_FLAGS] = (valid ? 1 : 0) | (owner ? 2 : 0) | (active ? 4 : 0) | (prev ? 8 : 0);
    ih[H_NIN] = n_in;
  }
  if (!valid) return;
  // the key and value of position p - 1 (D / 2 <= 64 words each: one per
  // lane), loaded beside the q|k|v copy so both take one round trip
  uint32_t kw = 0u, vw = 0u;
  if (prev && lane < D / 2) {
    const size_t row = ((((size_t)T.layer * P.B + kv_row_b(P, T.b)) * P.Hkv + T.g) * P.S + (p - 1)) * D;
    kw = ld_coh(reinterpret_cast<const uint32_t*>(P.kcache + row) + lane);
    vw = ld_coh(reinterpret_cast<const uint32_t*>(P.vcache + row) + lane);
  }
  stage_copy(cx, P.qkv + ((size_t)T.b * P.Hkv + T.g) * GR, raw, GR);
  if (prev && lane < D / 2) {
    float* kf1 = vf + D + D;  // after the bf16 bits of the new key and value
    float* vf1 = kf1 + D;
    kf1[2 * lane] = bf2f(kw & 0xffffu);
    kf1[2 * lane + 1] = bf2f(kw >> 16);
    vf1[2 * lane] = bf2f(vw & 0xffffu);
    vf1[2 * lane + 1] = bf2f(vw >> 16);
  }
  if (P.qk_norm) {
    // per-head RMSNorm of the G query heads and the key head, each over D with
    // its [D] gain, before RoPE (the raw q|k rows are contiguous)
    const uint16_t* gq = P.gains + (size_t)(2 * P.L + 1) * P.H + (size_t)T.layer * 2 * D;
    for (int h = 0; h <= G; ++h) {
      float ss = 0.f;
      for (int d = lane; d < D; d += 64) ss = fmaf(raw[h * D + d], raw[h * D + d], ss);
      const float f = 1.0f / sqrtf(wave_sum(ss) / (float)D + P.eps);
      const uint16_t* g = gq + (h < G ? 0 : D);
      for (int d = lane; d < D; d += 64) raw[h * D + d] = raw[h * D + d] * f * bf2f(g[d]);
    }
    wait_lgkm();
  }
  // whole-wave iterations: the (cos, sin) pair comes from lane jj of pre
  for (int base = 0; base < (G + 1) * Dh; base += 64) {
    const int idx = base + lane;
    const int h = idx / Dh, jj = idx - h * Dh;
    const float2 cs = make_float2(__uint_as_float(__shfl(pre.g[0].x, jj, 64)), __uint_as_float(__shfl(pre.g[0].y, jj, 64)));
    if (idx >= (G + 1) * Dh) continue;
    const float a = raw[h * D + jj], b = raw[h * D + jj + Dh];
    const float r0 = a * cs.x - b * cs.y, r1 = b * cs.x + a * cs.y;
    if (h < G) {
      q[h * D + jj] = r0;
      q[h * D + jj + Dh] = r1;
      qs[h * D + jj] = r0 * qscale;
      qs[h * D + jj + Dh] = r1 * qscale;
    } else {
      const uint32_t b0 = f2bf(r0), b1 = f2bf(r1);
      kf[jj] = bf2f(b0);
      kf[jj + Dh] = bf2f(b1);
      kvb[jj] = (uint16_t)b0;
      kvb[jj + Dh] = (uint16_t)b1;
    }
  }
  for (int d = lane; d < D; d += 64) {
    const uint32_t vb = f2bf(raw[(G + 1) * D + d]);
    vf[d] = bf2f(vb);
    kvb[D + d] = (uint16_t)vb;
  }
  if (n_in > 0) stage_att_prefill(P, cx, T, slot, n_in);
}

// offset of the second staged array of merge / argmax tasks
__device__ __forceinline__ int second_off(int n) { return (n + 255) & ~255; }

template <int NC>
__device__ __forceinline__ void stage_task(const Params& P, const Ctx& cx, const DevTask& T, int slot, int step,
                                           const StagePre& pre) {
  float* hdr = slot_ptr(cx, slot);
  float* data = hdr + kHdr;
  const int lane = cx.lane;
  switch (T.type) {
    case T_EMB: {
      if (T.b >= P.batch) break;
      int tok = step == 0 ? P.tokens_in[T.b] : ld_coh(P.tok_cur + T.b);
      if (tok < 0 || tok >= P.V) {
        if (lane == 0) __hip_atomic_fetch_or(P.status, kStatusBadToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tok = 0;
      }
      const uint16_t* row = P.embed + (size_t)tok * P.H;
      const int nl = (P.H * 2 + 1023) / 1024;
      for (int t = 0; t < nl; ++t) dma16<0>(row + t * 512 + lane * 8, data + t * 256);
      wait_all();
      break;
    }
    case T_ATT: stage_att(P, cx, T, slot, step, pre); break;
    case T_COMB: {
      if (T.b >= P.batch) break;
      const size_t head0 = (size_t)T.b * P.Hq + (size_t)T.g * P.G;
      // both copies in one round trip
      stage_copy(cx, P.part_ml + head0 * P.Nc * 2, data, P.G * P.Nc * 2, false);
      stage_copy(cx, P.part_acc + head0 * P.Nc * P.D, data + second_off(P.G * P.Nc * 2), P.G * P.Nc * P.D);
      break;
    }
    case T_ARGMAX: {
      if (T.b >= P.batch) break;
      stage_copy(cx, P.lm_val + (size_t)T.b * P.n_lm, data, P.n_lm, false);
      stage_copy(cx, reinterpret_cast<const float*>(P.lm_idx + (size_t)T.b * P.n_lm), data + second_off(P.n_lm),
                 P.n_lm);
      break;
    }
    default:
      if constexpr (NC == kMfmaCols) stage_matvec_m16(P, cx, T, slot);
      else stage_matvec<NC>(P, cx, T, slot, pre);
      break;
  }
}

template <int NC, bool PROF>
__device__ __forceinline__ void run_stager(const Params& P0, const Ctx& cx) {
  const Params& P = P0;
  int i = 0, nsmall = 0;
  int last0 = -1, last1 = -1, last2 = -1, last3 = -1;  // last task staged into each slot
  Waits wt;  // slot free, dependency event, staging, tasks
  waits_init<PROF>(P, cx, wt);
  for (int step = 0; step < P.n_steps; ++step) {
    const uint32_t epoch = P.epoch0 + (uint32_t)step;
    for (int qi = cx.q0; qi < cx.q1; ++qi, ++i) {
      const Params& P = fresh_params();
      const int id = task_at(P, cx, qi);
      const DevTask T = ld_task(P, id);
      const int slot = next_slot(nsmall, T.type);
      // the task whose retirement frees the slot (slot 3 overlays the others)
      const int prev = slot == kSlotDown ? i - 1 : max(slot == 0 ? last0 : slot == 1 ? last1 : last2, last3);
      uint64_t s0 = waits_now(wt);
      if (prev >= 0 && !spin_ctl(P, cx, C_RETIRED, prev + 1)) return;
      waits_add(wt, 0, s0);
      if (slot == 0) last0 = i; else if (slot == 1) last1 = i; else if (slot == 2) last2 = i; else last3 = i;
      StagePre pre;
      if (NC <= kMaxCols && (T.type == T_QKV || T.type == T_O || T.type == T_GU || T.type == T_D || T.type == T_LM))
        stage_matvec_pre(P, cx, T, slot, pre);
      else if (T.type == T_ATT)
        stage_att_pre(P, cx, T, step, pre);
      s0 = waits_now(wt);
      if (P.use_events) {
        const uint32_t mult = T.type == T_EMB ? epoch : epoch + 1;
        const uint32_t thr = (uint32_t)ld_uniform(reinterpret_cast<const int32_t*>(P.thresholds), T.dep);
        if (!wait_event(P, cx, T.dep, thr * mult)) return;
      }
      waits_add(wt, 1, s0);
      if (PROF && P.profile && cx.lane == 0) P.profile[((size_t)step * P.n_tasks + id) * kProfWords] = wall_clock64();
      if (qi == cx.q0) lds_st(&cx.ctl[C_STEPOK], step + 1);
      s0 = waits_now(wt);
      stage_task<NC>(P, cx, T, slot, step, pre);
      waits_add(wt, 2, s0);
      waits_count(wt, 3, 1);
      lds_st(&cx.ctl[C_STAGED], i + 1);
    }
  }
  waits_put(P, cx, wt);
}

// ---------------------------------------------------------------------------
// retirer (wave 1)
// ---------------------------------------------------------------------------

// Row blocks [a[w], b[w]] that stream wave w's piece of a matvec task touches
// (b < a: an empty piece); its partial sums hold rows of those blocks only.
struct PieceRows {
  int a[kStreams], b[kStreams];
};
__device__ __forceinline__ PieceRows piece_rows(const Ctx& cx, int slot) {
  static_assert(kStreams == 4, "two 16-byte reads hold the four waves' ranges");
  const int4 q0 = *reinterpret_cast<const int4*>(piece_words(cx, slot, 0));
  const int4 q1 = *reinterpret_cast<const int4*>(piece_words(cx, slot, 2));
  PieceRows pr;
  pr.a[0] = __builtin_amdgcn_readfirstlane(q0.x); pr.b[0] = __builtin_amdgcn_readfirstlane(q0.y);
  pr.a[1] = __builtin_amdgcn_readfirstlane(q0.z); pr.b[1] = __builtin_amdgcn_readfirstlane(q0.w);
  pr.a[2] = __builtin_amdgcn_readfirstlane(q1.x); pr.b[2] = __builtin_amdgcn_readfirstlane(q1.y);
  pr.a[3] = __builtin_amdgcn_readfirstlane(q1.z); pr.b[3] = __builtin_amdgcn_readfirstlane(q1.w);
  return pr;
}
// Sum of the stream waves' partials of row vrow (task-relative) in column c.
__device__ __forceinline__ float part_sum(const Params& P, const PieceRows& pr, const float* part, int c, int vrow) {
  const int rb = vrow >> 2;
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kStreams; ++w)
    if (rb >= pr.a[w] && rb <= pr.b[w])
      s += part[((size_t)w * P.ncap + c) * P.wave_vrows + (rb - pr.a[w]) * 4 + (vrow & 3)];
  return s;
}

template <int NC>
__device__ __forceinline__ void retire_matvec(const Params& P, const Ctx& cx, const DevTask& T, int slot, int step) {
  const float* hdr = slot_ptr(cx, slot);
  const float* res = hdr + kHdr + (size_t)P.ncap * slot_kp(P, slot);
  const float* part = part_ptr(cx, slot);
  const int ncols = P.batch;
  const int lane = cx.lane, R = T.row1 - T.row0;
  const PieceRows pr = piece_rows(cx, slot);
  if (T.type == T_LM) {
    const bool last = step == P.n_steps - 1;
    for (int c = 0; c < ncols; ++c) {
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int r = lane; r < R; r += 64) {
        const float v = part_sum(P, pr, part, c, r) * hdr[c];
        if (last && P.logits_out) P.logits_out[(size_t)c * P.V + T.row0 + r] = v;
        if (v > best || (v == best && T.row0 + r < bi)) { best = v; bi = T.row0 + r; }
      }
      wave_argmax(best, bi);
      if (lane == 0) {
        st_coh(P.lm_val + (size_t)c * P.n_lm + T.ordinal, best);
        st_coh(P.lm_idx + (size_t)c * P.n_lm + T.ordinal, bi);
      }
    }
    return;
  }
  for (int c = 0; c < ncols; ++c) {
    const float nf = hdr[c];  // RMS-norm factor of column c (QKV, GU)
    if (T.type == T_QKV) {
      float* dst = P.qkv + ((size_t)c * P.Hkv + T.g) * (P.G + 2) * P.D + T.row0;
      for (int r = lane; r < R; r += 64) st_coh(dst + r, part_sum(P, pr, part, c, r) * nf);
    } else if (T.type == T_GU) {
      float* dst = P.mlp + (size_t)c * P.F + T.row0;
      for (int r = lane; r < R; r += 64) {
        const int vr = 8 * (r >> 2) + (r & 3);
        const float gt = part_sum(P, pr, part, c, vr) * nf;
        const float up = part_sum(P, pr, part, c, vr + 4) * nf;
        st_coh(dst + r, gt / (1.0f + expf(-gt)) * up);
      }
    } else {  // O, D: residual add
      float* dst = P.x + (size_t)c * P.H + T.row0;
      const float* rs = res + (size_t)c * P.res_stride;
      for (int r = lane; r < R; r += 64) st_coh(dst + r, rs[r] + part_sum(P, pr, part, c, r));
    }
  }
}

// Matrix-core bodies: per row block, the stream waves' 16 x 16 partial tiles
// ([row][sequence]) added in wave order, then the RMS factor of each sequence
// (normalised inputs) and the epilogue. Lane l handles tile row l >> 2 and
// sequences 4 (l & 3) .. +3 (gate/up: output l >> 3, sequences 2 (l & 7), +1).
__device__ __forceinline__ void retire_matvec_m16(const Params& P, const Ctx& cx, const DevTask& T, int slot, int step) {
  const float* hdr = slot_ptr(cx, slot);
  const float* res = hdr + kHdr;
  const float* part = part_ptr(cx, slot);
  const int lane = cx.lane, R = T.row1 - T.row0;
  const PieceRows pr = piece_rows(cx, slot);
  const int ts = P.wave_tiles * 256;
  const bool normed = is_normed(T.type);
  if (T.type == T_GU) {
    const int j = lane >> 3, p2 = (lane & 7) * 2, nrb = (R + 7) / 8;
    const float f0 = hdr[p2], f1 = hdr[p2 + 1];
    for (int rb = 0; rb < nrb; ++rb) {
      float2 g = make_float2(0.f, 0.f), u = make_float2(0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kStreams; ++w)
        if (rb >= pr.a[w] && rb <= pr.b[w]) {
          const float* t = part + w * ts + (rb - pr.a[w]) * 256;
          const float2 a = *reinterpret_cast<const float2*>(t + j * 16 + p2);
          const float2 b = *reinterpret_cast<const float2*>(t + (j + 8) * 16 + p2);
          g.x += a.x; g.y += a.y; u.x += b.x; u.y += b.y;
        }
      const int o = rb * 8 + j;
      if (o < R) {
        const float gx = g.x * f0, gy = g.y * f1;
        if (p2 < P.batch) st_coh(P.mlp + (size_t)p2 * P.F + T.row0 + o, gx / (1.0f + expf(-gx)) * (u.x * f0));
        if (p2 + 1 < P.batch) st_coh(P.mlp + (size_t)(p2 + 1) * P.F + T.row0 + o, gy / (1.0f + expf(-gy)) * (u.y * f1));
      }
    }
    return;
  }
  const int n = lane >> 2, q4 = (lane & 3) * 4, nrb = (R + kMfmaRows - 1) / kMfmaRows;
  float fac[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) fac[e] = normed ? hdr[q4 + e] : 1.0f;
  const bool last = step == P.n_steps - 1;
  float best[4], ssum[4];
  int bi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { best[e] = -INFINITY; bi[e] = 0x7fffffff; ssum[e] = 0.f; }
  for (int rb = 0; rb < nrb; ++rb) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kStreams; ++w)
      if (rb >= pr.a[w] && rb <= pr.b[w]) {
        const float4 t = *reinterpret_cast<const float4*>(part + w * ts + (rb - pr.a[w]) * 256 + n * 16 + q4);
        v[0] += t.x; v[1] += t.y; v[2] += t.z; v[3] += t.w;
      }
    const int r = rb * kMfmaRows + n;
    if (r >= R) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = q4 + e;
      if (m >= P.batch) continue;
      const float y = v[e] * fac[e];
      if (T.type == T_LM) {
        if (last && P.logits_out) P.logits_out[(size_t)m * P.V + T.row0 + r] = y;
        if (y > best[e] || (y == best[e] && T.row0 + r < bi[e])) { best[e] = y; bi[e] = T.row0 + r; }
      } else if (T.type == T_QKV) {
        st_coh(P.qkv + ((size_t)m * P.Hkv + T.g) * (P.G + 2) * P.D + T.row0 + r, y);
      } else {  // O, D: residual add; the sum of squares of the new rows for the next RMSNorm
        const float xn = res[(size_t)m * P.res_stride + r] + y;
        st_coh(P.x + (size_t)m * P.H + T.row0 + r, xn);
        ssum[e] = fmaf(xn, xn, ssum[e]);
      }
    }
  }
  if (T.type == T_LM) {
    // the 16 lanes of one sequence quad (equal lane & 3): best value, then the smallest row
#pragma unroll
    for (int o = 4; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ov = __shfl_xor(best[e], o);
        const int oi = __shfl_xor(bi[e], o);
        if (ov > best[e] || (ov == best[e] && oi < bi[e])) { best[e] = ov; bi[e] = oi; }
      }
    if (lane < 4)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (q4 + e < P.batch) {
          st_coh(P.lm_val + (size_t)(q4 + e) * P.n_lm + T.ordinal, best[e]);
          st_coh(P.lm_idx + (size_t)(q4 + e) * P.n_lm + T.ordinal, bi[e]);
        }
  } else if (T.type == T_O || T.type == T_D) {
#pragma unroll
    for (int o = 4; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) ssum[e] += __shfl_xor(ssum[e], o);
    if (lane < 4)
#pragma unroll
      for (int e = 0; e < 4; ++e) st_coh(P.ssq + (size_t)T.ordinal * kMfmaCols + q4 + e, ssum[e]);
  }
}

// Merge the compute waves' softmax statistics and value sums for this chunk,
// add the newest position when this chunk owns it (and append it to the KV
// cache), and store the chunk partial.
__device__ __forceinline__ void retire_att(const Params& P, const Ctx& cx, const DevTask& T, int slot) {
  const float* hdr = slot_ptr(cx, slot);
  const int* ih = reinterpret_cast<const int*>(hdr);
  const int flags = ih[H_FLAGS];
  if (!(flags & 4)) return;  // sequence not in this call's batch
  const bool owner = flags & 2, prev = flags & 8;
  const int G = P.G, D = P.D, D4 = D / 4;
  const float* q = hdr + kHdr + att_raw_floats(P);
  const float* kf = q + G * D;
  const float* vf = kf + D;
  const uint32_t* kvw = reinterpret_cast<const uint32_t*>(vf + D);
  const float* kf1 = vf + 2 * D;  // position p - 1
  const float* vf1 = kf1 + D;
  const float* part = att_part_ptr(P, cx, slot);
  const float* pml = part + kStreams * G * D;  // (m, l) of [wave][head]
  const int lane = cx.lane, p = ih[H_P];
  // prefill: the scores of this call's earlier positions (staged keys), one
  // lane per (head, position), kept beside them in LDS
  const int n_in = ih[H_NIN];
  float* kin = prefill_kv_ptr(cx, slot);
  float* s_in = kin + (size_t)(P.ncap - 1) * 2 * D;  // [kMaxG][kPrefillMax] (n_in < ncap)
  if (n_in > 0) {
    const int h = lane / kPrefillMax, j = lane % kPrefillMax;
    if (h < G && j < n_in) {
      float a = 0.f;
      for (int d = 0; d < D; ++d) a = fmaf(q[h * D + d], kin[(size_t)j * 2 * D + d], a);
      s_in[h * kPrefillMax + j] = a * P.attn_scale;
    }
    wait_lgkm();
  }
  // scores of the new position and of p - 1 (their keys and values are the
  // staged ones)
  float sp[kMaxG], sq[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    sp[h] = -INFINITY;
    sq[h] = -INFINITY;
    if (h < G && owner) {
      float a = 0.f;
      for (int d = lane; d < D; d += 64) a = fmaf(q[h * D + d], kf[d], a);
      sp[h] = wave_sum(a) * P.attn_scale;
    }
    if (h < G && prev) {
      float a = 0.f;
      for (int d = lane; d < D; d += 64) a = fmaf(q[h * D + d], kf1[d], a);
      sq[h] = wave_sum(a) * P.attn_scale;
    }
  }
  // merge of the stream waves' partials and the staged positions: each lane
  // owns four dims of one head
  const size_t chunk0 = ((size_t)T.b * P.Hq + (size_t)T.g * G) * P.Nc + T.chunk;  // head 0 of the group
  const rsrc_t racc = make_rsrc(P.part_acc, 0xffffffffu);
  const rsrc_t rattn = make_rsrc(P.attn + (size_t)T.b * P.Hq * D + (size_t)T.g * G * D, (uint32_t)(G * D) * 4);
  for (int qd = lane; qd < G * D4; qd += 64) {
    const int h = qd / D4, d = (qd - h * D4) * 4;
    float s_new = sp[0], s_prev = sq[0];
#pragma unroll
    for (int hh = 1; hh < kMaxG; ++hh)
      if (h == hh) {
        s_new = sp[hh];
        s_prev = sq[hh];
      }
    float mw[kStreams], lw[kStreams];
    float4 aw[kStreams];
#pragma unroll
    for (int w = 0; w < kStreams; ++w) {
      mw[w] = pml[(w * G + h) * 2];
      lw[w] = pml[(w * G + h) * 2 + 1];
      aw[w] = *reinterpret_cast<const float4*>(part + (size_t)(w * G + h) * D + d);
    }
    float M = fmaxf(s_new, s_prev);
#pragma unroll
    for (int w = 0; w < kStreams; ++w) M = fmaxf(M, mw[w]);
    for (int j = 0; j < n_in; ++j) M = fmaxf(M, s_in[h * kPrefillMax + j]);
    float l = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kStreams; ++w) {
      const float e = mw[w] == -INFINITY ? 0.f : expf(mw[w] - M);
      l = fmaf(lw[w], e, l);
      a.x = fmaf(aw[w].x, e, a.x); a.y = fmaf(aw[w].y, e, a.y);
      a.z = fmaf(aw[w].z, e, a.z); a.w = fmaf(aw[w].w, e, a.w);
    }
    if (prev) {
      const float e = expf(s_prev - M);
      l += e;
      a.x = fmaf(e, vf1[d], a.x); a.y = fmaf(e, vf1[d + 1], a.y);
      a.z = fmaf(e, vf1[d + 2], a.z); a.w = fmaf(e, vf1[d + 3], a.w);
    }
    for (int j = 0; j < n_in; ++j) {  // prefill: this call's earlier positions
      const float e = expf(s_in[h * kPrefillMax + j] - M);
      const float* vj = kin + (size_t)j * 2 * D + D + d;
      l += e;
      a.x = fmaf(e, vj[0], a.x); a.y = fmaf(e, vj[1], a.y);
      a.z = fmaf(e, vj[2], a.z); a.w = fmaf(e, vj[3], a.w);
    }
    if (owner) {
      const float e = expf(s_new - M);
      l += e;
      a.x = fmaf(e, vf[d], a.x); a.y = fmaf(e, vf[d + 1], a.y);
      a.z = fmaf(e, vf[d + 2], a.z); a.w = fmaf(e, vf[d + 3], a.w);
    }
    u32x4 v;
    if (P.Nc == 1) {
      // the only chunk: this task is the merge (the graph has no COMB task),
      // so it stores the normalised output where the O projection reads it
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      v.x = __float_as_uint(inv * a.x); v.y = __float_as_uint(inv * a.y);
      v.z = __float_as_uint(inv * a.z); v.w = __float_as_uint(inv * a.w);
      __builtin_amdgcn_raw_buffer_store_b128(v, rattn, (uint32_t)((h * D + d) * 4), 0, kAuxCoherent);
      continue;
    }
    const size_t ci = chunk0 + (size_t)h * P.Nc;
    v.x = __float_as_uint(a.x); v.y = __float_as_uint(a.y); v.z = __float_as_uint(a.z); v.w = __float_as_uint(a.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, racc, (uint32_t)((ci * D + d) * 4), 0, kAuxCoherent);
    if (d == 0) {
      st_coh(P.part_ml + ci * 2, M);
      st_coh(P.part_ml + ci * 2 + 1, l);
    }
  }
  if (owner) {
    const size_t row = ((((size_t)T.layer * P.B + kv_row_b(P, T.b)) * P.Hkv + T.g) * P.S + p) * D;
    uint32_t* kc = reinterpret_cast<uint32_t*>(P.kcache + row);
    uint32_t* vc = reinterpret_cast<uint32_t*>(P.vcache + row);
    for (int w = lane; w < D / 2; w += 64) {
      st_coh(kc + w, kvw[w]);
      st_coh(vc + w, kvw[D / 2 + w]);
    }
  }
}

template <int NC>
__device__ __forceinline__ void retire_task(const Params& P, const Ctx& cx, const DevTask& T, int slot, int step) {
  const float* hdr = slot_ptr(cx, slot);
  const float* data = hdr + kHdr;
  const int lane = cx.lane;
  switch (T.type) {
    case T_EMB: {
      if (T.b >= P.batch) break;
      const uint32_t* row = reinterpret_cast<const uint32_t*>(data);  // bf16 pairs
      const rsrc_t r = make_rsrc(P.x + (size_t)T.b * P.H, (uint32_t)P.H * 4);
      float ss = 0.f;
      for (int k4 = lane * 4; k4 < P.H; k4 += 256) {
        const uint32_t a = row[k4 / 2], b = row[k4 / 2 + 1];
        u32x4 v;
        v.x = a << 16; v.y = a & 0xffff0000u; v.z = b << 16; v.w = b & 0xffff0000u;
        __builtin_amdgcn_raw_buffer_store_b128(v, r, k4 * 4, 0, kAuxCoherent);
        if constexpr (NC == kMfmaCols) {
          ss = fmaf(__uint_as_float(v.x), __uint_as_float(v.x), ss);
          ss = fmaf(__uint_as_float(v.y), __uint_as_float(v.y), ss);
          ss = fmaf(__uint_as_float(v.z), __uint_as_float(v.z), ss);
          ss = fmaf(__uint_as_float(v.w), __uint_as_float(v.w), ss);
        }
      }
      if constexpr (NC == kMfmaCols) {  // the sum of squares the first layer's RMSNorm reads
        ss = wave_sum(ss);
        if (lane == 0) st_coh(P.ssq + T.b, ss);
      }
      break;
    }
    case T_ATT: retire_att(P, cx, T, slot); break;
    case T_COMB: {
      if (T.b >= P.batch) break;
      const int G = P.G, D = P.D, Nc = P.Nc;
      float* ml = const_cast<float*>(data);  // (m, l) per (head, chunk); m becomes the weight
      const float* acc = data + second_off(G * Nc * 2);
      // per head: the largest chunk maximum M, then weight_c = exp(m_c - M) /
      // sum_c exp(m_c - M) l_c; the 16 lanes of row h handle head h (G <= 4)
      {
        const int h = lane >> 4, c0 = lane & 15;
        float M = -INFINITY;
        if (h < G)
          for (int c = c0; c < Nc; c += 16) M = fmaxf(M, ml[(h * Nc + c) * 2]);
        M = max16(M);
        float den = 0.f;
        if (h < G)
          for (int c = c0; c < Nc; c += 16) {
            const float mc = ml[(h * Nc + c) * 2];
            den += mc == -INFINITY ? 0.f : expf(mc - M) * ml[(h * Nc + c) * 2 + 1];
          }
        den = sum16(den);
        const float inv = den > 0.f ? 1.0f / den : 0.f;
        if (h < G)
          for (int c = c0; c < Nc; c += 16) {
            const float mc = ml[(h * Nc + c) * 2];
            ml[(h * Nc + c) * 2] = mc == -INFINITY ? 0.f : expf(mc - M) * inv;
          }
        wait_lgkm();
      }
      // weighted sum over chunks: each lane owns four dims of one head (16-byte
      // LDS reads, eight chunks in flight) and stores them as one 16-byte word
      const int D4 = D / 4;
      const rsrc_t r = make_rsrc(P.attn + (size_t)T.b * P.Hq * D + (size_t)T.g * G * D, (uint32_t)(G * D) * 4);
      for (int q = lane; q < G * D4; q += 64) {
        const int h = q / D4, d = (q - h * D4) * 4;
        const float* wc = ml + h * Nc * 2;
        const float* ac = acc + (size_t)h * Nc * D + d;
        float4 n = make_float4(0.f, 0.f, 0.f, 0.f);
        int c = 0;
        for (; c + 8 <= Nc; c += 8) {
          float4 a[8];
          float w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            a[j] = *reinterpret_cast<const float4*>(ac + (size_t)(c + j) * D);
            w[j] = wc[(c + j) * 2];
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            n.x = fmaf(w[j], a[j].x, n.x); n.y = fmaf(w[j], a[j].y, n.y);
            n.z = fmaf(w[j], a[j].z, n.z); n.w = fmaf(w[j], a[j].w, n.w);
          }
        }
        for (; c < Nc; ++c) {
          const float4 a = *reinterpret_cast<const float4*>(ac + (size_t)c * D);
          const float w = wc[c * 2];
          n.x = fmaf(w, a.x, n.x); n.y = fmaf(w, a.y, n.y); n.z = fmaf(w, a.z, n.z); n.w = fmaf(w, a.w, n.w);
        }
        u32x4 v;
        v.x = __float_as_uint(n.x); v.y = __float_as_uint(n.y); v.z = __float_as_uint(n.z); v.w = __float_as_uint(n.w);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (h * D + d) * 4, 0, kAuxCoherent);
      }
      break;
    }
    case T_ARGMAX: {
      if (T.b >= P.batch) break;
      const float* val = data;
      const int* ix = reinterpret_cast<const int*>(data + second_off(P.n_lm));
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int t = lane; t < P.n_lm; t += 64) {
        const float v = val[t];
        const int i2 = ix[t];
        if (v > best || (v == best && i2 < bi)) { best = v; bi = i2; }
      }
      wave_argmax(best, bi);
      if (lane == 0) {
        if (bi < 0 || bi >= P.V) bi = 0;  // every logit was NaN
        P.out_tokens[(size_t)step * P.out_stride + T.b] = bi;
        st_coh(P.tok_cur + T.b, bi);
      }
      break;
    }
    default:
      if constexpr (NC == kMfmaCols) retire_matvec_m16(P, cx, T, slot, step);
      else retire_matvec<NC>(P, cx, T, slot, step);
      break;
  }
}

template <int NC, bool PROF>
__device__ __forceinline__ void run_retirer(const Params& P0, const Ctx& cx) {
  const Params& P = P0;
  int i = 0, nsmall = 0;
  Waits wt;  // staged, computed, epilogue, tasks
  waits_init<PROF>(P, cx, wt);
  for (int step = 0; step < P.n_steps; ++step) {
    for (int qi = cx.q0; qi < cx.q1; ++qi, ++i) {
      const Params& P = fresh_params();
      const int id = task_at(P, cx, qi);
      const DevTask T = ld_task(P, id);
      const int slot = next_slot(nsmall, T.type);
      const uint64_t s0 = waits_now(wt);
      if (!spin_ctl(P, cx, C_STAGED, i + 1)) return;
      waits_add(wt, 0, s0);
      const uint64_t t_staged = wall_clock64();
      if (has_stream(T.type) && !spin_ctl(P, cx, C_DONE + ctl_slot(slot), kStreams)) return;
      const uint64_t t_computed = wall_clock64();
      waits_count(wt, 1, (uint32_t)(t_computed - t_staged));
      retire_task<NC>(P, cx, T, slot, step);
      wait_all();  // every store of the epilogue has completed
      waits_add(wt, 2, t_computed);
      waits_count(wt, 3, 1);
      if (cx.lane == 0) {
        if (P.use_events && id != P.drop_task)
          __hip_atomic_fetch_add(&P.counters[(size_t)T.trig * kEventWords + (cx.cu & (kStripes - 1)) * 32], 1u,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (PROF && P.profile) {
          uint64_t* rec = P.profile + ((size_t)step * P.n_tasks + id) * kProfWords;
          rec[1] = t_staged;
          rec[2] = t_computed;
          rec[3] = wall_clock64();
          if (has_stream(T.type))
            for (int w = 0; w < kStreams; ++w) {
              const uint32_t* pw = prof_words(cx, slot, w);
              rec[4 + w] = (uint64_t)pw[0] << 32 | pw[2];
              rec[8 + w] = pw[1];
            }
        }
        __hip_atomic_store(&cx.ctl[C_DONE + ctl_slot(slot)], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      lds_st(&cx.ctl[C_RETIRED], i + 1);
    }
  }
  waits_put(P, cx, wt);
}

#include "pipeline.h"
#include "mfma.h"

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

template <int NC, bool PROF>
__device__ __forceinline__ void run(const Params& P, int cu, int single) {
  extern __shared__ __align__(16) char smem[];
  Ctx cx;
  cx.ctl = reinterpret_cast<int*>(smem);
  float* base = reinterpret_cast<float*>(smem + kCtlBytes);
  cx.slots = base;
  cx.small_floats = P.small_floats;
  cx.parts = base + 2 * P.small_floats + P.big_floats;
  cx.part_floats = P.part_floats;
  cx.cu = cu;
  cx.single = single;
  if (single >= 0) {
    cx.q0 = 0;
    cx.q1 = 1;
  } else {
    cx.q0 = ld_uniform(P.queue_ptr, cu);
    cx.q1 = ld_uniform(P.queue_ptr, cu + 1);
  }
  cx.lane = threadIdx.x & 63;
  cx.recs = reinterpret_cast<StreamRec*>(cx.parts + 3 * P.part_floats);
  for (int j = threadIdx.x; j < kCtlBytes / 4; j += blockDim.x)
    cx.ctl[j] = j >= kOnesCtl && j < kOnesCtl + 4 ? 0x3F803F80 : 0;  // bf16 ones for the unnormalised inputs
  if (single < 0) {
    const int r0 = ld_uniform(P.srec_ptr, cu), r1 = ld_uniform(P.srec_ptr, cu + 1);
    cx.nrec = r1 - r0;
    const int32_t* src = reinterpret_cast<const int32_t*>(P.srecs + r0);
    int32_t* dst = reinterpret_cast<int32_t*>(cx.recs);
    for (int j = threadIdx.x; j < cx.nrec * 8; j += blockDim.x) dst[j] = src[j];
  } else {
    // one task: its record, in the slot the first task of a queue gets
    const DevTask T = ld_task(P, single);
    cx.nrec = has_stream(T.type) ? 1 : 0;
    if (threadIdx.x == 0 && cx.nrec) {
      StreamRec r;
      int nsmall = 0;
      r.tsbg = (uint32_t)T.type | (uint32_t)next_slot(nsmall, T.type) << 4 | (uint32_t)T.b << 6 | (uint32_t)T.g << 16;
      // as the host builds the records: column-major matvec tasks walk 8 row blocks per column pair
      r.lc = T.type == T_ATT ? (uint32_t)T.layer | (uint32_t)T.chunk << 16
                             : ((uint32_t)T.layer & 0xffffu) | (uint32_t)T.cm << 16;
      r.n_units = T.cm ? 8 * T.kb : T.n_units;
      r.kq = (uint32_t)T.kb;
      r.w_off = T.w_off;
      r.flip = 0;
      r.id = single;
      cx.recs[0] = r;
    }
  }
  __syncthreads();
  // wave index as a wave-uniform value: every role's control flow is scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0) run_stager<NC, PROF>(P, cx);
  else if (wave == 1) run_retirer<NC, PROF>(P, cx);
  else if constexpr (NC == kMfmaCols) run_stream_m16<MK_RING_M, MK_XRING_M, PROF>(P, cx, wave - kCtlWaves);
  else run_stream<kRing, NC, PROF>(P, cx, wave - kCtlWaves);
}

// One kernel per staged column count: each holds the code of its own variant
// only, which keeps the instruction working set of a workgroup small (it shares
// a 64 KiB instruction cache with a neighbouring compute unit). The per-task
// timestamps and wait counters live in separate persistent variants
// (mk_persistent_prof_*), launched only when a profile or wait-counter buffer
// is set.
#define MK_KERNELS(NC)                                                                                   \
  extern "C" __global__ void __launch_bounds__(kThreads) mk_persistent_b##NC(Params P) {               \
    run<NC, false>(P, blockIdx.x, -1);                                                                 \
  }                                                                                                    \
  extern "C" __global__ void __launch_bounds__(kThreads) mk_persistent_prof_b##NC(Params P) {          \
    run<NC, true>(P, blockIdx.x, -1);                                                                  \
  }                                                                                                    \
  extern "C" __global__ void __launch_bounds__(kThreads) mk_oplaunch_b##NC(Params P, int first) {      \
    run<NC, false>(P, blockIdx.x, first + blockIdx.x);                                                 \
  }
MK_KERNELS(1)
MK_KERNELS(2)
MK_KERNELS(3)
MK_KERNELS(4)
MK_KERNELS(16)
#undef MK_KERNELS

typedef void (*PersistentFn)(Params);
typedef void (*OpFn)(Params, int);
// [columns - 1]
static const PersistentFn kPersistent[kMaxCols] = {mk_persistent_b1, mk_persistent_b2, mk_persistent_b3,
                                                   mk_persistent_b4};
static const PersistentFn kPersistentProf[kMaxCols] = {mk_persistent_prof_b1, mk_persistent_prof_b2,
                                                       mk_persistent_prof_b3, mk_persistent_prof_b4};
static const OpFn kOplaunch[kMaxCols] = {mk_oplaunch_b1, mk_oplaunch_b2, mk_oplaunch_b3, mk_oplaunch_b4};
// the matrix-core bodies: one variant for every launch of up to kMfmaCols sequences
static_assert(kMfmaCols == 16, "kernel names");
static const PersistentFn kPersistentM = mk_persistent_b16, kPersistentProfM = mk_persistent_prof_b16;
static const OpFn kOplaunchM = mk_oplaunch_b16;

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
    const int col = kb * kUnitCols + i * 4;  // and col + 64
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
    if (r < R && col < J.K) {
      const uint2 a = *reinterpret_cast<const uint2*>(m + row * J.K + col);
      v.x = a.x;
      v.y = a.y;
    }
    if (r < R && col + 64 < J.K) {
      const uint2 b = *reinterpret_cast<const uint2*>(m + row * J.K + col + 64);
      v.z = b.x;
      v.w = b.y;
    }
    *reinterpret_cast<u32x4*>(dst + J.dst_off + u * kUnitBytes + lane * 16) = v;
  }
}

// The matrix-core arrangement (device.h): unit u = (row block rb, column block
// kb) of 16 rows x 32 columns, lane 16 * j + i holding columns [8j, 8j + 8) of
// row i; gate/up row blocks hold 8 gate rows and then the up rows of the same
// 8 outputs. Rows past the task's end and columns past K are zeros.
__device__ __forceinline__ const uint16_t* pack_row(const PackJob& J, const PackSrc* src, int G, int D, int L, int r,
                                                    int64_t& row) {
  const int ar = J.row0 + r;
  switch (J.type) {
    case T_QKV:
      if (ar < G * D) { row = (int64_t)J.g * G * D + ar; return src[J.layer].p[0]; }
      if (ar < (G + 1) * D) { row = (int64_t)J.g * D + ar - G * D; return src[J.layer].p[1]; }
      row = (int64_t)J.g * D + ar - (G + 1) * D;
      return src[J.layer].p[2];
    case T_O: row = ar; return src[J.layer].p[3];
    case T_D: row = ar; return src[J.layer].p[6];
    default: row = ar; return src[L].p[0];  // T_LM
  }
}

extern "C" __global__ void __launch_bounds__(256) mk_pack_m16(const PackJob* jobs, const PackSrc* src, uint8_t* dst,
                                                             int G, int D, int L) {
  const PackJob J = jobs[blockIdx.x];
  const int64_t lanes = (int64_t)J.n_vrb * J.KB * 64;
  const int R = J.row1 - J.row0;
  for (int64_t idx = threadIdx.x; idx < lanes; idx += blockDim.x) {
    const int64_t u = idx >> 6;
    const int lane = (int)(idx & 63);
    int rb, kb;
    if (J.cm) {  // item (column pair c, row block r) at c * cm + r; unit h of it: column block 2c + h
      const int64_t it = u >> 1;
      const int c = (int)(it / J.cm);
      rb = (int)(it - (int64_t)c * J.cm);
      kb = 2 * c + (int)(u & 1);
    } else {
      rb = (int)(u / J.KB);
      kb = (int)(u - (int64_t)rb * J.KB);
    }
    const int i = lane & 15, col = kb * 32 + (lane >> 4) * 8;
    int r;
    int64_t row = 0;
    const uint16_t* m;
    if (J.type == T_GU) {
      r = rb * 8 + (i & 7);
      m = src[J.layer].p[i < 8 ? 4 : 5];
      row = J.row0 + r;
    } else {
      r = rb * kMfmaRows + i;
      m = pack_row(J, src, G, D, L, r, row);
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && col < J.K) v = *reinterpret_cast<const u32x4*>(m + row * J.K + col);
    *reinterpret_cast<u32x4*>(dst + J.dst_off + u * kUnitBytes + lane * 16) = v;
  }
}

// ---------------------------------------------------------------------------
// host-side launchers (called from api.cpp)
// ---------------------------------------------------------------------------

hipError_t set_lds_limit(int bytes) {
  for (int c = 0; c <= kMaxCols; ++c) {
    const void* fns[3] = {
        reinterpret_cast<const void*>(c < kMaxCols ? kPersistent[c] : kPersistentM),
        reinterpret_cast<const void*>(c < kMaxCols ? kPersistentProf[c] : kPersistentProfM),
        reinterpret_cast<const void*>(c < kMaxCols ? kOplaunch[c] : kOplaunchM)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t persistent_occupancy(int lds, int* blocks_per_cu) {
  int worst = 1 << 30;
  for (int c = 0; c <= kMaxCols; ++c)
    for (const PersistentFn f : {c < kMaxCols ? kPersistent[c] : kPersistentM,
                                 c < kMaxCols ? kPersistentProf[c] : kPersistentProfM}) {
      int n = 0;
      hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(f), kThreads, lds);
      if (e != hipSuccess) return e;
      worst = n < worst ? n : worst;
    }
  *blocks_per_cu = worst;
  return hipSuccess;
}

// The variant for the call: staged columns = the call's batch.
hipError_t launch_persistent(const Params& P, int grid, int lds, bool mfma, hipStream_t s) {
  if (P.batch < 1 || P.batch > (mfma ? kMfmaCols : kMaxCols)) return hipErrorInvalidValue;
  Params p = P;
  void* args[] = {&p};
  const bool prof = P.profile || P.waits;
  const PersistentFn f = mfma ? (prof ? kPersistentProfM : kPersistentM)
                              : (prof ? kPersistentProf[P.batch - 1] : kPersistent[P.batch - 1]);
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(f), dim3(grid), dim3(kThreads), args, lds, s);
}

hipError_t launch_op(const Params& P, int first, int count, int lds, bool mfma, hipStream_t s) {
  if (P.batch < 1 || P.batch > (mfma ? kMfmaCols : kMaxCols)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma ? kOplaunchM : kOplaunch[P.batch - 1], dim3(count), dim3(kThreads), lds, s, P, first);
  return hipGetLastError();
}

hipError_t launch_pack(const PackJob* jobs, int n_jobs, const PackSrc* src, uint8_t* dst, int G, int D, int L,
                       bool mfma, hipStream_t s) {
  if (mfma) hipLaunchKernelGGL(mk_pack_m16, dim3(n_jobs), dim3(256), 0, s, jobs, src, dst, G, D, L);
  else hipLaunchKernelGGL(mk_pack, dim3(n_jobs), dim3(256), 0, s, jobs, src, dst, G, D, L);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// static workspace of the no-allocation entry point
// ---------------------------------------------------------------------------

// Zero-fill used to clear the static workspace's counters at every call (a
// kernel rather than a memset, so that a caller may capture the call).
__global__ void mk_fill_zero(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  if (words > 0xffffffffu) return hipErrorInvalidValue;
  const size_t blocks = std::min<size_t>((words + 255) / 256, 1024);
  hipLaunchKernelGGL(mk_fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                     static_cast<uint32_t>(words));
  return hipGetLastError();
}

}  // namespace mk

// The array itself. In host code its name is only a stand-in for the device
// symbol; its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[MK_NOALLOC_SCRATCH_BYTES];

namespace mk {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev].load(std::memory_order_acquire)) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev) return hipErrorInvalidDevice;  // the device must be current
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch[dev].store(ptr, std::memory_order_release);
  return hipSuccess;
}

void* noalloc_scratch(int dev) {
  return dev >= 0 && dev < kMaxDevices ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
}

}  // namespace mk
