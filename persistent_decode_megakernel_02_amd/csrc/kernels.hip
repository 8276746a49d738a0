// kernels.hip -- task bodies, the persistent decode megakernel and the
// per-operator ablation kernels, for gfx950 (MI355X, wave64).
//
// Runtime model (MPK digest, fr.news.hada.io, "Part 2. Runtime", "Workers"):
// every workgroup is a worker that stays resident for the whole launch and
// loops "take next task from my list -> run it -> notify its event".  The
// scheduler role of that design is replaced by lists fixed at build time
// (Ada-MK, gist.science, "L'Itinéraire Pré-planifié"), so a worker never asks
// anyone what to do next; it only waits until its task's event has fired.
//
// Memory protocol.  Activations produced by one worker and consumed by
// others (x, q/k/v, partials, o, a, LM partials) are written and read with
// device-coherent accesses (sc1: they bypass the non-coherent per-XCD L2
// state).  A producer drains its stores (s_waitcnt), joins its workgroup at a
// barrier and then one lane stores the step number into its own slot of the
// event; a consumer's wave 0 polls the event's slots (every slot, except that
// a wait on a distributed attention event reads only the step's merging
// splits), then the workgroup barrier releases the other waves.  Weights and the KV cache are
// never written by one worker and read by another inside a launch (a KV
// position is always re-read by the worker that wrote it), so they use plain
// or non-temporal loads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mk_internal.h"

namespace mk {

constexpr int NT = 512;  // threads per worker
constexpr int NW = NT / 64;
#ifndef MK_RPG1
#define MK_RPG1 2
#endif
// rows per staged-activation read at one sequence at the O-projection, gate/up and down projection,
// whose waves hold an even number of rows (QKV's three rows per wave would pay for a duplicate;
// the LM head measured slower with two)
constexpr int kRpg1 = MK_RPG1;
#ifndef MK_GEMV_CG
#define MK_GEMV_CG 4
#endif
constexpr int CG = MK_GEMV_CG;  // 16-byte weight chunks per lane per pipeline group
#ifndef MK_GEMV_DEPTH
#define MK_GEMV_DEPTH 2
#endif
constexpr int DEPTH = MK_GEMV_DEPTH;   // pipeline groups in flight per wave (8 KB per wave): a wave's loads complete in
                          // order, so a deeper queue delays the activation and flag loads behind it
constexpr int MISC_BYTES = 4096;
constexpr int ATT_MAXL = 5;   // most K/V 16-byte loads per thread per attention task (split <= 5 * 512 / (D / 8)) ...
constexpr int ATT_MAXL1 = 8;  // ... or 8 with one query head per KV head (split <= 8 * 512 / (D / 8))

// Pointers kept inside the parameter block are generic; casting them to the
// global address space lets the compiler emit global (not flat) memory
// instructions and track their completion precisely.
#define GAS __attribute__((address_space(1)))

typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

struct Misc {
  int32_t tok[16];      // tokens of this step (layer-0 QKV)
  double wred[NW][16];  // per-wave partial sums of squares (RMSNorm)
  float wval[NW][16];   // per-wave argmax values
  int32_t widx[NW][16]; // per-wave argmax indices
  double hr[16];        // QK-norm scales
  double ml[8][2];      // attention (max, sum) per head
  int32_t flag;
  double rsd[16];       // matrix-core GEMV: RMSNorm scale per sequence
  double kss[16];       // split-K QKV, last part: the other parts' sums of squares per sequence
  float lmv[16];        // matrix-core LM head: running (max, index) per sequence
  int32_t lmi[16];
  uint32_t cev, ctgt;   // the last (event, target) this worker's wait saw complete
  uint32_t qk_step, qk_id;  // step tag and (layer, sequence, KV head) of the rotated queries in LDS
  int32_t att_fail;         // sticky: an attention merge of this worker exceeded its poll budget
  int32_t lora_fail;        // a LoRA adapter sum of the current task was not published in its poll budget
  // streaming GEMV engine (batch <= 4)
  struct {
    uint32_t staged, done, abort;
    int32_t end_s;
    uint32_t end_i;
  } seg;
  double sg_rs[2][16];      // RMSNorm scale per sequence of the last two tasks
};
static_assert(sizeof(Misc) <= MISC_BYTES, "misc");

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf1(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

extern __shared__ __attribute__((aligned(16))) char g_lds[];

typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u_ __attribute__((ext_vector_type(4)));
// plain global load / store of any trivially copyable T (size 2 or a multiple of 4)
template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  T r;
  if constexpr (sizeof(T) == 2) {
    const uint16_t v = *(const GAS uint16_t*)p;
    __builtin_memcpy(&r, &v, 2);
  } else if constexpr (sizeof(T) == 8) {
    const v2u v = *(const GAS v2u*)p;
    __builtin_memcpy(&r, &v, 8);
  } else if constexpr (sizeof(T) % 16 == 0) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 16); ++i) {
      const v4u_ v = ((const GAS v4u_*)p)[i];
      __builtin_memcpy((char*)&r + 16 * i, &v, 16);
    }
  } else {
    static_assert(sizeof(T) % 4 == 0, "ldg size");
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) {
      const uint32_t v = ((const GAS uint32_t*)p)[i];
      __builtin_memcpy((char*)&r + 4 * i, &v, 4);
    }
  }
  return r;
}
// Load from a table that no kernel writes (task and event tables, per-task records): read
// through the constant address space, so a uniform address becomes a scalar load (it counts in
// lgkmcnt, not vmcnt, and so never waits behind a wave's weight loads).
template <typename T>
__device__ __forceinline__ T ldk(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "ldk size");
  T r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) {
    const uint32_t v = ((const __attribute__((address_space(4))) uint32_t*)p)[i];
    __builtin_memcpy((char*)&r + 4 * i, &v, 4);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void stg(T* p, const T& val) {
  if constexpr (sizeof(T) == 16) {
    v4u_ v;
    __builtin_memcpy(&v, &val, 16);
    *(GAS v4u_*)p = v;
  } else {
    static_assert(sizeof(T) == 4, "stg size");
    uint32_t v;
    __builtin_memcpy(&v, &val, 4);
    *(GAS uint32_t*)p = v;
  }
}

// device-coherent (sc1) scalar accesses for data shared between workers
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load((const GAS float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ldc_u(const uint32_t* p) {
  return __hip_atomic_load((const GAS uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ldc_i(const int32_t* p) {
  return __hip_atomic_load((const GAS int32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store((GAS float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store((GAS uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_i(int32_t* p, int32_t v) {
  __hip_atomic_store((GAS int32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 4 consecutive fp32 activations, device-coherent (sc1) 16-byte load.
__device__ __forceinline__ v4f ldc4(const float* base, uint32_t elem) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, elem * 4u, 0, 16 /* sc1 */);
}

// 16 bytes of a streamed, read-once weight row (non-temporal).
__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  v4u v = __builtin_nontemporal_load((const GAS v4u*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return ldg((const uint4*)p); }

// The thread index seen through an empty asm.  Lane-dependent addresses are
// then recomputed inside every task instead of being hoisted out of the
// persistent loop, where they would stay live across all tasks (and spill).
__device__ __forceinline__ int ltid() {
  int v = threadIdx.x;
  asm volatile("" : "+v"(v));
  return v;
}

// Cross-lane reductions in VALU (DPP row operations and the gfx950
// permlane swaps), no LDS traffic.  Only patterns within a row of 16 lanes are
// used (quad permutes, row mirrors), so every lane reads a valid source and
// the DPP moves need no fill value.  Every lane of a group receives the same,
// bit-identical result (each step adds the same two operands on all lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float xor16_pair(float v) {  // lanes i and i^16 both get v_i + v_{i^16}
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_pair(float v) {  // lanes i and i^32 both get v_i + v_{i^32}
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over aligned groups of N lanes (N = 4, 8, 16)
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);                 // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);                 // quad_perm [2,3,0,1]
  if (N >= 8) v += dpp<0x141>(v);    // row_half_mirror
  if (N >= 16) v += dpp<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return xor32_pair(xor16_pair(group_sum<16>(v))); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return xor32_pair_max(xor16_pair_max(v));
}
// fp64 versions: the two 32-bit halves move through the same lane permutation
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double xor16_pair_d(double v) {
  const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
  const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
  return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
}
__device__ __forceinline__ double xor32_pair_d(double v) {
  const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
  const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
  return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
}
__device__ __forceinline__ double xor16_pair_max_d(double v) {
  const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
  const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
  return fmax(__hiloint2double((int)h[0], (int)l[0]), __hiloint2double((int)h[1], (int)l[1]));
}
__device__ __forceinline__ double xor32_pair_max_d(double v) {
  const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
  const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
  return fmax(__hiloint2double((int)h[0], (int)l[0]), __hiloint2double((int)h[1], (int)l[1]));
}
template <int N>
__device__ __forceinline__ double group_sum_d(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  if (N >= 8) v += dpp_d<0x141>(v);
  if (N >= 16) v += dpp_d<0x140>(v);
  return v;
}
// group_sum_d over NV independent values at once (each step on all of them)
template <int N, int NV>
__device__ __forceinline__ void group_sum_d_n(double* v) {
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += dpp_d<0xB1>(v[k]);
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += dpp_d<0x4E>(v[k]);
  if (N >= 8)
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] += dpp_d<0x141>(v[k]);
  if (N >= 16)
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] += dpp_d<0x140>(v[k]);
}
__device__ __forceinline__ double wave_sum_d(double v) { return xor32_pair_d(xor16_pair_d(group_sum_d<16>(v))); }
__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, dpp_d<0xB1>(v));
  v = fmax(v, dpp_d<0x4E>(v));
  v = fmax(v, dpp_d<0x141>(v));
  v = fmax(v, dpp_d<0x140>(v));
  return xor32_pair_max_d(xor16_pair_max_d(v));
}

// larger value wins; equal values: lower index wins
__device__ __forceinline__ void amax_merge(float& v, int32_t& i, float v2, int32_t i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}
__device__ __forceinline__ void wave_amax(float& v, int32_t& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, 64);
    int32_t i2 = __shfl_xor(i, o, 64);
    amax_merge(v, i, v2, i2);
  }
}

__device__ __forceinline__ double silu_d(double z) { return z / (1.0 + exp(-z)); }

// ---------------------------------------------------------------------------
// events
// ---------------------------------------------------------------------------
// Attention merge forms.  dist: a worker for every attention task of the layer, so the splits
// of a head run together and the attention event has one slot per task, split-major (slot
// sp B Hkv + b Hkv + g).  Then, past ATT_MCH active splits (more than one burst of accumulator
// loads for a single merger), every active split merges a slice of its head group's outputs and
// signals; otherwise the split holding the current position merges them all and alone signals
// (without dist, in slot b Hkv + g, and a split may wait only on splits listed before it).
constexpr int ATT_MCH = 8;
__device__ __forceinline__ bool att_dist(const KParams& P) {
  return P.chunk == 0 && P.NS * P.B * P.Hkv <= P.n_workers;
}

// Event form.  Default: one 32-bit slot per producer holding the number of the last step it
// completed; an event fires for step t when every slot it waits on holds t (plain stores, no
// read-modify-write).  MK_EVENT_COUNTER=1 builds the counter form instead, to measure one
// against the other: one word per event, advanced by one device-scope atomic add per producer
// and step, firing for step t at fanin * t.  Every producer then signals every step (attention
// splits beyond the current length included, after their wait, so that no step's add can land
// before the previous step's event has fired).
#ifndef MK_EVENT_COUNTER
#define MK_EVENT_COUNTER 0
#endif
constexpr bool kEventCounter = MK_EVENT_COUNTER != 0;
__device__ __forceinline__ int att_active(const KParams& P, int s) { return (P.pos0 + s + 1 + P.S - 1) / P.S; }

// att: ev is a layer's attention event; cached: an attention task's wait, which first checks
// whether this worker's previous attention task already saw the same event complete
__device__ __forceinline__ bool wait_event(const KParams& P, uint32_t ev, uint32_t target, uint32_t task, Misc* m,
                                           uint64_t* tr = nullptr, bool att = false, bool cached = false) {
  if (ev == EV_NONE) return true;
  // the worker's attention tasks of a layer usually share one (sequence, KV head) and so one
  // event; slots only grow, so an event seen complete for this target still is
  if (cached && m->cev == ev && m->ctgt == target) {
    __syncthreads();
    if (tr && threadIdx.x == 0) tr[1] = wall_clock64();
    return true;
  }
  const int tid = ltid();
  if (tid < 64) {
    const int lane = tid;
    const EventRec e = ldk(P.events + ev);
    const uint32_t* f = P.flags + e.slot0;
    uint32_t fanin = e.fanin;
    uint32_t want = target;
    if constexpr (kEventCounter) {  // the event's one counter word, at fanin adds per step
      f = P.flags + ev;
      fanin = 1;
      // the LM head's event saw no adds in the steps run without it (prefill)
      const bool lm = ev == (uint32_t)(P.L * (P.Hkv + 4));
      want = e.fanin * (target - (lm ? P.lm_skip : 0u));
    } else if (att && att_dist(P)) {  // a dist attention event: only the slots of the step's signalling splits
      const int n_act = att_active(P, (int)(target - P.epoch) - 1);
      const uint32_t bh = (uint32_t)(P.B * P.Hkv);
      if (n_act > ATT_MCH) {
        fanin = (uint32_t)n_act * bh;
      } else {
        f += (uint32_t)(n_act - 1) * bh;
        fanin = bh;
      }
    }
    uint32_t polls = 0;
    int ok = 0;
    // a pass reads the slots in bursts of PW per lane, all in flight together (a slot index past
    // the fan-in re-reads the last slot), so one pass over up to 64 PW slots costs one round trip
    constexpr uint32_t PW = 4;
    for (;;) {
      bool mine = true;
      uint32_t seen = want;
      for (uint32_t i0 = 0; i0 < fanin; i0 += 64 * PW) {
        uint32_t v[PW];
#pragma unroll
        for (uint32_t k = 0; k < PW; ++k) v[k] = ldc_u(f + min(i0 + lane + 64 * k, fanin - 1));
#pragma unroll
        for (uint32_t k = 0; k < PW; ++k)
          if ((int32_t)(v[k] - want) < 0) {
            mine = false;
            seen = v[k];
          }
      }
      if (__all(mine)) {
        ok = 1;
        break;
      }
      ++polls;
      if ((polls & 63u) == 0) {
        if (ldc_u(P.status + ST_ABORT)) break;
        if (polls >= P.watchdog) {
          uint32_t zero = 0u;
          if (!mine && __hip_atomic_compare_exchange_strong((GAS uint32_t*)(P.status + ST_CODE), &zero, ERR_WATCHDOG,
                                                            __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            stc_u(P.status + ST_CU, blockIdx.x);
            stc_u(P.status + ST_TASK, task);
            stc_u(P.status + ST_EVENT, ev);
            stc_u(P.status + ST_SEEN, seen);
            stc_u(P.status + ST_WANT, want);
          }
          if (lane == 0) stc_u(P.status + ST_ABORT, 1u);
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      m->flag = ok;
      if (ok && cached) {
        m->cev = ev;
        m->ctgt = target;
      }
    }
  }
  __syncthreads();
  if (tr && threadIdx.x == 0) tr[1] = wall_clock64();
  return m->flag != 0;
}

__device__ __forceinline__ void signal_event(const KParams& P, uint32_t ev, uint32_t slot, uint32_t val) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's coherent stores have completed
  __syncthreads();                // ... and every other wave's
  if (threadIdx.x == 0) {
    if constexpr (kEventCounter)
      __hip_atomic_fetch_add((GAS uint32_t*)(P.flags + ev), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      stc_u(P.flags + ldk(P.events + ev).slot0 + slot, val);
  }
}

// ---------------------------------------------------------------------------
// tokens: argmax over the LM tiles' partial maxima (lowest index on ties)
// ---------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ void reduce_tokens(const KParams& P, Misc* m) {
  const int tid = ltid(), lane = tid & 63, w = tid >> 6;
  float bv[NB];
  int32_t bi[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    bv[b] = -INFINITY;
    bi[b] = 0x7fffffff;
  }
  for (int i = tid; i < P.n_lm; i += NT) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const LmPart* lp = P.lm_part + (size_t)b * P.n_lm + i;
      float v = ldc(&lp->val);
      int32_t ix = ldc_i(&lp->idx);
      amax_merge(bv[b], bi[b], v, ix);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    wave_amax(bv[b], bi[b]);
    if (lane == 0) {
      m->wval[w][b] = bv[b];
      m->widx[w][b] = bi[b];
    }
  }
  __syncthreads();
  if (tid < NB) {
    const int b = tid;
    float v = m->wval[0][b];
    int32_t ix = m->widx[0][b];
    for (int ww = 1; ww < NW; ++ww) amax_merge(v, ix, m->wval[ww][b], m->widx[ww][b]);
    m->tok[b] = (ix >= 0 && ix < P.V) ? ix : 0;  // all-NaN logits cannot index outside the vocabulary
  }
  __syncthreads();
}

// 32 bits of a value tagged with the step that wrote it, one 64-bit device-coherent access
__device__ __forceinline__ void st_tv(TV* p, uint32_t bits, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | bits;
  __hip_atomic_store((GAS uint64_t*)p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tv(const TV* p) {
  return __hip_atomic_load((const GAS uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tv_ok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
// an fp64 value as two tagged words: p[0] low half, p[1] high half
__device__ __forceinline__ void st_tvd(TV* p, double v, uint32_t tag) {
  st_tv(p, (uint32_t)__double2loint(v), tag);
  st_tv(p + 1, (uint32_t)__double2hiint(v), tag);
}
__device__ __forceinline__ double tvd_val(uint64_t lo, uint64_t hi) { return __hiloint2double((int)(uint32_t)hi, (int)(uint32_t)lo); }

// split-K partial sums: [operator region][part < kpart_max - 1][row][16 sequences], each an fp64 as
// two tagged words; regions WO (H + 1 rows), DN (H + 1), QKV (QKVR + 1); a region's last row holds
// a part's sums of squares (QKV).  (Sizes chosen arithmetically, not by selecting field addresses.)
__device__ __forceinline__ TV* kpart_row(const KParams& P, int op, int part, int row) {
  const size_t km = (size_t)(P.kpart_max - 1), rh = (size_t)P.H + 1, rq = (size_t)P.QKVR + 1;
  const size_t off = (size_t)(op == OP_DOWN) * km * rh + (size_t)(op == OP_QKV) * 2 * km * rh;
  const size_t rows = (size_t)(op == OP_QKV) * rq + (size_t)(op != OP_QKV) * rh;
  return P.kpart + (off + (size_t)part * rows + (size_t)row) * 32;
}

// ---------------------------------------------------------------------------
// GEMV task: rows [a0, a1) of one weight matrix against B activation vectors.
// Numerics: the staged activation x_k * gamma_k and every product with a bf16
// weight are exact in fp64; each row is summed in fp64 (lane-serial, then a
// fixed tree) and the result is rounded once to fp32 where it is stored.
// ---------------------------------------------------------------------------
// LO: compiled with the LoRA adapters (a separate instantiation, so that the plain GEMV keeps its
// registers)
template <int NB, bool LO, int RPG = 1>
__device__ __forceinline__ bool task_gemv(const KParams& P, const TaskRec& t, int s, bool mega, char* lds,
                                          uint64_t* tr) {
  const int op = (int)t.op, l = (int)t.layer;
  const int tid = ltid(), lane = tid & 63, w = tid >> 6;
  double* xs = (double*)lds;
  double* red = (double*)(lds + P.red_off);
  Misc* m = (Misc*)(lds + P.misc_off);
  const LayerW LW = ldk(P.layers + (op == OP_LM ? 0 : l));

  const uint16_t* W0;
  const uint16_t* W1 = nullptr;
  const uint16_t* gamma = nullptr;
  int K, RU = 1;
  switch (op) {
    case OP_QKV: W0 = LW.wqkv; K = P.H; gamma = LW.attn_norm; break;
    case OP_WO: W0 = LW.wo; K = P.QD; break;
    case OP_GU: W0 = LW.wg; W1 = LW.wu; K = P.H; RU = 2; gamma = LW.ffn_norm; break;
    case OP_DOWN: W0 = LW.wd; K = P.F; break;
    default: W0 = P.lm_head; K = P.H; gamma = P.final_norm; break;
  }
  const bool norm = gamma != nullptr;
  const bool embed_src = (op == OP_QKV && l == 0);
  const int u0 = (int)t.a0, nu = (int)t.a1 - (int)t.a0;
  // LoRA (Mirage article, "Case 2: LoRA + Linear", (W|B)(x|A x)): the tile also streams the
  // adapter A units [la0, la1) of its operator, stored right after the operator's R_op weight
  // units, as the first units of its own list (U < na), so that their sums u = A x are ready
  // early; each is published as soon as its row completes, as a step-tagged fp32 word, and every
  // tile of the operator reads all of them after its own rows.
  const bool lora = LO && t.lora_ev != EV_NONE;
  const int na = lora ? (int)(t.la1 - t.la0) : 0;
  // (arithmetic, not a choice between fields of P: a select of field addresses would make the
  // compiler keep a copy of the whole parameter block in scratch memory)
  const int R_op = (op == OP_QKV) * P.QKVR + (op == OP_GU) * P.F + (op == OP_WO || op == OP_DOWN) * P.H;
  const int a_off = R_op + (int)t.la0;  // unit U < na: A unit la0 + U; else weight unit u0 + U - na
  const int w_off = u0 - na;
  const int nut = nu + na;
  const int wbase = na * RU * NB;  // the weight rows' sums follow the adapter rows' in red
  const int lr = P.lora_r;
  const int lk = op == OP_QKV ? 0 : op == OP_WO ? 1 : op == OP_GU ? 2 : 3;
  TV* const ub = lora ? P.lora_u + (size_t)lk * P.B * 3 * lr : nullptr;  // [B][3 r] of this operator
  const uint32_t utag = (P.epoch + (uint32_t)s) * P.ntag + t.lora_ev + 1u;
  const int my_units = nut > w ? (nut - w + NW - 1) / NW : 0;
  const int my_rows = my_units * RU;
  // split-K (O- and down-projection): part kp of kn takes K elements [k_lo, k_hi), in whole
  // 8-element chunks; the row sums of the others go through kpart to the last part
  const int kp = (int)t.kp, kn = (int)t.kn;
  const int k_lo = kp * (K >> 3) / kn * 8, k_hi = (kp + 1) * (K >> 3) / kn * 8;
  const int kc = min(k_hi - k_lo, (P.xs_doubles / NB) / 512 * 512);
  const int ps = kc >> 2;  // one plane: elements (2p, 2p+1) of every 8-element chunk, kc/8 pairs
  const int nsl = (k_hi - k_lo + kc - 1) / kc;

  auto rowptr = [&](int r) -> const uint16_t* {
    const int ui = RU == 2 ? (r >> 1) : r;
    const uint16_t* base = (RU == 2 && (r & 1)) ? W1 : W0;
    const int U = w + NW * ui;
    if constexpr (LO) return base + (size_t)(U + (U < na ? a_off : w_off)) * K;
    else return base + (size_t)(u0 + U) * K;
  };

  // pipeline state for one slice.  With four sequences the activations read from LDS for a
  // chunk serve RPG rows (a group holds CG / RPG chunks of each of RPG rows): at one row per
  // read the reads would outrun LDS bandwidth.  RPG is chosen per operator (run_task).
  constexpr int CGE = CG / RPG;
  const int my_groups = (my_rows + RPG - 1) / RPG;  // row groups (a last odd row is paired with itself)
  uint4 buf[DEPTH][CG];
  int ir = 0, ig = 0, cr = 0, cgi = 0;
  int k0 = 0, nch8 = 0, GPR = 1;
  auto slice_setup = [&](int sl) {
    k0 = k_lo + sl * kc;
    const int ks = min(kc, k_hi - k0);
    nch8 = ks / 8;
    const int nch = (nch8 + 63) / 64;
    GPR = (nch + CGE - 1) / CGE;
    ir = ig = cr = cgi = 0;
  };
  // Loads are never predicated: lanes past the row end re-read the row's last
  // chunk (a clamped, in-bounds address) and are zeroed when consumed, so the
  // steady-state loop is branch-free and its waits count outstanding loads.
  auto issue_nocheck = [&](uint4 (&b)[CG]) {
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      const uint16_t* p = rowptr(RPG == 1 ? ir : min(ir * RPG + rr, my_rows - 1)) + k0;
#pragma unroll
      for (int c = 0; c < CGE; ++c) {
        const int j = min((ig * CGE + c) * 64 + lane, nch8 - 1);
        b[rr * CGE + c] = ldw(p + (size_t)j * 8);
      }
    }
    if (++ig == GPR) {
      ig = 0;
      ++ir;
    }
  };
  auto issue = [&](uint4 (&b)[CG]) {
    if (ir < my_groups) issue_nocheck(b);
  };

  double acc[RPG][NB];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[rr][b] = 0.0;
  int sl_cur = 0;
  auto consume = [&](const uint4 (&bw)[CG]) {
#pragma unroll
    for (int c = 0; c < CGE; ++c) {
      const int jr = (cgi * CGE + c) * 64 + lane;
      const bool ok = jr < nch8;
      const int j = ok ? jr : nch8 - 1;
      double wd[RPG][8];
#pragma unroll
      for (int rr = 0; rr < RPG; ++rr) {
        const uint4 q = bw[rr * CGE + c];
        const uint32_t wv[4] = {ok ? q.x : 0u, ok ? q.y : 0u, ok ? q.z : 0u, ok ? q.w : 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wd[rr][2 * e] = (double)bf_lo(wv[e]);
          wd[rr][2 * e + 1] = (double)bf_hi(wv[e]);
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // four planes per sequence, so that consecutive lanes read consecutive 16-byte pairs
        const double* xb = xs + (size_t)b * kc + j * 2;
        const v2d x0 = *(const v2d*)(xb);
        const v2d x1 = *(const v2d*)(xb + ps);
        const v2d x2 = *(const v2d*)(xb + 2 * ps);
        const v2d x3 = *(const v2d*)(xb + 3 * ps);
#pragma unroll
        for (int rr = 0; rr < RPG; ++rr) {
          double a = acc[rr][b];
          a = fma(wd[rr][0], x0.x, a);
          a = fma(wd[rr][1], x0.y, a);
          a = fma(wd[rr][2], x1.x, a);
          a = fma(wd[rr][3], x1.y, a);
          a = fma(wd[rr][4], x2.x, a);
          a = fma(wd[rr][5], x2.y, a);
          a = fma(wd[rr][6], x3.x, a);
          a = fma(wd[rr][7], x3.y, a);
          acc[rr][b] = a;
        }
      }
    }
    if (++cgi == GPR) {
      cgi = 0;
#pragma unroll
      for (int rr = 0; rr < RPG; ++rr) {
        const int r = cr * RPG + rr;  // the wave's row
        const int ui = RU == 2 ? (r >> 1) : r;
        const int rl = (w + NW * ui) * RU + (RU == 2 ? (r & 1) : 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const double v = wave_sum_d(acc[rr][b]);
          if (lane == 0 && (RPG == 1 || r < my_rows)) {
            const double tot = sl_cur == 0 ? v : red[rl * NB + b] + v;
            red[rl * NB + b] = tot;
            if constexpr (LO) {  // a completed adapter row: publish u = (A x) scaled like the weight rows
              const int U = w + NW * ui;
              if (U < na && sl_cur == nsl - 1) {
                double ss = 0.0;
                for (int ww = 0; ww < NW; ++ww) ss += m->wred[ww][b];
                const double rsb = norm ? 1.0 / sqrt(ss / (double)K + (double)P.eps) : 1.0;
                const int idx = (int)t.la0 + U + (RU == 2 ? (r & 1) * lr : 0);
                st_tv(ub + (size_t)b * 3 * lr + idx, __float_as_uint((float)(tot * rsb)), utag);
              }
            }
          }
          acc[rr][b] = 0.0;
        }
      }
      ++cr;
    }
  };

  // Weights do not depend on the event: start streaming before waiting.
  slice_setup(0);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(buf[d]);

  // LoRA: the tile's B rows (r bf16 per output row) do not depend on it either; up to two 16-byte
  // pieces per thread are requested now and parked in LDS after the rows are streamed
  const int bper = LO ? lr / 8 : 1;              // 16-byte pieces per B row
  const int nbq = lora ? nu * RU * bper : 0;     // pieces of the tile's B rows
  const bool bpre = lora && nbq <= 2 * NT;
  uint4 bq[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  // B row `row` of the tile (RU per unit; at gate/up the gate and up rows of unit row / 2)
  auto brow = [&](int row) -> const uint16_t* {
    const int ul = RU == 2 ? row >> 1 : row;
    const uintptr_t bm = (op == OP_QKV ? (uintptr_t)LW.b_qkv : 0) | (op == OP_WO ? (uintptr_t)LW.b_o : 0) |
                         (op == OP_DOWN ? (uintptr_t)LW.b_d : 0) |
                         (op == OP_GU ? (uintptr_t)((row & 1) ? LW.b_u : LW.b_g) : 0);
    return (const uint16_t*)bm + (size_t)(u0 + ul) * lr;
  };
  if constexpr (LO) {
    if (bpre)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int q = tid + k * NT;
        if (q < nbq) bq[k] = ldg((const uint4*)(brow(q / bper) + (q % bper) * 8));
      }
  }

  // a wait on the previous step is met by the launch boundary at the first step of a call
  if (mega && !(s == 0 && t.wait_lag) &&
      !wait_event(P, t.wait_ev, P.epoch + (uint32_t)s + 1u - t.wait_lag, t.tile, m, tr, t.op == OP_WO))
    return false;

  // layer-0 Q/K/V reads the embedding of this step's token
  if (embed_src) {
    if (P.force_tok) {
      if (tid < NB) m->tok[tid] = ldg(P.force_tok + (size_t)s * P.B + tid);
      __syncthreads();
    } else if (s == 0) {
      if (tid < NB) {
        const int32_t tk = ldg(P.pending + tid);
        m->tok[tid] = (tk >= 0 && tk < P.V) ? tk : 0;
      }
      __syncthreads();
    } else {
      reduce_tokens<NB>(P, m);
      if (t.tile == 0 && P.out_tokens && tid < NB) stg(P.out_tokens + (size_t)(s - 1) * P.B + tid, m->tok[tid]);
    }
    // this tile's share of x = embedding (read by the O-projection residual)
    const int h0 = (int)((int64_t)t.tile * P.H / P.n_qkv), h1 = (int)((int64_t)(t.tile + 1) * P.H / P.n_qkv);
    for (int i = h0 + tid; i < h1; i += NT)
#pragma unroll
      for (int b = 0; b < NB; ++b) stc(P.x + (size_t)b * P.H + i, bf1(ldg(P.embed + (size_t)m->tok[b] * P.H + i)));
  }

  // The residual this task adds to (O-projection, down projection) is read now,
  // after the wait, so the epilogue does not wait a round trip for it.
  const bool resid = op == OP_WO || op == OP_DOWN;
  float xpre = 0.f;
  if (resid && kp == kn - 1 && tid < nu * NB) {
    const int ul = tid / NB, b = tid - ul * NB;
    xpre = ldc(P.x + (size_t)b * P.H + u0 + ul);
  }

  for (int sl = 0; sl < nsl; ++sl) {
    sl_cur = sl;
    if (sl > 0) {
      __syncthreads();  // every wave is done with the previous slice of xs
      slice_setup(sl);
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) issue(buf[d]);
    }
    // ---- stage activations of this slice into LDS (x * gamma, exact in fp64); sum of squares on slice 0
    {
      const int ks = min(kc, k_hi - k0);
      double ss[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) ss[b] = 0.0;
      const int e_lo = (sl == 0 && norm) ? 0 : k0, e_hi = (sl == 0 && norm) ? K : k0 + ks;
      constexpr int SU = NB >= 8 ? 1 : 8 / NB;  // 16-byte loads in flight per thread and sequence
      for (int base = e_lo + tid * 4; base < e_hi; base += NT * 4 * SU) {
        v4f v[SU][NB];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const int e = base + u * NT * 4;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if (e < e_hi) {
              if (embed_src) {
                const uint16_t* er = P.embed + (size_t)m->tok[b] * P.H + e;
                const uint2 q = ldg((const uint2*)er);
                v[u][b] = v4f{bf_lo(q.x), bf_hi(q.x), bf_lo(q.y), bf_hi(q.y)};
              } else {
                const float* src;
                if constexpr (LO)  // the same choice without a select of field addresses (see R_op)
                  src = (const float*)((op == OP_WO ? (uintptr_t)(P.o + (size_t)b * P.QD) : 0) |
                                       (op == OP_DOWN ? (uintptr_t)(P.a + (size_t)b * P.F) : 0) |
                                       (op != OP_WO && op != OP_DOWN ? (uintptr_t)(P.x + (size_t)b * P.H) : 0));
                else
                  src = op == OP_WO ? P.o + (size_t)b * P.QD : op == OP_DOWN ? P.a + (size_t)b * P.F : P.x + (size_t)b * P.H;
                v[u][b] = ldc4(src, (uint32_t)e);
              }
            } else {
              v[u][b] = v4f{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const int e = base + u * NT * 4;
          if (e < e_hi) {
            float g4[4] = {1.f, 1.f, 1.f, 1.f};
            if (norm) {
              const uint2 gq = ldg((const uint2*)(gamma + e));
              g4[0] = bf_lo(gq.x);
              g4[1] = bf_hi(gq.x);
              g4[2] = bf_lo(gq.y);
              g4[3] = bf_hi(gq.y);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const v4f x = v[u][b];
              if (norm && sl == 0) {
                const double d0 = x.x, d1 = x.y, d2 = x.z, d3 = x.w;
                ss[b] += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
              }
              if (e >= k0 && e < k0 + ks) {
                const int el = e - k0;
                double* xb = xs + (size_t)b * kc + ((el >> 2) & 1) * 2 * ps + (el >> 3) * 2;
                *(v2d*)xb = v2d{(double)x.x * (double)g4[0], (double)x.y * (double)g4[1]};
                *(v2d*)(xb + ps) = v2d{(double)x.z * (double)g4[2], (double)x.w * (double)g4[3]};
              }
            }
          }
        }
      }
      if (norm && sl == 0) {  // per-wave partial sums; the scale itself is formed in the epilogue
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const double v = wave_sum_d(ss[b]);
          if (lane == 0) m->wred[w][b] = v;
        }
      }
      __syncthreads();
    }
    // ---- stream this slice's weight rows through the pipeline
    if (tr && sl == 0 && tid == 0) tr[2] = wall_clock64();
    // Nothing is outstanding here (staging waited for its loads, which were
    // issued after the prefetch); saying so explicitly gives the compiler an
    // exact count to start from, so the loop below waits only for the oldest
    // group instead of draining every load.
    __builtin_amdgcn_s_waitcnt(0);
    const int total = my_groups * GPR;
    int g = 0;
    for (; g + 2 * DEPTH <= total; g += DEPTH) {  // steady state: DEPTH groups always in flight
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        consume(buf[d]);
        issue_nocheck(buf[d]);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {  // drain
      if (g + d < total) {
        consume(buf[d]);
        if (g + d + DEPTH < total) issue_nocheck(buf[d]);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (g + DEPTH + d < total) consume(buf[d]);
  }
  __syncthreads();

  // ---- split-K: a part below the last publishes its row sums (fp64, two words tagged with the
  // step and the operator's event) and is done; the last part adds the others' in order of part,
  // its own last, polling a word not yet published (no adapters here: wbase is 0).  Not compiled
  // for one sequence, whose activations always fit one slice (with it, the compiler keeps a copy
  // of the parameter block in scratch memory).
  if constexpr (NB >= 2) {
    if (kn > 1) {
      const uint32_t ktag = (P.epoch + (uint32_t)s) * P.ntag + t.wait_ev + 1u;
      if (kp < kn - 1) {
        for (int i = tid; i < nu * NB; i += NT) {
          const int ul = i / NB, b = i - ul * NB;
          st_tvd(kpart_row(P, op, kp, u0 + ul) + b * 2, red[ul * NB + b], ktag);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        return true;
      }
      bool ok = true;
      for (int i = tid; i < nu * NB; i += NT) {
        const int ul = i / NB, b = i - ul * NB;
        double v = 0.0;
        for (int q = 0; q < kn - 1 && ok; ++q) {
          const TV* src = kpart_row(P, op, q, u0 + ul) + b * 2;
          uint64_t lo = ld_tv(src), hi = ld_tv(src + 1);
          for (uint32_t polls = 0; !(tv_ok(lo, ktag) && tv_ok(hi, ktag));) {
            if (++polls >= P.watchdog || ldc_u(P.status + ST_ABORT)) {
              ok = false;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
            lo = ld_tv(src);
            hi = ld_tv(src + 1);
          }
          v += tvd_val(lo, hi);
        }
        red[ul * NB + b] = v + red[ul * NB + b];
      }
      if (tid == 0) m->flag = 1;
      __syncthreads();
      if (!ok) {
        uint32_t zero = 0u;
        if (__hip_atomic_compare_exchange_strong((GAS uint32_t*)(P.status + ST_CODE), &zero, ERR_WATCHDOG,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          stc_u(P.status + ST_CU, blockIdx.x);
          stc_u(P.status + ST_TASK, t.tile);
          stc_u(P.status + ST_EVENT, t.sig_ev);
        }
        stc_u(P.status + ST_ABORT, 1u);
        m->flag = 0;
      }
      __syncthreads();
      if (!m->flag) return false;
    }
  }

  // ---- RMSNorm scale r = 1/sqrt(mean(x^2) + eps) in fp64, applied after the dot products
  double rs[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    double tot = 0.0;
    for (int ww = 0; ww < NW; ++ww) tot += m->wred[ww][b];
    rs[b] = norm ? 1.0 / sqrt(tot / (double)K + (double)P.eps) : 1.0;
  }

  // ---- LoRA: read the operator's adapter sums u = A x (fp32, the stored second half of the
  // concatenated operand), each a word tagged with this step, into LDS (the activation staging area
  // is free from here on); a word not yet published is polled, every mode (the publishing tiles
  // run in the same launch)
  const int nA = op == OP_QKV ? 3 * lr : op == OP_GU ? 2 * lr : lr;  // the operator's u per sequence
  double* uu = xs;                                                   // [NB][nA]
  uint4* bl = (uint4*)(xs + ((NB * nA + 1) & ~1));                   // [nbq] the tile's B rows
  if (lora) {
    if (bpre)
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (tid + k * NT < nbq) bl[tid + k * NT] = bq[k];
    // (the verdict goes through LDS: the workgroup-reduction builtins reserve static LDS, and the
    // workers take all of it dynamically)
    if (tid == 0) m->lora_fail = 0;
    __syncthreads();
    bool ok = true;
    for (int i = tid; i < NB * nA; i += NT) {
      const int b = i / nA, j = i - b * nA;
      const TV* up = ub + (size_t)b * 3 * lr + j;
      uint64_t v = ld_tv(up);
      for (uint32_t polls = 0; !tv_ok(v, utag);) {
        if (++polls >= P.watchdog || ldc_u(P.status + ST_ABORT)) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = ld_tv(up);
      }
      uu[i] = (double)__uint_as_float((uint32_t)v);
    }
    if (!ok) {
      uint32_t zero = 0u;
      if (__hip_atomic_compare_exchange_strong((GAS uint32_t*)(P.status + ST_CODE), &zero, ERR_WATCHDOG,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        stc_u(P.status + ST_CU, blockIdx.x);
        stc_u(P.status + ST_TASK, t.tile);
        stc_u(P.status + ST_EVENT, t.lora_ev);
      }
      stc_u(P.status + ST_ABORT, 1u);
      m->lora_fail = 1;
    }
    __syncthreads();
    if (m->lora_fail) return false;
  }
  // B row `row` of Bm [rows][r] against u[b][seg, seg + r), summed in fp64 in order (exact products)
  // tile row `row` (as brow) against u[b][seg, seg + r), in fp64 in order (exact products)
  auto lora_term = [&](int row, int seg, int b) -> double {
    const uint16_t* br = brow(row);
    const double* ur = uu + b * nA + seg;
    double acc = 0.0;
    for (int j = 0; j < lr; j += 8) {
      const uint4 q = bpre ? bl[row * bper + j / 8] : ldg((const uint4*)(br + j));
      const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fma((double)bf_lo(wv[e]), ur[j + 2 * e], acc);
        acc = fma((double)bf_hi(wv[e]), ur[j + 2 * e + 1], acc);
      }
    }
    return acc;
  };

  // ---- epilogue per operator
  if (op == OP_QKV) {
    for (int i = tid; i < nu * NB; i += NT) {
      const int ul = i / NB, b = i - ul * NB;
      double v = red[wbase + ul * NB + b] * rs[b];
      if (lora) {  // the row's adapter: q, k or v by its place in the KV-head group
        const int gi = (u0 + ul) % P.RG;
        v += lora_term(ul, gi < P.G * P.D ? 0 : gi < (P.G + 1) * P.D ? lr : 2 * lr, b);
      }
      stc(P.qkv + (size_t)b * P.QKVR + u0 + ul, (float)v);
    }
  } else if (resid) {
    for (int i = tid; i < nu * NB; i += NT) {
      const int ul = i / NB, b = i - ul * NB;
      float* xp = P.x + (size_t)b * P.H + u0 + ul;
      double y = red[wbase + ul * NB + b];
      if (lora) y += lora_term(ul, 0, b);
      stc(xp, (float)((double)(i == tid ? xpre : ldc(xp)) + y));
    }
  } else if (op == OP_GU) {
    for (int i = tid; i < nu * NB; i += NT) {
      const int ul = i / NB, b = i - ul * NB;
      double gt = red[wbase + (ul * 2) * NB + b] * rs[b];
      double up = red[wbase + (ul * 2 + 1) * NB + b] * rs[b];
      if (lora) {
        gt += lora_term(2 * ul, 0, b);
        up += lora_term(2 * ul + 1, lr, b);
      }
      stc(P.a + (size_t)b * P.F + u0 + ul, (float)(silu_d(gt) * up));
    }
  } else {  // OP_LM
    float bv[NB];
    int32_t bi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      bv[b] = -INFINITY;
      bi[b] = 0x7fffffff;
    }
    for (int ul = tid; ul < nu; ul += NT) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float logit = (float)(red[ul * NB + b] * rs[b]);
        if (P.out_logits) stg(P.out_logits + ((size_t)s * P.B + b) * P.V + u0 + ul, logit);
        amax_merge(bv[b], bi[b], logit, u0 + ul);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      wave_amax(bv[b], bi[b]);
      if (lane == 0) {
        m->wval[w][b] = bv[b];
        m->widx[w][b] = bi[b];
      }
    }
    __syncthreads();
    if (tid < NB) {
      float v = m->wval[0][tid];
      int32_t ix = m->widx[0][tid];
      for (int ww = 1; ww < NW; ++ww) amax_merge(v, ix, m->wval[ww][tid], m->widx[ww][tid]);
      LmPart* lp = P.lm_part + (size_t)tid * P.n_lm + t.tile;
      stc(&lp->val, v);
      stc_i(&lp->idx, ix);
    }
  }
  signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
  return true;
}

// ---------------------------------------------------------------------------
// GEMV task for B >= 8 sequences: a skinny GEMM on the matrix cores.
//   Y[rows x 16] = W[rows x K] . X[K x 16]  with v_mfma_f32_16x16x32_bf16
// (columns beyond B are zero).  Each fp32 activation is split exactly into
// three bf16 pieces, x = x0 + x1 + x2, so every product W * x_p is exact; the
// only rounding before the fp64 epilogue is the fp32 accumulation inside one
// wave's share of K.  The eight waves split every K slice and their partial
// sums are added in fp64.
// K goes through LDS in slices of MK_KS elements, staged as fp32 x * gamma
// (layout [8-element block][column][8 x fp32]) and split into the three pieces
// when a step reads them.  K is padded to whole slices: the padding's
// activations are zero and its weight loads re-read the row's last chunk.
// Each wave takes MK_KS / 8 elements (MK_SPS steps of 32) of every slice.  Rows
// go in tiles of 16, up to MT tiles per pass over K.  The weights stream
// through NBUF register buffers of NTB tile slots (NBUF * NTB = 16, at most 8
// buffers): with few tiles, more steps are in flight.
// Lane layout on gfx950: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16]
// and D[4(l/16)+r][l%16], e < 8, r < 4.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int MT = 8;                    // row tiles per pass
constexpr int MK_KS = 2048;              // K elements per staged slice (the host plans the same)
constexpr int MK_SPS = MK_KS / NW / 32;  // 32-element steps per wave per slice

// x = bf16(p0) + bf16(p1) + bf16(p2) exactly (truncations of x and of the exact remainders)
__device__ __forceinline__ void split3(float x, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
  const uint32_t u = __float_as_uint(x);
  const float r1 = x - __uint_as_float(u & 0xffff0000u);
  const uint32_t u1 = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
  p0 = u >> 16;
  p1 = u1 >> 16;
  p2 = __float_as_uint(r2) >> 16;
}

// Stage K elements [k0, k0 + MK_KS) of the B activation rows as fp32 x * gamma
// (zero beyond K).  Thread tid takes column tid % 16 and 8-element blocks
// tid / 16, tid / 16 + NT / 16, ...; IB blocks' loads are in flight together.
// src is the activation array (row stride `stride`), read with device-coherent
// loads; layer-0 Q/K/V reads the embedding rows instead.  src is a plain,
// uniform argument: a buffer resource built from a per-lane pointer would need
// a loop over its distinct values.
template <int NB>
__device__ __forceinline__ void mfma_stage(const KParams& P, const float* src, int stride, bool embed_src,
                                           const uint16_t* gamma, const Misc* m, int k0, int K, bool sumsq,
                                           char* lds, double& ss) {
  const int tid = ltid(), jcol = tid & 15;
  const bool norm = gamma != nullptr;
  const uint32_t scol = (uint32_t)jcol * (uint32_t)stride;  // this column's row, as a per-lane offset
  constexpr int items = (MK_KS / 8) * 16;
  constexpr int IB = 4;
  static_assert(items % (NT * IB) == 0, "staging items");
#pragma unroll 1
  for (int it0 = tid; it0 < items; it0 += NT * IB) {
    uint4 raw[IB][2], gqa[IB];
#pragma unroll
    for (int q = 0; q < IB; ++q) {
      const int kb = k0 + 8 * ((it0 + q * NT) >> 4);
      if (jcol < NB && kb < K) {
        if (embed_src) {
          raw[q][0] = ld16(P.embed + (size_t)m->tok[jcol] * P.H + kb);
        } else {
          raw[q][0] = __builtin_bit_cast(uint4, ldc4(src, scol + (uint32_t)kb));
          raw[q][1] = __builtin_bit_cast(uint4, ldc4(src, scol + (uint32_t)kb + 4u));
        }
        if (norm) gqa[q] = ld16(gamma + kb);
      }
    }
#pragma unroll
    for (int q = 0; q < IB; ++q) {
      const int it = it0 + q * NT, c = it >> 4, kb = k0 + 8 * c;
      float xv[8];
      if (jcol < NB && kb < K) {
        if (embed_src) {
          const uint32_t qw[4] = {raw[q][0].x, raw[q][0].y, raw[q][0].z, raw[q][0].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[2 * e] = bf_lo(qw[e]);
            xv[2 * e + 1] = bf_hi(qw[e]);
          }
        } else {
          const uint32_t xw[8] = {raw[q][0].x, raw[q][0].y, raw[q][0].z, raw[q][0].w,
                                  raw[q][1].x, raw[q][1].y, raw[q][1].z, raw[q][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = __uint_as_float(xw[e]);
        }
        if (norm) {
          const uint32_t gw[4] = {gqa[q].x, gqa[q].y, gqa[q].z, gqa[q].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double xd = xv[e];
            if (sumsq) ss += xd * xd;
            xv[e] = (float)(xd * (double)((e & 1) ? bf_hi(gw[e >> 1]) : bf_lo(gw[e >> 1])));
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = 0.f;
      }
      char* xb = lds + (size_t)(c * 16 + jcol) * 32;
      *(v4f*)(xb) = v4f{xv[0], xv[1], xv[2], xv[3]};
      *(v4f*)(xb + 16) = v4f{xv[4], xv[5], xv[6], xv[7]};
    }
  }
}

template <int NB, int NTB>
__device__ __forceinline__ bool gemv_mfma(const KParams& P, const TaskRec& t, int s, bool mega, char* lds, uint64_t* tr,
                                          int op, const uint16_t* W0, const uint16_t* W1, const uint16_t* gamma, int K,
                                          int RU) {
  constexpr int NBUF = (16 / NTB) > 8 ? 8 : 16 / NTB;
  static_assert(MK_SPS % NBUF == 0, "buffers per slice");
  const int l = (int)t.layer;
  const int tid = ltid(), lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;  // MFMA row / column index and K quarter of this lane
  double* red = (double*)(lds + P.red_off);
  Misc* m = (Misc*)(lds + P.misc_off);
  const bool norm = gamma != nullptr;
  const bool embed_src = (op == OP_QKV && l == 0);
  const int u0 = (int)t.a0, nu = (int)t.a1 - (int)t.a0;
  const int R = nu * RU, T = (R + 15) >> 4;
  // split-K (O- and down-projection): part kp of kn takes the K slices [sl0, sl0 + nsl)
  const int kp = (int)t.kp, kn = (int)t.kn, nsl_all = (K + MK_KS - 1) / MK_KS;
  const int sl0 = kp * nsl_all / kn;
  const int nsl = (kp + 1) * nsl_all / kn - sl0;
  const int npass = (T + MT - 1) / MT;
  const int gsteps = npass * nsl * MK_SPS;  // this wave's steps, over every pass and slice

  // the weights of this wave's step g (pass, slice, step), one 16-byte chunk per tile slot
  auto issue = [&](uint4 (&a)[NTB], int g) {
    if (g >= gsteps) return;
    const int pass = g / (nsl * MK_SPS), r = g - pass * nsl * MK_SPS;
    const int sl = r / MK_SPS, st = r - sl * MK_SPS;
    const int kk = min((sl0 + sl) * MK_KS + w * (MK_KS / NW) + 32 * st + 8 * lq, K - 8);
#pragma unroll
    for (int tt = 0; tt < NTB; ++tt) {
      const int row = min((min(pass * MT + tt, T - 1)) * 16 + li, R - 1);
      const int ui = RU == 2 ? (row >> 1) : row;
      const uint16_t* base = (RU == 2 && (row & 1)) ? W1 : W0;
      a[tt] = ldw(base + (size_t)(u0 + ui) * K + kk);
    }
  };
  uint4 A[NBUF][NTB];
  // weights do not depend on the event: the first NBUF steps go out before the wait
#pragma unroll
  for (int b = 0; b < NBUF; ++b) issue(A[b], b);

  if (mega && !(s == 0 && t.wait_lag) &&
      !wait_event(P, t.wait_ev, P.epoch + (uint32_t)s + 1u - t.wait_lag, t.tile, m, tr, t.op == OP_WO))
    return false;

  if (embed_src) {
    if (P.force_tok) {
      if (tid < NB) m->tok[tid] = ldg(P.force_tok + (size_t)s * P.B + tid);
      __syncthreads();
    } else if (s == 0) {
      if (tid < NB) {
        const int32_t tk = ldg(P.pending + tid);
        m->tok[tid] = (tk >= 0 && tk < P.V) ? tk : 0;
      }
      __syncthreads();
    } else {
      reduce_tokens<NB>(P, m);
      if (t.tile == 0 && P.out_tokens && tid < NB) stg(P.out_tokens + (size_t)(s - 1) * P.B + tid, m->tok[tid]);
    }
    const int h0 = (int)((int64_t)t.tile * P.H / P.n_qkv), h1 = (int)((int64_t)(t.tile + 1) * P.H / P.n_qkv);
    for (int i = h0 + tid; i < h1; i += NT)
#pragma unroll
      for (int b = 0; b < NB; ++b) stc(P.x + (size_t)b * P.H + i, bf1(ldg(P.embed + (size_t)m->tok[b] * P.H + i)));
  }

  double ss = 0.0;  // sum of squares of column tid % 16 (first pass)
  if (op == OP_LM && tid < NB) {
    m->lmv[tid] = -INFINITY;
    m->lmi[tid] = 0x7fffffff;
  }

  int g = 0;  // this wave's next step
  for (int pass = 0; pass < npass; ++pass) {
    const int tp0 = pass * MT, ntp = min(MT, T - tp0);
    v4f acc[NTB];
#pragma unroll
    for (int tt = 0; tt < NTB; ++tt) acc[tt] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < nsl; ++sl) {
      const int k0 = (sl0 + sl) * MK_KS;
      __syncthreads();  // the previous slice (or pass) is no longer read
      const bool sumsq = norm && pass == 0;
      if (op == OP_WO) mfma_stage<NB>(P, P.o, P.QD, false, nullptr, m, k0, K, false, lds, ss);
      else if (op == OP_DOWN) mfma_stage<NB>(P, P.a, P.F, false, nullptr, m, k0, K, false, lds, ss);
      else mfma_stage<NB>(P, P.x, P.H, embed_src, gamma, m, k0, K, sumsq, lds, ss);
      __syncthreads();
      if (tr && pass == 0 && sl == 0 && tid == 0) tr[2] = wall_clock64();
      // ---- this wave's MK_SPS steps of the slice; each consumes buffer b, then refills it
      // with the step NBUF ahead (which may belong to the next slice or pass)
      for (int st0 = 0; st0 < MK_SPS; st0 += NBUF) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
          const int cblk = (w * (MK_KS / NW) + 32 * (st0 + b)) / 8 + lq;  // 8-element block of this lane
          const char* xb = lds + (size_t)(cblk * 16 + li) * 32;
          const v4f xa = *(const v4f*)(xb), xc = *(const v4f*)(xb + 16);
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xc.x, xc.y, xc.z, xc.w};
          uint32_t p0[8], p1[8], p2[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) split3(xv[e], p0[e], p1[e], p2[e]);
          const bf16x8 b0 = __builtin_bit_cast(bf16x8, make_uint4(p0[0] | (p0[1] << 16), p0[2] | (p0[3] << 16), p0[4] | (p0[5] << 16), p0[6] | (p0[7] << 16)));
          const bf16x8 b1 = __builtin_bit_cast(bf16x8, make_uint4(p1[0] | (p1[1] << 16), p1[2] | (p1[3] << 16), p1[4] | (p1[5] << 16), p1[6] | (p1[7] << 16)));
          const bf16x8 b2 = __builtin_bit_cast(bf16x8, make_uint4(p2[0] | (p2[1] << 16), p2[2] | (p2[3] << 16), p2[4] | (p2[5] << 16), p2[6] | (p2[7] << 16)));
#pragma unroll
          for (int tt = 0; tt < NTB; ++tt) {
            if (tt < ntp) {
              const bf16x8 a = __builtin_bit_cast(bf16x8, A[b][tt]);
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[tt], 0, 0, 0);
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[tt], 0, 0, 0);
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, acc[tt], 0, 0, 0);
            }
          }
          issue(A[b], g + NBUF);
          ++g;
        }
      }
    }
    // ---- add the eight waves' partial tiles in fp64 (the staging area is free now)
    __syncthreads();
    float* part = (float*)lds;  // [wave][tile][256]
#pragma unroll
    for (int tt = 0; tt < NTB; ++tt)
      if (tt < ntp)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[((size_t)w * MT + tt) * 256 + (lq * 4 + r) * 16 + li] = acc[tt][r];
    if (pass == 0 && norm) {  // per-wave sums of squares per column: lanes with equal (lane & 15) share a column
      double v = ss;
      v = xor16_pair_d(v);
      v = xor32_pair_d(v);
      if (lane < 16) m->wred[w][lane] = v;
    }
    __syncthreads();
    const int rows = min(R - tp0 * 16, ntp * 16);
    for (int i = tid; i < rows * NB; i += NT) {
      const int rr = i / NB, b = i - rr * NB;
      const int tt = rr >> 4, ri = rr & 15;
      double v = 0.0;
      for (int ww = 0; ww < NW; ++ww) v += (double)part[((size_t)ww * MT + tt) * 256 + ri * 16 + b];
      red[rr * NB + b] = v;
    }
    if (kn > 1) {
      // split-K: a part below the last publishes its row sums (fp64, as two words tagged with the
      // step and the operator's input event, which differs per layer) and, at QKV, its sums of
      // squares; the last part adds the others' in order of part, its own last, polling a word
      // not yet published.  Only the last part runs the epilogue.
      const uint32_t ktag = (P.epoch + (uint32_t)s) * P.ntag + t.wait_ev + 1u;
      const int prow0 = u0 * RU + tp0 * 16;
      const int srow = (op == OP_QKV) * P.QKVR + (op != OP_QKV) * P.H;  // the sums-of-squares row
      const bool pss = norm && pass == 0;
      __builtin_amdgcn_s_waitcnt(0);  // this task's earlier stores (layer 0: its share of x) are done
      __syncthreads();                // red complete
      if (kp < kn - 1) {
        for (int i = tid; i < rows * NB; i += NT) {
          const int rr = i / NB, b = i - rr * NB;
          st_tvd(kpart_row(P, op, kp, prow0 + rr) + b * 2, red[rr * NB + b], ktag);
        }
        if (pss && tid < NB) {
          double tot = 0.0;
          for (int ww = 0; ww < NW; ++ww) tot += m->wred[ww][tid];
          st_tvd(kpart_row(P, op, kp, srow) + tid * 2, tot, ktag);
        }
        continue;  // next pass
      }
      bool ok = true;
      auto poll_sum = [&](int row, int b) -> double {
        double v = 0.0;
        for (int q = 0; q < kn - 1 && ok; ++q) {
          const TV* src = kpart_row(P, op, q, row) + b * 2;
          uint64_t lo = ld_tv(src), hi = ld_tv(src + 1);
          for (uint32_t polls = 0; !(tv_ok(lo, ktag) && tv_ok(hi, ktag));) {
            if (++polls >= P.watchdog || ldc_u(P.status + ST_ABORT)) {
              ok = false;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
            lo = ld_tv(src);
            hi = ld_tv(src + 1);
          }
          v += tvd_val(lo, hi);
        }
        return v;
      };
      for (int i = tid; i < rows * NB; i += NT) {
        const int rr = i / NB, b = i - rr * NB;
        red[rr * NB + b] = poll_sum(prow0 + rr, b) + red[rr * NB + b];
      }
      if (pss && tid < NB) m->kss[tid] = poll_sum(srow, tid);
      if (tid == 0) m->flag = 1;
      __syncthreads();
      if (!ok) {
        uint32_t zero = 0u;
        if (__hip_atomic_compare_exchange_strong((GAS uint32_t*)(P.status + ST_CODE), &zero, ERR_WATCHDOG,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          stc_u(P.status + ST_CU, blockIdx.x);
          stc_u(P.status + ST_TASK, t.tile);
          stc_u(P.status + ST_EVENT, t.sig_ev);
        }
        stc_u(P.status + ST_ABORT, 1u);
        m->flag = 0;
      }
      __syncthreads();
      if (!m->flag) return false;
    }
    // ---- epilogue for this pass's rows (the RMSNorm scale per sequence, formed once, in LDS)
    if (tid < NB) {
      double tot = (kn > 1 && norm) ? m->kss[tid] : 0.0;  // split: the other parts' first, in order
      for (int ww = 0; ww < NW; ++ww) tot += m->wred[ww][tid];
      m->rsd[tid] = norm ? 1.0 / sqrt(tot / (double)K + (double)P.eps) : 1.0;
    }
    __syncthreads();
    const double* rs = m->rsd;
    const int pu0 = u0 + tp0 * 16 / RU, pnu = rows / RU;
    if (op == OP_QKV) {
      for (int i = tid; i < pnu * NB; i += NT) {
        const int ul = i / NB, b = i - ul * NB;
        stc(P.qkv + (size_t)b * P.QKVR + pu0 + ul, (float)(red[ul * NB + b] * rs[b]));
      }
    } else if (op == OP_WO || op == OP_DOWN) {
      for (int i = tid; i < pnu * NB; i += NT) {
        const int ul = i / NB, b = i - ul * NB;
        float* xp = P.x + (size_t)b * P.H + pu0 + ul;
        stc(xp, (float)((double)ldc(xp) + red[ul * NB + b]));
      }
    } else if (op == OP_GU) {
      for (int i = tid; i < pnu * NB; i += NT) {
        const int ul = i / NB, b = i - ul * NB;
        const double gt = red[(ul * 2) * NB + b] * rs[b];
        const double up = red[(ul * 2 + 1) * NB + b] * rs[b];
        stc(P.a + (size_t)b * P.F + pu0 + ul, (float)(silu_d(gt) * up));
      }
    } else {  // OP_LM
      if (P.out_logits)
        for (int ul = tid; ul < pnu; ul += NT)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            stg(P.out_logits + ((size_t)s * P.B + b) * P.V + pu0 + ul, (float)(red[ul * NB + b] * rs[b]));
      // this pass's (max, lowest index) per sequence: thread (b, c) scans rows c, c + TPB, ... of
      // sequence b, then the TPB threads of b (adjacent lanes of one wave) combine theirs
      constexpr int TPB = NT / NB;
      const int b = tid / TPB, c = tid - b * TPB;
      float v = -INFINITY;
      int32_t ix = 0x7fffffff;
      for (int ul = c; ul < pnu; ul += TPB) amax_merge(v, ix, (float)(red[ul * NB + b] * rs[b]), pu0 + ul);
#pragma unroll
      for (int o = TPB / 2; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o, 64);
        const int32_t i2 = __shfl_xor(ix, o, 64);
        amax_merge(v, ix, v2, i2);
      }
      if (c == 0) {
        float rv = m->lmv[b];
        int32_t ri = m->lmi[b];
        amax_merge(rv, ri, v, ix);
        m->lmv[b] = rv;
        m->lmi[b] = ri;
      }
    }
  }
  if (op == OP_LM) {
    __syncthreads();
    if (tid < NB) {
      LmPart* lp = P.lm_part + (size_t)tid * P.n_lm + t.tile;
      stc(&lp->val, m->lmv[tid]);
      stc_i(&lp->idx, m->lmi[tid]);
    }
  }
  if (t.sig_ev != EV_NONE) {
    signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
  } else {  // a split-K part below the last: its tagged sums are complete once stored
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  return true;
}

// The weight buffers are shaped by the tile count of the task's first pass.
template <int NB>
__device__ __forceinline__ bool task_gemv_mfma(const KParams& P, const TaskRec& t, int s, bool mega, char* lds,
                                               uint64_t* tr) {
  const int op = (int)t.op, l = (int)t.layer;
  const LayerW LW = ldk(P.layers + (op == OP_LM ? 0 : l));
  const uint16_t* W0;
  const uint16_t* W1 = nullptr;
  const uint16_t* gamma = nullptr;
  int K, RU = 1;
  switch (op) {
    case OP_QKV: W0 = LW.wqkv; K = P.H; gamma = LW.attn_norm; break;
    case OP_WO: W0 = LW.wo; K = P.QD; break;
    case OP_GU: W0 = LW.wg; W1 = LW.wu; K = P.H; RU = 2; gamma = LW.ffn_norm; break;
    case OP_DOWN: W0 = LW.wd; K = P.F; break;
    default: W0 = P.lm_head; K = P.H; gamma = P.final_norm; break;
  }
  const int T = (((int)t.a1 - (int)t.a0) * RU + 15) >> 4;
  static_assert(MT == 8, "the buffer shapes below cover up to eight tiles per pass");
  if (T <= 1) return gemv_mfma<NB, 1>(P, t, s, mega, lds, tr, op, W0, W1, gamma, K, RU);
  if (T <= 2) return gemv_mfma<NB, 2>(P, t, s, mega, lds, tr, op, W0, W1, gamma, K, RU);
  if (T <= 4) return gemv_mfma<NB, 4>(P, t, s, mega, lds, tr, op, W0, W1, gamma, K, RU);
  return gemv_mfma<NB, 8>(P, t, s, mega, lds, tr, op, W0, W1, gamma, K, RU);
}

// ---------------------------------------------------------------------------
// Attention task (sequence b, KV head g, split sp): QK-norm + RoPE of the G
// query heads (and of k when this split holds the current position, which it
// then appends to the cache), scores over the split's positions, and the
// split's softmax partial: max m, sum l = sum_j e^{t_j - m}, and the
// unnormalised acc = sum_j e^{t_j - m} v_j (FlashDecoding-style split-KV, as
// in the Mirage article's attention search space).  Everything is evaluated
// in fp64; partials are stored as tagged fp64 words.  The merge
//   M = max_s m_s;  den = sum_s e^{m_s - M} l_s;  o = sum_s e^{m_s - M} acc_s / den
// adds the splits in ascending order and rounds o once to fp32.  It is done by
// the split holding the current position, or, past ATT_MCH active splits with
// a worker per attention task, by every active split for a slice of the
// outputs (the forms are described with att_dist).
// ---------------------------------------------------------------------------
// the same coherent 8-byte load through a buffer resource: one 32-bit lane offset
// and a scalar offset, so a burst of such loads holds no 64-bit addresses
__device__ __forceinline__ uint64_t ld_tv_b(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 16 /* sc1 */);
  return ((uint64_t)v.y << 32) | v.x;
}

// NL: K/V 16-byte loads per thread (the split covers at most NL * PPB positions)
// QR: compiled with the reuse of rotated queries (left out where registers are scarce)
template <int G, int LPP, int NL, bool QR>
__device__ __forceinline__ bool task_attn(const KParams& P, const TaskRec& t, int s, bool mega, char* lds,
                                          uint64_t* tr) {
  constexpr int D = LPP * 8, PPB = NT / LPP;
  const int Hkv = P.Hkv, S = P.S;
  const int bg = (int)t.a0, b = bg / Hkv, g = bg - b * Hkv, sp = (int)t.a1, l = (int)t.layer;
  // prefill graph: virtual sequence b is token pos0 + s chunk + b of sequence kv_seq, whose keys and
  // values an append task has already written to the cache; padding tokens only signal
  const bool chunked = P.chunk > 0;
  const int pos = chunked ? P.pos0 + s * P.chunk + b : P.pos0 + s, N = pos + 1;
  if (chunked && pos >= P.pos_end) {
    if (sp == 0) signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
    return true;
  }
  const int n_act = (pos + S) / S;  // splits holding positions 0..pos
  constexpr int MCH = ATT_MCH;  // single merger: accumulator splits in flight per thread
  const bool dist = att_dist(P);
  const bool slice = dist && n_act > MCH;
  if (sp >= n_act) {  // split beyond the current length: nothing to do
    if constexpr (kEventCounter) {  // ... but its add, in step (dist: every attention task signals)
      if (dist) {
        Misc* mm = (Misc*)(lds + P.misc_off);
        if (mega && !wait_event(P, t.wait_ev, P.epoch + (uint32_t)s + 1u, t.tile, mm, tr, false, false)) return false;
        signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
      }
    }
    return true;
  }
  const int tid = ltid(), lane = tid & 63, w = tid >> 6;
  const int j0 = sp * S, j1 = min(j0 + S, N);
  const bool has_cur = (j1 == N);  // this split holds the current position (and merges)
  const bool cur = has_cur && !chunked;  // ... and computes and appends its key and value (decode)
  const int jc = cur ? pos : j1;  // cached positions [j0, jc)
  const int lp = tid % LPP, po = tid / LPP;
  const size_t head = ((size_t)(l * P.kvB + (chunked ? P.kv_seq : b)) * Hkv + g) * P.max_seq;
  uint16_t* Kh = P.kc + head * D;
  uint16_t* Vh = P.vc + head * D;
  const uint32_t tag = (P.epoch + (uint32_t)s) * P.ntag + t.sig_ev + 1u;

  // cached K/V do not depend on this step: load them before waiting (decode; in the prefill
  // graph they were written in this launch by other compute units, and are read after the wait)
  uint4 kr[NL], vr[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int j = j0 + po + i * PPB;
    if (!chunked && po + i * PPB < S && j < jc) {
      kr[i] = ld16(Kh + (size_t)j * D + lp * 8);
      vr[i] = ld16(Vh + (size_t)j * D + lp * 8);
    } else {
      kr[i] = vr[i] = make_uint4(0, 0, 0, 0);
    }
  }

  // Without dist, a worker's attention tasks of a layer are consecutive in its list and share
  // one (sequence, KV head): a split that does not hold the current position reuses the rotated
  // queries that the worker's previous task left in LDS.
  Misc* m = (Misc*)(lds + P.misc_off);
  const uint32_t qk_step = P.epoch + (uint32_t)s + 1u, qk_id = (uint32_t)(l * P.B * Hkv + bg);
  const bool reuse = QR && !dist && !has_cur && m->qk_step == qk_step && m->qk_id == qk_id;

  // so do this thread's RoPE factors (and QK-norm gains): item tid is (head tid / (D/2), pair tid % (D/2))
  constexpr int half = D / 2;
  const int nh = G + (cur ? 1 : 0);  // heads to rotate (q heads, then k)
  const bool rot = !reuse && tid < nh * half;
  const int rh = tid / half, rk = tid - rh * half;
  double rc = 0.0, rsn = 0.0, g0 = 1.0, g1 = 1.0;
  if (rot) {
    rc = ldg(P.rope_cos + (size_t)pos * half + rk);
    rsn = ldg(P.rope_sin + (size_t)pos * half + rk);
    if (P.qk_norm) {
      const LayerW LW = ldk(P.layers + l);
      const uint16_t* gm = rh < G ? LW.q_norm : LW.k_norm;
      g0 = (double)bf1(ldg(gm + rk));
      g1 = (double)bf1(ldg(gm + rk + half));
    }
  }

  // (with dist a worker holds at most one attention task of a layer: nothing to reuse)
  if (mega && !wait_event(P, t.wait_ev, P.epoch + (uint32_t)s + 1u, t.tile, m, tr, false, !dist)) return false;
  if (chunked) {  // device-coherent loads of this launch's appends (two 8-byte halves)
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int j = j0 + po + i * PPB;
      if (po + i * PPB < S && j < jc) {
        const uint64_t* kp = (const uint64_t*)(Kh + (size_t)j * D + lp * 8);
        const uint64_t* vp = (const uint64_t*)(Vh + (size_t)j * D + lp * 8);
        const uint64_t k0 = __hip_atomic_load((const GAS uint64_t*)kp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t k1 = __hip_atomic_load((const GAS uint64_t*)(kp + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t v0 = __hip_atomic_load((const GAS uint64_t*)vp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t v1 = __hip_atomic_load((const GAS uint64_t*)(vp + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        kr[i] = make_uint4((uint32_t)k0, (uint32_t)(k0 >> 32), (uint32_t)k1, (uint32_t)(k1 >> 32));
        vr[i] = make_uint4((uint32_t)v0, (uint32_t)(v0 >> 32), (uint32_t)v1, (uint32_t)(v1 >> 32));
      }
    }
  }

  float* raw = (float*)lds;                    // [(G+2) D]: q heads, k, v as stored (fp32)
  double* qrot = (double*)(raw + (G + 2) * D); // [G D]
  uint16_t* kcur = (uint16_t*)(qrot + G * D);  // [D]
  uint16_t* vcur = kcur + D;                   // [D]
  double* sc = (double*)(vcur + D);            // [G S]
  uint16_t* vsm = (uint16_t*)(sc + G * ((S + 1) & ~1));  // [S D] this split's values (bf16)
  double* accw = (double*)(vsm + S * D);       // P.V partial sums, then the merge's scratch

  const float* src = P.qkv + (size_t)b * P.QKVR + (size_t)g * P.RG;
  if (!reuse)
    for (int i = tid * 4; i < (G + 2) * D; i += NT * 4) *(v4f*)(raw + i) = ldc4(src, (uint32_t)i);
  // the cached values, position-major, for the P.V pass
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int jr = po + i * PPB;
    if (jr < S && j0 + jr < jc) *(uint4*)(vsm + jr * D + lp * 8) = vr[i];
  }
  __syncthreads();
  if (P.qk_norm && !reuse) {
    for (int h = w; h < nh; h += NW) {
      double ss = 0.0;
      for (int d = lane; d < D; d += 64) ss += (double)raw[h * D + d] * (double)raw[h * D + d];
      ss = wave_sum_d(ss);
      if (lane == 0) m->hr[h] = 1.0 / sqrt(ss / (double)D + (double)P.eps);
    }
    __syncthreads();
  }
  if (rot) {
    const int h = rh, k = rk;
    double x0 = raw[h * D + k], x1 = raw[h * D + k + half];
    if (P.qk_norm) {
      x0 = (x0 * m->hr[h]) * g0;
      x1 = (x1 * m->hr[h]) * g1;
    }
    const double y0 = x0 * rc - x1 * rsn, y1 = x0 * rsn + x1 * rc;
    if (h < G) {
      qrot[h * D + k] = y0;
      qrot[h * D + k + half] = y1;
    } else {  // the rotated key is an fp32 value; the cache holds it in bf16
      kcur[k] = f2bf((float)y0);
      kcur[k + half] = f2bf((float)y1);
    }
  }
  if (cur)
    for (int i = tid; i < D; i += NT) vcur[i] = vsm[(pos - j0) * D + i] = f2bf(raw[(G + 1) * D + i]);
  if (QR && tid == 0) {
    m->qk_step = qk_step;
    m->qk_id = qk_id;
  }
  __syncthreads();

  // ---- scores t_j = (q_h . k_j) / sqrt(D); LPP lanes share one position.  Heads go
  // one at a time so that only one head's query slice and sums occupy registers.
  // The current position's key (rotated above) joins the cached ones first.
  const int n = j1 - j0;
  if (cur)
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (j0 + po + i * PPB == pos) kr[i] = *(const uint4*)(kcur + lp * 8);
  // Dot products of every (head, position block) first, then their 16-lane sums
  // side by side, so the reduction chains overlap instead of running head after head.
  double dots[G][NL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    double q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = qrot[h * D + lp * 8 + e];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = fma(q[2 * e], (double)bf_lo(kw[e]), a);
        a = fma(q[2 * e + 1], (double)bf_hi(kw[e]), a);
      }
      dots[h][i] = a;
    }
  }
  group_sum_d_n<LPP, G * NL>(&dots[0][0]);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int jr = po + i * PPB;
      if (jr < n && lp == 0) sc[h * S + jr] = dots[h][i] * P.attn_scale;
    }
  __syncthreads();
  // ---- split softmax statistics per head
  for (int h = w; h < G; h += NW) {
    double mx = -INFINITY;
    for (int jr = lane; jr < n; jr += 64) mx = fmax(mx, sc[h * S + jr]);
    mx = wave_max_d(mx);
    double ls = 0.0;
    for (int jr = lane; jr < n; jr += 64) {
      const double p = exp(sc[h * S + jr] - mx);
      sc[h * S + jr] = p;
      ls += p;
    }
    ls = wave_sum_d(ls);
    if (lane == 0) {
      m->ml[h][0] = mx;
      m->ml[h][1] = ls;
    }
  }
  __syncthreads();
  // ---- unnormalised P.V: thread (q, r) sums e^{t_j - m} v_j[d] for the four outputs
  // d = 4q..4q+3 of the group's G heads (one 8-byte read of the split's values per position)
  // over positions j = r, r + RPV, ... in ascending order; the RPV partial sums of an output
  // are then added in order of r.
  constexpr int GD = G * D, NQ = GD / 4, RPV = NT / NQ;
  static_assert(NQ * RPV == NT, "P.V thread layout");
  double pv = 0.0;
  {
    const int q = tid % NQ, r = tid / NQ;
    const int h = (4 * q) / D, d0 = 4 * q - h * D;
    const double* ph = sc + h * S;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (int j4 = r; j4 < n; j4 += 4 * RPV) {  // 4 positions' LDS reads in flight
      double pp[4];
      uint2 vv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jr = min(j4 + u * RPV, n - 1);
        pp[u] = ph[jr];
        vv[u] = *(const uint2*)(vsm + jr * D + d0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j4 + u * RPV < n) {
          a0 = fma(pp[u], (double)bf_lo(vv[u].x), a0);
          a1 = fma(pp[u], (double)bf_hi(vv[u].x), a1);
          a2 = fma(pp[u], (double)bf_lo(vv[u].y), a2);
          a3 = fma(pp[u], (double)bf_hi(vv[u].y), a3);
        }
    }
    *(v2d*)(accw + r * GD + 4 * q) = v2d{a0, a1};
    *(v2d*)(accw + r * GD + 4 * q + 2) = v2d{a2, a3};
  }
  __syncthreads();
  if (tid < GD)
#pragma unroll
    for (int r = 0; r < RPV; ++r) pv += accw[r * GD + tid];
  // ---- this split's partial, tagged with the step
  const size_t pbase = ((size_t)bg * P.NS + sp) * G;
  if (tid < GD) st_tvd(P.part_acc + (pbase * D + tid) * 2, pv, tag);
  if (tid < G) {
    st_tvd(P.part_ml + ((pbase + tid) * 2) * 2, m->ml[tid][0], tag);
    st_tvd(P.part_ml + ((pbase + tid) * 2 + 1) * 2, m->ml[tid][1], tag);
  }
  if (tr && tid == 0) tr[2] = wall_clock64();  // partial stored
  if (!has_cur && !slice) {  // the merger checks this split's partial by its tags
    if constexpr (kEventCounter) {
      if (dist) {
        signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
        return true;
      }
    }
    __syncthreads();
    return true;
  }
  // ---- merge the splits of (b, g), polling the others' partials:
  //   slice: this split merges outputs [e0, e0 + ne) of the group's G D, item i of its
  //   slice being (split i / ne, output e0 + i % ne), at most MI items per thread in flight;
  //   otherwise: thread tid merges output tid, MCH splits in flight at a time.
  // The (m_s, l_s) words and the first accumulator words are requested together, so the
  // merge costs one round trip; the weights e^{m_s - M} are formed once per (head, split).
  // Either way output e is sum_s e^{m_s - M} acc_s[e] / den, summed in ascending s.
  const size_t b0 = (size_t)bg * P.NS;
  uint32_t polls = 0;
  const uint32_t wdog = P.watchdog;
  bool ok_all = true;
  __syncthreads();                    // every thread is done reading the P.V scratch and m->ml
  double* mls = accw;                 // [G][n_act][2], reuses the P.V scratch
  double* scl = accw + 2 * G * n_act; // [G][n_act] weights e^{m_s - M}
  double* accs = scl + G * n_act;     // slice: [n_act][ne] the slice's accumulators
  constexpr int MI = 2;               // slice: items in flight per thread
  constexpr uint32_t SSTR = G * D * 16;  // bytes between consecutive splits of one accumulator element
  const int npair = G * n_act;
  const int e0 = slice ? sp * GD / n_act : 0, ne = slice ? (sp + 1) * GD / n_act - e0 : GD;
  const int tot = ne * n_act;
  const bool mine = !slice && tid < G * D;  // this thread merges element tid of the group's G heads
  const int h_me = tid / D;
  // byte offsets: accumulator element tid of split s2 at tid * 16 + s2 * SSTR (lo word, then hi);
  // (m, l) of (head h, split s2) at (s2 * G + h) * 32 (m lo, m hi, l lo, l hi)
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(P.part_acc + b0 * G * D * 2), (short)0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc((void*)(P.part_ml + b0 * G * 4), (short)0, 0x7fffffff, 0x00020000);
  const uint32_t va = (uint32_t)tid * 16u;
  auto pair_off = [&](int i) -> uint32_t {
    const int h = i / n_act, s2 = i - h * n_act;
    return (uint32_t)(s2 * G + h) * 32u;
  };
  uint64_t pw[4] = {0, 0, 0, 0};
  if (tid < npair) {
    const uint32_t vo = pair_off(tid);
#pragma unroll
    for (int k = 0; k < 4; ++k) pw[k] = ld_tv_b(rm, vo, 8u * k);
  }
  uint64_t wl[MCH], wh[MCH];
  // slice: byte offset of item i
  auto item_off = [&](int i) -> uint32_t {
    const int s2 = i / ne, el = i - s2 * ne;
    return (uint32_t)s2 * SSTR + (uint32_t)(e0 + el) * 16u;
  };
  if (slice) {
#pragma unroll
    for (int k = 0; k < MI; ++k)
      if (tid + k * NT < tot) {
        const uint32_t vo = item_off(tid + k * NT);
        wl[k] = ld_tv_b(ra, vo, 0u);
        wh[k] = ld_tv_b(ra, vo + 8u, 0u);
      }
  } else {
#pragma unroll
    for (int k = 0; k < MCH; ++k)
      if (mine && k < n_act) {
        wl[k] = ld_tv_b(ra, va, k * SSTR);
        wh[k] = ld_tv_b(ra, va + 8u, k * SSTR);
      }
  }
  for (int i = tid; i < npair; i += NT) {
    const uint32_t vo = pair_off(i);
    if (i != tid)
#pragma unroll
      for (int k = 0; k < 4; ++k) pw[k] = ld_tv_b(rm, vo, 8u * k);
    while (ok_all && !(tv_ok(pw[0], tag) && tv_ok(pw[1], tag) && tv_ok(pw[2], tag) && tv_ok(pw[3], tag))) {
      if (++polls > wdog) ok_all = false;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int k = 0; k < 4; ++k) pw[k] = ld_tv_b(rm, vo, 8u * k);
    }
    mls[i * 2] = tvd_val(pw[0], pw[1]);
    mls[i * 2 + 1] = tvd_val(pw[2], pw[3]);
  }
  // checks the tags of a burst of accumulator words, re-reading those not yet written
  auto settle = [&](int c0) {
#pragma unroll
    for (int k = 0; k < MCH; ++k)
      if (mine && c0 + k < n_act)
        while (ok_all && !(tv_ok(wl[k], tag) && tv_ok(wh[k], tag))) {
          if (++polls > wdog) ok_all = false;
          __builtin_amdgcn_s_sleep(1);
          wl[k] = ld_tv_b(ra, va, (c0 + k) * SSTR);
          wh[k] = ld_tv_b(ra, va + 8u, (c0 + k) * SSTR);
        }
  };
  double av[MCH];  // the first MCH accumulators
  if (slice) {
    // the slice's items in bursts of MI per thread, each checked and parked in LDS
    for (int c0 = 0; c0 < tot; c0 += MI * NT) {
      if (c0 > 0)
#pragma unroll
        for (int k = 0; k < MI; ++k)
          if (c0 + tid + k * NT < tot) {
            const uint32_t vo = item_off(c0 + tid + k * NT);
            wl[k] = ld_tv_b(ra, vo, 0u);
            wh[k] = ld_tv_b(ra, vo + 8u, 0u);
          }
#pragma unroll
      for (int k = 0; k < MI; ++k) {
        const int i = c0 + tid + k * NT;
        if (i < tot) {
          const uint32_t vo = item_off(i);
          while (ok_all && !(tv_ok(wl[k], tag) && tv_ok(wh[k], tag))) {
            if (++polls > wdog) ok_all = false;
            __builtin_amdgcn_s_sleep(1);
            wl[k] = ld_tv_b(ra, vo, 0u);
            wh[k] = ld_tv_b(ra, vo + 8u, 0u);
          }
          accs[i] = tvd_val(wl[k], wh[k]);
        }
      }
    }
  } else {
    settle(0);
#pragma unroll
    for (int k = 0; k < MCH; ++k) av[k] = tvd_val(wl[k], wh[k]);
  }
  __syncthreads();
  // per head h, wave h (lanes over splits): M = max_s m_s, the weights e^{m_s - M}, and
  // den = sum_s e^{m_s - M} l_s (a fixed tree, the same on every lane)
  if (w < G) {
    const int h = w;
    double M = -INFINITY;
    for (int s2 = lane; s2 < n_act; s2 += 64) M = fmax(M, mls[(h * n_act + s2) * 2]);
    M = wave_max_d(M);
    double dsum = 0.0;
    for (int s2 = lane; s2 < n_act; s2 += 64) {
      const double e = exp(mls[(h * n_act + s2) * 2] - M);
      scl[h * n_act + s2] = e;
      dsum += e * mls[(h * n_act + s2) * 2 + 1];
    }
    dsum = wave_sum_d(dsum);
    if (lane == 0) m->ml[h][1] = dsum;
  }
  __syncthreads();
  if (slice && tid < ne) {
    const int e = e0 + tid;
    const double* sw = scl + (e / D) * n_act;
    double num = 0.0;
#pragma unroll 8
    for (int s2 = 0; s2 < n_act; ++s2) num += sw[s2] * accs[s2 * ne + tid];
    if (ok_all) stc(P.o + (size_t)b * P.QD + (size_t)(g * G) * D + e, (float)(num / m->ml[e / D][1]));
  }
  if (mine) {
    const double* sw = scl + h_me * n_act;
    const double den = m->ml[h_me][1];
    double num = 0.0;
#pragma unroll
    for (int k = 0; k < MCH; ++k)
      if (k < n_act) num += sw[k] * av[k];
    for (int c0 = MCH; c0 < n_act && ok_all; c0 += MCH) {
#pragma unroll
      for (int k = 0; k < MCH; ++k)
        if (c0 + k < n_act) {
          wl[k] = ld_tv_b(ra, va, (c0 + k) * SSTR);
          wh[k] = ld_tv_b(ra, va + 8u, (c0 + k) * SSTR);
        }
      settle(c0);
#pragma unroll
      for (int k = 0; k < MCH; ++k)
        if (c0 + k < n_act) num += sw[c0 + k] * tvd_val(wl[k], wh[k]);
    }
    if (ok_all) stc(P.o + (size_t)b * P.QD + (size_t)(g * G) * D + tid, (float)(num / den));
  }
  // Append this position's K/V to the cache.  Only later steps read it, after
  // the signal below; issued here, the stores complete alongside those of o
  // instead of stalling the scores (a store's registers are reusable only
  // once it has completed).
  if (cur && tid < LPP) {
    stg((uint4*)(Kh + (size_t)pos * D + tid * 8), *(const uint4*)(kcur + tid * 8));
    stg((uint4*)(Vh + (size_t)pos * D + tid * 8), *(const uint4*)(vcur + tid * 8));
  }
  if (!ok_all) {
    uint32_t zero = 0u;
    if (__hip_atomic_compare_exchange_strong((GAS uint32_t*)(P.status + ST_CODE), &zero, ERR_WATCHDOG,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
      stc_u(P.status + ST_CU, blockIdx.x);
      stc_u(P.status + ST_TASK, t.tile);
      stc_u(P.status + ST_EVENT, t.sig_ev);
    }
    stc_u(P.status + ST_ABORT, 1u);
    m->att_fail = 1;
  }
  signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
  // the same verdict for every thread (read after the signal's barrier; never cleared within a
  // launch); other workers' aborts are seen at this worker's next wait
  return m->att_fail == 0;
}

template <int G, int LPP, bool QR>
__device__ __forceinline__ bool attn_nl(const KParams& P, const TaskRec& t, int s, bool mega, char* lds, uint64_t* tr) {
  constexpr int PPB = NT / LPP;
  if (P.S <= PPB) return task_attn<G, LPP, 1, QR>(P, t, s, mega, lds, tr);
  if (P.S <= 2 * PPB) return task_attn<G, LPP, 2, QR>(P, t, s, mega, lds, tr);
  if constexpr (G == 1)  // longer splits only where one head's scores are in registers
    if (P.S > ATT_MAXL * PPB) return task_attn<G, LPP, ATT_MAXL1, QR>(P, t, s, mega, lds, tr);
  return task_attn<G, LPP, ATT_MAXL, QR>(P, t, s, mega, lds, tr);
}

#include "gemv_stream.inc"

// The streaming engine (gemv_stream.inc) is switched off: its first GPU run ended in a memory
// fault whose cause is not yet found (a CPU emulation of the same launches finds no out-of-bounds
// access).  Until it is, GEMV tasks run as per-task GEMVs (task_gemv).
constexpr bool kStreamEngine = false;

// Prefill graph: the rotated keys and the values of one KV-head group, for every token of the chunk,
// go to the cache with device-coherent stores (the attention tasks that read them run on other
// compute units of the same launch).  The arithmetic is a decoding attention task's for its current
// position: QK-norm with the same fp64 lane sums and wave tree, RoPE in fp64, the key rounded to
// fp32 and then bf16, the value to bf16.  One wave per token.
__device__ __forceinline__ bool task_append(const KParams& P, const TaskRec& t, int s, bool mega, char* lds,
                                            uint64_t* tr) {
  const int g = (int)t.a0, l = (int)t.layer, D = P.D, half = D / 2, C = P.chunk;
  const int tid = ltid(), lane = tid & 63, w = tid >> 6;
  Misc* m = (Misc*)(lds + P.misc_off);
  if (mega && !wait_event(P, t.wait_ev, P.epoch + (uint32_t)s + 1u, t.tile, m, tr)) return false;
  uint16_t* kst = (uint16_t*)lds;  // [C][D] rotated keys, bf16
  uint16_t* vst = kst + C * D;     // [C][D] values, bf16
  const LayerW LW = ldk(P.layers + l);
  for (int b = w; b < C; b += NW) {
    const int pos = P.pos0 + s * C + b;
    if (pos >= P.pos_end) continue;
    const float* kraw = P.qkv + (size_t)b * P.QKVR + (size_t)g * P.RG + (size_t)P.G * D;
    const float* vraw = kraw + D;
    double hr = 1.0;
    if (P.qk_norm) {
      double ss = 0.0;
      for (int d = lane; d < D; d += 64) {
        const double x = (double)ldc(kraw + d);
        ss += x * x;
      }
      ss = wave_sum_d(ss);
      hr = 1.0 / sqrt(ss / (double)D + (double)P.eps);
    }
    for (int k = lane; k < half; k += 64) {
      double x0 = (double)ldc(kraw + k), x1 = (double)ldc(kraw + k + half);
      if (P.qk_norm) {
        x0 = (x0 * hr) * (double)bf1(ldg(LW.k_norm + k));
        x1 = (x1 * hr) * (double)bf1(ldg(LW.k_norm + k + half));
      }
      const double rc = ldg(P.rope_cos + (size_t)pos * half + k), rsn = ldg(P.rope_sin + (size_t)pos * half + k);
      const double y0 = x0 * rc - x1 * rsn, y1 = x0 * rsn + x1 * rc;
      kst[b * D + k] = f2bf((float)y0);
      kst[b * D + k + half] = f2bf((float)y1);
    }
    for (int d = lane; d < D; d += 64) vst[b * D + d] = f2bf(ldc(vraw + d));
  }
  __syncthreads();
  const size_t head = ((size_t)(l * P.kvB + P.kv_seq) * P.Hkv + g) * P.max_seq;
  for (int i = tid; i < C * D / 2; i += NT) {
    const int b = (2 * i) / D, e = 2 * i - b * D;
    const int pos = P.pos0 + s * C + b;
    if (pos >= P.pos_end) continue;
    stc_u((uint32_t*)(P.kc + (head + pos) * D + e), *(const uint32_t*)(kst + b * D + e));
    stc_u((uint32_t*)(P.vc + (head + pos) * D + e), *(const uint32_t*)(vst + b * D + e));
  }
  signal_event(P, t.sig_ev, t.sig_slot, P.epoch + (uint32_t)s + 1u);
  return true;
}

template <int NB, bool LO>
__device__ __forceinline__ bool run_task(const KParams& P, const TaskRec& t, int s, bool mega, char* lds,
                                         uint64_t* tr = nullptr) {
  if (t.op == OP_APPEND) return task_append(P, t, s, mega, lds, tr);
  if (t.op == OP_ATTN) {
    constexpr bool QR = NB < 8;  // at B >= 8 the matrix-core GEMV leaves no registers for it
    if (P.D == 64) {
      switch (P.G) {
        case 1: return attn_nl<1, 8, QR>(P, t, s, mega, lds, tr);
        case 2: return attn_nl<2, 8, QR>(P, t, s, mega, lds, tr);
        default: return attn_nl<4, 8, QR>(P, t, s, mega, lds, tr);
      }
    }
    switch (P.G) {
      case 1: return attn_nl<1, 16, QR>(P, t, s, mega, lds, tr);
      case 2: return attn_nl<2, 16, QR>(P, t, s, mega, lds, tr);
      default: return attn_nl<4, 16, QR>(P, t, s, mega, lds, tr);
    }
  }
  if constexpr (NB >= 8) return task_gemv_mfma<NB>(P, t, s, mega, lds, tr);
  else if constexpr (NB == 1 && kRpg1 > 1) {
    if (t.op == OP_WO || t.op == OP_GU || t.op == OP_DOWN) return task_gemv<NB, LO, kRpg1>(P, t, s, mega, lds, tr);
    return task_gemv<NB, LO, 1>(P, t, s, mega, lds, tr);
  } else if constexpr (NB < 4) return task_gemv<NB, LO, 1>(P, t, s, mega, lds, tr);
  // four sequences: each staged-activation read serves four rows where a wave's rows come in
  // fours or the pairing wastes as much (down projection, QKV, LM head), two elsewhere (a wave
  // holds two O-projection rows; fourteen gate/up rows would leave two slots of sixteen idle)
  else if (t.op == OP_WO || t.op == OP_GU) return task_gemv<NB, LO, 2>(P, t, s, mega, lds, tr);
  else return task_gemv<NB, LO, 4>(P, t, s, mega, lds, tr);
}

// The megakernel: one launch runs n_steps decode steps of the whole model.
template <int NB, bool LO>
__global__ __launch_bounds__(NT, 1) void mk_persistent(KParams P) {
  char* lds = g_lds;
  const uint32_t off = ldk(P.list_off + blockIdx.x), n = ldk(P.list_len + blockIdx.x);
  if (threadIdx.x == 0) {
    Misc* m = (Misc*)(lds + P.misc_off);
    m->cev = EV_NONE;
    m->att_fail = 0;
    if constexpr (NB < 8) m->qk_step = 0u;  // no rotated queries in LDS yet
  }
  __syncthreads();
  if constexpr (NB <= 4 && kStreamEngine) {
    // attention tasks one by one; every run of GEMV tasks between them as one streaming segment
    const SegList L{P.cu_tasks + off, 0u, n, P.n_steps, 0};
    int s = 0;
    uint32_t i = 0;
    while (s < P.n_steps && n > 0) {
      const TaskRec t = ldk(P.tasks + seg_index(L, i));
      if (t.op == OP_ATTN) {
        uint64_t* tr = (P.trace && s == P.trace_step) ? P.trace + ((size_t)blockIdx.x * P.trace_stride + i) * 4 : nullptr;
        if (tr && threadIdx.x == 0) tr[0] = wall_clock64();
        if (!run_task<NB, LO>(P, t, s, true, lds, tr)) return;
        if (tr && threadIdx.x == 0) tr[3] = wall_clock64();
        seg_step(L, s, i);
      } else if (!run_segment<NB>(P, L, s, i, lds, true)) {
        return;
      }
    }
  } else {
    for (int s = 0; s < P.n_steps; ++s) {
      for (uint32_t i = 0; i < n; ++i) {
        const TaskRec t = ldk(P.tasks + ldk(P.cu_tasks + off + i));
        uint64_t* tr = (P.trace && s == P.trace_step) ? P.trace + ((size_t)blockIdx.x * P.trace_stride + i) * 4 : nullptr;
        if (tr && threadIdx.x == 0) tr[0] = wall_clock64();
        if (!run_task<NB, LO>(P, t, s, true, lds, tr)) return;
        if (tr && threadIdx.x == 0) tr[3] = wall_clock64();
      }
    }
  }
  if (blockIdx.x == 0 && P.chunk == 0) {
    // last step's token: wait for every LM tile of the final step (the prefill graph has none)
    Misc* m = (Misc*)(lds + P.misc_off);
    const uint32_t ev_lm = (uint32_t)(P.L * (P.Hkv + 4));
    if (!wait_event(P, ev_lm, P.epoch + (uint32_t)P.n_steps, 0xffffffffu, m)) return;
    reduce_tokens<NB>(P, m);
    if (threadIdx.x < NB) {
      if (P.out_tokens) stg(P.out_tokens + (size_t)(P.n_steps - 1) * P.B + threadIdx.x, m->tok[threadIdx.x]);
      stg(P.pending + threadIdx.x, m->tok[threadIdx.x]);
    }
  }
}

// Ablation: one launch per operator instance, same tasks on the same workers.
template <int NB, bool LO>
__global__ __launch_bounds__(NT, 1) void mk_per_op(KParams P) {
  char* lds = g_lds;
  if (threadIdx.x == 0) {
    Misc* m = (Misc*)(lds + P.misc_off);
    m->att_fail = 0;
    if constexpr (NB < 8) m->qk_step = 0u;  // no rotated queries in LDS yet
  }
  __syncthreads();
  // a worker's tasks of this operator instance are a contiguous stretch of its list (the lists
  // are in topological order), located by the host: no scan of the operator's other tasks
  const uint32_t w = blockIdx.x, nw = (uint32_t)P.n_workers, r = (uint32_t)P.op_range;
  const uint32_t j1 = ldk(P.range_start + (r + 1u) * nw + w), off = ldk(P.list_off + w);
  for (uint32_t j = ldk(P.range_start + r * nw + w); j < j1; ++j) {
    const int i = (int)ldk(P.cu_tasks + off + j);
    const TaskRec t = ldk(P.tasks + i);
    if constexpr (NB <= 4 && kStreamEngine) {
      if (t.op != OP_ATTN) {  // a segment of one task
        const SegList L{nullptr, (uint32_t)i, 1u, 1, P.step};
        int s = 0;
        uint32_t li = 0;
        (void)run_segment<NB>(P, L, s, li, lds, false);
        continue;
      }
    }
    run_task<NB, LO>(P, t, P.step, false, lds);
  }
}

template <int NB>
__global__ __launch_bounds__(NT, 1) void mk_finish_tokens(KParams P) {
  Misc* m = (Misc*)(g_lds + P.misc_off);
  reduce_tokens<NB>(P, m);
  if (threadIdx.x < NB) {
    if (P.out_tokens) stg(P.out_tokens + (size_t)P.step * P.B + threadIdx.x, m->tok[threadIdx.x]);
    stg(P.pending + threadIdx.x, m->tok[threadIdx.x]);
  }
}

// ---------------------------------------------------------------------------
// host-side launch helpers.  The kernels are instantiated for one batch size
// per translation unit (MK_NB = 1, 2, 4, 8, 16), so that the units compile in
// parallel; the unit built without MK_NB holds the probes and the dispatch.
// ---------------------------------------------------------------------------
static inline size_t worker_lds_bytes(const KParams& P) { return (size_t)P.misc_off + MISC_BYTES; }

#define MK_CAT2(a, b) a##b
#define MK_CAT(a, b) MK_CAT2(a, b)

#ifdef MK_NB
// LoRA kernels exist for batch <= 4 (the library refuses adapters at larger batches)
constexpr bool kLoraBuilt = MK_NB <= 4;

template <int NB, bool LO>
static hipError_t launch_nb(int kind, const KParams& P, hipStream_t st) {
  const size_t sh = worker_lds_bytes(P);
  KParams Q = P;
  if (kind == 0) {
    void* args[] = {&Q};
    return hipLaunchCooperativeKernel((const void*)mk_persistent<NB, LO>, dim3(P.n_workers), dim3(NT), args, sh, st);
  } else if (kind == 1) {
    hipLaunchKernelGGL((mk_per_op<NB, LO>), dim3(P.n_workers), dim3(NT), sh, st, Q);
  } else if (kind == 3) {
    // cooperative: tasks of the launch wait on each other (attention mergers, LoRA adapter rows)
    void* args[] = {&Q};
    return hipLaunchCooperativeKernel((const void*)mk_per_op<NB, LO>, dim3(P.n_workers), dim3(NT), args, sh, st);
  } else {
    hipLaunchKernelGGL(mk_finish_tokens<NB>, dim3(1), dim3(NT), sh, st, Q);
  }
  return hipGetLastError();
}

template <int NB, bool LO>
static hipError_t set_attrs_lo() {
  const int sh = 163840;
  hipError_t e = hipFuncSetAttribute((const void*)mk_persistent<NB, LO>, hipFuncAttributeMaxDynamicSharedMemorySize, sh);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)mk_per_op<NB, LO>, hipFuncAttributeMaxDynamicSharedMemorySize, sh);
}

template <int NB>
static hipError_t set_attrs() {
  const int sh = 163840;
  hipError_t e = set_attrs_lo<NB, false>();
  if (e != hipSuccess) return e;
  if constexpr (kLoraBuilt) {
    e = set_attrs_lo<NB, true>();
    if (e != hipSuccess) return e;
  }
  return hipFuncSetAttribute((const void*)mk_finish_tokens<NB>, hipFuncAttributeMaxDynamicSharedMemorySize, sh);
}

hipError_t MK_CAT(launch_b, MK_NB)(int kind, const KParams& P, hipStream_t st) {
  if constexpr (kLoraBuilt)
    if (P.lora_r > 0) return launch_nb<MK_NB, true>(kind, P, st);
  return launch_nb<MK_NB, false>(kind, P, st);
}
hipError_t MK_CAT(set_attrs_b, MK_NB)() { return set_attrs<MK_NB>(); }
int MK_CAT(coresident_b, MK_NB)(size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)mk_persistent<MK_NB, false>, NT, lds) != hipSuccess)
    return -1;
  if constexpr (kLoraBuilt) {
    int lo = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&lo, (const void*)mk_persistent<MK_NB, true>, NT, lds) != hipSuccess)
      return -1;
    per_cu = std::min(per_cu, lo);
  }
  return per_cu;
}
#else
// ---------------------------------------------------------------------------
// Plain streaming read of a buffer: the achievable HBM read rate with the same
// loads the GEMV tasks use (16-byte non-temporal, one contiguous block per
// workgroup), and a kernel of known traffic for calibrating byte counters.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void mk_read_probe(const uint16_t* __restrict__ p, size_t per_wg16, uint32_t* out) {
  const uint16_t* q = p + (size_t)blockIdx.x * per_wg16 * 8;
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i < per_wg16; i += (size_t)NT * 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t j = i + (size_t)u * NT;
      v[u] = j < per_wg16 ? ldw(q + j * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads; never true for the zero-filled buffer
}

// Copy of one half of a buffer into the other (known read and write volume).
__global__ __launch_bounds__(NT) void mk_copy_probe(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t per_wg16) {
  const uint4* q = src + (size_t)blockIdx.x * per_wg16;
  uint4* o = dst + (size_t)blockIdx.x * per_wg16;
  for (size_t i = threadIdx.x; i < per_wg16; i += (size_t)NT * 4) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t j = i + (size_t)u * NT;
      v[u] = j < per_wg16 ? ldw((const uint16_t*)(q + j)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t j = i + (size_t)u * NT;
      if (j < per_wg16) stg(o + j, v[u]);
    }
  }
}

hipError_t launch_copy_probe(void* buf, size_t bytes, int n_wg, hipStream_t st) {
  const size_t half16 = bytes / 32;
  const size_t per_wg16 = half16 / (size_t)n_wg;
  hipLaunchKernelGGL(mk_copy_probe, dim3(n_wg), dim3(NT), 0, st, (const uint4*)buf, (uint4*)buf + half16, per_wg16);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, size_t bytes, int n_wg, uint32_t* out, hipStream_t st) {
  const size_t per_wg16 = bytes / 16 / (size_t)n_wg;
  hipLaunchKernelGGL(mk_read_probe, dim3(n_wg), dim3(NT), 0, st, (const uint16_t*)buf, per_wg16, out);
  return hipGetLastError();
}

size_t lds_bytes(const KParams& P) { return worker_lds_bytes(P); }

// Token staging of mk_prefill_noalloc: a static device array (every context on a device shares
// it; calls that overlap on one device race for it).  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, resolved once per device with that
// device current, and only that address is ever handed to kernels or copies.
constexpr int kNoAllocTokens = 1 << 16;
static __device__ __align__(256) int32_t scratch[kNoAllocTokens];
static int32_t* g_scratch_ptr[64];
static bool g_scratch_ok[64];
static std::mutex g_scratch_mu;

hipError_t noalloc_token_staging(int device, int32_t** ptr) {
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ok[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = (int32_t*)p;
    g_scratch_ok[device] = true;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

#define MK_DECL(nb)                                                         \
  hipError_t launch_b##nb(int kind, const KParams& P, hipStream_t st); \
  hipError_t set_attrs_b##nb();                                        \
  int coresident_b##nb(size_t lds);
MK_DECL(1)
MK_DECL(2)
MK_DECL(4)
MK_DECL(8)
MK_DECL(16)

hipError_t prepare_kernels(int B) {
  switch (B) {
    case 1: return set_attrs_b1();
    case 2: return set_attrs_b2();
    case 4: return set_attrs_b4();
    case 8: return set_attrs_b8();
    default: return set_attrs_b16();
  }
}

// kind: 0 persistent (cooperative), 1 one operator instance, 2 final token, 3 attention operator instance
hipError_t launch(int kind, const KParams& P, hipStream_t st) {
  switch (P.B) {
    case 1: return launch_b1(kind, P, st);
    case 2: return launch_b2(kind, P, st);
    case 4: return launch_b4(kind, P, st);
    case 8: return launch_b8(kind, P, st);
    default: return launch_b16(kind, P, st);
  }
}

int max_coresident_workers(int B, size_t lds) {
  switch (B) {
    case 1: return coresident_b1(lds);
    case 2: return coresident_b2(lds);
    case 4: return coresident_b4(lds);
    case 8: return coresident_b8(lds);
    default: return coresident_b16(lds);
  }
}
#endif

}  // namespace mk
