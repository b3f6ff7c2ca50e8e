// device_common.h -- small gfx950 device helpers shared by the route and
// align kernels: bf16 rounding and ordered keys, wave64 reductions and scans
// on DPP lane moves, and the release/acquire ticket hand-off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mr {

constexpr int kWave = 64;

// ------------------------------------------------------------- bf16 keys --

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs; an
// overflow carries into the exponent and becomes infinity).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Monotone 16-bit code of a bf16 value: a larger value gets a larger code,
// and -0 gets the code of +0 so the two compare equal.
__device__ __forceinline__ uint32_t bf16_order(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ uint32_t bf16_from_order(uint32_t o) {
  return (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu);
}

// 32-bit selection key of expert e with fp32 logit z: the order code of
// bf16(z) in the high half and 0xFFFF - e in the low half.  Unsigned max
// picks the larger rounded logit and, among equal ones, the lower id (the
// tie rule of the one-launch router page, Modifications).  Every real key
// is >= 0x007F0000, so 0 marks an empty slot.
__device__ __forceinline__ uint32_t make_key(float z, uint32_t e) {
  return (bf16_order(f32_to_bf16_rne(z)) << 16) | (0xFFFFu - e);
}

__device__ __forceinline__ uint32_t key_id(uint32_t key) { return 0xFFFFu - (key & 0xFFFFu); }

__device__ __forceinline__ float key_value(uint32_t key) {
  return bf16_to_f32(bf16_from_order(key >> 16));
}

// ------------------------------------------------------ wave64 collectives --

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // Lanes whose source is outside the row read 0 (the `old` operand).
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within 16
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kQuadRev = 0x1B;        // quad_perm [3,2,1,0]
constexpr int kRowRor8 = 0x128;       // lane i <- lane (i + 8) mod 16 within 16: i ^ 8

// Max over the 64 lanes, left in every lane (no scalar round trip): DPP
// within rows of 16, then gfx950's permlane16/permlane32 swaps pair each lane
// with lane^16 and lane^32.  Every lane must be active.
__device__ __forceinline__ uint32_t wave_max_all_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  v = max(v, dpp_u32<kRowHalfMirror>(v));
  v = max(v, dpp_u32<kRowMirror>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}

// Max over each half of the wave (lanes 0..31 and 32..63), left in every
// lane of that half: DPP within rows of 16, then the permlane16 swap pairs
// rows 0 and 1, and rows 2 and 3.  Every lane must be active.
__device__ __forceinline__ uint32_t half_max_all_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  v = max(v, dpp_u32<kRowHalfMirror>(v));
  v = max(v, dpp_u32<kRowMirror>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(a[0], a[1]);
}

// Value held by lane (lane ^ J), for J = 1, 2, 4, 8 (DPP inside a row of 16;
// J = 4 is the half-row mirror 7 - i = i ^ 7 followed by a quad reversal,
// i ^ 3) and J = 16, 32 (gfx950's permlane16 / permlane32 swaps, which hand
// each lane both its own row and the partner row).  Every lane active.
template <int J>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int lane) {
  if constexpr (J == 1) {
    return dpp_u32<kQuadXor1>(v);
  } else if constexpr (J == 2) {
    return dpp_u32<kQuadXor2>(v);
  } else if constexpr (J == 4) {
    return dpp_u32<kQuadRev>(dpp_u32<kRowHalfMirror>(v));
  } else if constexpr (J == 8) {
    return dpp_u32<kRowRor8>(v);
  } else if constexpr (J == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? a[0] : a[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? a[0] : a[1];
  }
}

// Sorts N (a power of two) keys held in registers into descending order
// with a bitonic network (all indices compile-time: no register indexing).
template <int N>
__device__ __forceinline__ void sort_desc_u32(uint32_t (&a)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t x = a[i], y = a[l];
          if ((i & k) == 0) {
            a[i] = max(x, y);
            a[l] = min(x, y);
          } else {
            a[i] = min(x, y);
            a[l] = max(x, y);
          }
        }
      }
}

// The k largest of the wave's keys (each lane's N keys sorted descending,
// every key unique or zero): round j takes the wave-wide maximum of the
// lanes' heads, lane j keeps it, and the lane that held it drops its head.
// Returns lane j's key for j < k (0 elsewhere).  Every lane must be active.
// Modifies a[].
template <int N>
__device__ __forceinline__ uint32_t topk_full_u32(uint32_t (&a)[N], int k, int lane) {
  uint32_t mine = 0u;
  for (int j = 0; j < k; ++j) {
    const uint32_t top = wave_max_all_u32(a[0]);
    mine = (lane == j) ? top : mine;
    // keep = all ones except in the lane whose head was taken; there the
    // list shifts up by one (a sorted list never grows along the shift, so
    // the minimum picks the shifted value exactly where keep is 0)
    const uint32_t keep = (uint32_t)(a[0] != top) * 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i + 1 < N; ++i) a[i] = min(a[i], a[i + 1] | keep);
    a[N - 1] &= keep;
  }
  return mine;
}

// Keys per lane that the fast selection rounds shift.
constexpr int kHotKeys = 4;

// Same result as topk_full_u32 (a[] is left as it was): the rounds shift
// only the first kHotKeys keys of each list, since one lane rarely holds
// more than a few of the k largest.  If some lane gave up all of them, its
// later keys were never offered, and the rounds are redone on the full
// lists.
template <int N>
__device__ __forceinline__ uint32_t topk_sorted_u32(uint32_t (&a)[N], int k, int lane) {
  if constexpr (N <= kHotKeys) {
    uint32_t f[N];
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = a[i];
    return topk_full_u32(f, k, lane);
  } else {
    uint32_t h[kHotKeys];
#pragma unroll
    for (int i = 0; i < kHotKeys; ++i) h[i] = a[i];
    uint32_t mine = 0u, pops = 0u;
    for (int j = 0; j < k; ++j) {
      const uint32_t top = wave_max_all_u32(h[0]);
      mine = (lane == j) ? top : mine;
      const bool taken = h[0] == top;
      pops += taken ? 1u : 0u;
      const uint32_t keep = taken ? 0u : 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i + 1 < kHotKeys; ++i) h[i] = min(h[i], h[i + 1] | keep);
      h[kHotKeys - 1] &= keep;
    }
    if (__builtin_amdgcn_ballot_w64(pops >= (uint32_t)kHotKeys) == 0) return mine;
    uint32_t f[N];
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = a[i];
    return topk_full_u32(f, k, lane);
  }
}

// topk_sorted_u32 for two independent lists at once: the two dependency
// chains interleave, so two selections take little longer than one.
template <int N>
__device__ __forceinline__ void topk_sorted2_u32(uint32_t (&a)[N], uint32_t (&b)[N], int k, int lane,
                                                 uint32_t &mine_a, uint32_t &mine_b) {
  constexpr int H = N < kHotKeys ? N : kHotKeys;
  uint32_t ha[H], hb[H];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    ha[i] = a[i];
    hb[i] = b[i];
  }
  mine_a = 0u;
  mine_b = 0u;
  uint32_t pa = 0u, pb = 0u;
  for (int j = 0; j < k; ++j) {
    const uint32_t ta = wave_max_all_u32(ha[0]);
    const uint32_t tb = wave_max_all_u32(hb[0]);
    mine_a = (lane == j) ? ta : mine_a;
    mine_b = (lane == j) ? tb : mine_b;
    const bool xa = ha[0] == ta, xb = hb[0] == tb;
    pa += xa ? 1u : 0u;
    pb += xb ? 1u : 0u;
    const uint32_t keep_a = xa ? 0u : 0xFFFFFFFFu;
    const uint32_t keep_b = xb ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i + 1 < H; ++i) {
      ha[i] = min(ha[i], ha[i + 1] | keep_a);
      hb[i] = min(hb[i], hb[i + 1] | keep_b);
    }
    ha[H - 1] &= keep_a;
    hb[H - 1] &= keep_b;
  }
  if constexpr (N > kHotKeys) {
    if (__builtin_amdgcn_ballot_w64(pa >= (uint32_t)kHotKeys) != 0) {
      uint32_t f[N];
#pragma unroll
      for (int i = 0; i < N; ++i) f[i] = a[i];
      mine_a = topk_full_u32(f, k, lane);
    }
    if (__builtin_amdgcn_ballot_w64(pb >= (uint32_t)kHotKeys) != 0) {
      uint32_t f[N];
#pragma unroll
      for (int i = 0; i < N; ++i) f[i] = b[i];
      mine_b = topk_full_u32(f, k, lane);
    }
  }
}

// Sum over the 64 lanes (fixed butterfly order, so deterministic); every
// lane must be active.  Returns a wave-uniform value.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kQuadXor1>(v);
  v += dpp_f32<kQuadXor2>(v);
  v += dpp_f32<kRowHalfMirror>(v);
  v += dpp_f32<kRowMirror>(v);
  float a = readlane_f32(v, 0), b = readlane_f32(v, 16);
  float c = readlane_f32(v, 32), d = readlane_f32(v, 48);
  return (a + b) + (c + d);
}

// Inclusive prefix sum over the 64 lanes; every lane must be active.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
  v += dpp_u32<kRowShr1>(v);
  v += dpp_u32<kRowShr2>(v);
  v += dpp_u32<kRowShr4>(v);
  v += dpp_u32<kRowShr8>(v);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  v += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT/64 waves); `tmp` is
// LDS scratch of NT/64 + 1 words.  Returns the exclusive prefix for this
// thread and writes the block total to *total.  Contains barriers: every
// thread of the block must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t *tmp, uint32_t *total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_incl_scan_u32(v, lane);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = tmp[w];
    base += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// ------------------------------------------------------- grid hand-off ---
//
// Blocks of one launch exchange data through agent-coherent accesses: a
// relaxed agent-scope atomic store is a write-through store (sc1) that is
// complete once the issuing wave's store counter drains, and a relaxed
// agent-scope atomic load (sc1) reads the coherent copy, never a stale line
// in another XCD's L2.  Every hand-off therefore goes: data stores (st_agent)
// -> each wave waits for its own stores -> barrier -> one relaxed atomic per
// block -> the receiving block's loads (ld_agent).  No L2 write-back or
// invalidate is needed, so hundreds of blocks can take tickets without
// serialising on cache maintenance.

__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Batched coherent loads.  Each reads like a relaxed agent-scope atomic load
// (sc1: fetched past this XCD's L2, so never a stale copy of data another XCD
// wrote through), but the eight loads of a batch are all issued before one
// wait; the compiler waits for every atomic load before issuing the next.
// The loads and the wait sit in one asm statement, so no result register is
// read or copied before its data has arrived.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_coh;
__device__ __forceinline__ void ld_coherent8(uint32_t (&v)[8], const uint32_t *const (&a)[8]) {
  asm volatile(
      "global_load_dword %0, %8, off sc1\n\t"
      "global_load_dword %1, %9, off sc1\n\t"
      "global_load_dword %2, %10, off sc1\n\t"
      "global_load_dword %3, %11, off sc1\n\t"
      "global_load_dword %4, %12, off sc1\n\t"
      "global_load_dword %5, %13, off sc1\n\t"
      "global_load_dword %6, %14, off sc1\n\t"
      "global_load_dword %7, %15, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
// Sixteen 16-byte coherent loads, one wait (see ld_coherent8).
__device__ __forceinline__ void ld_coherent16(u32x4_coh (&v)[16], const u32x4_coh *const (&a)[16]) {
  asm volatile(
      "global_load_dwordx4 %0, %16, off sc1\n\t"
      "global_load_dwordx4 %1, %17, off sc1\n\t"
      "global_load_dwordx4 %2, %18, off sc1\n\t"
      "global_load_dwordx4 %3, %19, off sc1\n\t"
      "global_load_dwordx4 %4, %20, off sc1\n\t"
      "global_load_dwordx4 %5, %21, off sc1\n\t"
      "global_load_dwordx4 %6, %22, off sc1\n\t"
      "global_load_dwordx4 %7, %23, off sc1\n\t"
      "global_load_dwordx4 %8, %24, off sc1\n\t"
      "global_load_dwordx4 %9, %25, off sc1\n\t"
      "global_load_dwordx4 %10, %26, off sc1\n\t"
      "global_load_dwordx4 %11, %27, off sc1\n\t"
      "global_load_dwordx4 %12, %28, off sc1\n\t"
      "global_load_dwordx4 %13, %29, off sc1\n\t"
      "global_load_dwordx4 %14, %30, off sc1\n\t"
      "global_load_dwordx4 %15, %31, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
      : "memory");
}

// N (1, 2, 4 or 8) 16-byte coherent loads, one wait (see ld_coherent8).
template <int N>
__device__ __forceinline__ void ld_coherent_x4(u32x4_coh (&v)[N], const u32x4_coh *const (&a)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "1, 2, 4 or 8 loads");
  if constexpr (N == 1) {
    asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=&v"(v[0]) : "v"(a[0]) : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "global_load_dwordx4 %0, %2, off sc1\n\t"
        "global_load_dwordx4 %1, %3, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "global_load_dwordx4 %0, %4, off sc1\n\t"
        "global_load_dwordx4 %1, %5, off sc1\n\t"
        "global_load_dwordx4 %2, %6, off sc1\n\t"
        "global_load_dwordx4 %3, %7, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  } else {
    asm volatile(
        "global_load_dwordx4 %0, %8, off sc1\n\t"
        "global_load_dwordx4 %1, %9, off sc1\n\t"
        "global_load_dwordx4 %2, %10, off sc1\n\t"
        "global_load_dwordx4 %3, %11, off sc1\n\t"
        "global_load_dwordx4 %4, %12, off sc1\n\t"
        "global_load_dwordx4 %5, %13, off sc1\n\t"
        "global_load_dwordx4 %6, %14, off sc1\n\t"
        "global_load_dwordx4 %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
  }
}

// Waits until every global store and atomic this wave issued has completed
// (s_waitcnt with all counters at zero).
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Every thread of a block calls this after its st_agent writes.  Returns true
// in every thread of the block that took the last of `count` tickets; that
// block may then ld_agent everything the other blocks wrote before their
// tickets.  Contains barriers: every thread of the block must call it.
__device__ __forceinline__ bool last_block_ticket(uint32_t *ticket, uint32_t count, uint32_t *lds_flag) {
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (t == count - 1) ? 1u : 0u;
  }
  __syncthreads();
  return *lds_flag != 0u;
}

__device__ __forceinline__ void reset_counter(uint32_t *c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded waits: iterations of s_sleep(2) (about 128 cycles each).
constexpr int kStartSpin = 8192;        // ~0.5 ms
constexpr int kPublishSpin = 1 << 22;   // ~0.2 s

// Lets a block that has finished its own part help with the work the
// winning block publishes.  It may wait only once every one of the `nblocks`
// blocks of the grid has begun: the blocks it waits for are then all
// resident and never wait themselves, so the wait ends.  If not every block
// has begun within kStartSpin polls, or the publication does not come
// within kPublishSpin polls, the block does not help (the winner does all
// the work).  Returns true, with acquire semantics for every thread, if the
// block may help.  Contains barriers: every thread must call it.
__device__ __forceinline__ bool join_after_publish(const uint32_t *started, uint32_t nblocks,
                                                   const uint32_t *published, uint32_t *lds_flag) {
  if (threadIdx.x == 0) {
    uint32_t ok = 0;
    for (int it = 0; it < kStartSpin; ++it) {
      if (__hip_atomic_load(started, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= nblocks) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ok) {
      ok = 0;
      for (int it = 0; it < kPublishSpin; ++it) {
        if (__hip_atomic_load(published, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          ok = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    *lds_flag = ok;
  }
  __syncthreads();
  return *lds_flag != 0u;
}

// Winner side of join_after_publish: after its st_agent writes, every wave
// waits for its stores, then thread 0 raises the flag.  Every thread of the
// block must call it.
__device__ __forceinline__ void publish(uint32_t *published) {
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(published, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Next item of a shared work queue (block-uniform).  Contains barriers.
__device__ __forceinline__ uint32_t next_work_item(uint32_t *queue, uint32_t *lds_slot) {
  __syncthreads();
  if (threadIdx.x == 0)
    *lds_slot = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *lds_slot;
}

// Counts block exits; the last block to leave returns true (and then owns
// every counter of the launch, which nobody else touches any more).  The
// counters are only ever accessed with agent-scope atomics; each wave waits
// for its own outstanding atomics before the exit ticket, so every earlier
// counter update of every block has been performed when the last block sees
// its ticket.
__device__ __forceinline__ bool last_to_exit(uint32_t *exited, uint32_t nblocks, uint32_t *lds_flag) {
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(exited, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (t == nblocks - 1) ? 1u : 0u;
  }
  __syncthreads();
  return *lds_flag != 0u;
}

// ---------------------------------------------------------- bf16 dot ----

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// 16-byte streaming load (non-temporal hint: data read once per launch).
__device__ __forceinline__ uint4 ld_stream_16(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// acc + sum_{j<8} a_j * b_j for two 16-byte vectors of 8 bf16 each (fp32
// accumulation through v_dot2_f32_bf16; bf16 x bf16 products are exact).
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
  return acc;
}

}  // namespace mr
