// Device helpers shared by the forward and backward kernels (gfx950):
// MFMA and 16-bit packing wrappers, LDS swizzles, the HBM->LDS copy, wave
// reductions, launch-order maps and barriers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace fa {


enum Kind : int { KF16 = 0, KBF16 = 1, KFP8 = 2 };
enum OutKind : int { OF16 = 0, OBF16 = 1, OF32 = 3 };

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_tr __attribute__((vector_size(8)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

template <typename T>
__device__ __forceinline__ T bitcast(const u32x4& x) {
  T r;
  __builtin_memcpy(&r, &x, sizeof(T));
  return r;
}

template <int KIND>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (KIND == KBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8>(a), bitcast<half8>(b), c, 0, 0, 0);
  }
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed 16-bit, round to nearest even (v_cvt_pk_{f16,bf16}_f32).
template <int KIND>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  uint32_t u;
  if constexpr (KIND == KBF16) {
    const bf16x2_t v = {(__bf16)x, (__bf16)y};
    __builtin_memcpy(&u, &v, 4);
  } else {
    const half2_t v = {(_Float16)x, (_Float16)y};
    __builtin_memcpy(&u, &v, 4);
  }
  return u;
}

// acc + a.lo + a.hi for a packed pair of 16-bit values (v_dot2c_f32_*).
template <int KIND>
__device__ __forceinline__ float add_pair(uint32_t a, float acc) {
  if constexpr (KIND == KBF16) {
    bf16x2_t x, one = {(__bf16)1.0f, (__bf16)1.0f};
    __builtin_memcpy(&x, &a, 4);
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
  } else {
    half2_t x, one = {(_Float16)1.0f, (_Float16)1.0f};
    __builtin_memcpy(&x, &a, 4);
    return __builtin_amdgcn_fdot2(x, one, acc, false);
  }
}

template <int KIND>
__device__ __forceinline__ float unpack_lo(uint32_t x) {
  uint16_t u = (uint16_t)(x & 0xffffu);
  if constexpr (KIND == KBF16) {
    return __uint_as_float((uint32_t)u << 16);
  } else {
    _Float16 h;
    __builtin_memcpy(&h, &u, 2);
    return (float)h;
  }
}

template <int KIND>
__device__ __forceinline__ float unpack_hi(uint32_t x) {
  uint16_t u = (uint16_t)(x >> 16);
  if constexpr (KIND == KBF16) {
    return __uint_as_float((uint32_t)u << 16);
  } else {
    _Float16 h;
    __builtin_memcpy(&h, &u, 2);
    return (float)h;
  }
}

// XOR swizzles of the 16-byte chunks of one LDS row (row r, chunk c is
// stored at chunk c ^ swz(r)). They depend on the row pitch in bytes (RB:
// 256 for 16-bit data at D=128, 128 for 16-bit at D=64 or fp8 at D=128, 64
// for fp8 at D=64), because the pitch decides which rows share LDS banks.
// The K swizzle spreads the 16 rows that one ds_read_b128 phase touches over
// all 64 banks. The V swizzle for 16-bit data spreads the four rows that one
// transposing read (ds_read_b64_tr_b16) touches over four different 64-byte
// bank groups. A half-wave of fp8 V reads (ds_read_b64_tr_b8) touches eight
// rows, {0,1,2,3,8,9,10,11} + 4*hl, two 16-byte chunks each: at a 128-byte
// pitch the even rows share one 128-byte half of the banks and the odd rows
// the other, so the swizzle gives the four even (odd) rows four different
// chunk pairs (the K pattern would pair them up, a two-way conflict on every
// V read); at a 64-byte pitch the K pattern already separates them. Every
// swizzle depends on the row index mod 16 only.
template <int RB>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (RB == 256) return r & 15;
  else if constexpr (RB == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}
template <int RB, bool TR8>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (TR8 && RB == 128) return (((r >> 1) & 1) | ((r >> 2) & 2)) << 1;
  else if constexpr (TR8) return swz_k<RB>(r);
  else if constexpr (RB == 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r >> 1) & 1) << 2;
}

// 16 bytes per lane from base + voff (HBM) to LDS at lds_wave + 16 * lane
// (global_load_lds_dwordx4). One asm statement sets M0 (the LDS destination,
// wave-uniform), waits the one wait state the hardware needs between an M0
// write and an LDS-DMA load, and issues the load; M0 is declared clobbered,
// so the compiler restores it only if it needs it (it does not here: no
// restore instructions, 80 scalar moves fewer per unrolled loop of the
// headline kernel than a save/restore around each load, 0.3-2.6 % faster,
// same results). Being asm, the load is not seen as a producer of later
// LDS reads: the kernels wait for these loads explicitly (s_waitcnt vmcnt)
// and order them against LDS readers with barriers.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_wave) {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_wave)
      : "memory", "m0");
  __builtin_amdgcn_sched_barrier(0);
}

// max of two floats that are never NaN (scores, -inf, running maxima), as
// one v_max_f32: fmaxf would first quiet possible signalling NaNs of
// operands the compiler cannot see the origin of (a lane exchange, a loop
// variable), one extra instruction per operand on every tile
__device__ __forceinline__ float max_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // After the swap each lane holds its own value and its partner's (l ^ 32).
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_f32(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Map the launch-order workgroup id to a logical tile so that each XCD
// (workgroups are dealt round-robin over the 8 XCDs) receives a contiguous
// range of tiles: the query blocks of one head then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int xcd = w & 7, local = w >> 3;
  const int base = n >> 3, rem = n & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + local;
}
// The same with the launch order cut into groups of `unit` adjacent blocks
// (the blocks of one head, or of the heads sharing one key/value head) dealt
// round-robin to the XCDs: XCD x runs groups x, x+8, ... (needs n/unit to be
// a multiple of 8). Used when the groups differ in work (variable lengths):
// every XCD then gets a share of every sequence.
__device__ __forceinline__ int xcd_deal(int w, int unit) {
  const int xcd = w & 7, local = w >> 3;
  const int g = local / unit;
  return (xcd + 8 * g) * unit + (local - g * unit);
}

// Launch order for grids whose blocks differ in work (causal masks). The
// grid holds total = U * nblk blocks: U units (heads) in groups of G that
// read the same K/V, nblk blocks per unit, rank 0 being a unit's block with
// the most work. Whole groups are dealt round-robin to the 8 XCDs (a
// group's K/V stays in one L2) and each XCD runs its blocks by rank across
// all of its units, not unit by unit: the most work first, so that a slot
// freed late takes a short block; with snake (the whole grid resident at
// once) the higher-work half in falling order and then the rest in rising
// order, so that launch positions i and i + half, which share a CU, add up
// to about the same work. The last rem groups (the group count modulo 8)
// go first, most work first, spread over the XCDs; the others follow as
// above with the XCDs rotated by a fixed amount.
__device__ __forceinline__ void xcd_lpt(int w, int total, int nblk, int G, int rem, bool snake,
                                        int& unit, int& rank) {
  const int U = total / nblk;
  const int urem = rem * G;
  const int nrem = urem * nblk;
  if (w < nrem) {
    rank = w / urem;
    unit = U - urem + (w - rank * urem);
    return;
  }
  w -= nrem;
  const int xcd = w & 7, loc = w >> 3;
  const int ux = (U - urem) / 8;                  // units per XCD
  const int half = snake ? (nblk / 2) * ux : total;
  const int i = loc < half ? loc : loc - half;
  rank = loc < half ? i / ux : nblk - 1 - i / ux;
  const int r = i - (i / ux) * ux;
  unit = ((r / G) * 8 + xcd) * G + r % G;
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// (lgkmcnt) but not for its HBM->LDS loads, which are waited for explicitly
// (wait_loads) before the tile that reads them. The scheduling fences keep
// the compiler from moving instructions across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Wait until at most N of this wave's HBM->LDS loads are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
  return *(const __attribute__((address_space(3))) T*)(uintptr_t)addr;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011): ten rounds, each taking the two 128-bit
// products of counter words 0 and 2 with the round multipliers and mixing
// their halves with words 1 and 3 and the key; the key advances by the two
// Weyl constants between rounds. c is the counter on entry, the output on
// return.
// The 128-bit product m * c as (lo, hi) from four 32 x 32 + 64 -> 64-bit
// multiply-adds (v_mad_u64_u32): with m = mh:ml and c = ch:cl,
// t = cl*mh + hi(cl*ml) and t2 = ch*ml + lo(t) cannot overflow, lo =
// lo(cl*ml) + 2^32 lo(t2) and hi = ch*mh + hi(t) + hi(t2).
__device__ __forceinline__ void mul64wide(uint64_t m, uint64_t c, uint64_t& lo, uint64_t& hi) {
  const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
  const uint32_t cl = (uint32_t)c, ch = (uint32_t)(c >> 32);
  const uint64_t p0 = (uint64_t)cl * ml;
  const uint64_t t = (uint64_t)cl * mh + (p0 >> 32);
  const uint64_t t2 = (uint64_t)ch * ml + (uint32_t)t;
  lo = (uint32_t)p0 | (t2 << 32);
  hi = (uint64_t)ch * mh + ((t >> 32) + (t2 >> 32));
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t lo0, hi0, lo1, hi1;
    mul64wide(M0, c[0], lo0, hi0);
    mul64wide(M1, c[2], lo1, hi1);
    c[0] = hi1 ^ c[1] ^ k0;
    c[1] = lo1;
    c[2] = hi0 ^ c[3] ^ k1;
    c[3] = lo0;
  }
}

}  // namespace fa
