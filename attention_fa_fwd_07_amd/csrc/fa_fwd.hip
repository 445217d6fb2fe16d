// FlashAttention forward for MI355X (gfx950, CDNA4), HIP.
//
// One workgroup computes a block of BM = 128 query rows of one (batch, head)
// and streams the keys and values through LDS in tiles of BN rows: the
// FlashAttention-2 order, with the outer loop over query blocks and an
// online softmax that keeps the running row maximum and row sum, so that the
// score matrix S and the probabilities P never leave registers
// ("ops-transformer FlashAttention on Ascend: build, run and tune",
// ai6s.net/6a31724f..., section 1.2). The per-tile pipeline is the one the
// runtime trace on "Tracing npu_flash_attention through the CANN runtime"
// (ai6s.net/6a114bb2..., layer 5) shows: the loads of the next K/V tile
// overlap the matrix products and the softmax of the current one.
//
// gfx950 mapping:
//  * 4 waves of 64 lanes; wave w owns query rows [32w, 32w+32) of the block.
//  * Both products run on MFMA v_mfma_f32_32x32x16_{f16,bf16}, computed
//    transposed: S^T = K Q^T and O^T = V^T P^T. In the 32x32 accumulator
//    layout a lane then owns one query column and 16 key (or head-dim) rows,
//    so the row max and row sum of the softmax are in-lane reductions plus
//    one exchange between the two 32-lane halves (v_permlane32_swap), and the
//    rescale of O by exp(m_old - m_new) is one multiply per register.
//  * The S^T accumulator is converted to the P^T operand of the second
//    product in registers (no LDS round trip), with the key order inside a
//    16-key step chosen to match the accumulator layout.
//  * K and V tiles go from HBM straight into LDS (global_load_lds, 16 bytes
//    per lane), double buffered, in an XOR-swizzled layout chosen per head
//    dim; K is read with ds_read_b128, V with the transposing
//    ds_read_b64_tr_b16, which delivers V^T fragments directly.
//  * Tail guards: rows past Sq or Sk are clamped to the last valid row, so
//    every load reads mapped memory holding finite values; keys past Sk and
//    keys above the causal diagonal are set to -inf before the softmax, and
//    the softmax subtracts a guarded maximum so that (-inf) - (-inf) never
//    occurs. Padding query columns are computed and never stored. This
//    follows the tail-guard and 0 x NaN lessons of "Hygon FlashAttention:
//    fixed-defect review" (chatdocs.ruinique.com/hygon/flash-attention-
//    fixed-bugs, items 2 and 3); all offsets are 64-bit (item 1); the build
//    keeps IEEE infinities (-fno-finite-math-only, item 8).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <float.h>

#include "fa_mi355x.h"

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

struct Params {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  const float* descale_q;
  const float* descale_k;
  const float* descale_v;
  int64_t Sq;
  int64_t Sk;
  int32_t nqb;          // query blocks per (batch, head)
  int32_t total;        // B * H * nqb workgroups
  float scale_log2;     // |scale| * log2(e)
  int32_t negate;       // scale < 0: Q fragments are negated (exact)
};

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

// XOR swizzles of the 16-byte chunks of one LDS row (row r, chunk c is stored
// at chunk c ^ swz(r)). They depend on the head dim because the row pitch in
// bytes does: the K swizzle spreads the 16 rows that one ds_read_b128 phase
// touches over all 64 banks; the V swizzle spreads the four rows that one
// transposing read touches over four different 64-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r >> 1) & 1) << 2;
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // After the swap each lane holds its own value and its partner's (l ^ 32).
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
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

template <int D, int BN, bool CAUSAL, int KIND, int OUT>
__global__ __launch_bounds__(256) void fa_fwd_kernel(Params p) {
  constexpr int BM = 128;
  constexpr int C = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BN * D * 2;         // bytes of one K or V tile
  constexpr int NDS = D / 16;              // k-steps of the first product
  constexpr int NKB = BN / 32;             // 32-key blocks per tile
  constexpr int NDB = D / 32;              // 32-wide head-dim blocks of O
  constexpr int LOADS = BN * C / 256;      // 16-byte loads per thread per tile
  constexpr bool SPLIT_P = (KIND == KBF16);  // bf16: P = hi + lo
  static_assert(LOADS * 256 == BN * C, "tile must split evenly over 256 lanes");

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K0 K1 V0 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;     // lane half
  const int l32 = lane & 31;

  // ---- work decomposition (64-bit offsets) ----
  const int t = xcd_remap(blockIdx.x, p.total);
  const int bh = t / p.nqb;
  int qb = t - bh * p.nqb;
  if constexpr (CAUSAL) qb = p.nqb - 1 - qb;   // longest rows first
  const int64_t Sq = p.Sq, Sk = p.Sk;
  const int64_t q0 = (int64_t)qb * BM;
  const int64_t in_elt = (KIND == KFP8) ? 1 : 2;
  const char* qhead = p.q + (int64_t)bh * Sq * D * in_elt;
  const char* khead = p.k + (int64_t)bh * Sk * D * in_elt;
  const char* vhead = p.v + (int64_t)bh * Sk * D * in_elt;

  const int64_t qrow = q0 + wave * 32 + l32;          // this lane's query
  const int64_t qrow_ld = qrow < Sq ? qrow : Sq - 1;   // clamped for the load

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
  u32x4 qf[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    qf[ds] = *(const u32x4*)(qhead + (qrow_ld * D + ds * 16 + hl * 8) * 2);
    if (p.negate) qf[ds] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  // ---- tile range ----
  int64_t kend = Sk;
  if constexpr (CAUSAL) {
    const int64_t last_q = q0 + BM - 1;
    kend = last_q + 1 < Sk ? last_q + 1 : Sk;
  }
  const int ntiles = (int)((kend + BN - 1) / BN);

  auto load_tile = [&](int j, int buf) {
    const int64_t row0 = (int64_t)j * BN;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int pidx = i * 256 + tid;       // physical chunk in the tile
      const int r = pidx / C;
      const int pc = pidx % C;
      int64_t grow = row0 + r;
      grow = grow < Sk ? grow : Sk - 1;
      const int64_t koff = (grow * D + (pc ^ swz_k<D>(r)) * 8) * 2;
      const int64_t voff = (grow * D + (pc ^ swz_v<D>(r)) * 8) * 2;
      char* kdst = smem + buf * TILE + (i * 256 + wave * 64) * 16;
      char* vdst = smem + (2 + buf) * TILE + (i * 256 + wave * 64) * 16;
      __builtin_amdgcn_global_load_lds((const void*)(khead + koff), LDS_PTR(void, kdst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vhead + voff), LDS_PTR(void, vdst), 16, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets (loop invariant) ----
  // K: lane reads row kb*32 + l32, logical chunk 2*ds + hl.
  int koffs[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) koffs[ds] = (l32 * C + ((2 * ds + hl) ^ swz_k<D>(l32))) * 16;
  // V (transposing reads): within each 16-lane group, lane i supplies row
  // 16*step + 4*hl + (i/4) [+8 for the second read] and head-dim columns
  // 32*db + 16*((lane/16)&1) + 4*(i%4) .. +4; the read returns to lane i the
  // four keys of its head-dim column.
  const int gi = lane & 15;
  const int vr = 4 * hl + (gi >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (gi & 3);   // column within a 32-block
  int voffs[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = vr + 8 * e;   // row within a 16-row step (swizzle is step invariant)
      const int col = 32 * db + vcol;
      voffs[db][e] = (r * C + ((col >> 3) ^ swz_v<D>(r))) * 16 + (col & 7) * 2;
    }
  }

  // ---- accumulators ----
  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = (f32x16){};
  float m_run = -INFINITY;   // running max of scaled scores, log2 units
  float l_run = 0.f;         // this lane's partial row sum (16 of the 32 rows per block)
  const float c = p.scale_log2;

  load_tile(0, 0);

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < ntiles) load_tile(j + 1, buf ^ 1);

    const int64_t kt0 = (int64_t)j * BN;
    // Causal: a wave whose rows all lie above this tile's first key has
    // nothing to add (all its scores here are masked).
    if (CAUSAL && kt0 > q0 + wave * 32 + 31) continue;

    const char* kb_lds = smem + buf * TILE;
    const char* vb_lds = smem + (2 + buf) * TILE;

    // ---- S^T = K Q^T for NKB blocks of 32 keys ----
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      u32x4 kf[NDS];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) kf[ds] = *(const u32x4*)(kb_lds + kb * 32 * C * 16 + koffs[ds]);
      s[kb] = (f32x16){};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) s[kb] = mfma32<KIND>(kf[ds], qf[ds], s[kb]);
    }

    // ---- masks: keys past Sk, keys above the diagonal (32-bit, tile-relative) ----
    const bool need_mask = (kt0 + BN > Sk) || (CAUSAL && kt0 + BN - 1 > q0 + wave * 32);
    if (need_mask) {
      const int64_t kv = Sk - kt0;                        // valid keys in this tile (may exceed BN)
      const int kvalid = kv < BN ? (int)kv : BN;
      const int64_t qr = qrow - kt0;                      // last visible key, tile-relative
      const int qlim = CAUSAL ? (qr < BN ? (int)qr : BN) : BN;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool dead = (key >= kvalid) || (key > qlim);
          s[kb][r] = dead ? -INFINITY : s[kb][r];
        }
      }
    }

    // ---- online softmax (log2 domain) ----
    // The running maximum only moves when the tile's maximum exceeds it by
    // more than 2^8 (in any lane of the wave): P is then bounded by 256, which
    // fp16, bf16 and the fp32 accumulators hold exactly as well as values
    // below 1, and the rescale of O is skipped on almost every tile. The
    // final O / l and lse do not depend on which reference maximum was used.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_max_halves(mx);
    const float m_cand = fmaxf(m_run, mx * c);
    const bool grow = m_cand > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_use = (m_cand == -INFINITY) ? 0.f : m_cand;   // no (-inf) - (-inf)
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    u32x4 pf[NKB * 2];                    // P^T operand, one per 16-key step
    u32x4 pl[SPLIT_P ? NKB * 2 : 1];      // bf16 only: rounding residual of P
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_use));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = pack2<KIND>(pv[8 * half + 2 * e], pv[8 * half + 2 * e + 1]);
          l_run = add_pair<KIND>(f[e], l_run);     // l sums the P that multiplies V
        }
        pf[kb * 2 + half] = f;
        if constexpr (SPLIT_P) {
          u32x4 g;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = pack2<KIND>(pv[8 * half + 2 * e] - unpack_lo<KIND>(f[e]),
                               pv[8 * half + 2 * e + 1] - unpack_hi<KIND>(f[e]));
            l_run = add_pair<KIND>(g[e], l_run);
          }
          pl[kb * 2 + half] = g;
        }
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int st = 0; st < BN / 16; ++st) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const fp16x4_tr x0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            LDS_PTR(fp16x4_tr, vb_lds + st * 16 * C * 16 + voffs[db][0]));
        const fp16x4_tr x1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            LDS_PTR(fp16x4_tr, vb_lds + st * 16 * C * 16 + voffs[db][1]));
        u32x2 y0, y1;
        __builtin_memcpy(&y0, &x0, 8);
        __builtin_memcpy(&y1, &x1, 8);
        const u32x4 a = (u32x4){y0[0], y0[1], y1[0], y1[1]};
        acc_o[db] = mfma32<KIND>(a, pf[st], acc_o[db]);
        if constexpr (SPLIT_P) acc_o[db] = mfma32<KIND>(a, pl[st], acc_o[db]);
      }
    }
  }

  // ---- epilogue: O = O / l, lse = (m + log2 l) * ln 2 ----
  const float l_tot = wave_sum_halves(l_run);
  const float inv_l = 1.f / l_tot;
  if (qrow < Sq) {
    char* orow = p.o + ((int64_t)bh * Sq + qrow) * D * (OUT == OF32 ? 4 : 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hl;   // 4 consecutive head-dim entries
        const float o0 = acc_o[db][4 * g + 0] * inv_l;
        const float o1 = acc_o[db][4 * g + 1] * inv_l;
        const float o2 = acc_o[db][4 * g + 2] * inv_l;
        const float o3 = acc_o[db][4 * g + 3] * inv_l;
        if constexpr (OUT == OF32) {
          *(f32x4*)(orow + d * 4) = (f32x4){o0, o1, o2, o3};
        } else {
          constexpr int PK = (OUT == OBF16) ? KBF16 : KF16;
          *(u32x2*)(orow + d * 2) = (u32x2){pack2<PK>(o0, o1), pack2<PK>(o2, o3)};
        }
      }
    }
    if (hl == 0) {
      p.lse[(int64_t)bh * Sq + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
    }
  }
}

}  // namespace fa

// ============================== host side ==============================

namespace {

using fa::Params;
typedef void (*KernelFn)(Params);

template <int D, bool CAUSAL, int KIND, int OUT>
KernelFn pick() {
  return fa::fa_fwd_kernel<D, 64, CAUSAL, KIND, OUT>;
}

template <int D, int KIND, int OUT>
KernelFn pick_c(bool causal) {
  return causal ? pick<D, true, KIND, OUT>() : pick<D, false, KIND, OUT>();
}

template <int KIND, int OUT>
KernelFn pick_d(int64_t D, bool causal) {
  return D == 64 ? pick_c<64, KIND, OUT>(causal) : pick_c<128, KIND, OUT>(causal);
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int64_t dtype_size(fa_dtype_t t) {
  switch (t) {
    case FA_F16: case FA_BF16: return 2;
    case FA_FP8_E4M3: return 1;
    case FA_F32: return 4;
  }
  return 0;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_str(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE";
    case FA_ERR_UNSUPPORTED_HEAD_DIM: return "FA_ERR_UNSUPPORTED_HEAD_DIM";
    case FA_ERR_UNSUPPORTED_DTYPE: return "FA_ERR_UNSUPPORTED_DTYPE";
    case FA_ERR_UNSUPPORTED_LAYOUT: return "FA_ERR_UNSUPPORTED_LAYOUT";
    case FA_ERR_UNSUPPORTED_DROPOUT: return "FA_ERR_UNSUPPORTED_DROPOUT";
    case FA_ERR_BAD_SCALE: return "FA_ERR_BAD_SCALE";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED";
    case FA_ERR_ALIASING: return "FA_ERR_ALIASING";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                   fa_layout_t layout, float scale, int causal, float keep_prob,
                   fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                   const float* descale_q, const float* descale_k, const float* descale_v,
                   hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return FA_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  const bool ok_pair = (in_dtype == FA_F16 && (o_dtype == FA_F16 || o_dtype == FA_F32)) ||
                       (in_dtype == FA_BF16 && (o_dtype == FA_BF16 || o_dtype == FA_F32)) ||
                       (in_dtype == FA_FP8_E4M3 && (o_dtype == FA_F16 || o_dtype == FA_F32));
  if (!ok_pair) return FA_ERR_UNSUPPORTED_DTYPE;
  if (in_dtype == FA_FP8_E4M3) {
    if (!descale_q || !descale_k || !descale_v) return FA_ERR_NULL_POINTER;
    return FA_ERR_UNSUPPORTED_DTYPE;   // fp8 kernels are not built yet
  }
  if (layout != FA_LAYOUT_BNSD) return FA_ERR_UNSUPPORTED_LAYOUT;
  if (keep_prob != 1.0f) return FA_ERR_UNSUPPORTED_DROPOUT;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;

  // sizes: element counts must fit comfortably in 64-bit byte offsets and
  // the grid in 31 bits.
  const int64_t lim = (int64_t)1 << 40;
  if (B > lim / H || Sq > lim || Sk > lim) return FA_ERR_BAD_SHAPE;
  const int64_t BH = B * H;
  if (BH > (lim / Sq) || BH > (lim / Sk)) return FA_ERR_BAD_SHAPE;
  const int64_t nqb = (Sq + 127) / 128;
  if (nqb > INT32_MAX || BH * nqb > INT32_MAX) return FA_ERR_BAD_SHAPE;

  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;

  const int64_t ie = dtype_size(in_dtype), oe = dtype_size(o_dtype);
  const int64_t nq = BH * Sq * D * ie, nk = BH * Sk * D * ie;
  const int64_t no = BH * Sq * D * oe, nl = BH * Sq * 4;
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nk) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) ||
      overlaps(o, no, lse, nl))
    return FA_ERR_ALIASING;

  Params p;
  p.q = (const char*)q;
  p.k = (const char*)k;
  p.v = (const char*)v;
  p.o = (char*)o;
  p.lse = lse;
  p.descale_q = descale_q;
  p.descale_k = descale_k;
  p.descale_v = descale_v;
  p.Sq = Sq;
  p.Sk = Sk;
  p.nqb = (int32_t)nqb;
  p.total = (int32_t)(BH * nqb);
  // A zero scale would turn masked scores into (-inf) * 0 = NaN; the
  // smallest normal factor gives the same result (every visible score maps
  // to exp2(0) = 1) and keeps -inf masks intact.
  p.scale_log2 = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
  p.negate = scale < 0.f;

  const bool cz = causal != 0;
  KernelFn fn = nullptr;
  if (in_dtype == FA_F16) {
    fn = (o_dtype == FA_F32) ? pick_d<fa::KF16, fa::OF32>(D, cz) : pick_d<fa::KF16, fa::OF16>(D, cz);
  } else if (in_dtype == FA_BF16) {
    fn = (o_dtype == FA_F32) ? pick_d<fa::KBF16, fa::OF32>(D, cz) : pick_d<fa::KBF16, fa::OBF16>(D, cz);
  }
  if (!fn) return FA_ERR_UNSUPPORTED_DTYPE;

  hipLaunchKernelGGL(fn, dim3((unsigned)p.total), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

}  // extern "C"
