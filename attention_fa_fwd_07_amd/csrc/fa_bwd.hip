// FlashAttention backward for MI355X (gfx950, CDNA4), HIP.
//
// Given Q, K, V, the forward output O, its gradient dO and the per-row
// logsumexp of the forward, the gradients of O = softmax(scale*QK^T + mask) V
// are, per (batch, head) and with P recomputed from lse:
//   P  = exp(scale*QK^T - lse)        (masked entries 0)
//   dV = P^T dO
//   dP = dO V^T
//   dS = P * (dP - Delta),  Delta_i = sum_j P_ij dP_ij = sum_d dO_id O_id
//   dQ = scale * dS K,      dK = scale * dS^T Q
// (the derivative of the softmax: d softmax(x)/dx = diag(p) - p p^T). The
// forward's lse is what makes P recomputable tile by tile, so S, P, dP and
// dS never reach HBM here either. "Hygon FlashAttention: fixed-defect
// review" (chatdocs.ruinique.com/hygon/flash-attention-fixed-bugs, item 13)
// reports a dQ pass that stepped V by K's row stride; K and V carry their
// own row pitch throughout this file.
//
// Three kernels, all on MFMA v_mfma_f32_32x32x16_{f16,bf16} for the products:
//  * pre: Delta = rowsum(dO * O) and lse2 = lse * log2(e) per query row into
//    the caller's workspace; rows past Sq and rows that see no key get
//    lse2 = +inf, so that their P is exactly 0 without a mask.
//  * dkv: one workgroup per 128 keys of one (batch, key/value head), 32 keys
//    per wave, K in registers and V in LDS; it walks the query tiles (32
//    rows) of every query head that shares the key/value head, with Q, dO,
//    lse2 and Delta of a tile loaded HBM->LDS one tile ahead. Per tile:
//    S = Q K^T and dP = dO V^T (accumulator: a lane owns one key and 16
//    queries), then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read
//    transposed from LDS (ds_read_b64_tr_b16), P and dS converted to the
//    B operand in registers. Summing over the heads of a group inside the
//    workgroup keeps dK, dV deterministic (no atomics).
//  * dq: the forward's structure, one workgroup per 128 query rows, K and V
//    tiles (32 keys) streamed through LDS: S^T = K Q^T, dP^T = V dO^T, then
//    dQ^T += K^T dS^T with K^T read transposed.
//
// Dropout (DROP): the forward's mask Z (Philox4x64-10, counter (2t + half,
// query row, b*H + h, 0) per 16 keys of a 32-key tile t) is drawn again;
// P * Z / keep_prob multiplies dO in dV, and dP * Z / keep_prob is the
// gradient reaching P. The dq kernel holds the forward's layout (a lane owns
// one query row and the 16 keys of one Philox block per tile). In the dkv
// kernel a lane owns one key and 16 query rows, so each lane draws the block
// of one (row, half) of its wave's tile, reduces it to 16 keep bits and the
// lanes exchange the bits through 128 bytes of LDS per wave.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <float.h>

#include "fa_mi355x.h"
#include "fa_device.h"

namespace fa {

struct BwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  char* dq;
  char* dk;
  char* dv;
  float* lse2;          // workspace [B*H*Sqp]: lse * log2(e), +inf where P must be 0
  float* delta;         // workspace [B*H*Sqp]: rowsum(dO * O)
  int64_t Sq, Sk;
  int64_t Sqp;          // Sq rounded up to a multiple of 32
  int64_t k_ss, v_ss;   // elements from one K (V) row to the next
  int64_t moff;         // causal: key j is visible to query i iff j <= i + moff
  int32_t H, Hkv;
  int32_t nblk;         // blocks per head (dq) or per key/value head (dkv)
  int32_t total;        // workgroups of the launch
  // causal launch order (xcd_lpt): qmajor > 0 orders the blocks by work
  // across each XCD's heads, in groups of qmajor heads sharing K/V; qrem
  // groups beyond a multiple of 8 go first; qsnake pairs long and short
  // blocks when the whole grid is resident
  int32_t qmajor, qrem, qsnake;
  float scale;          // S = scale * Q K^T (dQ and dK carry it with its sign)
  float c;              // max(|scale| * log2(e), FLT_MIN)
  int32_t negate;       // scale < 0: the register operand of S is negated (exact)
  uint64_t seed, rng_off;   // dropout: Philox key
  uint32_t keep_thr;        // a 16-bit draw below this keeps its P
  float inv_keep;
};

constexpr float kLog2e = 1.4426950408889634f;

// ---- Delta and lse2 per query row; LPR lanes per row, 8 elements each ----
template <int D, int KIND>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t R = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int ch = tid % LPR;
  const bool valid = R < rows;
  int64_t bh = 0, i = 0;
  if (valid) {
    bh = R / p.Sqp;
    i = R - bh * p.Sqp;
  }
  const bool live = valid && i < p.Sq;
  float acc = 0.f;
  if (live) {
    const int64_t off = ((bh * p.Sq + i) * D + ch * 8) * 2;
    const u32x4 a = *(const u32x4*)(p.o + off);
    const u32x4 g = *(const u32x4*)(p.dout + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(unpack_lo<KIND>(a[e]), unpack_lo<KIND>(g[e]), acc);
      acc = __builtin_fmaf(unpack_hi<KIND>(a[e]), unpack_hi<KIND>(g[e]), acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (valid && ch == 0) {
    float l2 = INFINITY;
    if (live) {
      const float l = p.lse[bh * p.Sq + i];
      l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
    p.lse2[R] = l2;
    p.delta[R] = live ? acc : 0.f;
  }
}

// Fragment reads shared by both kernels. A tile is stored with 16-byte
// chunk c of row r at chunk c ^ SW(r) (SW from fa_device.h: swz_k for row
// reads only, swz_v where a tile is also read transposed).
//
// Row fragment (A or B operand with the lane's row = l32, k = head dim
// 16*ds + 8*hl .. +8): one ds_read_b128.
template <int RB, int SWSEL>
__device__ __forceinline__ int swz(int r) {
  if constexpr (SWSEL == 0) return swz_k<RB>(r);
  else return swz_v<RB, false>(r);
}

template <int RB, int SWSEL>
__device__ __forceinline__ u32x4 row_frag(uint32_t base, int row, int ds, int hl) {
  return lds_load<u32x4>(base + row * RB + ((((2 * ds + hl) ^ swz<RB, SWSEL>(row))) << 4));
}

// Transposed fragment (A operand, lane's row = head-dim column 32*db + l32,
// k = the 16 tile rows of step st in the order 4*hl + 0..3, 8 + 4*hl + 0..3,
// which is the row order of a 32x32 accumulator's registers 8*st .. 8*st+7):
// two ds_read_b64_tr_b16. Within each 16-lane group, lane i supplies row
// 16*st + 4*hl + i/4 (+8 for the second read) and the 4 columns
// 32*db + 16*((lane/16)&1) + 4*(i%4) .. +4; the read returns to lane i the
// four rows of its own column.
template <int RB, int SWSEL>
__device__ __forceinline__ uint32_t tr_addr(uint32_t base, int lane, int hl, int db, int e) {
  const int gi = lane & 15;
  const int r = 4 * hl + (gi >> 2) + 8 * e;
  const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
  return base + r * RB + (((col >> 3) ^ swz<RB, SWSEL>(r)) << 4) + (col & 7) * 2;
}

__device__ __forceinline__ u32x4 tr_frag(uint32_t a0, uint32_t a1) {
  u32x2 y[2];
  const fp16x4_tr x0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) fp16x4_tr*)(uintptr_t)a0);
  const fp16x4_tr x1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) fp16x4_tr*)(uintptr_t)a1);
  __builtin_memcpy(&y[0], &x0, 8);
  __builtin_memcpy(&y[1], &x1, 8);
  return (u32x4){y[0][0], y[0][1], y[1][0], y[1][1]};
}

// HBM -> LDS copy of `rows` rows of RB bytes (row pitch `pitch` bytes in
// HBM) into a swizzled tile at `dst`, by all NL lanes of the workgroup; rows
// at or past `rmax` (relative) read row rmax - 1, a legal row with finite
// values. RB/16 chunks per row, NL*16 bytes per instruction.
template <int RB, int SWSEL, int ROWS, int NL>
__device__ __forceinline__ void copy_tile(const char* src, int64_t pitch, int64_t rmax, uint32_t dst, int tid) {
  constexpr int C = RB / 16;
  constexpr int N = ROWS * C / NL;
  static_assert(ROWS * C % NL == 0, "tile must split evenly over the lanes");
  // the LDS destination goes to M0: wave-uniform
  const uint32_t wdst = __builtin_amdgcn_readfirstlane(dst + (tid & ~63) * 16);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int pidx = i * NL + tid;
    const int r = pidx / C;
    const int pc = pidx % C;
    const int64_t rr = r < rmax ? r : rmax - 1;
    dma16(src, (uint32_t)(rr * pitch + ((pc ^ swz<RB, SWSEL>(r)) << 4)), wdst + i * NL * 16);
  }
}

// 8 scores (accumulator registers 8*st .. 8*st+7) -> B operand, RNE.
template <int KIND>
__device__ __forceinline__ u32x4 pack8(const f32x16& x, int st) {
  u32x4 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = pack2<KIND>(x[8 * st + 2 * e], x[8 * st + 2 * e + 1]);
  return f;
}

template <int OUT>
__device__ __forceinline__ void store4(char* row, int d, float a, float b, float c, float e) {
  if constexpr (OUT == OF32) {
    *(f32x4*)(row + d * 4) = (f32x4){a, b, c, e};
  } else {
    constexpr int PK = (OUT == OBF16) ? KBF16 : KF16;
    *(u32x2*)(row + d * 2) = (u32x2){pack2<PK>(a, b), pack2<PK>(c, e)};
  }
}

// 16 keep bits of one Philox block: bit n set iff 16-bit value n of the
// output lies below the threshold
__device__ __forceinline__ uint32_t keep_bits16(uint64_t c0, uint64_t c1, uint64_t c2, const BwdParams& p) {
  uint64_t c[4] = {c0, c1, c2, 0ull};
  philox4x64_10(c, p.seed, p.rng_off);
  uint32_t m = 0;
#pragma unroll
  for (int n = 0; n < 16; ++n) m |= ((uint32_t)(c[n >> 2] >> (16 * (n & 3))) & 0xffffu) < p.keep_thr ? (1u << n) : 0u;
  return m;
}

// ============================== dK, dV ==============================
template <int D, bool CAUSAL, int KIND, int OUT, bool DROP>
struct BwdDkv {
  static constexpr int NW = 4;                // waves, 32 keys each
  static constexpr int BK = 32 * NW;          // keys per workgroup
  static constexpr int BQ = 32;               // query rows per tile
  static constexpr int RB = D * 2;            // bytes per row
  static constexpr int NDS = D / 16;          // k-steps over the head dim
  static constexpr int NDB = D / 32;          // 32-wide head-dim blocks
  static constexpr int TQ = BQ * RB;          // one Q or dO tile
  static constexpr int BUF = 2 * TQ + 256;    // Q, dO, lse2[32], Delta[32]
  static constexpr int VOFF = 0;              // V block (BK rows)
  static constexpr int ROFF = BK * RB;        // ring of two tile buffers
  static constexpr int ZOFF = ROFF + 2 * BUF; // dropout: keep bits, 32 rows x 4 bytes per wave
  static constexpr int SMEM = ZOFF + (DROP ? NW * 128 : 0);

  const BwdParams& p;
  uint32_t lds0;
  int tid, lane, wave, hl, l32;
  int64_t k0, kw0;
  int b, kvh, group;
  int qt0, nqt, ntot;                         // query tiles qt0 .. nqt-1 per head
  u32x4 kf[NDS];
  f32x16 acc_k[NDB], acc_v[NDB];
  // this lane's fragment addresses in tile buffer 0 (the buffer, the dO tile
  // and the 16-row step are compile-time offsets added to them, so they fold
  // into the read instructions): Q rows, V rows of this wave's keys,
  // transposed Q (and dO) fragments, lse2/Delta. The causal instances (more
  // live state) keep one Q row base, one V row base and one transposed-read
  // base per row half and form each fragment's address with an XOR in the loop.
  static constexpr int NQA = CAUSAL ? 1 : NDS;
  static constexpr int NVA = CAUSAL ? 1 : NDS;
  static constexpr int NTA = CAUSAL ? 1 : NDB;
  uint32_t qa[NQA], va[NVA], ta[NTA][2], la;

  __device__ __forceinline__ BwdDkv(const BwdParams& p_, char* smem) : p(p_) {
    lds0 = (uint32_t)(uintptr_t)LDS_PTR(char, smem);
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hl = lane >> 5;
    l32 = lane & 31;
    int bkv, kb;
    if (CAUSAL && p.qmajor > 0) {   // key blocks by work across each XCD's heads (block 0 the most)
      xcd_lpt(blockIdx.x, p.total, p.nblk, 1, p.qrem, p.qsnake != 0, bkv, kb);
    } else {
      const int t = xcd_remap(blockIdx.x, p.total);
      bkv = t / p.nblk;
      kb = t - bkv * p.nblk;
    }
    b = bkv / p.Hkv;
    kvh = bkv - b * p.Hkv;
    group = p.H / p.Hkv;
    k0 = (int64_t)kb * BK;
    kw0 = k0 + 32 * wave;
    nqt = (int)(p.Sqp / BQ);
    qt0 = 0;
    if constexpr (CAUSAL) {
      // first query tile that sees key k0: rows q with k0 <= q + moff
      const int64_t q = k0 - p.moff;
      qt0 = q <= 0 ? 0 : (q >= p.Sqp ? nqt : (int)(q / BQ));
    }
    ntot = group * (nqt - qt0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      acc_k[db] = (f32x16){};
      acc_v[db] = (f32x16){};
    }
    const uint32_t qb0 = lds0 + ROFF;
    const uint32_t vb = lds0 + VOFF + 32 * wave * RB;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (ds < NQA) qa[ds] = qb0 + l32 * RB + (((2 * ds + hl) ^ swz<RB, 1>(l32)) << 4);
      if (ds < NVA) va[ds] = vb + l32 * RB + (((2 * ds + hl) ^ swz<RB, 0>(l32)) << 4);
    }
#pragma unroll
    for (int db = 0; db < NTA; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) ta[db][e] = tr_addr<RB, 1>(qb0, lane, hl, db, e);
    la = qb0 + 2 * TQ + 4 * hl * 4;
  }

  __device__ __forceinline__ const char* kvbase(const char* t, int64_t ss) const {
    return t + (((int64_t)b * p.Hkv + kvh) * p.Sk * ss) * 2;
  }

  // tile `it` of the flattened (head of the group, query tile) loop -> buffer
  __device__ __forceinline__ void load_tile(int it, int buf) {
    const int per = nqt - qt0;
    const int hh = it / per;
    const int qt = qt0 + (it - hh * per);
    const int64_t bh = (int64_t)b * p.H + (int64_t)kvh * group + hh;
    const int64_t q0 = (int64_t)qt * BQ;
    const int64_t rmax = p.Sq - q0;          // >= 1 unless the tile lies past Sq
    const uint32_t dst = lds0 + ROFF + buf * BUF;
    const int64_t qoff = (bh * p.Sq + q0) * D * 2;
    copy_tile<RB, 1, BQ, 64 * NW>(p.q + qoff, RB, rmax > 0 ? rmax : 1, dst, tid);
    copy_tile<RB, 1, BQ, 64 * NW>(p.dout + qoff, RB, rmax > 0 ? rmax : 1, dst + TQ, tid);
    if (tid < 16) {
      // lanes 0..7: lse2[q0 .. q0+32), lanes 8..15: Delta (the workspace
      // holds lse2, then Delta, each B*H*Sqp floats)
      const int64_t idx = bh * p.Sqp + q0;
      const uint32_t off = (uint32_t)(((tid < 8 ? idx : idx + (int64_t)(p.delta - p.lse2)) + 4 * (tid & 7)) * 4);
      dma16((const char*)p.lse2, off, dst + 2 * TQ);
    }
  }

  __device__ __forceinline__ void run() {
    if (ntot > 0) load_tile(0, 0);
    // V rows k0 .. k0+BK into LDS; K rows of this wave into registers
    copy_tile<RB, 0, BK, 64 * NW>(kvbase(p.v, p.v_ss) + k0 * p.v_ss * 2, p.v_ss * 2, p.Sk - k0, lds0 + VOFF, tid);
    {
      const int64_t key = kw0 + l32 < p.Sk ? kw0 + l32 : p.Sk - 1;
      const char* kr = kvbase(p.k, p.k_ss) + key * p.k_ss * 2;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        kf[ds] = *(const u32x4*)(kr + (16 * ds + 8 * hl) * 2);
        if (p.negate) kf[ds] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      }
    }
    for (int it = 0; it < ntot; it += 2) {
      step<0>(it);
      if (it + 1 < ntot) step<1>(it + 1);
    }
    wait_loads<0>();   // no copy into LDS may outlive the workgroup (ntot = 0)
    store();
  }

  // LDS addresses of this lane's Q and V row fragments of k-step ds. The
  // chunk index is (2*ds + hl) ^ swz(row), and the row base (1 KiB-aligned
  // block, whole rows) has zero chunk bits, so the address of k-step ds is
  // that of k-step 0 with ds XORed into bits 5 and up; the causal instances
  // form it in the loop (an XOR opaque to the compiler, so that it is not
  // hoisted into a register per k-step) to stay within the register budget.
  // ds (and db below) are unrolled loop indices: compile-time immediates.
  __device__ __forceinline__ uint32_t q_addr(int ds) const {
    if constexpr (NQA == NDS) {
      return qa[ds];
    } else {
      uint32_t a;
      asm volatile("v_xor_b32 %0, %2, %1" : "=v"(a) : "v"(qa[0]), "n"(ds << 5));
      return a;
    }
  }
  __device__ __forceinline__ uint32_t v_addr(int ds) const {
    if constexpr (NVA == NDS) {
      return va[ds];
    } else {
      uint32_t a;
      asm volatile("v_xor_b32 %0, %2, %1" : "=v"(a) : "v"(va[0]), "n"(ds << 5));
      return a;
    }
  }
  // the same for the transposed reads of head-dim block db (tr_addr): the
  // block enters the chunk index as 4*db, above the two chunk bits that the
  // lane picks, so it is db XORed into address bits 6 and up
  __device__ __forceinline__ uint32_t t_addr(int db, int e) const {
    if constexpr (NTA == NDB) {
      return ta[db][e];
    } else {
      uint32_t a;
      asm volatile("v_xor_b32 %0, %2, %1" : "=v"(a) : "v"(ta[0][e]), "n"(db << 6));
      return a;
    }
  }

  // query tile `it` in buffer B (= it % 2, a compile-time value so that the
  // LDS offsets fold into the instructions)
  template <int B>
  __device__ __forceinline__ void step(int it) {
    wait_loads<0>();
    lds_barrier();
    if (it + 1 < ntot) load_tile(it + 1, B ^ 1);
    tile<B>(it);
  }

  template <int B>
  __device__ __forceinline__ void tile(int it) {
    constexpr uint32_t off = B * BUF;
    const int per = nqt - qt0;
    const int hh = it / per;
    const int64_t q0 = (int64_t)(qt0 + (it - hh * per)) * BQ;
    if constexpr (CAUSAL) {
      // every key of this wave lies above the diagonal for all 32 rows
      if (kw0 > q0 + BQ - 1 + p.moff) return;
    }
    uint32_t zbits = 0;   // dropout: bit r = keep bit of this lane's key in row r
    if constexpr (DROP) {
      // this lane draws row q0 + l32, half hl of the wave's 32-key tile and
      // stores its 16 keep bits; the word of row r holds half 0 in bits
      // 0..15 and half 1 in bits 16..31
      const int64_t bhq = (int64_t)b * p.H + (int64_t)kvh * group + hh;
      const uint32_t m = keep_bits16((uint64_t)(2 * (kw0 / 32) + hl), (uint64_t)(q0 + l32), (uint64_t)bhq, p);
      const uint32_t zb = lds0 + ZOFF + wave * 128;
      *LDS_PTR(uint16_t, zb + l32 * 4 + hl * 2) = (uint16_t)m;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // key offset l32 of the tile: half (l32/4)&1, value 4*(l32/8) + l32%4
      const int bit = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 w = lds_load<u32x4>(zb + (8 * g + 4 * hl) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) zbits |= ((w[e] >> bit) & 1u) << (4 * g + e);
      }
    }

    // S = Q K^T, dP = dO V^T: lane = key (l32), rows = queries
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) s = mfma32<KIND>(lds_load<u32x4>(q_addr(ds) + off), kf[ds], s);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      dp = mfma32<KIND>(lds_load<u32x4>(q_addr(ds) + off + TQ), lds_load<u32x4>(v_addr(ds)), dp);

    // P = exp2(S*c - lse2), dS = P * (dP - Delta); register r holds query
    // row 8*(r/4) + 4*hl + r%4 of the tile
    bool need_mask = false;
    int lim = 0;
    if constexpr (CAUSAL) {
      // masked iff key > q + moff, i.e. row < kw0 + l32 - moff - q0
      need_mask = kw0 + 31 > q0 + p.moff;
      const int64_t x = kw0 + l32 - p.moff - q0 - 4 * hl;
      lim = x < -64 ? -64 : (x > 64 ? 64 : (int)x);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l2 = lds_load<f32x4>(la + off + 8 * g * 4);
      const f32x4 dl = lds_load<f32x4>(la + off + 128 + 8 * g * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float x = __builtin_fmaf(s[r], p.c, -l2[e]);
        if (CAUSAL && need_mask && (8 * g + e) < lim) x = -INFINITY;
        const float pr = __builtin_amdgcn_exp2f(x);
        if constexpr (DROP) {
          const float z = ((zbits >> r) & 1u) ? p.inv_keep : 0.f;
          s[r] = pr * z;
          dp[r] = pr * (dp[r] * z - dl[e]);
        } else {
          s[r] = pr;
          dp[r] = pr * (dp[r] - dl[e]);
        }
      }
    }
    u32x4 pf[2], dsf[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      pf[st] = pack8<KIND>(s, st);
      dsf[st] = pack8<KIND>(dp, st);
    }
    // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t so = off + st * 16 * RB;
        const uint32_t t0 = t_addr(db, 0), t1 = t_addr(db, 1);
        const u32x4 a = tr_frag(t0 + so + TQ, t1 + so + TQ);
        acc_v[db] = mfma32<KIND>(a, pf[st], acc_v[db]);
        const u32x4 qt = tr_frag(t0 + so, t1 + so);
        acc_k[db] = mfma32<KIND>(qt, dsf[st], acc_k[db]);
      }
    }
  }

  __device__ __forceinline__ void store() {
    const int64_t key = kw0 + l32;
    if (key >= p.Sk) return;
    constexpr int GE = (OUT == OF32) ? 4 : 2;
    const int64_t kvrow = ((int64_t)b * p.Hkv + kvh) * p.Sk + key;
    char* dkr = p.dk + kvrow * D * GE;
    char* dvr = p.dv + kvrow * D * GE;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hl;
        store4<OUT>(dkr, d, acc_k[db][4 * g] * p.scale, acc_k[db][4 * g + 1] * p.scale,
                    acc_k[db][4 * g + 2] * p.scale, acc_k[db][4 * g + 3] * p.scale);
        store4<OUT>(dvr, d, acc_v[db][4 * g], acc_v[db][4 * g + 1], acc_v[db][4 * g + 2], acc_v[db][4 * g + 3]);
      }
    }
  }
};

// ================================ dQ ================================
template <int D, bool CAUSAL, int KIND, int OUT, bool DROP>
struct BwdDq {
  static constexpr int NW = 4;                // waves, 32 query rows each
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 32;               // keys per tile
  static constexpr int RB = D * 2;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int TILE = BN * RB;
  static constexpr int BUF = 2 * TILE;        // K (read both ways), V
  static constexpr int SMEM = 2 * BUF;

  const BwdParams& p;
  uint32_t lds0;
  int tid, lane, wave, hl, l32;
  int64_t bh, q0, qw0, qrow;
  const char* khead;
  const char* vhead;
  int ntiles, jlast;
  float l2, dl;
  u32x4 qf[NDS], dof[NDS];
  f32x16 acc[NDB];
  // LDS addresses of this lane's fragments in buffer 0 (the buffer and the
  // 16-key step go into the reads' immediate offsets): K and V row
  // fragments per k-step, transposed K fragments per head-dim block and read
  uint32_t ka[NDS], va[NDS], ta[NDB][2];

  __device__ __forceinline__ BwdDq(const BwdParams& p_, char* smem) : p(p_) {
    lds0 = (uint32_t)(uintptr_t)LDS_PTR(char, smem);
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hl = lane >> 5;
    l32 = lane & 31;
    int qb;
    if (CAUSAL && p.qmajor > 0) {   // query blocks by length across each XCD's heads
      int u, rank;
      xcd_lpt(blockIdx.x, p.total, p.nblk, p.qmajor, p.qrem, p.qsnake != 0, u, rank);
      bh = u;
      qb = p.nblk - 1 - rank;
    } else {
      const int t = xcd_remap(blockIdx.x, p.total);
      bh = t / p.nblk;
      qb = t - (int)bh * p.nblk;
      if constexpr (CAUSAL) qb = p.nblk - 1 - qb;   // longest rows first
    }
    const int b = (int)(bh / p.H);
    const int h = (int)(bh - (int64_t)b * p.H);
    const int kvh = h / (p.H / p.Hkv);
    khead = p.k + ((int64_t)b * p.Hkv + kvh) * p.Sk * p.k_ss * 2;
    vhead = p.v + ((int64_t)b * p.Hkv + kvh) * p.Sk * p.v_ss * 2;
    q0 = (int64_t)qb * BM;
    qw0 = q0 + 32 * wave;
    qrow = qw0 + l32;
    int64_t kend = p.Sk;
    if constexpr (CAUSAL) {
      kend = q0 + BM + p.moff < p.Sk ? q0 + BM + p.moff : p.Sk;
      if (kend < 0) kend = 0;
    }
    ntiles = (int)((kend + BN - 1) / BN);
    jlast = ntiles - 1;
    if constexpr (CAUSAL) {
      const int64_t last = qw0 + 31 + p.moff;
      const int64_t jl = last < 0 ? -1 : last / BN;
      jlast = jl < jlast ? (int)jl : jlast;
    }
    if (qw0 >= p.Sq) jlast = -1;
    const int64_t qr = qrow < p.Sq ? qrow : p.Sq - 1;
    const char* qp = p.q + (bh * p.Sq + qr) * D * 2;
    const char* op = p.dout + (bh * p.Sq + qr) * D * 2;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qf[ds] = *(const u32x4*)(qp + (16 * ds + 8 * hl) * 2);
      if (p.negate) qf[ds] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      dof[ds] = *(const u32x4*)(op + (16 * ds + 8 * hl) * 2);
    }
    // rows past Sq: P = 0 through lse2 = +inf
    l2 = qrow < p.Sq ? p.lse2[bh * p.Sqp + qrow] : INFINITY;
    dl = qrow < p.Sq ? p.delta[bh * p.Sqp + qrow] : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      ka[ds] = lds0 + l32 * RB + (((2 * ds + hl) ^ swz<RB, 1>(l32)) << 4);
      va[ds] = lds0 + TILE + l32 * RB + (((2 * ds + hl) ^ swz<RB, 0>(l32)) << 4);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) ta[db][e] = tr_addr<RB, 1>(lds0, lane, hl, db, e);
  }

  __device__ __forceinline__ void load_tile(int j, int buf) {
    const int64_t r0 = (int64_t)j * BN;
    const uint32_t dst = lds0 + buf * BUF;
    copy_tile<RB, 1, BN, 64 * NW>(khead + r0 * p.k_ss * 2, p.k_ss * 2, p.Sk - r0, dst, tid);
    copy_tile<RB, 0, BN, 64 * NW>(vhead + r0 * p.v_ss * 2, p.v_ss * 2, p.Sk - r0, dst + TILE, tid);
  }

  // tile j in buffer BUF (= j % 2, a compile-time value so that the LDS
  // offsets fold into the instructions)
  template <int B>
  __device__ __forceinline__ void step(int j) {
    wait_loads<0>();
    lds_barrier();
    if (j + 1 < ntiles) load_tile(j + 1, B ^ 1);
    if (j <= jlast) tile<B>(j);
  }

  __device__ __forceinline__ void run() {
    if (ntiles > 0) load_tile(0, 0);
    for (int j = 0; j < ntiles; j += 2) {
      step<0>(j);
      if (j + 1 < ntiles) step<1>(j + 1);
    }
    store();
  }

  template <int B>
  __device__ __forceinline__ void tile(int j) {
    constexpr uint32_t off = B * BUF;
    const int64_t kt0 = (int64_t)j * BN;
    uint32_t zm = 0;
    if constexpr (DROP) zm = keep_bits16((uint64_t)(2 * j + hl), (uint64_t)qrow, (uint64_t)bh, p);
    // S^T = K Q^T, dP^T = V dO^T: lane = query (l32), rows = keys
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) s = mfma32<KIND>(lds_load<u32x4>(ka[ds] + off), qf[ds], s);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) dp = mfma32<KIND>(lds_load<u32x4>(va[ds] + off), dof[ds], dp);
    // the transposed K fragments of dQ^T += K^T dS^T: without dropout read
    // now, so that their LDS latency runs during the exponentials below (the
    // dropout instances have no registers to spare for them)
    u32x4 kt[2][NDB];
    auto read_kt = [&]() {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          kt[st][db] = tr_frag(ta[db][0] + off + st * 16 * RB, ta[db][1] + off + st * 16 * RB);
    };
    if constexpr (!DROP) read_kt();
    // keys past Sk or above the diagonal: P = 0. Register r holds key
    // kt0 + 8*(r/4) + 4*hl + r%4.
    const bool need_mask = (kt0 + BN > p.Sk) || (CAUSAL && kt0 + BN - 1 > qw0 + p.moff);
    if (need_mask) {
      // a real branch: tiles inside the keys and below the diagonal skip
      // the compare-and-select on every score
      asm volatile("");
      const int64_t kv = p.Sk - kt0;
      int lim = kv < BN ? (int)kv : BN;
      if constexpr (CAUSAL) {
        int64_t qr = qrow + p.moff - kt0 + 1;
        if (qr < 0) qr = 0;
        lim = qr < lim ? (int)qr : lim;
      }
      lim -= 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3)) >= lim ? -INFINITY : s[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // c > 0: a masked score (-inf) stays -inf
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.c, -l2));
      if constexpr (DROP) {
        // register r holds Philox value r of this lane's block
        const float z = ((zm >> r) & 1u) ? p.inv_keep : 0.f;
        dp[r] = pr * (dp[r] * z - dl);
      } else {
        dp[r] = pr * (dp[r] - dl);
      }
    }
    // dQ^T += K^T dS^T
    if constexpr (DROP) read_kt();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u32x4 dsf = pack8<KIND>(dp, st);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = mfma32<KIND>(kt[st][db], dsf, acc[db]);
    }
  }

  __device__ __forceinline__ void store() {
    if (qrow >= p.Sq) return;
    constexpr int GE = (OUT == OF32) ? 4 : 2;
    char* row = p.dq + (bh * p.Sq + qrow) * D * GE;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hl;
        store4<OUT>(row, d, acc[db][4 * g] * p.scale, acc[db][4 * g + 1] * p.scale,
                    acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
      }
    }
  }
};

// Two waves per SIMD; the D = 128 dropout instances, whose Philox state does
// not fit beside the 32 K fragments and the two 64-register accumulators of
// that budget (the compiler spilled about 30 VGPRs to scratch), get one.
template <int D, bool DROP>
constexpr int dkv_waves_per_simd() { return (DROP && D == 128) ? 1 : 2; }

template <int D, bool CAUSAL, int KIND, int OUT, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dkv_waves_per_simd<D, DROP>())))
void fa_bwd_dkv_kernel(BwdParams p) {
  using Blk = BwdDkv<D, CAUSAL, KIND, OUT, DROP>;
  __shared__ __attribute__((aligned(1024))) char smem[Blk::SMEM];
  Blk blk(p, smem);
  blk.run();
}

template <int D, bool CAUSAL, int KIND, int OUT, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dq_kernel(BwdParams p) {
  using Blk = BwdDq<D, CAUSAL, KIND, OUT, DROP>;
  __shared__ __attribute__((aligned(1024))) char smem[Blk::SMEM];
  Blk blk(p, smem);
  blk.run();
}

}  // namespace fa

// ============================== host side ==============================

namespace {

using fa::BwdParams;
typedef void (*BwdFn)(BwdParams);
typedef void (*PreFn)(BwdParams, int64_t);

template <int D, bool CAUSAL, int KIND, int OUT>
void pick_pair(bool drop, BwdFn& dkv, BwdFn& dq) {
  dkv = drop ? fa::fa_bwd_dkv_kernel<D, CAUSAL, KIND, OUT, true> : fa::fa_bwd_dkv_kernel<D, CAUSAL, KIND, OUT, false>;
  dq = drop ? fa::fa_bwd_dq_kernel<D, CAUSAL, KIND, OUT, true> : fa::fa_bwd_dq_kernel<D, CAUSAL, KIND, OUT, false>;
}

template <int D, int KIND, int OUT>
void pick_c(bool causal, bool drop, BwdFn& dkv, BwdFn& dq) {
  if (causal) pick_pair<D, true, KIND, OUT>(drop, dkv, dq);
  else pick_pair<D, false, KIND, OUT>(drop, dkv, dq);
}

template <int D, int KIND>
void pick_o(bool f32, bool causal, bool drop, BwdFn& dkv, BwdFn& dq) {
  if (f32) pick_c<D, KIND, fa::OF32>(causal, drop, dkv, dq);
  else pick_c<D, KIND, KIND == fa::KBF16 ? fa::OBF16 : fa::OF16>(causal, drop, dkv, dq);
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

constexpr int64_t kMaxDim = int64_t(1) << 40;

int64_t bwd_rows(int64_t B, int64_t H, int64_t Sq) { return B * H * ((Sq + 31) / 32 * 32); }

}  // namespace

static fa_status_t bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                       int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D, float scale, fa_mask_t mask,
                       float keep_prob, uint64_t seed, uint64_t rng_off, fa_dtype_t in_dtype,
                       fa_dtype_t grad_dtype, void* workspace, int64_t workspace_size,
                       hipStream_t stream);

extern "C" {

int64_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t Sq) {
  if (B < 1 || H < 1 || Sq < 1 || B > kMaxDim || H > kMaxDim || Sq > kMaxDim) return -1;
  if (B * H > kMaxDim / Sq) return -1;
  const int64_t rows = bwd_rows(B, H, Sq);
  // lse2 and Delta are read with 32-bit byte offsets from the workspace start
  if (rows * 8 > INT32_MAX) return -1;
  return rows * 8;
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D, float scale, fa_mask_t mask,
                   fa_dtype_t in_dtype, fa_dtype_t grad_dtype, void* workspace,
                   int64_t workspace_size, hipStream_t stream) {
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Sq, Sk, D, scale, mask, 1.0f, 0, 0,
                    in_dtype, grad_dtype, workspace, workspace_size, stream);
}

fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                           float scale, fa_mask_t mask, float keep_prob, uint64_t seed,
                           uint64_t offset, fa_dtype_t in_dtype, fa_dtype_t grad_dtype,
                           void* workspace, int64_t workspace_size, hipStream_t stream) {
  if (!(keep_prob > 0.f && keep_prob <= 1.f)) return FA_ERR_UNSUPPORTED_DROPOUT;
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Sq, Sk, D, scale, mask, keep_prob,
                    seed, offset, in_dtype, grad_dtype, workspace, workspace_size, stream);
}

}  // extern "C"

static fa_status_t bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                       int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D, float scale, fa_mask_t mask,
                       float keep_prob, uint64_t seed, uint64_t rng_off, fa_dtype_t in_dtype,
                       fa_dtype_t grad_dtype, void* workspace, int64_t workspace_size,
                       hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || H_kv < 1 || Sq < 1 || Sk < 1) return FA_ERR_BAD_SHAPE;
  if (B > kMaxDim || H > kMaxDim || Sq > kMaxDim || Sk > kMaxDim) return FA_ERR_BAD_SHAPE;
  if (H % H_kv != 0) return FA_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
  if (grad_dtype != in_dtype && grad_dtype != FA_F32) return FA_ERR_UNSUPPORTED_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL_TOP_LEFT && mask != FA_MASK_CAUSAL_BOTTOM_RIGHT)
    return FA_ERR_UNSUPPORTED_MASK;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;
  const int64_t need = fa_bwd_workspace_size(B, H, Sq);
  if (need < 0) return FA_ERR_BAD_SHAPE;
  if (B * H_kv > kMaxDim / Sk) return FA_ERR_BAD_SHAPE;
  const int64_t nqb = (Sq + 127) / 128, nkb = (Sk + 127) / 128;
  if (B * H * nqb > INT32_MAX || B * H_kv * nkb > INT32_MAX) return FA_ERR_BAD_SHAPE;
  // one K/V row pitch must fit the 32-bit per-lane load offsets
  if (D * 2 * 128 > INT32_MAX) return FA_ERR_BAD_SHAPE;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
                       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
  if (al & 15) return FA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;
  if (!workspace || workspace_size < need) return FA_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 255) return FA_ERR_MISALIGNED;
  const int64_t ge = grad_dtype == FA_F32 ? 4 : 2;
  const int64_t nq = B * H * Sq * D * 2, nkv = B * H_kv * Sk * D * 2, nl = B * H * Sq * 4;
  const int64_t gq = B * H * Sq * D * ge, gkv = B * H_kv * Sk * D * ge;
  const void* in_p[6] = {q, k, v, o, dout, lse};
  const int64_t in_n[6] = {nq, nkv, nkv, nq, nq, nl};
  void* out_p[4] = {dq, dk, dv, workspace};
  const int64_t out_n[4] = {gq, gkv, gkv, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out_p[i], out_n[i], in_p[j], in_n[j])) return FA_ERR_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out_p[i], out_n[i], out_p[j], out_n[j])) return FA_ERR_ALIASING;
  }

  BwdParams p;
  p.q = (const char*)q;
  p.k = (const char*)k;
  p.v = (const char*)v;
  p.o = (const char*)o;
  p.dout = (const char*)dout;
  p.lse = lse;
  p.dq = (char*)dq;
  p.dk = (char*)dk;
  p.dv = (char*)dv;
  const int64_t rows = bwd_rows(B, H, Sq);
  p.lse2 = (float*)workspace;
  p.delta = (float*)workspace + rows;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Sqp = (Sq + 31) / 32 * 32;
  p.k_ss = D;
  p.v_ss = D;
  p.moff = mask == FA_MASK_CAUSAL_BOTTOM_RIGHT ? Sk - Sq : 0;
  p.H = (int32_t)H;
  p.Hkv = (int32_t)H_kv;
  p.scale = scale;
  p.c = fmaxf(fabsf(scale) * fa::kLog2e, FLT_MIN);
  p.negate = scale < 0.f;
  const bool drop = keep_prob != 1.0f;
  p.seed = seed;
  p.rng_off = rng_off;
  p.keep_thr = 0;
  p.inv_keep = 1.f;
  if (drop) {
    const long t = lrintf(keep_prob * 65536.0f);
    p.keep_thr = (uint32_t)(t < 1 ? 1 : (t > 65535 ? 65535 : t));
    p.inv_keep = 1.0f / keep_prob;
  }
  const bool causal = mask != FA_MASK_NONE;
  const bool f32 = grad_dtype == FA_F32;

  PreFn pre;
  BwdFn dkv, dq_fn;
  if (D == 64) {
    if (in_dtype == FA_BF16) { pre = fa::fa_bwd_pre_kernel<64, fa::KBF16>; pick_o<64, fa::KBF16>(f32, causal, drop, dkv, dq_fn); }
    else { pre = fa::fa_bwd_pre_kernel<64, fa::KF16>; pick_o<64, fa::KF16>(f32, causal, drop, dkv, dq_fn); }
  } else {
    if (in_dtype == FA_BF16) { pre = fa::fa_bwd_pre_kernel<128, fa::KBF16>; pick_o<128, fa::KBF16>(f32, causal, drop, dkv, dq_fn); }
    else { pre = fa::fa_bwd_pre_kernel<128, fa::KF16>; pick_o<128, fa::KF16>(f32, causal, drop, dkv, dq_fn); }
  }
  const int rpb = 256 / (int)(D / 8);
  hipLaunchKernelGGL(pre, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream, p, rows);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  // causal grids with at least 8 key/value heads: blocks by work across
  // each XCD's heads; pairing of long and short blocks when the groups
  // divide over the XCDs and the grid is resident (two workgroups per CU)
  const bool lpt = causal && B * H_kv >= 8;
  p.qrem = (int32_t)((B * H_kv) % 8);
  BwdParams pk = p;
  pk.nblk = (int32_t)nkb;
  pk.total = (int32_t)(B * H_kv * nkb);
  pk.qmajor = lpt ? 1 : 0;
  pk.qsnake = lpt && p.qrem == 0 && pk.total <= 512;
  hipLaunchKernelGGL(dkv, dim3((unsigned)pk.total), dim3(256), 0, stream, pk);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  BwdParams pq = p;
  pq.nblk = (int32_t)nqb;
  pq.total = (int32_t)(B * H * nqb);
  pq.qmajor = lpt ? (int32_t)(H / H_kv) : 0;
  pq.qsnake = lpt && p.qrem == 0 && pq.total <= 512;
  hipLaunchKernelGGL(dq_fn, dim3((unsigned)pq.total), dim3(256), 0, stream, pq);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
