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
//    per lane), through a ring of two buffers (the next tile in flight while
//    one is computed on), in an XOR-swizzled layout chosen per head dim; K
//    is read with ds_read_b128, V with the transposing ds_read_b64_tr_b16,
//    which delivers V^T fragments directly.
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
#include <type_traits>
#include <mutex>

#include "fa_mi355x.h"

#include "fa_device.h"

namespace fa {

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
  int32_t H;            // query heads
  int32_t Hkv;          // key/value heads (divides H; query head h uses h / (H / Hkv))
  // element strides of (batch, head, row): q and o share theirs, k and v
  // theirs (BNSD: H*S*D, S*D, D; BSHD: S*H*D, D, H*D); rows are contiguous
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t moff;         // causal: key j is visible to query i iff j <= i + moff
  // variable lengths: cumulative query and key lengths of the B sequences
  // ([B+1] each, device); nullptr for fixed lengths Sq, Sk. Rows of sequence
  // b start at row cu[b] of the packed tensors; Sq, Sk are then the packed
  // totals, lse is [H, total_q], and a bottom-right diagonal (br) is placed
  // per sequence.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t br;
  int32_t xcd_unit;     // > 0: launch-order groups dealt round-robin to the XCDs
  // causal launch order (xcd_lpt): qmajor > 0 orders the blocks by length
  // across each XCD's heads, in groups of qmajor heads sharing K/V; qrem
  // groups beyond a multiple of 8 go first; qsnake pairs long and short
  // blocks when the whole grid is resident
  int32_t qmajor, qrem, qsnake;
  // dropout: the keep test of key j for query row i of query head bh uses
  // Philox4x64-10 keyed by (seed, rng_off); a kept P is scaled by inv_keep
  uint64_t seed, rng_off;
  uint32_t keep_thr;    // a 16-bit draw below this keeps its P
  float inv_keep;
  float scale_log2;     // |scale| * log2(e)
  int32_t negate;       // scale < 0: Q fragments are negated (exact)
  // split-KV only: key-tile ranges per query block, partial results
  int32_t nsplit;       // ranges per query block (workgroups per block)
  float* ws_o;          // [nsplit][B*H*Sq][D] fp32, O of each range (normalised)
  float* ws_lse;        // [nsplit][B*H*Sq] fp32, lse of each range (-inf: no key)
};


// One workgroup: NW waves, BM = 32 * NW query rows, 32 per wave.
// Keys and values stream through LDS in tiles of BN rows, in a ring of NB
// buffers per tensor: the loads of tile j+NB-1 are issued right after the
// barrier that opens tile j and waited for before the barrier that opens
// tile j+NB-1, so they have NB-1 tiles of compute to arrive. Per tile each
// wave runs S^T = K Q^T, the mask, the online softmax and O^T += V^T P^T;
// several waves share each SIMD, so one wave's matrix products overlap
// another's softmax.
//
// fp8 (e4m3fn) inputs: S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4
// on the codes (unit block scales); the per-tensor descales of Q and K are
// folded into the softmax scale. O^T += V^T P^T runs in fp16: P is fp16 as
// for fp16 inputs, and the V codes, read transposed from LDS with
// ds_read_b64_tr_b8, are converted exactly to fp16 (every e4m3fn value is
// an fp16 value); the descale of V multiplies O in the epilogue.
//
// Dropout (DROP): P is computed and summed into l as without it; the P
// multiplied by V has each dropped entry set to 0, and the epilogue scales O
// by 1/keep_prob. The keep test of the 16 keys a lane holds in a 32-key tile
// j (registers r = 0..15: key 32j + 8*(r/4) + 4*hl + r%4) uses one Philox
// call with counter (2j + hl, query row, b*H + h, 0): 16-bit value r of the
// output (bits 16r .. 16r+15, word 0 lowest) below keep_thr keeps key r.
template <int D, int BN_, int NW_, int NB_, bool CAUSAL, int KIND, int OUT, bool SPLIT,
          bool DROP = false>
struct FwdTile {
  static constexpr bool F8 = (KIND == KFP8);
  static constexpr int MK = F8 ? KF16 : KIND;     // type of the P.V product
  static constexpr int BN = BN_;                  // keys per tile
  static constexpr int NW = NW_;                  // waves per workgroup
  static constexpr int NB = NB_;                  // K/V tile buffers (ring)
  static constexpr int BM = 32 * NW;              // query rows per workgroup
  static constexpr int ES = F8 ? 1 : 2;           // bytes per input element
  static constexpr int RB = D * ES;               // bytes per K/V row
  static constexpr int C = RB / 16;               // 16-byte chunks per K/V row
  static constexpr int TILE = BN * RB;            // bytes of one K or V tile buffer
  static constexpr int NDS = F8 ? D / 64 : D / 16;  // k-steps of S = K Q^T
  static constexpr int NKB = BN / 32;             // 32-key blocks per tile
  static constexpr int NDB = D / 32;              // 32-wide head-dim blocks of O
  static constexpr int NST = BN / 16;             // 16-key steps of O += V^T P^T
  static constexpr int NCH = BN * C;              // 16-byte chunks per tile
  static constexpr int LWAVES = NCH / 64 < NW ? NCH / 64 : NW;   // waves that issue the HBM->LDS loads
  static constexpr int NT = 64 * LWAVES;          // lanes that issue them
  static constexpr int LOADS = NCH / NT;          // loads per lane, tile and tensor
  static constexpr bool SPLIT_P = (KIND == KBF16);  // bf16: P = hi + lo
  static constexpr int SMEM = 2 * NB * TILE;      // K ring, then V ring
  static_assert(NB >= 2 && (NB - 2) * 2 * LOADS < 64, "ring depth: the loads in flight must fit the vmcnt field");
  static_assert(NCH % 64 == 0 && NCH % NT == 0 && (NT & (NT - 1)) == 0, "tile must split evenly over the lanes");
  static_assert((NT / C) % 16 == 0, "swizzle period must divide the rows per load");
  static_assert(!DROP || (NKB == 1 && !SPLIT), "dropout: one 32-key block per tile, no split");

  typedef typename std::conditional<F8, i32x8, u32x4>::type qfrag_t;

  const Params& p;
  uint32_t lds0;                    // LDS byte address of the tile buffers
  int tid, lane, wave, hl, l32;
  int bh, ntiles, jlast;           // tiles 0 .. ntiles-1 of this block (split-KV: of its range)
  int split;
  int64_t Sq, Sk, q0, qw0, qrow;
  const char* khead;
  const char* vhead;
  int kpitch;                       // bytes from one K/V row to the next in HBM
  int64_t qbase;                    // element offset of this (batch, head) in q and o
  int64_t lse_base;                 // index of this block's row 0 in lse
  int64_t moff;                     // causal: key j is visible to query i iff j <= i + moff
  bool idle;                        // variable lengths: no row of this block exists
  float c;                          // softmax scale in log2 units (fp8: times dq * dk)

  qfrag_t qf[NDS];
  uint32_t kaddr0;                  // K fragment address of k-step 0 (buffer 0)
  uint32_t vaddr[NDB][F8 ? 1 : 2];  // V transposing-read addresses (buffer 0, step 0)
  uint32_t goff_k, goff_v;          // this lane's byte offsets in a full tile (first load)
  f32x16 acc_o[NDB];
  float m_run, l_run;
  float neg_m;                      // -m_run, or 0 while m_run = -inf (the exponent's offset)
  float thr;                        // m_run + the slack of the last move_ref (see there)
  int jmask;                        // tiles j >= jmask need the key mask
  int jfull;                        // tiles j < jfull lie wholly below Sk

  __device__ __forceinline__ FwdTile(const Params& pp, char* sm) : p(pp) {
    lds0 = (uint32_t)(uintptr_t)LDS_PTR(char, sm);
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hl = lane >> 5;
    l32 = lane & 31;
    int t = p.xcd_unit ? xcd_deal(blockIdx.x, p.xcd_unit) : xcd_remap(blockIdx.x, p.total);
    split = 0;
    if constexpr (SPLIT) {
      split = t % p.nsplit;          // the ranges of a block are adjacent, on one XCD
      t /= p.nsplit;
    }
    bh = t / p.nqb;
    int qb = t - bh * p.nqb;
    if constexpr (CAUSAL) {
      qb = p.nqb - 1 - qb;   // longest rows first
      if (!SPLIT && p.qmajor > 0) {   // blocks by length across each XCD's heads
        int rank;
        xcd_lpt(blockIdx.x, p.total, p.nqb, p.qmajor, p.qrem, p.qsnake != 0, bh, rank);
        qb = p.nqb - 1 - rank;
      }
    }
    Sq = p.Sq;
    Sk = p.Sk;
    q0 = (int64_t)qb * BM;
    moff = p.moff;
    idle = false;
    {
      const int b = bh / p.H;
      const int h = bh - b * p.H;
      const int kvh = h / (p.H / p.Hkv);
      int64_t koff = (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
      qbase = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
      lse_base = (int64_t)bh * Sq;
      if (p.cu_q) {
        // sequence b: its start and length, clamped into the packed tensors
        // (malformed arrays give undefined results, never a stray access)
        int64_t qs = p.cu_q[b], qe = p.cu_q[b + 1];
        int64_t ks = p.cu_k[b], ke = p.cu_k[b + 1];
        qs = qs < 0 ? 0 : (qs > Sq ? Sq : qs);
        qe = qe < qs ? qs : (qe > Sq ? Sq : qe);
        ks = ks < 0 ? 0 : (ks > Sk ? Sk : ks);
        ke = ke < ks ? ks : (ke > Sk ? Sk : ke);
        lse_base = (int64_t)h * Sq + qs;      // lse [H, total_q]
        qbase = qs * p.q_ss + (int64_t)h * p.q_sh;
        koff = ks * p.k_ss + (int64_t)kvh * p.k_sh;
        Sq = qe - qs;
        Sk = ke - ks;
        if (p.br) moff = Sk - Sq;
        idle = q0 >= Sq;                      // past this sequence's last row
      }
      khead = p.k + koff * ES;
      vhead = p.v + koff * ES;
      kpitch = (int)(p.k_ss * ES);
    }
    if (idle) return;
    qw0 = q0 + wave * 32;
    qrow = qw0 + l32;
    c = p.scale_log2;
    if constexpr (F8) c = fmaxf(c * (*p.descale_q) * (*p.descale_k), FLT_MIN);

    int64_t kend = Sk;
    if constexpr (CAUSAL) {
      kend = (q0 + BM + moff) < Sk ? (q0 + BM + moff) : Sk;
      if (kend < 0) kend = 0;   // every row of the block lies above the diagonal
    }
    ntiles = (int)((kend + BN - 1) / BN);
    if constexpr (SPLIT) {
      // range `split` of nsplit near-equal ranges of the block's tiles
      // (empty when there are more ranges than tiles). The range becomes a
      // problem of its own: its first key is key 0 (K and V start there,
      // Sk and the causal offset move with it), so the loop below is the
      // one of a whole block.
      const int per = (ntiles + p.nsplit - 1) / p.nsplit;
      int jb = split * per;
      const int je = jb + per < ntiles ? jb + per : ntiles;
      if (jb > je) jb = je;
      const int64_t k0 = (int64_t)jb * BN;
      khead += k0 * kpitch;
      vhead += k0 * kpitch;
      const int64_t kmax = (int64_t)je * BN;
      Sk = (kmax < Sk ? kmax : Sk) - k0;
      moff -= k0;
      ntiles = je - jb;
    }
    jlast = ntiles - 1;   // last tile this wave needs
    if constexpr (CAUSAL) {
      const int64_t last_key = qw0 + 31 + moff;   // last key any row of this wave sees
      const int64_t jl = last_key < 0 ? -1 : last_key / BN;
      jlast = jl < jlast ? (int)jl : jlast;
    }
    if (qw0 >= Sq) jlast = -1;   // all rows of this wave lie past Sq
    {
      // the first tile that reaches past Sk or, causal, past the diagonal
      // of one of this wave's rows; the tiles before it need no mask
      int64_t jm = Sk / BN;
      if constexpr (CAUSAL) {
        const int64_t x = qw0 + moff + 1 - BN;
        const int64_t jc = x < 0 ? 0 : x / BN + 1;
        jm = jc < jm ? jc : jm;
      }
      jmask = __builtin_amdgcn_readfirstlane(jm < ntiles ? (int)jm : ntiles);
      const int64_t jf = Sk / BN;
      jfull = __builtin_amdgcn_readfirstlane(jf < ntiles ? (int)jf : ntiles);
    }

    // Q fragments (B operand of S^T = K Q^T), kept in registers; rows past
    // Sq read the last row (their results are never stored). Negative
    // scales negate Q (exact).
    const char* qrowp = p.q + (qbase + (qrow < Sq ? qrow : Sq - 1) * p.q_ss) * ES;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if constexpr (F8) {
        // 32 consecutive codes: d = 64*ds + 32*hl .. +32
        const u32x4 a = *(const u32x4*)(qrowp + 64 * ds + 32 * hl);
        const u32x4 b = *(const u32x4*)(qrowp + 64 * ds + 32 * hl + 16);
        const uint32_t sg = p.negate ? 0x80808080u : 0u;
        qf[ds] = (i32x8){(int)(a[0] ^ sg), (int)(a[1] ^ sg), (int)(a[2] ^ sg), (int)(a[3] ^ sg),
                         (int)(b[0] ^ sg), (int)(b[1] ^ sg), (int)(b[2] ^ sg), (int)(b[3] ^ sg)};
      } else {
        qf[ds] = *(const u32x4*)(qrowp + (ds * 16 + hl * 8) * 2);
        if (p.negate) qf[ds] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      }
    }

    // K (ds_read_b128): row l32 of a 32-key block. 16-bit: logical chunk
    // 2*ds + hl; fp8: chunks 4*ds + 2*hl and the next one (32 codes).
    // Chunk c of row r is stored at chunk c ^ swz_k(r).
    // The k-step part of the chunk index (ds * KSTEP) shares no bit with the
    // rest, so the address of k-step ds is kaddr0 ^ (ds * KSTEP * 16).
    kaddr0 = lds0 + l32 * RB + (((F8 ? 2 * hl : hl) ^ swz_k<RB>(l32)) << 4);
    // V, 16-bit (ds_read_b64_tr_b16): within each 16-lane group, lane i
    // supplies row 16*step + 4*hl + (i/4) [+8 for the second read] and
    // head-dim columns 32*db + 16*((lane/16)&1) + 4*(i%4) .. +4; the read
    // returns to lane i the four keys of its head-dim column.
    // V, fp8 (ds_read_b64_tr_b8): lane i supplies row 16*step +
    // 8*((i/2)/4) + 4*hl + (i/2)%4 and columns 32*db + 16*((lane/16)&1) +
    // 8*(i%2) .. +8; the read returns to lane i the eight keys of its column.
    // Both key orders match the accumulator layout of S^T. The swizzle of
    // a row only depends on its index mod 16, so one address per (db, read)
    // serves every step.
    const int gi = lane & 15;
    const int dh = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if constexpr (F8) {
        const int j = gi >> 1;
        const int r = 8 * (j >> 2) + 4 * hl + (j & 3);
        const int ch = 2 * db + dh;
        vaddr[db][0] = lds0 + NB * TILE + r * RB + ((ch ^ swz_v<RB, true>(r)) << 4) + 8 * (gi & 1);
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 4 * hl + (gi >> 2) + 8 * e;
          const int col = 32 * db + 16 * dh + 4 * (gi & 3);
          vaddr[db][e] = lds0 + NB * TILE + r * RB + (((col >> 3) ^ swz_v<RB, false>(r)) << 4) + (col & 7) * 2;
        }
      }
    }
    // HBM->LDS (lanes 0..NT-1 only): lane chunk i*NT + tid of a tile; one
    // wave writes a contiguous KiB of LDS per instruction, so the swizzle is
    // applied to the global source offset. Load i covers rows r + i*NT/C;
    // the swizzle only depends on the row mod 16, so every load of a lane
    // uses the same chunk and the offsets differ by i*(NT/C) rows.
    {
      const int r = (tid & (NT - 1)) / C;
      const int pc = tid % C;
      goff_k = (uint32_t)(r * kpitch + ((pc ^ swz_k<RB>(r)) << 4));
      goff_v = (uint32_t)(r * kpitch + ((pc ^ swz_v<RB, F8>(r)) << 4));
    }

#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] = (f32x16){};
    m_run = -INFINITY;
    neg_m = 0.f;
    thr = -INFINITY;
    l_run = 0.f;
  }

  // ---- HBM -> LDS: tile j of K or V into buffer buf (lanes 0..NT-1) ----
  // Rows past Sk read the last row (only the final tile can have them).
  template <bool IS_V>
  __device__ __forceinline__ void load_one(int j, int buf) {
    if (wave >= LWAVES) return;   // only the first LWAVES waves issue loads
    const int64_t row0 = (int64_t)j * BN;
    const char* base = (IS_V ? vhead : khead) + row0 * kpitch;
    const uint32_t dst = lds0 + (IS_V ? NB + buf : buf) * TILE + wave * 64 * 16;
    const uint32_t goff = IS_V ? goff_v : goff_k;
    if (j < jfull) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dma16(base + (int64_t)i * (NT / C) * kpitch, goff, dst + i * NT * 16);
    } else {
      const int rmax = (int)(Sk - 1 - row0);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int pidx = i * NT + tid;
        const int r = pidx / C;
        const int pc = pidx % C;
        const int rr = r < rmax ? r : rmax;
        const int sw = IS_V ? swz_v<RB, F8>(r) : swz_k<RB>(r);
        dma16(base, (uint32_t)(rr * kpitch + ((pc ^ sw) << 4)), dst + i * NT * 16);
      }
    }
  }
  __device__ __forceinline__ void load_tile(int j, int buf) {
    load_one<false>(j, buf);
    load_one<true>(j, buf);
  }

  // V^T fragment (A operand of O^T += V^T P^T) of 16-key step st, head-dim block db
  __device__ __forceinline__ u32x4 v_frag(uint32_t voff, int st, int db) {
    if constexpr (F8) {
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(uintptr_t)(vaddr[db][0] + voff + st * 16 * RB));
      // codes 0..3 of a dword hold keys 4w .. 4w+3 of this lane's column
      uint32_t r[4];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)x[w], 1.0f, false);
        const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)x[w], 1.0f, true);
        __builtin_memcpy(&r[2 * w], &lo, 4);
        __builtin_memcpy(&r[2 * w + 1], &hi, 4);
      }
      return (u32x4){r[0], r[1], r[2], r[3]};
    } else {
      u32x2 y[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const fp16x4_tr x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (__attribute__((address_space(3))) fp16x4_tr*)(uintptr_t)(vaddr[db][e] + voff + st * 16 * RB));
        __builtin_memcpy(&y[e], &x, 8);
      }
      return (u32x4){y[0][0], y[0][1], y[1][0], y[1][1]};
    }
  }

  // ---- S^T = K Q^T for one tile (buffer BUF) ----
  // The K fragments are read first (read_k) and the MFMA chain runs once
  // they are in registers (mma_s), so the LDS latency is paid once per
  // tile instead of once per MFMA.
  typedef typename std::conditional<F8, i32x8, u32x4>::type kfrag_t;

  static constexpr int KSTEP = F8 ? 4 : 2;   // chunks per k-step

  template <int BUF>
  __device__ __forceinline__ void read_k(kfrag_t (&kf)[NKB][NDS]) {
    constexpr uint32_t koff = BUF * TILE;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const uint32_t ka = kaddr0 ^ (uint32_t)(ds * KSTEP * 16);
        if constexpr (F8) {
          const u32x4 a = lds_load<u32x4>(ka + koff + kb * 32 * RB);
          const u32x4 b = lds_load<u32x4>((ka ^ 16) + koff + kb * 32 * RB);
          kf[kb][ds] = (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        } else {
          kf[kb][ds] = lds_load<u32x4>(ka + koff + kb * 32 * RB);
        }
      }
    }
  }

  __device__ __forceinline__ void mma_s(const kfrag_t (&kf)[NKB][NDS], f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        if constexpr (F8)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[kb][ds], qf[ds], s[kb], 0, 0, 0, 127, 0, 127);
        else
          s[kb] = mfma32<KIND>(kf[kb][ds], qf[ds], s[kb]);
      }
    }
  }

  template <int BUF>
  __device__ __forceinline__ void gemm_s(f32x16 (&s)[NKB]) {
    kfrag_t kf[NKB][NDS];
    read_k<BUF>(kf);
    mma_s(kf, s);
    constexpr int KPIPE = 4;
    if constexpr (!F8 && NKB == 1 && NDS > KPIPE) {
      // KPIPE reads in flight ahead of the MFMA that consumes them.
      __builtin_amdgcn_sched_group_barrier(0x100, KPIPE, 0);
#pragma unroll
      for (int i = 0; i < NDS - KPIPE; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KPIPE, 0);
    }
  }

  // ---- mask, online softmax and P for tile j ----
  __device__ __forceinline__ void mask_s(int j, f32x16 (&s)[NKB]) {
    const int64_t kt0 = (int64_t)j * BN;
    // mask: keys past Sk, keys above the diagonal. key = kt0 + kb*32 +
    // 8*(r/4) + 4*hl + r%4 is dead if it is >= Sk or > this row's query:
    // compare the compile-time part with a per-lane limit.
    if (j >= jmask) {
      // keeps this a branch: full tiles (all but the last, or the diagonal
      // ones) then skip the compare-and-select on every score
      asm volatile("");
      const int64_t kv = Sk - kt0;
      int lim = kv < BN ? (int)kv : BN;
      if constexpr (CAUSAL) {
        int64_t qr = qrow + moff - kt0 + 1;
        if (qr < 0) qr = 0;
        lim = qr < lim ? (int)qr : lim;
      }
      lim -= 4 * hl;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3)) >= lim ? -INFINITY : s[kb][r];
    }
  }

  __device__ __forceinline__ void rescale_s(const f32x16 (&s)[NKB]) {
    // Online softmax (log2 domain) with a reference maximum m_run: P =
    // exp2(S*c - m_run), O and l accumulate relative to it, and moving it
    // rescales O and l by exp2(m_old - m_new). While a row has few
    // comparable keys (this lane's part of l below 4, in units of the
    // reference) the reference follows the running maximum exactly, so the
    // largest P is exactly 1 and carries no fp16 rounding error: with only
    // a few keys of similar weight, that error would not average out. After
    // that, a new maximum less than 2 above the reference keeps it (P then
    // stays below 4, its rounding stays relative), which skips the rescale
    // on most tiles of long rows.
    move_ref(max_cand(s));
  }

  // this tile's row maximum in log2 units (scaled by c)
  __device__ __forceinline__ float max_cand(const f32x16 (&s)[NKB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_max_halves(mx);
    return mx * c;
  }

  // Moves the reference when some row of the wave has a maximum mxc above
  // m_run + slack, slack (log2 units) = 2 once this lane's half of l is at
  // least 4 (it bounds the row's l from below), else 0. thr caches m_run +
  // slack as of the last call that entered the branch: l only grows in
  // between, so the cached slack is never larger than the current one and
  // the cheap test below lets through every tile the exact test would; the
  // exact test then decides, and refreshes thr.
  __device__ __forceinline__ void move_ref(float mxc) {
    if (__builtin_amdgcn_ballot_w64(mxc > thr) != 0) {
      const float m_cand = max_f32(m_run, mxc);
      const float slack = l_run >= 4.0f ? 2.0f : 0.0f;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + slack) != 0) {
        const float m_new = (m_cand == -INFINITY) ? 0.f : m_cand;   // no (-inf) - (-inf)
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
        m_run = m_cand;
        neg_m = -m_new;
      }
      thr = m_run + (l_run >= 4.0f ? 2.0f : 0.0f);
    }
  }

  // keep masks of this lane's 8 register pairs for tile j: value pair
  // (2q, 2q+1) is the q-th 32-bit half of the Philox output
  __device__ __forceinline__ void drop_masks(int j, uint32_t (&dm)[8]) {
    uint64_t c[4] = {(uint64_t)(2 * j + hl), (uint64_t)qrow, (uint64_t)bh, 0ull};
    philox4x64_10(c, p.seed, p.rng_off);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t w = (uint32_t)(c[q >> 1] >> (32 * (q & 1)));
      dm[q] = ((w & 0xffffu) < p.keep_thr ? 0x0000ffffu : 0u) | ((w >> 16) < p.keep_thr ? 0xffff0000u : 0u);
    }
  }

  __device__ __forceinline__ void exp_p(const f32x16 (&s)[NKB], u32x4 (&pf)[NST], u32x4 (&pl)[SPLIT_P ? NST : 1],
                                        const uint32_t (&dm)[8]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 f, g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * half + 2 * e;
          const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, neg_m));
          const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, neg_m));
          f[e] = pack2<MK>(x0, x1);
          l_run = add_pair<MK>(f[e], l_run);     // l sums the P that multiplies V
          if constexpr (SPLIT_P) {
            g[e] = pack2<MK>(x0 - unpack_lo<MK>(f[e]), x1 - unpack_hi<MK>(f[e]));
            l_run = add_pair<MK>(g[e], l_run);
          }
          if constexpr (DROP) {   // l keeps every P; V sees the kept ones
            f[e] &= dm[4 * half + e];
            if constexpr (SPLIT_P) g[e] &= dm[4 * half + e];
          }
        }
        pf[kb * 2 + half] = f;
        if constexpr (SPLIT_P) pl[kb * 2 + half] = g;
      }
    }
  }

  __device__ __forceinline__ void softmax(int j, f32x16 (&s)[NKB], u32x4 (&pf)[NST], u32x4 (&pl)[SPLIT_P ? NST : 1],
                                          const uint32_t (&dm)[8]) {
    mask_s(j, s);
    rescale_s(s);
    exp_p(s, pf, pl, dm);
  }

  // ---- O^T += V^T P^T for one tile (buffer BUF); the V fragments of step
  // st+1 are read while the MFMAs of step st run ----
  template <int BUF>
  __device__ __forceinline__ void read_v0(u32x4 (&v0)[NDB]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) v0[db] = v_frag(BUF * TILE, 0, db);
  }

  template <int BUF>
  __device__ __forceinline__ void gemm_pv(const u32x4 (&pf)[NST], const u32x4 (&pl)[SPLIT_P ? NST : 1],
                                          const u32x4 (&v0)[NDB]) {
    constexpr uint32_t voff = BUF * TILE;
    u32x4 vf[2][NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vf[0][db] = v0[db];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + 1 < NST) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf[(st + 1) & 1][db] = v_frag(voff, st + 1, db);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc_o[db] = mfma32<MK>(vf[st & 1][db], pf[st], acc_o[db]);
        if constexpr (SPLIT_P) acc_o[db] = mfma32<MK>(vf[st & 1][db], pl[st], acc_o[db]);
      }
    }
  }

  // ---- one tile: S, mask, online softmax, O += V^T P^T ----
  template <int BUF>
  __device__ __forceinline__ void tile(int j) {
    f32x16 s[NKB];
    u32x4 pf[NST];
    u32x4 pl[SPLIT_P ? NST : 1];
    uint32_t dm[8];
    if constexpr (DROP) drop_masks(j, dm);
    gemm_s<BUF>(s);
    // plain instances: the first 16-key step's V fragments are read before
    // the softmax, so their LDS latency runs during it (the split and
    // dropout instances have no registers to spare for them)
    constexpr bool EARLY_V = !SPLIT && !DROP;
    u32x4 v0[NDB];
    if constexpr (EARLY_V) read_v0<BUF>(v0);
    softmax(j, s, pf, pl, dm);
    if constexpr (!EARLY_V) read_v0<BUF>(v0);
    gemm_pv<BUF>(pf, pl, v0);
  }

  template <int BUF>
  __device__ __forceinline__ void step(int j) {
    // this wave's part of tile j has landed once at most the loads of the
    // younger tiles in flight (j+1 .. j+NB-2) are outstanding; the barrier
    // then makes the whole tile visible and frees buffer (j-1) % NB, last
    // read while computing tile j-1
    if (j + NB - 2 < ntiles) wait_loads<(NB - 2) * 2 * LOADS>();
    else wait_loads<0>();
    lds_barrier();
    if (j + NB - 1 < ntiles) load_tile(j + NB - 1, (BUF + NB - 1) % NB);
    // Causal: a wave whose rows all lie above this tile's first key has
    // nothing to add (all its scores here are masked).
    if (j > jlast) return;
    tile<BUF>(j);
  }

  // steps j+B .. j+NB-1 (tile j+b in buffer b); false
  // once past the last tile
  template <int B>
  __device__ __forceinline__ bool steps_from(int j) {
    if constexpr (B == NB) {
      return true;
    } else {
      if (j + B >= ntiles) return false;
      step<B>(j + B);
      return steps_from<B + 1>(j);
    }
  }

  __device__ __forceinline__ void run() {
    if (idle) return;   // uniform over the workgroup: no barrier is left waiting
    // tile j lives in buffer j % NB; tiles j+1 .. j+NB-1 are in flight
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
      if (i < ntiles) load_tile(i, i);
    for (int j = 0; j < ntiles; j += NB)
      if (!steps_from<0>(j)) break;
    store();
  }

  // ---- epilogue: O = O / l (fp8: times the V descale), lse = (m + log2 l) * ln 2 ----
  __device__ __forceinline__ void store() {
    const float l_tot = wave_sum_halves(l_run);
    if constexpr (SPLIT) {
      store_partial(l_tot);
      return;
    }
    // l = 0: the row sees no key (a diagonal shifted left of it); O = 0 and
    // lse = -inf by definition
    const bool any = l_tot > 0.f;
    float inv_l = any ? 1.f / l_tot : 0.f;
    if constexpr (F8) inv_l *= *p.descale_v;
    if constexpr (DROP) inv_l *= p.inv_keep;
    if (qrow >= Sq) return;
    char* orow = p.o + (qbase + qrow * p.q_ss) * (OUT == OF32 ? 4 : 2);
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
      p.lse[lse_base + qrow] = any ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
  }

  // split-KV epilogue: this range's O (normalised by its own l; fp8: times
  // the V descale) and lse, fp32; a row that saw no key in the range gets
  // O = 0 and lse = -inf, which the merge weighs by exp(-inf) = 0.
  __device__ __forceinline__ void store_partial(float l_tot) {
    if (qrow >= Sq) return;
    const bool any = l_tot > 0.f;
    float inv_l = any ? 1.f / l_tot : 0.f;
    if constexpr (F8) inv_l *= *p.descale_v;
    const int64_t rows = (int64_t)(p.total / p.nsplit / p.nqb) * Sq;   // B*H*Sq
    const int64_t r = (int64_t)split * rows + (int64_t)bh * Sq + qrow;
    float* orow = p.ws_o + r * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hl;
        *(f32x4*)(orow + d) = (f32x4){acc_o[db][4 * g + 0] * inv_l, acc_o[db][4 * g + 1] * inv_l,
                                      acc_o[db][4 * g + 2] * inv_l, acc_o[db][4 * g + 3] * inv_l};
      }
    }
    if (hl == 0)
      p.ws_lse[r] = any ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
};

// ---- split-KV merge: for each row, lse = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) * O_s over the nsplit ranges (a row whose
// ranges all saw no key keeps O = 0, lse = -inf). One lane per four
// head-dim entries of a row; memory-bound. ----
struct MergeParams {
  const float* ws_o;
  const float* ws_lse;
  char* o;
  float* lse;
  int64_t rows;         // B*H*Sq, in (batch, head, row) order
  int32_t nsplit;
  int32_t H;
  int64_t Sq;
  int64_t q_sb, q_sh, q_ss;   // element strides of o (as Params)
};

template <int D, int OUT>
__global__ __launch_bounds__(256) void fa_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;
  const int d = (int)(gid % TPR) * 4;
  if (row >= p.rows) return;
  float m = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) m = fmaxf(m, p.ws_lse[(int64_t)s * p.rows + row]);
  if (m == -INFINITY) m = 0.f;       // no key in any range: every weight below is 0
  float sum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.nsplit; ++s) {
    const int64_t r = (int64_t)s * p.rows + row;
    const float w = expf(p.ws_lse[r] - m);
    if (w == 0.f) continue;          // range without a key (its O is 0 anyway)
    sum += w;
    acc += w * *(const f32x4*)(p.ws_o + r * D + d);
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  acc *= inv;
  const int64_t bh = row / p.Sq, srow = row - bh * p.Sq;
  const int64_t b = bh / p.H, h = bh - b * p.H;
  const int64_t oel = b * p.q_sb + h * p.q_sh + srow * p.q_ss + d;
  if constexpr (OUT == OF32) {
    *(f32x4*)(p.o + oel * 4) = acc;
  } else {
    constexpr int PK = (OUT == OBF16) ? KBF16 : KF16;
    *(u32x2*)(p.o + oel * 2) = (u32x2){pack2<PK>(acc[0], acc[1]), pack2<PK>(acc[2], acc[3])};
  }
  if (d == 0) p.lse[row] = sum > 0.f ? m + logf(sum) : -INFINITY;
}

// Tiles in a ring of FA_NBUF buffers per tensor: two, 2 x 2 x 32 x D x 2
// bytes (32 KiB) for 32-key 16-bit tiles at D = 128. The loads of tile j+1
// then have the compute of tile j to arrive, which covers them: against a
// ring of three (48 KiB) two measured 0.2-0.7 % faster on every D = 128
// workload and 1.4 % on the dropout forward, same outputs bit for bit
// (deeper rings gave nothing either). At least three waves per SIMD, so the
// register budget is capped at a third of the file.
#ifndef FA_NBUF
#define FA_NBUF 2
#endif
// Waves per workgroup (32 query rows each): four, i.e. three workgroups per
// CU. (Causal D = 64 ran faster with 8-wave workgroups while each XCD took
// its heads one after the other; with the blocks ordered by length across
// the heads, 4-wave workgroups are 14 % faster there too. The tile code
// keeps any power-of-two wave count.)
__host__ __device__ constexpr int waves_for(int d, bool causal) { return 4; }
// Keys per tile: 64 where a K/V row is 128 bytes (fp8 at D=128, anything at
// D=64: the ring still leaves room for three workgroups per CU;
// measured 7.5 % faster on B1 H32 S8192 D128 fp8 causal, 8.5 % on B3 H12
// S4097 D64 causal, 17 % on B1 H8 S512 D64), 32 for 16-bit data at D=128
// (64 would leave one workgroup per CU).
__host__ __device__ constexpr int keys_for(int kind, int d) { return (kind == KFP8 || d == 64) ? 64 : 32; }
// 16-bit data at D = 64 (a 64-key tile is 8 KiB per tensor): always a ring
// of two buffers (32 KiB) and at most 128 VGPRs, so four workgroups can
// share a CU.
// Its LDS is dynamic and the host sizes it per launch: 32 KiB (four
// workgroups per CU) for grids of at least DYN_LDS_MIN_GRID workgroups, else
// 48 KiB, which keeps three per CU. Measured against the ring of three at
// three per CU (same outputs bit for bit): B4 H32 S4096 D64 fp16 2.4 %
// faster non-causal and 3.8 % causal at four per CU, B3 H12 S4097 D64
// causal (1188 workgroups) 4 % faster at three per CU and 0.6 % at four (the
// longest causal blocks run longer when four workgroups share a SIMD).
__host__ __device__ constexpr bool dyn_lds(int kind, int d) { return d == 64 && kind != KFP8; }
__host__ __device__ constexpr int nbuf_for(int kind, int d) { return dyn_lds(kind, d) ? 2 : FA_NBUF; }
__host__ __device__ constexpr int waves_per_simd(int kind, int d) { return dyn_lds(kind, d) ? 4 : 3; }
constexpr int DYN_LDS_SMEM = 2 * 2 * 64 * 64 * 2;       // two buffers of K and of V
constexpr int DYN_LDS_SMEM_3 = 48 * 1024;               // three workgroups per CU
constexpr int64_t DYN_LDS_MIN_GRID = 2048;

template <int D, bool CAUSAL, int KIND, int OUT, bool SPLIT>
__global__ __launch_bounds__(64 * waves_for(D, CAUSAL)) __attribute__((amdgpu_waves_per_eu(waves_per_simd(KIND, D)))) void fa_fwd_kernel(Params p) {
  using Blk = FwdTile<D, keys_for(KIND, D), waves_for(D, CAUSAL), nbuf_for(KIND, D), CAUSAL, KIND, OUT, SPLIT>;
  if constexpr (dyn_lds(KIND, D)) {
    static_assert(Blk::SMEM == DYN_LDS_SMEM, "host and kernel disagree on the LDS size");
    extern __shared__ __attribute__((aligned(1024))) char dyn_smem[];
    Blk blk(p, dyn_smem);
    blk.run();
  } else {
    __shared__ __attribute__((aligned(1024))) char smem[Blk::SMEM];
    Blk blk(p, smem);
    blk.run();
  }
}

// The forward with dropout: a separate instance (the keep test adds one
// Philox call per lane and tile, so it gets the register budget of two
// waves per SIMD).
template <int D, bool CAUSAL, int KIND, int OUT>
__global__ __launch_bounds__(64 * waves_for(D, CAUSAL)) __attribute__((amdgpu_waves_per_eu(2))) void fa_fwd_drop_kernel(Params p) {
  using Blk = FwdTile<D, 32, waves_for(D, CAUSAL), FA_NBUF, CAUSAL, KIND, OUT, false, true>;
  __shared__ __attribute__((aligned(1024))) char smem[Blk::SMEM];
  Blk blk(p, smem);
  blk.run();
}

}  // namespace fa

// ============================== host side ==============================

namespace {

using fa::Params;
typedef void (*KernelFn)(Params);
typedef void (*MergeFn)(fa::MergeParams);

template <int D, bool CAUSAL, int KIND, int OUT, bool SPLIT>
KernelFn pick() {
  return fa::fa_fwd_kernel<D, CAUSAL, KIND, OUT, SPLIT>;
}

template <int D, int KIND, int OUT, bool SPLIT>
KernelFn pick_c(bool causal) {
  return causal ? pick<D, true, KIND, OUT, SPLIT>() : pick<D, false, KIND, OUT, SPLIT>();
}

template <int KIND, int OUT, bool SPLIT>
KernelFn pick_d(int64_t D, bool causal) {
  return D == 64 ? pick_c<64, KIND, OUT, SPLIT>(causal) : pick_c<128, KIND, OUT, SPLIT>(causal);
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

// Everything fa_fwd and fa_fwd_splitkv check before any HIP call, and the
// launch parameters that follow from the arguments.
struct Call {
  Params p;
  int nw;               // waves per workgroup
  int64_t BH, nqb, D;
  bool causal;
  fa_dtype_t in_dtype, o_dtype;
  int64_t nq, nk, no, nl;   // byte sizes of q, k (and v), o, lse
};

// dynamic LDS bytes of a forward launch of `grid` workgroups (0: the
// instance's LDS is static)
unsigned fwd_lds_bytes(const Call& c, int64_t grid) {
  const int kind = c.in_dtype == FA_FP8_E4M3 ? fa::KFP8 : (c.in_dtype == FA_BF16 ? fa::KBF16 : fa::KF16);
  if (!fa::dyn_lds(kind, (int)c.D)) return 0;
  return grid >= fa::DYN_LDS_MIN_GRID ? fa::DYN_LDS_SMEM : fa::DYN_LDS_SMEM_3;
}

fa_status_t check_call(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                       fa_layout_t layout, float scale, fa_mask_t mask, float keep_prob,
                       fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                       const float* descale_q, const float* descale_k, const float* descale_v,
                       Call& c) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return FA_ERR_BAD_SHAPE;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0 || H > INT32_MAX) return FA_ERR_BAD_SHAPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL_TOP_LEFT && mask != FA_MASK_CAUSAL_BOTTOM_RIGHT)
    return FA_ERR_UNSUPPORTED_MASK;
  const int causal = mask != FA_MASK_NONE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  const bool ok_pair = (in_dtype == FA_F16 && (o_dtype == FA_F16 || o_dtype == FA_F32)) ||
                       (in_dtype == FA_BF16 && (o_dtype == FA_BF16 || o_dtype == FA_F32)) ||
                       (in_dtype == FA_FP8_E4M3 && (o_dtype == FA_F16 || o_dtype == FA_F32));
  if (!ok_pair) return FA_ERR_UNSUPPORTED_DTYPE;
  if (in_dtype == FA_FP8_E4M3) {
    if (!descale_q || !descale_k || !descale_v) return FA_ERR_NULL_POINTER;
    if (((uintptr_t)descale_q | (uintptr_t)descale_k | (uintptr_t)descale_v) & 3) return FA_ERR_MISALIGNED;
  }
  if (layout != FA_LAYOUT_BNSD && layout != FA_LAYOUT_BSHD) return FA_ERR_UNSUPPORTED_LAYOUT;
  if (keep_prob != 1.0f) return FA_ERR_UNSUPPORTED_DROPOUT;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;

  // sizes: element counts must fit comfortably in 64-bit byte offsets and
  // the grid in 31 bits.
  const int64_t lim = (int64_t)1 << 40;
  if (B > lim / H || Sq > lim || Sk > lim) return FA_ERR_BAD_SHAPE;
  const int64_t BH = B * H;
  if (BH > (lim / Sq) || BH > (lim / Sk)) return FA_ERR_BAD_SHAPE;
  const int nw = fa::waves_for((int)D, causal != 0);
  const int64_t nqb = (Sq + 32 * nw - 1) / (32 * nw);   // 32 * nw query rows per workgroup
  if (nqb > INT32_MAX || BH * nqb > INT32_MAX) return FA_ERR_BAD_SHAPE;

  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;

  const int64_t ie = dtype_size(in_dtype), oe = dtype_size(o_dtype);
  c.nq = BH * Sq * D * ie;
  c.nk = B * Hkv * Sk * D * ie;
  c.no = BH * Sq * D * oe;
  c.nl = BH * Sq * 4;
  if (overlaps(o, c.no, q, c.nq) || overlaps(o, c.no, k, c.nk) || overlaps(o, c.no, v, c.nk) ||
      overlaps(lse, c.nl, q, c.nq) || overlaps(lse, c.nl, k, c.nk) || overlaps(lse, c.nl, v, c.nk) ||
      overlaps(o, c.no, lse, c.nl))
    return FA_ERR_ALIASING;

  Params& p = c.p;
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
  p.nsplit = 1;
  p.ws_o = nullptr;
  p.ws_lse = nullptr;
  p.H = (int32_t)H;
  p.Hkv = (int32_t)Hkv;
  if (layout == FA_LAYOUT_BNSD) {
    p.q_sb = H * Sq * D; p.q_sh = Sq * D; p.q_ss = D;
    p.k_sb = Hkv * Sk * D; p.k_sh = Sk * D; p.k_ss = D;
  } else {   // BSHD
    p.q_sb = Sq * H * D; p.q_sh = D; p.q_ss = H * D;
    p.k_sb = Sk * Hkv * D; p.k_sh = D; p.k_ss = Hkv * D;
  }
  // the row offsets of one K/V tile (up to 64 rows) must fit the 32-bit
  // per-lane load offsets
  if (p.k_ss * ie * 64 > INT32_MAX) return FA_ERR_BAD_SHAPE;
  p.moff = mask == FA_MASK_CAUSAL_BOTTOM_RIGHT ? Sk - Sq : 0;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.br = mask == FA_MASK_CAUSAL_BOTTOM_RIGHT;
  p.xcd_unit = 0;
  // causal: q-block-major order inside each XCD when there are at least 8
  // key/value head groups; the resident-grid variant when they divide
  // evenly over the XCDs and every workgroup fits on the 256 CUs at once
  // (three 4-wave or one 8-wave workgroup per CU)
  p.qmajor = (causal && B * Hkv >= 8) ? (int32_t)(H / Hkv) : 0;
  p.qrem = (int32_t)((B * Hkv) % 8);
  p.qsnake = p.qrem == 0 && BH * nqb <= 256 * (nw == 4 ? 3 : 1);
  p.seed = 0;
  p.rng_off = 0;
  p.keep_thr = 0;
  p.inv_keep = 1.f;
  c.nw = nw;
  c.BH = BH;
  c.nqb = nqb;
  c.D = D;
  c.causal = causal != 0;
  c.in_dtype = in_dtype;
  c.o_dtype = o_dtype;
  return FA_OK;
}

template <bool SPLIT>
KernelFn pick_kernel(const Call& c) {
  if (SPLIT) {   // partial results are fp32 whatever the output type
    if (c.in_dtype == FA_F16) return pick_d<fa::KF16, fa::OF32, SPLIT>(c.D, c.causal);
    if (c.in_dtype == FA_BF16) return pick_d<fa::KBF16, fa::OF32, SPLIT>(c.D, c.causal);
    return pick_d<fa::KFP8, fa::OF32, SPLIT>(c.D, c.causal);
  }
  if (c.in_dtype == FA_F16)
    return (c.o_dtype == FA_F32) ? pick_d<fa::KF16, fa::OF32, false>(c.D, c.causal) : pick_d<fa::KF16, fa::OF16, false>(c.D, c.causal);
  if (c.in_dtype == FA_BF16)
    return (c.o_dtype == FA_F32) ? pick_d<fa::KBF16, fa::OF32, false>(c.D, c.causal) : pick_d<fa::KBF16, fa::OBF16, false>(c.D, c.causal);
  return (c.o_dtype == FA_F32) ? pick_d<fa::KFP8, fa::OF32, false>(c.D, c.causal) : pick_d<fa::KFP8, fa::OF16, false>(c.D, c.causal);
}

template <int KIND, int OUT>
KernelFn pick_drop_d(int64_t D, bool causal) {
  if (D == 64) return causal ? fa::fa_fwd_drop_kernel<64, true, KIND, OUT> : fa::fa_fwd_drop_kernel<64, false, KIND, OUT>;
  return causal ? fa::fa_fwd_drop_kernel<128, true, KIND, OUT> : fa::fa_fwd_drop_kernel<128, false, KIND, OUT>;
}

KernelFn pick_drop(const Call& c) {
  if (c.in_dtype == FA_F16)
    return (c.o_dtype == FA_F32) ? pick_drop_d<fa::KF16, fa::OF32>(c.D, c.causal) : pick_drop_d<fa::KF16, fa::OF16>(c.D, c.causal);
  if (c.in_dtype == FA_BF16)
    return (c.o_dtype == FA_F32) ? pick_drop_d<fa::KBF16, fa::OF32>(c.D, c.causal) : pick_drop_d<fa::KBF16, fa::OBF16>(c.D, c.causal);
  return (c.o_dtype == FA_F32) ? pick_drop_d<fa::KFP8, fa::OF32>(c.D, c.causal) : pick_drop_d<fa::KFP8, fa::OF16>(c.D, c.causal);
}

MergeFn pick_merge(const Call& c) {
  if (c.o_dtype == FA_F32) return c.D == 64 ? fa::fa_merge_kernel<64, fa::OF32> : fa::fa_merge_kernel<128, fa::OF32>;
  if (c.o_dtype == FA_BF16) return c.D == 64 ? fa::fa_merge_kernel<64, fa::OBF16> : fa::fa_merge_kernel<128, fa::OBF16>;
  return c.D == 64 ? fa::fa_merge_kernel<64, fa::OF16> : fa::fa_merge_kernel<128, fa::OF16>;
}

constexpr int kMaxSplits = 256;

// Key ranges per query block when the caller passes num_splits = 0. A split
// pays for its fp32 partial results, the merge and a second launch only
// where the plain grid leaves most of the GPU idle: blocks for fewer than
// half the resident slots (three 4-wave workgroups per CU) and key ranges
// of at least 16 32-key tiles. Then it aims at one full round of the slots.
// Measured on fp16 D = 128: B1 H4 S8192 (256 blocks) 200 -> 158 us at 3
// ranges, causal 172 -> 114; B2 H2 S4096 (128 blocks) 95 -> 59 at 6; B1 H1
// S32768 641 -> 540 at 3; with 512 blocks (B1 H16 S4096, B2 H16 S2048
// causal) every split was slower than the plain kernel.
int auto_splits(int64_t BH, int64_t nqb, int64_t Sk, int nw) {
  const int64_t resident = 256 * (nw == 4 ? 3 : 1);
  const int64_t base = BH * nqb;
  if (2 * base > resident) return 1;
  int64_t s = (resident + base - 1) / base;
  const int64_t by_tiles = ((Sk + 31) / 32) / 16;
  if (s > by_tiles) s = by_tiles;
  if (s > 64) s = 64;
  return s < 1 ? 1 : (int)s;
}

int64_t workspace_bytes(int64_t BH, int64_t Sq, int64_t D, int nsplit) {
  if (nsplit <= 1) return 0;
  const int64_t o_bytes = (int64_t)nsplit * BH * Sq * D * 4;
  return ((o_bytes + 255) / 256) * 256 + (int64_t)nsplit * BH * Sq * 4;
}

}  // namespace

// Workspace of fa_fwd_splitkv_noalloc: a static device array, held by every
// GPU the library runs on until the process ends. In host code `scratch` is
// a host-side stand-in; its device address comes from hipGetSymbolAddress,
// once per device (with that device current), and only that address is
// handed to kernels.
static constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, which must be the
// device of `stream`.
fa_status_t scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
    if (sdev != dev) return FA_ERR_SCRATCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return FA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
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
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_UNSUPPORTED_MASK: return "FA_ERR_UNSUPPORTED_MASK";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH";
  }
  return "FA_ERR_UNKNOWN";
}

fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                      fa_layout_t layout, float scale, fa_mask_t mask, float keep_prob,
                      fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                      const float* descale_q, const float* descale_k, const float* descale_v,
                      int num_splits, void* workspace, int64_t workspace_size,
                      hipStream_t stream) {
  Call c;
  const fa_status_t st = check_call(q, k, v, o, lse, B, H, H_kv, Sq, Sk, D, layout, scale, mask,
                                    keep_prob, in_dtype, o_dtype, descale_q, descale_k, descale_v, c);
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_BAD_SHAPE;
  const int ns = num_splits ? num_splits : auto_splits(c.BH, c.nqb, Sk, c.nw);
  if (c.BH * c.nqb * ns > INT32_MAX) return FA_ERR_BAD_SHAPE;
  if ((c.BH * Sq * (D / 4) + 255) / 256 > INT32_MAX) return FA_ERR_BAD_SHAPE;   // merge grid
  const int64_t need = workspace_bytes(c.BH, Sq, D, ns);
  if (need > 0) {
    if (!workspace || workspace_size < need) return FA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255) return FA_ERR_MISALIGNED;
    if (overlaps(workspace, need, q, c.nq) || overlaps(workspace, need, k, c.nk) ||
        overlaps(workspace, need, v, c.nk) || overlaps(workspace, need, o, c.no) ||
        overlaps(workspace, need, lse, c.nl))
      return FA_ERR_ALIASING;
  }
  if (ns == 1) {   // one range: the plain kernel writes O and lse directly
    hipLaunchKernelGGL(pick_kernel<false>(c), dim3((unsigned)c.p.total), dim3(64 * c.nw), fwd_lds_bytes(c, c.p.total), stream, c.p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  Params p = c.p;
  p.nsplit = ns;
  p.total = (int32_t)(c.BH * c.nqb * ns);
  p.ws_o = (float*)workspace;
  const int64_t o_bytes = (int64_t)ns * c.BH * Sq * D * 4;
  p.ws_lse = (float*)((char*)workspace + ((o_bytes + 255) / 256) * 256);
  hipLaunchKernelGGL(pick_kernel<true>(c), dim3((unsigned)p.total), dim3(64 * c.nw), fwd_lds_bytes(c, p.total), stream, p);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  fa::MergeParams m;
  m.ws_o = p.ws_o;
  m.ws_lse = p.ws_lse;
  m.o = (char*)o;
  m.lse = lse;
  m.rows = c.BH * Sq;
  m.nsplit = ns;
  m.H = (int32_t)H;
  m.Sq = Sq;
  m.q_sb = c.p.q_sb;
  m.q_sh = c.p.q_sh;
  m.q_ss = c.p.q_ss;
  const int64_t lanes = m.rows * (D / 4);
  hipLaunchKernelGGL(pick_merge(c), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream, m);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                   fa_layout_t layout, float scale, int causal, float keep_prob,
                   fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                   const float* descale_q, const float* descale_k, const float* descale_v,
                   hipStream_t stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, Sq, Sk, D, layout, scale,
                   causal ? FA_MASK_CAUSAL_TOP_LEFT : FA_MASK_NONE, keep_prob, in_dtype, o_dtype,
                   descale_q, descale_k, descale_v, 1, nullptr, 0, stream);
}

int64_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                      int causal, int num_splits) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || (D != 64 && D != 128)) return -1;
  if (num_splits < 0 || num_splits > kMaxSplits) return -1;
  const int64_t lim = (int64_t)1 << 40;
  if (B > lim / H || Sq > lim || Sk > lim || B * H > lim / Sq || B * H > lim / Sk) return -1;
  const int nw = fa::waves_for((int)D, causal != 0);
  const int64_t nqb = (Sq + 32 * nw - 1) / (32 * nw);
  const int ns = num_splits ? num_splits : auto_splits(B * H, nqb, Sk, nw);
  return workspace_bytes(B * H, Sq, D, ns);
}

fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                           fa_layout_t layout, float scale, int causal, float keep_prob,
                           fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                           const float* descale_q, const float* descale_k, const float* descale_v,
                           int num_splits, void* workspace, int64_t workspace_size,
                           hipStream_t stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, Sq, Sk, D, layout, scale,
                   causal ? FA_MASK_CAUSAL_TOP_LEFT : FA_MASK_NONE, keep_prob, in_dtype, o_dtype,
                   descale_q, descale_k, descale_v, num_splits, workspace, workspace_size, stream);
}

fa_status_t fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                   fa_layout_t layout, float scale, int causal, float keep_prob,
                                   fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                                   const float* descale_q, const float* descale_k,
                                   const float* descale_v, int num_splits, hipStream_t stream) {
  // the same checks as fa_fwd_ex, before any HIP call
  Call c;
  const fa_status_t st = check_call(q, k, v, o, lse, B, H, H, Sq, Sk, D, layout, scale,
                                    causal ? FA_MASK_CAUSAL_TOP_LEFT : FA_MASK_NONE, keep_prob,
                                    in_dtype, o_dtype, descale_q, descale_k, descale_v, c);
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_BAD_SHAPE;
  const int ns = num_splits ? num_splits : auto_splits(c.BH, c.nqb, Sk, c.nw);
  const int64_t need = workspace_bytes(c.BH, Sq, D, ns);
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const fa_status_t s2 = scratch_address(stream, &ws);
    if (s2 != FA_OK) return s2;
  }
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, Sq, Sk, D, layout, scale,
                   causal ? FA_MASK_CAUSAL_TOP_LEFT : FA_MASK_NONE, keep_prob, in_dtype, o_dtype,
                   descale_q, descale_k, descale_v, ns, ws, need > 0 ? kScratchBytes : 0, stream);
}

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int64_t B, int64_t H, int64_t H_kv, int64_t total_q, int64_t total_k,
                          int64_t max_seqlen_q, int64_t D, float scale, fa_mask_t mask,
                          float keep_prob, fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                          const float* descale_q, const float* descale_k, const float* descale_v,
                          hipStream_t stream) {
  // the packed tensors are checked as one sequence-major batch of total_q
  // query and total_k key rows
  Call c;
  const fa_status_t st = check_call(q, k, v, o, lse, 1, H, H_kv, total_q, total_k, D, FA_LAYOUT_BSHD,
                                    scale, mask, keep_prob, in_dtype, o_dtype, descale_q, descale_k,
                                    descale_v, c);
  if (st != FA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL_POINTER;
  if (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3) return FA_ERR_MISALIGNED;
  if (B < 1 || B > INT32_MAX / 2 || max_seqlen_q < 1 || max_seqlen_q > total_q) return FA_ERR_BAD_SHAPE;
  const int64_t nqb = (max_seqlen_q + 32 * c.nw - 1) / (32 * c.nw);
  if (B * H * nqb > INT32_MAX) return FA_ERR_BAD_SHAPE;
  Params p = c.p;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.moff = 0;
  p.nqb = (int32_t)nqb;
  p.total = (int32_t)(B * H * nqb);
  p.qmajor = 0;
  p.qsnake = 0;
  p.qrem = 0;
  // sequences differ in work: deal each key/value head's blocks (else each
  // head's) round-robin to the 8 XCDs so they stay balanced and the blocks
  // sharing K/V still share one XCD's L2
  if ((B * H_kv) % 8 == 0)
    p.xcd_unit = (int32_t)((H / H_kv) * nqb);
  else if ((B * H) % 8 == 0)
    p.xcd_unit = (int32_t)nqb;
  hipLaunchKernelGGL(pick_kernel<false>(c), dim3((unsigned)p.total), dim3(64 * c.nw), fwd_lds_bytes(c, p.total), stream, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                           fa_layout_t layout, float scale, fa_mask_t mask, float keep_prob,
                           uint64_t seed, uint64_t offset, fa_dtype_t in_dtype,
                           fa_dtype_t o_dtype, const float* descale_q, const float* descale_k,
                           const float* descale_v, hipStream_t stream) {
  if (!(keep_prob > 0.f && keep_prob <= 1.f)) return FA_ERR_UNSUPPORTED_DROPOUT;
  Call c;
  const fa_status_t st = check_call(q, k, v, o, lse, B, H, H_kv, Sq, Sk, D, layout, scale, mask,
                                    1.0f, in_dtype, o_dtype, descale_q, descale_k, descale_v, c);
  if (st != FA_OK) return st;
  if (keep_prob == 1.f) {   // nothing is dropped
    hipLaunchKernelGGL(pick_kernel<false>(c), dim3((unsigned)c.p.total), dim3(64 * c.nw), fwd_lds_bytes(c, c.p.total), stream, c.p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  Params p = c.p;
  long t = lrintf(keep_prob * 65536.0f);
  p.keep_thr = (uint32_t)(t < 1 ? 1 : (t > 65535 ? 65535 : t));
  p.inv_keep = 1.0f / keep_prob;
  p.seed = seed;
  p.rng_off = offset;
  hipLaunchKernelGGL(pick_drop(c), dim3((unsigned)p.total), dim3(64 * c.nw), 0, stream, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
