// Split-K decode of absorbed MLA for 128 query rows per work-group over an
// e4m3 cache with per-token fp32 scales (gfx950).
//
// The method and the division of a tile's work between the four waves are
// those of decode_wide.hip (scores: wave w owns query rows 32w .. 32w+31;
// P . V: wave w owns latent columns (DC/4) w .. for all 128 rows, P through
// LDS, one tile late).  The difference is the tile image: the e4m3 bytes
// stay in LDS as copied (row pair m = bytes 16m .. 16m+15 of the latent, then
// of the RoPE key, token t at byte (32 m + t) 16), so there is no bf16 image,
// no decode pass over the tile and no second barrier per tile:
//   scores: the e4m3 MFMA (32x32x64 f8f6f4) takes the key bytes as copied
//     (two 16-byte LDS reads per lane and 64-deep k-step) against the query
//     split once into two e4m3 parts under a per-row power-of-two scale
//     (QF8 below);
//   V^T fragment (P . V A operand, bf16 MFMA): column c, the eight tokens of
//     the P fragment it meets: one 8-bit transposing LDS read (each lane i
//     of a 16-lane group receives byte i % 8 of the words of lanes i / 8,
//     i / 8 + 2, ..., i / 8 + 14, which address those tokens' halves of the
//     column's row pair), four e4m3 -> bf16 conversions (exact: every e4m3
//     value is a bf16 value).
// The keys' scale multiplies the raw scores and the values' scale is carried
// by P (WideSoftmax<true>).  A staged tile is half a bf16 image's bytes, so
// two tiles are kept in flight; their scales come with them by DMA.  Copy
// lanes past a sequence's length re-read its first record and scale.
#include <type_traits>

#include "decode_common.h"
#include "mla_device.h"
#include "mla_kernels.h"
#include "split_plan.h"
#include "tile_ops.h"
#include "wide_common.h"

namespace mla {
namespace {

template <int DC>
struct F8Wide {
  using Gm = Geo<DC>;
  using F = Fp8Geo<DC>;
  static constexpr int NW = 4, ROWS = 32 * NW, NBW = Gm::NB / NW;
  static constexpr int AHEAD = 2;                    // tiles in flight
  static constexpr int NBUF = AHEAD + 2;             // + the tile scored and the one in P . V
  static constexpr int RAW = F::BYTES;               // one staged tile
  static constexpr int NQ = (F::NINS + NW - 1) / NW;  // row-pair copies per wave per tile
  static constexpr int NI = NQ + 1;                  // + the scales
  static constexpr int PB = NW * 2 * 1024;           // P of one tile
  static_assert(Gm::KS == F::NP, "one score k-step per row pair");
};

// 4-byte global -> LDS copy (lane i writes LDS `lds` + 4 i), as lds_dma16.
__device__ __forceinline__ void lds_dma4(const void* base_any, uint32_t voff, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(base_any);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(base), "s"(dst)
      : "memory", "m0");
}

// The copy of one tile: instruction q < NQ moves row pairs 2 ins, 2 ins + 1
// (ins = q NW + w; the last round's surplus waves repeat an instruction of
// that round, writing the same bytes, so that every wave issues the same
// number of copies and one vmcnt value fits all); q = NQ moves the tile's
// 32 scales (lanes 32 .. 63 repeat them into the slot's unused half).
template <int DC>
struct F8Dma {
  using X = F8Wide<DC>;
  const char* run;
  int64_t rope_off;
  const float* scl;
  uint32_t lane_off, sc_off, raw_lds, sc_lds;
  int w;
  bool active;
  __device__ __forceinline__ void issue(int q) const {
    if (!active) return;
    if (q < X::NQ) {
      int ins = q * X::NW + w;
      if (ins >= Fp8Geo<DC>::NINS) ins -= X::NW * X::NQ - Fp8Geo<DC>::NINS;
      const int m0 = 2 * ins;  // pairs m0, m0 + 1 never straddle the latent and the RoPE key
      const int64_t off = m0 < Geo<DC>::GC / 2 ? (int64_t)m0 * 16 : rope_off + (int64_t)(m0 - Geo<DC>::GC / 2) * 16;
      lds_dma16(run + off, lane_off, uniform(raw_lds + ins * 1024));
    } else {
      lds_dma4(scl, sc_off, sc_lds);
    }
  }
};

// Eight e4m3 values (bytes 0..7 of lo | hi) as bf16, exactly.
__device__ __forceinline__ bf16x8 e4m3x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) i32x2* lds_i32x2_ptr;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short s16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// The query block as operands of the e4m3 score product (the 32x32x64
// f8f6f4 MFMA, whose A operand is the K fragment exactly as copied): lane
// (row r = lane % 32, k-half kh = lane / 32) holds, for 64-deep k-step j,
// the 32 consecutive values 64 j + 32 kh .. +31 of query row r in two e4m3
// parts with one power-of-two scale 2^s per row (the same on both of its
// lanes):  hi = e4m3(q / 2^s),  lo = e4m3((q - hi 2^s) / 2^(s - 4)).
// s puts the row's largest magnitude in [128, 256), inside e4m3's range;
// hi keeps 4 significant bits of each value and lo the next 4, so hi + lo
// carry a bf16 query to about 2^-8 of each value.  The MFMA multiplies each
// part by its scale (E8M0 bytes sh, sl), so both products accumulate into one
// chain.
template <int DC>
struct QF8 {
  static constexpr int NJ = (DC + 64) / 64;
  i32x8 hi[NJ], lo[NJ];
  int sh, sl;
};

template <int DC>
__device__ __forceinline__ void make_qf8(const bf16x8 (&qf)[Geo<DC>::KS], QF8<DC>& q) {
  constexpr int KS = Geo<DC>::KS, NJ = QF8<DC>::NJ;
  static_assert(KS == 4 * NJ, "four 16-deep k-steps per 64-deep step");
  // the row's largest magnitude (bf16 magnitudes order as integers), over
  // this lane's values and its partner lane's (lane ^ 32)
  uint32_t mx = 0;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 u = __builtin_bit_cast(uint4, qf[ks]);
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = max(mx, max(d[i] & 0x7fffu, (d[i] >> 16) & 0x7fffu));
  }
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
  // exponent e of the largest magnitude (bf16 bits 14..7); s = e - 7, kept
  // where both 2^s and 2^(s - 4) are normal fp32 values
  const int e = (int)(mx >> 7) - 127;
  const int sc = max(e - 7, -122);
  q.sh = sc + 127;
  q.sl = sc + 123;
  const float f_hi = __builtin_bit_cast(float, (uint32_t)(sc + 127) << 23);
  const float f_lo = __builtin_bit_cast(float, (uint32_t)(sc + 123) << 23);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    // this lane's 32 values: k-steps 4j + 2kh and 4j + 2kh + 1, both halves.
    // Lane r holds half 0 of every k-step and lane r + 32 half 1; the swap
    // gives the low lane the partner's half 1 of k-steps 4j, 4j + 1 and the
    // high lane the partner's half 0 of k-steps 4j + 2, 4j + 3.
    const uint4 a0 = __builtin_bit_cast(uint4, qf[4 * j]), a2 = __builtin_bit_cast(uint4, qf[4 * j + 2]);
    const uint4 a1 = __builtin_bit_cast(uint4, qf[4 * j + 1]), a3 = __builtin_bit_cast(uint4, qf[4 * j + 3]);
    const uint32_t x0[4] = {a0.x, a0.y, a0.z, a0.w}, x2[4] = {a2.x, a2.y, a2.z, a2.w};
    const uint32_t x1[4] = {a1.x, a1.y, a1.z, a1.w}, x3[4] = {a3.x, a3.y, a3.z, a3.w};
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto p02 = __builtin_amdgcn_permlane32_swap(x0[i], x2[i], false, false);
      const auto p13 = __builtin_amdgcn_permlane32_swap(x1[i], x3[i], false, false);
      v[i] = p02[0];       // values 0 .. 7
      v[4 + i] = p02[1];   // values 8 .. 15
      v[8 + i] = p13[0];   // values 16 .. 23
      v[12 + i] = p13[1];  // values 24 .. 31
    }
    int h[8], l[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      s16x2 hb = {0, 0};
      hb = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hb, __builtin_bit_cast(bf16x2, v[2 * m]), f_hi, false);
      hb = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hb, __builtin_bit_cast(bf16x2, v[2 * m + 1]), f_hi, true);
      h[m] = __builtin_bit_cast(int, hb);
      const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)h[m], f_hi, false);
      const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)h[m], f_hi, true);
      const float y0 = __builtin_bit_cast(float, v[2 * m] << 16) - b0[0];
      const float y1 = __builtin_bit_cast(float, v[2 * m] & 0xffff0000u) - b0[1];
      const float y2 = __builtin_bit_cast(float, v[2 * m + 1] << 16) - b1[0];
      const float y3 = __builtin_bit_cast(float, v[2 * m + 1] & 0xffff0000u) - b1[1];
      s16x2 lb = {0, 0};
      lb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lb, y0, y1, f_lo, false);
      lb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lb, y2, y3, f_lo, true);
      l[m] = __builtin_bit_cast(int, lb);
    }
    q.hi[j] = i32x8{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
    q.lo[j] = i32x8{l[0], l[1], l[2], l[3], l[4], l[5], l[6], l[7]};
  }
}

// The scaled e4m3 score MFMA in inline asm, so that it stays where it is
// placed between the copy instructions, with the hazard handling of the
// bf16 chain helpers (s_nop 1 before each MFMA; the last one carries the
// wait states a VALU read of its result needs).  sa, sb: E8M0 scale bytes.
__device__ __forceinline__ void mf8_first(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(acc)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void mf8_acc(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(acc)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void mf8_last(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile(
      "s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(acc)
      : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// S^T = K . Q^T of one staged tile: per 64-deep k-step j, lane (token t,
// k-half kh) reads its 32 key bytes (row pairs 4 j + 2 kh and 4 j + 2 kh + 1
// of token t) and two scaled MFMAs add K . hi and K . lo, with the next
// tile's copy spread over the steps.
template <int DC, class Pre = NoPre>
__device__ __forceinline__ f32x16 score_f8(const char* tb, const QF8<DC>& q, const F8Dma<DC>& dma, Pre&& pre = Pre{}) {
  constexpr int NJ = QF8<DC>::NJ, PD = 2, NI = F8Wide<DC>::NI;
  static_assert(NJ >= NI, "at most one copy instruction per k-step");
  const int lane = opaque_lane();
  const char* kb = tb + (64 * (lane >> 5) + (lane & 31)) * 16;
  auto kread = [&](int j) {
    const uint4 x = *(const uint4*)(kb + j * 2048);
    const uint4 y = *(const uint4*)(kb + j * 2048 + 512);
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };
  i32x8 kr[NJ];
#pragma unroll
  for (int j = 0; j < PD; ++j) kr[j] = kread(j);
  constexpr int kOne = 127;  // E8M0 2^0: the keys are used as stored
  f32x16 s;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j + PD < NJ) kr[j + PD] = kread(j + PD);
#pragma unroll
    for (int c = 0; c < NI; ++c)
      if ((c * NJ) / NI == j) dma.issue(c);
    if (j == NJ - 4) pre.load();  // the lagged P . V's first operands, eight MFMAs ahead of it
    if (j == 0) mf8_first(s, kr[j], q.hi[j], kOne, q.sh);
    else mf8_acc(s, kr[j], q.hi[j], kOne, q.sh);
    if (j + 1 < NJ) mf8_acc(s, kr[j], q.lo[j], kOne, q.sl);
    else mf8_last(s, kr[j], q.lo[j], kOne, q.sl);
  }
  __builtin_amdgcn_sched_barrier(0);
  return s;
}

// The V^T fragment of column block nb, k-half j of a staged tile: lane
// (G = lane / 16, i = lane % 16) gets column 32 nb + 16 (G % 2) + i of
// tokens 16 j + 4 (G / 2) + {0, 1, 2, 3, 8, 9, 10, 11}, the token order of
// the P fragments (the score MFMA's output layout, which P keeps).
__device__ __forceinline__ bf16x8 v_frag_f8(const char* vb, int nb, int j) {
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_ptr)(lds_void_ptr)(vb + nb * 1024 + j * 256));
  return e4m3x8((uint32_t)r[0], (uint32_t)r[1]);
}

// P . V of one staged tile for this wave's column blocks over all four row
// blocks (the order of pv_rows), with the softmax steps of the next tile
// between the column blocks.  Source lane (G, s) of a transposing read
// addresses bytes 8 (s % 2) .. +7 of row pair 2 nb + G % 2 of token
// 16 j + 4 (G / 2) + e % 4 + 8 (e / 4), e = s / 2 (result byte e of the
// receiving lanes).
// The no-op publication hook of pv_f8.
struct NoPublish {
  __device__ __forceinline__ void operator()() const {}
};

template <int DC>
struct F8PvOperands {
  static constexpr int NBW = Geo<DC>::NB / 4;
  const char* vb;
  const char* pb;
  int w;
  bf16x8 pf[4][2];
  bf16x8 c0, c1;
  __device__ __forceinline__ F8PvOperands(const char* tb, const char* pb_, int w_) : pb(pb_), w(w_) {
    const int lane = opaque_lane();
    const int G = lane >> 4, s = lane & 15;
    const int e = s >> 1;
    vb = tb + (32 * (G & 1) + 4 * (G >> 1) + (e & 3) + 8 * (e >> 2)) * 16 + 8 * (s & 1);
  }
  // P of all four row blocks and the first column block's V (read by the
  // score chain before its end, so that the first P . V MFMA finds them).
  __device__ __forceinline__ void load() {
    const int lane = opaque_lane();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int j = 0; j < 2; ++j) pf[rb][j] = *(const bf16x8*)(pb + (rb * 2 + j) * 1024 + lane * 16);
    c0 = v_frag_f8(vb, w * NBW, 0);
    c1 = v_frag_f8(vb, w * NBW, 1);
  }
};

template <int DC, bool STEPS, class SM, class Pub = NoPublish>
__device__ __forceinline__ void pv_f8(const F8PvOperands<DC>& op, f32x16 (&O)[4][Geo<DC>::NB / 4], SM& sm,
                                      const Pub& pub = Pub{}) {
  constexpr int NBW = Geo<DC>::NB / 4;
  const char* vb = op.vb;
  const int w = op.w;
  // softmax steps per column block, front-loaded (the last block gets none)
  // so that the softmax's tail and the publication of its results (pub)
  // run under the last block's MFMAs
  constexpr int SPB = (SM::STEPS + NBW - 2) / (NBW - 1);
  bf16x8 c0 = op.c0, c1 = op.c1;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    bf16x8 n0 = c0, n1 = c1;
    if (cb + 1 < NBW) {
      n0 = v_frag_f8(vb, w * NBW + cb + 1, 0);
      n1 = v_frag_f8(vb, w * NBW + cb + 1, 1);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      O[rb][cb] = mfma32(c0, op.pf[rb][0], O[rb][cb]);
      O[rb][cb] = mfma32(c1, op.pf[rb][1], O[rb][cb]);
    }
    if constexpr (STEPS) {
#pragma unroll
      for (int j = 0; j < SPB; ++j)
        if (cb * SPB + j < SM::STEPS) sm.step(cb * SPB + j);
      if (cb * SPB < SM::STEPS && (cb + 1) * SPB >= SM::STEPS) pub();
    }
    c0 = n0;
    c1 = n1;
  }
}

template <int DC>
__global__ void __launch_bounds__(256)
    decode_f8_kernel(DecodeParams p, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table) {
  using X = F8Wide<DC>;
  using Gm = Geo<DC>;
  constexpr int NW = X::NW, ROWS = X::ROWS, NBW = X::NBW, NBUF = X::NBUF, RAW = X::RAW, AHEAD = X::AHEAD;
  constexpr int NI = X::NI, PB = X::PB;
  constexpr int KST = DC / 32;            // query k-steps staged through LDS (half the latent)
  constexpr int CPR = 2 * KST;            // staged 16-byte chunks per row
  constexpr int SROW = CPR * 16;          // staged bytes per row
  constexpr int RPI = 1024 / SROW;        // rows per copy instruction

  __shared__ __attribute__((aligned(1024))) char raw[NBUF * RAW];
  __shared__ __attribute__((aligned(1024))) char qstg[NW * 32 * SROW];
  __shared__ __attribute__((aligned(1024))) char pbuf[2 * PB];
  __shared__ __attribute__((aligned(16))) float tscale[NBUF][2 * kTile];
  __shared__ __attribute__((aligned(16))) float alph[2][ROWS];
  __shared__ __attribute__((aligned(16))) int rflag[2][NW];
  __shared__ float fin_l[ROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware placement (as in decode_wide_kernel).
  int u = blockIdx.x;
  if ((gridDim.x & 7) == 0) u = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int g = u / p.RG, rg = u % p.RG;

  int b = -1, t0 = 0, t1 = 0, L = 0;
  with_plan(seq_lens, p.B, p.P, lane, [&](const auto& pl) {
    int s_b = 0;
    if (g < pl.total) pl.locate_slot(g, lane, b, s_b);
    if (b >= 0) {
      t0 = (g - s_b) * pl.W;
      t1 = min(t0 + pl.W, pl.tiles(b, lane));
      L = pl.length(b);
    }
  });
  b = uniform(b);
  if (b < 0) return;
  t0 = uniform(t0);
  const int n = uniform(t1) - t0;  // tiles of this part (>= 1)
  L = uniform(L);
  const int32_t* bt = block_table + (int64_t)b * p.bt_stride;
  const int rowbase = rg * ROWS;
  const uint32_t raw_lds = lds_offset(raw);

  // The copy of part tile t from page `page` (lane-derived values recomputed
  // per tile rather than kept live).
  auto make_dma = [&](int t, int page, bool active) {
    const TileSrc s = tile_src(p, page, t0 + t, L);
    const int ol = opaque_lane();
    const int tok = (ol & 31) < s.nv ? (ol & 31) : 0;
    return F8Dma<DC>{s.run, p.rope_off, p.kv_scale + s.page_slot,
                     (uint32_t)tok * (uint32_t)p.token_stride + 16u * (uint32_t)(ol >> 5), 4u * (uint32_t)tok,
                     raw_lds + (t % NBUF) * RAW, lds_offset(tscale[t % NBUF]), w, active};
  };

  // ---- prologue: the pages of tiles 0 .. AHEAD, the query block (half
  // staged through LDS as in decode_wide_kernel), tiles 0 and 1.
  const int qrow0 = rowbase + 32 * w;
  const char* qseq = (const char*)(p.q_lat + (int64_t)b * p.R * DC);
  char* stg = qstg + w * 32 * SROW;
  const int page0 = tile_page_load(p, bt, t0);
  const int page1 = n > 1 ? tile_page_load(p, bt, t0 + 1) : 0;
  int page_pf = AHEAD < n ? tile_page_load(p, bt, t0 + AHEAD) : 0;
  {
    const int ol = opaque_lane();
    const int rr = ol / CPR, cs = ol % CPR;
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int r = j * RPI + rr;
      const int rg_ = min(qrow0 + r, p.R - 1);            // rows past R re-read row R-1 (discarded)
      const int chunk = cs ^ (r & (CPR - 1) & 15);
      lds_dma16(qseq, (uint32_t)(rg_ * DC * 2 + chunk * 16), lds_offset(stg + j * 1024));
    }
  }
  bf16x8 qf[Gm::KS];
  const int ln0 = opaque_lane();
  const int qrow = qrow0 + (ln0 & 31);
  {
    const int qr_ = min(qrow, p.R - 1);
    const bf16x8* ql = (const bf16x8*)(p.q_lat + ((int64_t)b * p.R + qr_) * DC + 8 * (ln0 >> 5));
    const bf16x8* qr = (const bf16x8*)(p.q_rope + ((int64_t)b * p.R + qr_) * 64 + 8 * (ln0 >> 5));
#pragma unroll
    for (int ks = KST; ks < DC / 16; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
    for (int ks = DC / 16; ks < Gm::KS; ++ks) qf[ks] = qr[2 * (ks - DC / 16)];
  }
  {
    const F8Dma<DC> d0 = make_dma(0, uniform(page0), true);
#pragma unroll
    for (int q = 0; q < NI; ++q) d0.issue(q);
  }
  if (n > 1) {
    const F8Dma<DC> d1 = make_dma(1, uniform(page1), true);
#pragma unroll
    for (int q = 0; q < NI; ++q) d1.issue(q);
  }
#pragma unroll
  for (int ks = KST; ks < Gm::KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  asm volatile("" ::"v"(page_pf));
  // everything but tile 1's copy (the last NI instructions, when it exists)
  if (n > 1) vm_wait<NI>();
  else vm_wait<0>();
  block_sync();  // tile 0, its scales and the staged query are in LDS for every wave
  {
    const int col_ = ln0 & 31, hf = ln0 >> 5;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const int c = 2 * ks + hf;
      qf[ks] = *(const bf16x8*)(stg + col_ * SROW + ((c ^ (col_ & (CPR - 1) & 15)) << 4));
    }
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) asm volatile("" ::"v"(qf[ks]));
    if (qrow >= p.R) {
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks) qf[ks] = bf16x8{};
    }
  }
  QF8<DC> q8;
  make_qf8<DC>(qf, q8);

  const int my_row = rowbase + 32 * w + col;
  const int limit = min(L - p.S + 1 + my_row / p.H, L);  // first position this lane's row may not see
  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x16 O[4][NBW];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) O[rb][cb] = f32x16{};

  // One tile step: (a) tile i and its scales are in LDS (tile i + 1 may still
  // be in flight), P of tile i - 1 is visible, every wave is done with tile
  // i - 2 (whose slots take tile i + 2); (b) the copy of tile i + 2 spread
  // over the scores of tile i; (c) the softmax of tile i with, from the
  // second tile on (PV), the P . V of tile i - 1; (d) P and the factors of
  // tile i published.
  auto tile_step = [&](int i, auto pv_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    const int t = t0 + i;
    if (i + 1 < n) vm_wait<NI>();  // tile i and the page read before tile i + 1's copy
    else vm_wait<0>();
    block_sync();
    int4 fl = int4{0, 0, 0, 0};
    if constexpr (PV) fl = *(const int4*)rflag[(i - 1) & 1];
    // the page of tile i + AHEAD + 1, read before this step's copy is issued
    const int page_cur = uniform(page_pf);
    if (i + AHEAD + 1 < n) page_pf = tile_page_load(p, bt, t + AHEAD + 1);
    const F8Dma<DC> dma = make_dma(i + AHEAD, page_cur, i + AHEAD < n);
    const int pos0 = t * kTile;
    F8PvOperands<DC> pv(raw + ((i + NBUF - 1) % NBUF) * RAW, pbuf + ((i - 1) & 1) * PB, w);
    WideSoftmax<true> sm{PV ? score_f8<DC>(raw + (i % NBUF) * RAW, q8, dma, pv)
                            : score_f8<DC>(raw + (i % NBUF) * RAW, q8, dma),
                         tscale[i % NBUF], limit - pos0 - 4 * half, p.scale_log2, m_run, l_run, half};
    // Publish P and the rescale factor of tile i (their buffers [i & 1] were
    // last read in iteration i - 1, before this iteration's barrier).
    auto publish = [&]() {
      const int ol = opaque_lane();
      char* pw = pbuf + (i & 1) * PB + (w * 2) * 1024 + ol * 16;
      *(bf16x8*)pw = sm.pf0;
      *(bf16x8*)(pw + 1024) = sm.pf1;
      if (ol < 32) alph[i & 1][32 * w + ol] = sm.alpha;
      const bool any = PV && __any(sm.alpha != 1.0f);
      if (ol == 0) rflag[i & 1][w] = any;
    };
    if constexpr (PV) {
      if (fl.x | fl.y | fl.z | fl.w) {
        float a[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[rb] = alph[(i - 1) & 1][32 * rb + col];
        rescale_rows<NBW>(O, a);
      }
      pv_f8<DC, true>(pv, O, sm, publish);
    } else {
      sm.all();
      publish();
    }
  };
  tile_step(0, std::false_type{});
#pragma nounroll
  for (int i = 1; i < n; ++i) tile_step(i, std::true_type{});
  // ---- drain: P . V of the last tile
  block_sync();
  {
    const int pbi = (n - 1) & 1;
    if (rflag[pbi][0] | rflag[pbi][1] | rflag[pbi][2] | rflag[pbi][3]) {
      float a[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[rb] = alph[pbi][32 * rb + col];
      rescale_rows<NBW>(O, a);
    }
    NoSteps none;
    F8PvOperands<DC> pv(raw + ((n - 1) % NBUF) * RAW, pbuf + pbi * PB, w);
    pv.load();
    pv_f8<DC, false>(pv, O, none);
  }

  // ---- normalise and write this part's partial and lse
  const float l_tot = pair_sum(l_run);
  if (half == 0) fin_l[32 * w + col] = l_tot;
  if (half == 0 && my_row < p.R)
    p.lse_part[(int64_t)g * p.R + my_row] =
        l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
  block_sync();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int ln = opaque_lane();
    const int r = rowbase + 32 * rb + (ln & 31);
    const float lt = fin_l[32 * rb + (ln & 31)];
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (r < p.R) store_partial<NBW>(p, O[rb], inv, ((int64_t)g * p.R + r) * DC + w * NBW * 32, ln >> 5);
  }
}

template <int DC>
hipError_t launch_f8_one(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_f8_kernel<DC>), dim3(p.P * p.RG), dim3(256), 0, stream, p, p.seq_lens, p.block_table);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_wide_fp8(const DecodeParams& p, int d_latent, hipStream_t stream) {
  return d_latent == 512 ? launch_f8_one<512>(p, stream) : launch_f8_one<256>(p, stream);
}

}  // namespace mla
