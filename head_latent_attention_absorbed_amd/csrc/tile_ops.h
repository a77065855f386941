// Tile products and online softmax shared by the latent decode and the
// MLA-form prefill (gfx950).
//
// A tile is 32 tokens.  Its scores against 32 query rows are one chain of
// 32x32x16 bf16 MFMAs, S^T[t, r] = sum_d K[t, d] Q[r, d], with K read from the
// LDS tile and Q held in registers; P = softmax(S) stays in the registers the
// score MFMAs leave it in, which is the B-operand layout of the second
// product O^T[c, r] += sum_t V[t, c] P[r, t], whose A operand comes from
// transposing LDS reads of the same tile.  The softmax is online (the BLASST
// abstract on the "GQA-to-MLA" Daily Papers listing builds on the same running
// max and sum), in exp2, and re-bases the running max only when it grows by
// more than 2^8, so rescaling the accumulators is rare.
//
// LDS tile layout (granule-major): row g (512 bytes) holds 16-byte granule g
// (8 bf16 values) of all 32 tokens, token t at slot t ^ (4 * (g & 1)).  One
// DMA instruction fills two rows; the K-operand reads of eight lanes cover one
// contiguous 128-byte run, and the sixteen lanes of a transposing V read hit
// 32 distinct banks.
#pragma once
#include "mla_device.h"

namespace mla {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRebase = 8.0f;  // log2 of the largest unnormalised weight kept between re-bases
constexpr int kPvAhead = 2;      // V blocks read ahead of their MFMAs
constexpr int kScoreAhead = 4;   // K fragments read ahead of their MFMAs

// Tile geometry for a latent (or key) width DC plus the 64-wide RoPE key.
template <int DC>
struct Geo {
  static constexpr int GC = DC * 2 / 16;         // latent granules per token (bf16)
  static constexpr int GR = 64 * 2 / 16;         // RoPE granules per token (d_rope = 64)
  static constexpr int GPT = GC + GR;            // granule rows per tile
  static constexpr int TILE_BYTES = GPT * kRow;
  static constexpr int KS = (DC + 64) / 16;      // k-steps of the score product
  static constexpr int NB = DC / 32;             // 32-column blocks of O^T
};

// The no-op copy hook of score_mfma (no DMA spread over the MFMAs).
struct NoDma {
  __device__ __forceinline__ void issue(int) const {}
};

// Score MFMAs with VGPR accumulators.  The hardware forwards an MFMA result
// to the accumulator input of the next MFMA of the same chain; a VALU read of
// the result needs wait states that the compiler cannot see through inline
// asm, so the last MFMA of every chain (mfma_v_last) carries them in the
// same asm statement: a separate statement of nops would not order the
// compiler's own copies of the result after it.
// The other direction needs them too: an MFMA may read a VGPR only two wait
// states after a VALU instruction wrote it, and the compiler may place such a
// write (say a v_accvgpr_read bringing back an operand it parked in an AGPR)
// right before the asm, so each MFMA here starts with s_nop 1.
__device__ __forceinline__ void mfma_v_first(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_last(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc)
               : "v"(a), "v"(b));
}

// The no-op read-ahead hook of score_mfma.
struct NoPre {
  static constexpr int AT = -1;
  __device__ __forceinline__ void load() {}
};

// S^T = K . Q^T of one 32-token tile (32 tokens x this wave's 32 rows):
// A = token `col`, granule 2ks + half, from LDS; B = the query fragments.
// NDMA > 0 spreads that many instructions of the next tile's copy over
// the MFMA stream; pre.load() runs before the MFMA of k-step Pre::AT (the
// operand reads of whatever follows the chain, issued while it runs).
template <int DC, int NDMA, class Dma, class Pre>
__device__ __forceinline__ f32x16 score_mfma(const char* tb, const bf16x8 (&qf)[Geo<DC>::KS], const Dma& dma,
                                             Pre& pre) {
  using Gm = Geo<DC>;
  constexpr int PD = kScoreAhead;  // k-steps of K fragments read ahead of their MFMA
  const int lane = opaque_lane();
  const int half = lane >> 5, col = lane & 31;
  const char* kb = tb + half * kRow + ((col ^ (half << 2)) << 4);
  bf16x8 kf[Gm::KS];
#pragma unroll
  for (int ks = 0; ks < PD; ++ks) kf[ks] = *(const bf16x8*)(kb + ks * 2 * kRow);
  // The score accumulators are kept in VGPRs (inline-asm MFMAs): the
  // accumulator registers are all taken by O^T, and left to itself the
  // compiler would park part of O^T in VGPRs around every tile.  Program
  // order is the issue order: read ks + PD, then the MFMA of k-step ks.
  // Dependent MFMAs on one accumulator issue back to back (the hardware
  // forwards the accumulation), so one chain suffices.
  f32x16 sacc;
  static_assert(NDMA == 0 || Gm::KS % NDMA == 0, "DMA instructions must divide the k-steps");
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    if (ks + PD < Gm::KS) kf[ks + PD] = *(const bf16x8*)(kb + (ks + PD) * 2 * kRow);
    if constexpr (NDMA > 0) {
      if (ks % (Gm::KS / NDMA) == 0) dma.issue(ks / (Gm::KS / NDMA));  // next tile's copy, spread out
    }
    if (ks == Pre::AT) pre.load();
    if (ks == 0) mfma_v_first(sacc, kf[ks], qf[ks]);
    else if (ks + 1 < Gm::KS) mfma_v_acc(sacc, kf[ks], qf[ks]);
    else mfma_v_last(sacc, kf[ks], qf[ks]);
  }
  // The score product is its own scheduling region: nothing that follows
  // (the softmax, or the lagged P.V of the previous tile) is hoisted into it.
  __builtin_amdgcn_sched_barrier(0);
  return sacc;
}
template <int DC, int NDMA, class Dma>
__device__ __forceinline__ f32x16 score_mfma(const char* tb, const bf16x8 (&qf)[Geo<DC>::KS], const Dma& dma) {
  NoPre none;
  return score_mfma<DC, NDMA>(tb, qf, dma, none);
}

// Online-softmax update of one tile's scores, in kSoftmaxSteps steps that
// can be spread over the MFMAs of the previous tile's P.V (step() with
// increasing j; all() runs them back to back).  Produces P (the B operand of
// the P.V product, pf0 | pf1) and the factor alpha by which the accumulators
// must be multiplied before this tile's P.V is added (1 unless the row
// maximum grew by more than 2^kRebase).  Lane (col, half) holds row `col`,
// tokens 8(i/4) + 4 half + i%4 of the tile in value i.
//
// `full` (wave-uniform) says every position of the tile is visible to every
// row: then the maximum is taken over the raw scores (the scale is positive)
// and each weight is exp2(s * scale - m) with one fused multiply-add, with no
// masking and no guard (m is finite), in 10 steps.  For an e4m3 tile the raw
// scores are first multiplied by their tokens' scales (the keys' scale), and
// the weights by them again after the sum (the values' scale, carried by P).
constexpr int kSoftmaxSteps = 13;
template <bool FP8>
struct Softmax {
  f32x16 v;          // raw scores, then scaled masked scores, then weights (in place)
  const float* tsc;  // fp8: the tile's per-token scales (LDS)
  int pos0, limit;   // tile position in the sequence, first masked position of this row
  float slog2;       // softmax scale * log2(e)
  float& m_run;
  float& l_run;
  bool full = false;
  float tsv[16];
  float mt, m_new, alpha;
  bf16x8 pf0, pf1;

  __device__ __forceinline__ void step(int j) {
    if (full) {
      fast_step(j);
      return;
    }
    const int half = opaque_lane() >> 5;
    if (j < 4) {  // scaled, masked scores, four at a time
      if constexpr (FP8) {
        const f32x4 s4 = *(const f32x4*)(tsc + 8 * j + 4 * half);
#pragma unroll
        for (int c = 0; c < 4; ++c) tsv[4 * j + c] = s4[c];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * j + c;
        const int tau = 8 * (i >> 2) + 4 * half + (i & 3);
        float zi = v[i] * slog2;
        if constexpr (FP8) zi *= tsv[i];
        v[i] = (pos0 + tau < limit) ? zi : -__builtin_inff();
      }
    } else if (j == 4) {
      mt = v[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, v[i]);
    } else if (j == 5) {
      mt = pair_max(mt);
      const bool rebase = mt > m_run + kRebase;
      m_new = rebase ? mt : m_run;
      alpha = rebase ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // exp2(-inf) = 0 on the first visible tile
      l_run *= alpha;
      m_run = m_new;
    } else if (j < 10) {  // weights, four at a time
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * (j - 6) + c;
        // A row that has seen no visible position yet keeps m = -inf with all
        // its scores at -inf; exp2(-inf - -inf) would be NaN, so masked
        // entries give 0.
        v[i] = (v[i] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(v[i] - m_new);
      }
    } else if (j == 10) {
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t += v[i];
      l_run += t;
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] *= tsv[i];
      }
    } else if (j == 11) {
      float w8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = v[i];
      pf0 = pack_bf16x8(w8);
    } else if (j == 12) {
      float w8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = v[8 + i];
      pf1 = pack_bf16x8(w8);
    }
  }
  __device__ __forceinline__ void fast_step(int j) {
    if (j == 0) {
      if constexpr (FP8) {  // the tokens' scales apply to the keys: scale the raw scores first
        const int half = opaque_lane() >> 5;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 s4 = *(const f32x4*)(tsc + 8 * q + 4 * half);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            tsv[4 * q + c] = s4[c];
            v[4 * q + c] *= s4[c];
          }
        }
      }
      mt = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
#pragma unroll
      for (int i = 4; i < 8; ++i) mt = fmaxf(mt, v[i]);
    } else if (j == 1) {
      if constexpr (FP8) {
        const int half = opaque_lane() >> 5;
#pragma unroll
        for (int q = 2; q < 4; ++q) {
          const f32x4 s4 = *(const f32x4*)(tsc + 8 * q + 4 * half);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            tsv[4 * q + c] = s4[c];
            v[4 * q + c] *= s4[c];
          }
        }
      }
#pragma unroll
      for (int i = 8; i < 16; ++i) mt = fmaxf(mt, v[i]);
    } else if (j == 2) {
      mt = pair_max(mt) * slog2;
      const bool rebase = mt > m_run + kRebase;
      m_new = rebase ? mt : m_run;
      alpha = rebase ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // exp2(-inf) = 0 on the first visible tile
      l_run *= alpha;
      m_run = m_new;
    } else if (j < 7) {  // weights, four at a time
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * (j - 3) + c;
        v[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], slog2, -m_new));
      }
    } else if (j == 7) {
      float t0 = v[0] + v[1], t1 = v[2] + v[3], t2 = v[4] + v[5], t3 = v[6] + v[7];
      float t4 = v[8] + v[9], t5 = v[10] + v[11], t6 = v[12] + v[13], t7 = v[14] + v[15];
      l_run += ((t0 + t1) + (t2 + t3)) + ((t4 + t5) + (t6 + t7));
      if constexpr (FP8) {  // and to the values: P carries them into P.V
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] *= tsv[i];
      }
    } else if (j == 8) {
      float w8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = v[i];
      pf0 = pack_bf16x8(w8);
    } else if (j == 9) {
      float w8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = v[8 + i];
      pf1 = pack_bf16x8(w8);
    }
  }
  __device__ __forceinline__ void all() {
#pragma unroll
    for (int j = 0; j < kSoftmaxSteps; ++j) step(j);
  }
};

// Scores of one tile and the whole softmax update (the unpipelined order).
template <int DC, bool FP8, int NDMA, class Dma>
__device__ __forceinline__ void score_tile(const char* tb, const float* tsc, const bf16x8 (&qf)[Geo<DC>::KS],
                                           float& m_run, float& l_run, int pos0, int limit, bool full, float slog2,
                                           bf16x8& pf0, bf16x8& pf1, float& alpha, const Dma& dma) {
  Softmax<FP8> sm{score_mfma<DC, NDMA>(tb, qf, dma), tsc, pos0, limit, slog2, m_run, l_run};
  sm.full = full;
  sm.all();
  pf0 = sm.pf0;
  pf1 = sm.pf1;
  alpha = sm.alpha;
}

// O^T += V^T . P^T for one tile over NBK 32-column blocks starting at `tb`
// (a tile, or a tile advanced by 4 granule rows per skipped block); the four
// transposed reads of block nb + AH are issued before the two MFMAs of block
// nb.  Source lane (group G = lane/16, i = lane%16) reads token
// 16 j2 + 8 h + 4 (G/2) + i/4 and columns 32 nb + 16 (G%2) + 4 (i%4) .. +3.
template <int DC, int AH, bool FIRST, int NBK>
__device__ __forceinline__ void pv_tile(const char* tb, bf16x8 pf0, bf16x8 pf1, f32x16 (&O)[NBK]) {
  static_assert(NBK <= Geo<DC>::NB, "more blocks than latent columns");
  const int lane = opaque_lane();
  const int half = lane >> 5;
  const int i16 = lane & 15, grp = lane >> 4;
  const int jj = i16 >> 2, qq = i16 & 3, ch = grp & 1;
  const int godd = qq >> 1;
  const char* vb = tb + (2 * ch + godd) * kRow + (((4 * half + jj) ^ (godd << 2)) << 4) + ((qq & 1) << 3);
  struct VF { s16x4 x0, x1, y0, y1; };
  auto vread = [&](int nb) {
    const char* a = vb + nb * 4 * kRow;
    VF f;
    f.x0 = lds_read_tr16(a);
    f.x1 = lds_read_tr16(a + 8 * 16);
    f.y0 = lds_read_tr16(a + 16 * 16);
    f.y1 = lds_read_tr16(a + 24 * 16);
    return f;
  };
  VF vf[NBK];
#pragma unroll
  for (int nb = 0; nb < AH; ++nb) vf[nb] = vread(nb);
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb) {
    if (nb + AH < NBK) vf[nb + AH] = vread(nb + AH);
    const VF& cur = vf[nb];
    const s16x8 a0 = {cur.x0[0], cur.x0[1], cur.x0[2], cur.x0[3], cur.x1[0], cur.x1[1], cur.x1[2], cur.x1[3]};
    const s16x8 a1 = {cur.y0[0], cur.y0[1], cur.y0[2], cur.y0[3], cur.y1[0], cur.y1[1], cur.y1[2], cur.y1[3]};
    O[nb] = mfma32((bf16x8)a0, pf0, FIRST ? f32x16{} : O[nb]);  // the first tile starts the sums
    O[nb] = mfma32((bf16x8)a1, pf1, O[nb]);
  }
  // Order: the reads of the first AH blocks, then per block (reads of block
  // nb + AH, MFMAs of block nb).
  __builtin_amdgcn_sched_group_barrier(0x100, 4 * AH, 1);
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb) {
    if (nb + AH < NBK) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
  }
}

// Multiply the accumulators by alpha (rare: the row maximum grew by more than
// 2^kRebase).  Element-wise through AGPR-constrained blocks, so the
// accumulators stay in AGPRs and one temporary VGPR suffices; the leading
// wait states cover an MFMA that may just have written them (the compiler's
// hazard check does not look inside inline asm).
template <int NBK>
__device__ __forceinline__ void rescale(f32x16 (&O)[NBK], float alpha) {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = O[nb][i];
      float tmp;
      asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32_e32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                   : "+a"(x), "=&v"(tmp)
                   : "v"(alpha));
      O[nb][i] = x;
    }
  }
  // an MFMA may read the accumulators two wait states after the last write
  asm volatile("s_nop 1" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace
}  // namespace mla
