// Split-K decode of absorbed MLA over a paged latent cache (gfx950).
//
// Absorbing W_UK into the query turns every head into a reader of the same
// cache record [c_KV | k_rope] (the MQA form of MLA in the GQLA abstract on
// the "GQA-to-MLA" Daily Papers listing; the absorb itself is described on the
// TransMLA review page, key_machinery).  So the query rows of all heads form
// one dense operand against each 32-token tile, and both products of a tile
// are 32x32x16 bf16 MFMAs:
//
//   S^T[t, r] = sum_d K[t, d] Q[r, d]      A = tile (LDS), B = query (registers)
//   O^T[c, r] += sum_t V[t, c] P[r, t]     A = tile via transposing LDS reads,
//                                          B = P, which S^T already leaves in
//                                          the B-operand lane layout
//
// Each wave owns 32 query rows (r = s*H + h) and keeps, per row, the running
// max m, the running sum l and O^T[512 or 256, 32] in accumulators; the
// softmax is online (BLASST abstract on the same listing relies on the same
// running state), with the max only re-based when it grows by more than 2^8
// so the accumulator rescale is rare.  A work-group of NW waves shares each
// tile; tiles stream through an LDS ring (direct global->LDS DMA for bf16,
// register-staged e4m3->bf16 decode for fp8).  The token axis of the whole
// batch is cut into G equal parts; each (part, sequence) pair writes one
// normalised partial and its log-sum-exp.
//
// LDS tile layout (granule-major): row g (512 bytes) holds 16-byte granule g
// (8 bf16 values) of all 32 tokens, token t at slot t ^ (4 * (g & 1)).  One
// DMA instruction fills two rows; the K-operand reads of eight lanes cover one
// contiguous 128-byte run, and the sixteen lanes of a transposing V read hit
// 32 distinct banks.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRebase = 8.0f;  // log2 of the largest unnormalised weight kept between re-bases
constexpr int kTab = 128;  // tiles per LDS source-table fill
constexpr int kPvAhead = 2;     // V blocks read ahead of their MFMAs
constexpr int kScoreAhead = 4;  // K fragments read ahead of their MFMAs

__device__ __forceinline__ int seq_of_tile(const int* cu, int B, int k) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= k) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int NI, int MAXLATER>
__device__ __forceinline__ void wait_dma_groups(int later) {
  // Tiles complete in issue order; `later` (<= MAXLATER) DMA groups of NI
  // loads were issued after the one being waited for.
  static_assert(NI * MAXLATER <= 63, "vmcnt range");
  if constexpr (MAXLATER == 0) {
    vm_wait<0>();
  } else if constexpr (MAXLATER == 1) {
    if (later <= 0) vm_wait<0>(); else vm_wait<NI>();
  } else {
    static_assert(MAXLATER == 2, "ring depth");
    if (later <= 0) vm_wait<0>();
    else if (later == 1) vm_wait<NI>();
    else vm_wait<NI * 2>();
  }
}

template <int DC>
struct Geo {
  static constexpr int GC = DC * 2 / 16;         // latent granules per token (bf16)
  static constexpr int GR = 64 * 2 / 16;         // RoPE granules per token (d_rope = 64)
  static constexpr int GPT = GC + GR;            // granule rows per tile
  static constexpr int TILE_BYTES = GPT * kRow;
  static constexpr int KS = (DC + 64) / 16;      // k-steps of the score product
  static constexpr int NB = DC / 32;             // 32-column blocks of O^T
};


// The token a lane moves in every tile-load instruction: slot lane % 32 of
// row 2m + lane / 32 holds token (lane % 32) ^ (4 * (lane / 32)).
__device__ __forceinline__ int load_token(int lane) { return (lane & 31) ^ ((lane >> 5) << 2); }

// Byte offset of granule row pair (g0, g0+1) inside a cache record (GB-byte
// granules: 16 for bf16, 8 for e4m3).  g0 is even, so a pair never straddles
// the latent and the RoPE key.
template <int DC, int GB>
__device__ __forceinline__ int64_t granule_offset(const DecodeParams& p, int g0) {
  return g0 < Geo<DC>::GC ? (int64_t)g0 * GB : p.rope_off + (int64_t)(g0 - Geo<DC>::GC) * GB;
}

// Issue this wave's DMA loads of one tile.  `run` is the address of the
// tile's first token (page base + slot offset); `lane_off` is this lane's
// load_token times the token stride, plus 16 bytes on the odd row of a pair.
template <int DC, int NW>
__device__ __forceinline__ void issue_tile_dma(const DecodeParams& p, const char* run, uint32_t lane_off,
                                               uint32_t buf_lds, int w) {
  constexpr int NI = Geo<DC>::GPT / (2 * NW);
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int g0 = 2 * (q * NW + w);
    lds_dma16(run + granule_offset<DC, 16>(p, g0), lane_off, uniform(buf_lds + (q * NW + w) * 1024));
  }
}

// The same copy, one instruction at a time, so that the instructions can be
// spread over the MFMA stream of the score product instead of being issued in
// one burst (a burst stalls the wave while the texture unit accepts it).
template <int DC, int NW>
struct TileDma {
  static constexpr int NI = Geo<DC>::GPT / (2 * NW);
  const char* run;
  int64_t rope_off;
  uint32_t lane_off, buf_lds;
  int w;
  __device__ __forceinline__ void issue(int q) const {
    const int g0 = 2 * (q * NW + w);
    const int64_t off = g0 < Geo<DC>::GC ? (int64_t)g0 * 16 : rope_off + (int64_t)(g0 - Geo<DC>::GC) * 16;
    lds_dma16(run + off, lane_off, uniform(buf_lds + (q * NW + w) * 1024));
  }
};
struct NoDma {
  __device__ __forceinline__ void issue(int) const {}
};

// Zero the slots of tokens nv..31 of a tile (the last, partial tile of a
// sequence): their DMA'd contents are whatever the page held past the length.
template <int DC, int NW>
__device__ __forceinline__ void zero_tail(char* tb, int nv, int tid) {
  for (int i = tid; i < Geo<DC>::GPT * kTile; i += NW * kWave) {
    const int g = i >> 5, slot = i & 31;
    if ((slot ^ ((g & 1) << 2)) >= nv) *(uint4*)(tb + g * kRow + slot * 16) = uint4{0, 0, 0, 0};
  }
}

// fp8 tile: 8 e4m3 bytes per bf16 granule, loaded into registers, decoded
// exactly (every e4m3 value is a bf16 value) and written to the same layout;
// tokens past the length are written as zeros.
template <int DC, int NW>
struct Fp8Stage {
  static constexpr int NI = Geo<DC>::GPT / (2 * NW);  // granules per lane
  static constexpr int CH = NI < 9 ? NI : 9;          // granules kept in flight
  uint2 v[CH];

  __device__ __forceinline__ void load_chunk(const DecodeParams& p, const char* run, uint32_t lane_off8, int c0,
                                             int w) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int qq = c0 + q;
      if (qq < NI) {
        const int g0 = 2 * (qq * NW + w);
        v[q] = *(const uint2*)(run + granule_offset<DC, 8>(p, g0) + lane_off8);
      }
    }
  }
  __device__ __forceinline__ void store_chunk(char* buf, int c0, int w, int lane, bool valid) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int qq = c0 + q;
      if (qq < NI) {
        bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].x, 1.0f, false);
        bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].x, 1.0f, true);
        bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].y, 1.0f, false);
        bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].y, 1.0f, true);
        bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        if (!valid) r = bf16x8{};
        *(bf16x8*)(buf + (qq * NW + w) * 1024 + lane * 16) = r;
      }
    }
  }
};

// Score MFMAs with VGPR accumulators.  The hardware forwards an MFMA result
// to the accumulator input of the next MFMA of the same chain; a VALU read of
// the result needs wait states that the compiler cannot see through inline
// asm, so every chain ends with mfma_v_drain before its values are used.
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
__device__ __forceinline__ void mfma_v_drain(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}

// S^T = K . Q^T of one 32-token tile (32 tokens x this wave's 32 rows):
// A = token `col`, granule 2ks + half, from LDS; B = the query fragments.
// NDMA > 0 spreads that many instructions of the next tile's copy over
// the MFMA stream.
template <int DC, int NDMA, class Dma>
__device__ __forceinline__ f32x16 score_mfma(const char* tb, const bf16x8 (&qf)[Geo<DC>::KS], const Dma& dma) {
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
    if (ks == 0) mfma_v_first(sacc, kf[ks], qf[ks]);
    else mfma_v_acc(sacc, kf[ks], qf[ks]);
  }
  mfma_v_drain(sacc);
  // The score product is its own scheduling region: nothing that follows
  // (the softmax, or the lagged P.V of the previous tile) is hoisted into it.
  __builtin_amdgcn_sched_barrier(0);
  return sacc;
}

// Online-softmax update of one tile's scores, in kSoftmaxSteps steps that
// can be spread over the MFMAs of the previous tile's P.V (step() with
// increasing j; all() runs them back to back).  Produces P (the B operand of
// the P.V product, pf0 | pf1) and the factor alpha by which the accumulators
// must be multiplied before this tile's P.V is added (1 unless the row
// maximum grew by more than 2^kRebase).  Lane (col, half) holds row `col`,
// tokens 8(i/4) + 4 half + i%4 of the tile in value i.
//
// `full` (bf16 only, wave-uniform) says every position of the tile is visible
// to every row: then the maximum is taken over the raw scores (the scale is
// positive) and each weight is exp2(s * scale - m) with one fused
// multiply-add, with no masking and no guard (m is finite), in 10 steps.
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
    if (!FP8 && full) {
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
      mt = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
#pragma unroll
      for (int i = 4; i < 8; ++i) mt = fmaxf(mt, v[i]);
    } else if (j == 1) {
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

// O^T += V^T . P^T for one tile; the four transposed reads of block nb + AH
// are issued before the two MFMAs of block nb.  Source lane (group G = lane/16,
// i = lane%16) reads token 16 j2 + 8 h + 4 (G/2) + i/4 and columns
// 32 nb + 16 (G%2) + 4 (i%4) .. +3.
template <int DC, int AH, bool FIRST>
__device__ __forceinline__ void pv_tile(const char* tb, bf16x8 pf0, bf16x8 pf1, f32x16 (&O)[Geo<DC>::NB]) {
  using Gm = Geo<DC>;
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
  VF vf[Gm::NB];
#pragma unroll
  for (int nb = 0; nb < AH; ++nb) vf[nb] = vread(nb);
#pragma unroll
  for (int nb = 0; nb < Gm::NB; ++nb) {
    if (nb + AH < Gm::NB) vf[nb + AH] = vread(nb + AH);
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
  for (int nb = 0; nb < Gm::NB; ++nb) {
    if (nb + AH < Gm::NB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
  }
}

// Multiply the accumulators by alpha (rare: the row maximum grew by more than
// 2^kRebase).  Element-wise through AGPR-constrained blocks, so the
// accumulators stay in AGPRs and one temporary VGPR suffices; the leading
// wait states cover an MFMA that may just have written them (the compiler's
// hazard check does not look inside inline asm).
template <int DC>
__device__ __forceinline__ void rescale(f32x16 (&O)[Geo<DC>::NB], float alpha) {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int nb = 0; nb < Geo<DC>::NB; ++nb) {
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

// Write NBK accumulator blocks (32 latent columns each, starting at element
// offset `base` of o_part) scaled by inv, as fp16 or fp32.
template <int NBK>
__device__ __forceinline__ void store_partial(const DecodeParams& p, const f32x16* O, float inv, int64_t base,
                                              int half) {
  if (p.o_half) {
    // Lane pair (l, l + 32) swaps packed halves so that each lane stores 8
    // consecutive columns: with column quarters q0..q3 of an 8-column group
    // split 4 + 4 over the pair, the swap gives the lower lane the odd group
    // and the upper lane the even one.
    _Float16* dst = (_Float16*)p.o_part + base + 8 * (1 - half);
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x2 v = {(_Float16)(O[nb][2 * j] * inv), (_Float16)(O[nb][2 * j + 1] * inv)};
        h[j] = __builtin_bit_cast(uint32_t, v);
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {  // 8-column groups (2pr, 2pr + 1)
        const auto r0 = __builtin_amdgcn_permlane32_swap(h[4 * pr + 2], h[4 * pr], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(h[4 * pr + 3], h[4 * pr + 1], false, false);
        const uint4 v = {r0[0], r1[0], r0[1], r1[1]};
        *(uint4*)(dst + 32 * nb + 16 * pr) = v;
      }
      __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time
    }
  } else {
    float* dst = (float*)p.o_part + base + 4 * half;
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const f32x4 v = {O[nb][4 * ig] * inv, O[nb][4 * ig + 1] * inv, O[nb][4 * ig + 2] * inv,
                         O[nb][4 * ig + 3] * inv};
        *(f32x4*)(dst + 32 * nb + 8 * ig) = v;
      }
      __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time
    }
  }
}

// Pitch of one row of a staged fp16 partial: the row plus 16 bytes, so that
// the rows of one LDS write instruction start in different banks.
template <int DC>
constexpr int stage_pitch() { return DC * 2 + 16; }

// The same write as store_partial<NB> for fp16 partials, through LDS: the
// wave puts its 32 normalised rows into `stage` (row = lane % 32), then
// writes them back out with every store instruction covering whole rows
// (DC * 2 contiguous bytes), instead of 32 rows x 32 bytes per instruction.
// `stage` is this wave's own region; nothing else may use it meanwhile.
template <int DC>
__device__ __forceinline__ void store_partial_staged(const DecodeParams& p, const f32x16* O, float inv, int64_t slot,
                                                     int rowbase, char* stage) {
  constexpr int NB = DC / 32;
  constexpr int PITCH = stage_pitch<DC>();
  const int lane = opaque_lane();
  const int half = lane >> 5, col = lane & 31;
  char* mine = stage + col * PITCH + 16 * (1 - half);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16x2 v = {(_Float16)(O[nb][2 * j] * inv), (_Float16)(O[nb][2 * j + 1] * inv)};
      h[j] = __builtin_bit_cast(uint32_t, v);
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {  // 8-column groups (2pr, 2pr + 1), as in store_partial
      const auto r0 = __builtin_amdgcn_permlane32_swap(h[4 * pr + 2], h[4 * pr], false, false);
      const auto r1 = __builtin_amdgcn_permlane32_swap(h[4 * pr + 3], h[4 * pr + 1], false, false);
      *(uint4*)(mine + 64 * nb + 32 * pr) = uint4{r0[0], r1[0], r0[1], r1[1]};
    }
    __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time
  }
  // A wave's LDS accesses complete in order, so the reads below see the writes.
  constexpr int LPR = DC / 8;       // lanes per row (16 bytes each)
  constexpr int RPI = kWave / LPR;  // rows per store instruction
  const int sub = lane / LPR, gi = lane % LPR;
#pragma unroll 4
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + sub;
    const uint4 x = *(const uint4*)(stage + r * PITCH + 16 * gi);
    if (rowbase + r < p.R) *(uint4*)((_Float16*)p.o_part + (slot * p.R + rowbase + r) * DC + 8 * gi) = x;
  }
}

template <int DC, bool FP8, int NW, int NBUF>
__global__ void __launch_bounds__(NW * kWave)
    decode_kernel(DecodeParams p, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table,
                  const float* __restrict__ kv_scale) {
  using Gm = Geo<DC>;
  constexpr int TB = Gm::TILE_BYTES;
  constexpr int NI = Gm::GPT / (2 * NW);
  constexpr int AHEAD = NBUF - 1;  // tiles in flight ahead of the one computed
  static_assert(Gm::GPT % (2 * NW) == 0, "tile rows must split evenly over the waves");
  static_assert(AHEAD >= 1, "ring too small");
  static_assert(FP8 || NI * AHEAD <= 63, "DMA groups must fit vmcnt");
  static_assert(!FP8 || AHEAD == 1, "fp8 tiles are staged one ahead");

  __shared__ __attribute__((aligned(1024))) char tiles[NBUF * TB];
  __shared__ __attribute__((aligned(16))) float tscale[FP8 ? NBUF * kTile : 4];
  __shared__ int cu[kMaxBatch + 1];
  __shared__ int4 tab[kTab];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware placement: consecutive work items (the row groups of one token
  // part, then neighbouring parts) land on the same XCD, whose L2 they share.
  int u = blockIdx.x;
  if ((gridDim.x & 7) == 0) u = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int g = u / p.RG, rg = u % p.RG;

  if (w == 0) build_tile_prefix(seq_lens, p.B, cu, lane);
  block_sync();
  const int N = uniform(cu[p.B]);
  const int Wt = (N + p.G - 1) / p.G;
  const int k0 = g * Wt;
  const int k1 = min(k0 + Wt, N);
  if (k0 >= k1) return;

  const int row = rg * (32 * NW) + 32 * w + col;  // this lane's query row (S^T column)
  const uint32_t tiles_lds = lds_offset(tiles);

  // The first segment's query rows are touched (one dword per 128-byte line)
  // while the tile-table reads are in flight, so that the wave's own query
  // loads below hit L2 instead of making a further trip to HBM.
  int bc = uniform(seq_of_tile(cu, p.B, k0));
  uint32_t touch = 0;
  {
    const char* qa = (const char*)(p.q_lat + ((int64_t)bc * p.R + rg * (32 * NW)) * DC);
    const char* qb = (const char*)(p.q_rope + ((int64_t)bc * p.R + rg * (32 * NW)) * 64);
    const int rows = min(32 * NW, p.R - rg * (32 * NW));
    const int la = rows * DC * 2 / 128, lb = rows * 64 * 2 / 128;
    for (int i = tid; i < la + lb; i += NW * kWave)
      touch += i < la ? *(const uint32_t*)(qa + 128 * i) : *(const uint32_t*)(qb + 128 * (i - la));
  }

  // ---- tile source table: page, position and valid-token count of each tile
  // this part loads, kTab tiles at a time in LDS, so that starting a tile's
  // copy needs no memory round trip (a block-table read in the loop would).
  int tab0 = k0;
  auto fill_tab = [&](int from) {  // all threads; followed by block_sync()
    for (int i = tid; i < kTab; i += NW * kWave) {
      const int kk = from + i;
      if (kk < k1) {
        const int b = seq_of_tile(cu, p.B, kk);
        const int pos0 = (kk - cu[b]) * kTile;
        const int page = block_table[(int64_t)b * p.bt_stride + (pos0 >> p.block_shift)];
        tab[i] = int4{page, pos0, min(seq_lens[b] - pos0, kTile), 0};
      }
    }
  };
  fill_tab(k0);
  asm volatile("" ::"v"(touch));  // the touches complete together with the table reads
  block_sync();

  // ---- tile loader: next tile to load (kl) and its source.
  int kl = k0;
  int spage = 0, spos = 0, snv = 0;
  const char* src = p.c_kv;
  auto locate = [&]() {  // source of tile kl < k1 (called by all waves together)
    if (kl - tab0 == kTab) {
      block_sync();
      tab0 = kl;
      fill_tab(kl);
      block_sync();
    }
    const int4 e = tab[kl - tab0];
    spage = uniform(e.x);
    spos = uniform(e.y);
    snv = uniform(e.z);
    src = p.c_kv + (int64_t)spage * p.block_stride + (int64_t)(spos & (p.block_size - 1)) * p.token_stride;
  };
  locate();
  auto dma_next = [&]() {  // bf16: start the copy of tile kl into its ring slot
    const int ol = opaque_lane();
    const uint32_t lane_off = (uint32_t)load_token(ol) * (uint32_t)p.token_stride + 16u * (ol >> 5);
    issue_tile_dma<DC, NW>(p, src, lane_off, tiles_lds + ((kl - k0) % NBUF) * TB, w);
    ++kl;
    if (kl < k1) locate();
  };

  Fp8Stage<DC, NW> stage;
  auto stage_finish = [&]() {  // fp8: decode the loaded tile kl into its ring slot
    const int nbuf = (kl - k0) % NBUF;
    const int ol = opaque_lane();
    const uint32_t lane_off8 = (uint32_t)load_token(ol) * (uint32_t)p.token_stride + 8u * (ol >> 5);
    const bool valid = load_token(ol) < snv;
    stage.store_chunk(tiles + nbuf * TB, 0, w, ol, valid);
    for (int c0 = Fp8Stage<DC, NW>::CH; c0 < Fp8Stage<DC, NW>::NI; c0 += Fp8Stage<DC, NW>::CH) {
      stage.load_chunk(p, src, lane_off8, c0, w);
      stage.store_chunk(tiles + nbuf * TB, c0, w, ol, valid);
    }
    if (w == 0 && lane < kTile) {
      const float sc = kv_scale[(int64_t)spage * p.block_size + (spos & (p.block_size - 1)) + lane];
      tscale[nbuf * kTile + lane] = lane < snv ? sc : 0.0f;
    }
    ++kl;
    if (kl < k1) locate();
  };
  auto stage_start = [&]() {
    const int ol = opaque_lane();
    const uint32_t lane_off8 = (uint32_t)load_token(ol) * (uint32_t)p.token_stride + 8u * (ol >> 5);
    stage.load_chunk(p, src, lane_off8, 0, w);
  };

  if constexpr (FP8) {
    stage_start();
    stage_finish();
    block_sync();
  }

  // Before computing tile k: its data is in LDS and visible to all waves, and
  // the next copy is started (bf16) or its loads are issued (fp8).
  // FULL: every position of the tile is visible to every row (so it lies
  // inside the sequence and needs no zero fill either).
  auto tile_begin = [&](int k, int cub, int L, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int buf = (k - k0) % NBUF;
    if constexpr (!FP8) {
      wait_dma_groups<NI, AHEAD - 1>(kl - 1 - k);
      block_sync();
      if (!FULL && (k - cub + 1) * kTile > L) {  // last tile of the sequence, partially filled
        zero_tail<DC, NW>(tiles + buf * TB, L - (k - cub) * kTile, tid);
        block_sync();
      }
    } else {
      if (kl < k1) stage_start();
    }
  };
  auto tile_end = [&]() {
    if constexpr (FP8) {
      if (kl < k1) stage_finish();
      block_sync();
    }
  };

  // ---- segments: maximal runs of this part's tiles inside one sequence
  int k = k0;
  while (true) {
    const int cub = uniform(cu[bc]);
    const int kend = min(uniform(cu[bc + 1]), k1);
    const int L = seq_lens[bc];
    const int limit = min(L - p.S + 1 + row / p.H, L);
    const int lim_all = L - p.S + 1;  // positions below this are visible to every query row

    bf16x8 qf[Gm::KS];
    if (row < p.R) {
      const int ln = opaque_lane();
      const int qrow = rg * (32 * NW) + 32 * w + (ln & 31);
      const bf16x8* ql = (const bf16x8*)(p.q_lat + ((int64_t)bc * p.R + qrow) * DC + 8 * (ln >> 5));
      const bf16x8* qr = (const bf16x8*)(p.q_rope + ((int64_t)bc * p.R + qrow) * 64 + 8 * (ln >> 5));
#pragma unroll
      for (int ks = 0; ks < DC / 16; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
      for (int ks = DC / 16; ks < Gm::KS; ++ks) qf[ks] = qr[2 * (ks - DC / 16)];
    } else {
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks) qf[ks] = bf16x8{};
    }
    // Let the compiler see the query loads complete here, so it places no
    // waits for them inside the tile loop (where they would also drain the
    // in-flight tile DMA).  On the part's first segment the first tile
    // copies are started after the queries were requested, and the wait
    // leaves them in flight.
    if (!FP8 && k == k0) {
#pragma unroll
      for (int i = 0; i < AHEAD; ++i)
        if (kl < k1) dma_next();
      if (kl - k0 == AHEAD) vm_wait<NI * AHEAD>(); else vm_wait<0>();
    } else {
      vm_wait<0>();
    }
    f32x16 O[Gm::NB];
    float m_run = -__builtin_inff(), l_run = 0.0f;
    bf16x8 pf0, pf1;
    float alpha;

    // One tile.  The first tile of a segment starts the accumulators with its
    // P.V (a zero accumulator input), so O needs no initialisation and no
    // rescale there (alpha is 0 or 1 on a first tile, and O would be 0).
    auto one_tile = [&](auto first_tag, auto full_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      constexpr bool FULL = decltype(full_tag)::value;
      tile_begin(k, cub, L, full_tag);
      const int buf = (k - k0) % NBUF;
      if (!FP8 && kl < k1) {
        // the copy of tile kl (AHEAD tiles on) is issued inside the score product
        const int ol = opaque_lane();
        const TileDma<DC, NW> dma{src, p.rope_off,
                                  (uint32_t)load_token(ol) * (uint32_t)p.token_stride + 16u * (ol >> 5),
                                  tiles_lds + (uint32_t)(((kl - k0) % NBUF) * TB), w};
        score_tile<DC, FP8, TileDma<DC, NW>::NI>(tiles + buf * TB, tscale + buf * kTile, qf, m_run, l_run,
                                                 (k - cub) * kTile, limit, FULL, p.scale_log2, pf0, pf1, alpha,
                                                 dma);
        ++kl;
        if (kl < k1) locate();
      } else {
        score_tile<DC, FP8, 0>(tiles + buf * TB, tscale + buf * kTile, qf, m_run, l_run, (k - cub) * kTile, limit,
                               FULL, p.scale_log2, pf0, pf1, alpha, NoDma{});
      }
      if constexpr (!FIRST) {
        if (__any(alpha != 1.0f)) rescale<DC>(O, alpha);
      }
      pv_tile<DC, kPvAhead, FIRST>(tiles + buf * TB, pf0, pf1, O);
      tile_end();
      ++k;
    };
    // The segment's first tile starts the sums (general path); then the tiles
    // every row sees in full run branch-free; then the masked tail.
    one_tile(std::true_type{}, std::false_type{});
    const int kfull = min(kend, cub + lim_all / kTile);
    while (k < kfull) one_tile(std::false_type{}, std::integral_constant<bool, !FP8>{});
    while (k < kend) one_tile(std::false_type{}, std::false_type{});

    // ---- normalise and write this (sequence, part) partial
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
    const int64_t slot = (int64_t)bc + g;
    // The lse goes first: vector stores count in vmcnt, so any wait the
    // compiler places before a later store (a spilled address being reloaded)
    // would otherwise also wait for the whole partial to be written.
    {
      // lane-derived indices recomputed here rather than kept live (and
      // spilled) across the tile loop
      const int ln = opaque_lane();
      const int lhalf = ln >> 5, lcol = ln & 31;
      const int lrow = rg * (32 * NW) + 32 * w + lcol;
      if (lrow < p.R && lhalf == 0) p.lse_part[slot * p.R + lrow] = lse;
      // After the part's last tile the ring is idle (every copy has landed and
      // been consumed), so an fp16 partial is staged through it.
      constexpr bool STAGE_FITS = NW * 32 * stage_pitch<DC>() <= NBUF * TB;
      if (STAGE_FITS && p.o_half && kend == k1) {
        block_sync();
        store_partial_staged<DC>(p, O, inv, slot, rg * (32 * NW) + 32 * w, tiles + w * 32 * stage_pitch<DC>());
      } else if (lrow < p.R) {
        store_partial<Gm::NB>(p, O, inv, (slot * p.R + lrow) * DC, lhalf);
      }
    }
    ++bc;
    while (bc < p.B - 1 && uniform(cu[bc + 1]) == uniform(cu[bc])) ++bc;
    if (k >= k1) break;
  }
}

template <int DC, bool FP8, int NW, int NBUF>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const int grid = p.G * p.RG;
  hipLaunchKernelGGL((decode_kernel<DC, FP8, NW, NBUF>), dim3(grid), dim3(NW * kWave), 0, stream, p,
                     p.seq_lens, p.block_table, p.kv_scale);
  return hipGetLastError();
}

// Four-wave groups (128 query rows) run one work-group per CU on a 4-tile
// ring (bf16; 2 for the staged fp8 path).  One- and two-wave groups run two
// work-groups per CU on a 2-tile ring.
template <int DC, bool FP8>
hipError_t launch_dc(const DecodeParams& p, int nw, hipStream_t stream) {
  if constexpr (FP8) {
    if (nw == 4) return launch_one<DC, FP8, 4, 2>(p, stream);
    if (nw == 2) return launch_one<DC, FP8, 2, 2>(p, stream);
    return launch_one<DC, FP8, 1, 2>(p, stream);
  } else {
    if (nw == 4) return launch_one<DC, FP8, 4, 4>(p, stream);
    if (nw == 2) return launch_one<DC, FP8, 2, 2>(p, stream);
    return launch_one<DC, FP8, 1, 2>(p, stream);
  }
}

// ---------------------------------------------------------------------------
// Prefill in the MLA form (keys and values reconstructed per head, as the
// prefill-decode separation of the TPLA abstract keeps for the compute-bound
// prefill): every position of a prompt attends causally to the positions up
// to it, per head, over K = [W_UK c ; k_rope] (128 + 64) and V = c W_UV (128)
// made by mla_prefill_kv.  The tile products, the online softmax and P.V
// are the decode's, at latent width 128: a 32-token tile of K (24 granule
// rows) and of V (16 rows) in the same granule-major LDS layout, one wave per
// 32 query positions of one head, four waves per work-group.  The keys and
// values are stored in that layout already (tile-native), so a tile is two
// contiguous 8 KiB copies plus the shared RoPE keys gathered from the
// records, all global->LDS DMA into a two-slot ring.
constexpr int kPfRows = 128;  // query positions per work-group
constexpr int kPfBuf = 2;     // ring slots: one tile computed while the next lands

// Three work-groups per CU (registers held to 168 per lane, a 40 KiB ring
// each): the tile loop is a chain of dependent MFMA and softmax steps, so
// more waves per SIMD pay more than a deeper ring (measured on the 2 x 4096
// DeepSeek-V3 prompt batch: 2252 us with a 4-slot ring at two groups per CU,
// 2018 us like this).
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
prefill_kernel(PrefillParams p) {
  using Gm = Geo<128>;
  constexpr int KROWS = Gm::GPT;   // 24 granule rows of K
  constexpr int VROWS = 16;        // 16 granule rows of V
  constexpr int TB = (KROWS + VROWS) * kRow;
  constexpr int NI = (KROWS + VROWS) / 8;  // DMA instructions per wave per tile (2 rows each, 4 waves)
  __shared__ __attribute__((aligned(1024))) char tiles[kPfBuf * TB];

  const int w = uniform(threadIdx.x >> 6);
  // XCD-aware placement: work item u = (sequence, head, query tile), longest
  // rows first; the grid (a multiple of 8) is dealt so that consecutive work
  // items land on the same XCD, which keeps each head's keys and values in
  // one L2 while its query tiles, all starting from key tile 0, re-read them.
  const int ntile = (p.P + kPfRows - 1) / kPfRows;
  const int u = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
  if (u >= ntile * p.H * p.B) return;
  const int pair = u / ntile;
  const int b = pair / p.H, h = pair % p.H;
  const int qt = ntile - 1 - u % ntile;  // longest rows first
  const int L = min(p.seq_lens[b], p.P);
  const int q0 = qt * kPfRows;
  if (q0 >= L) return;
  const int nkt = (min(L, q0 + kPfRows) + kTile - 1) / kTile;  // key tiles this group needs
  const int64_t tok0 = (int64_t)b * p.P;

  // Tile kt into ring slot s.  Instruction q of wave w fills granule rows
  // 2c, 2c + 1 with c = 4 q + w: rows 0..15 from the key tile, 16..23 from
  // the records' RoPE keys (lane l brings position 32 kt + (l % 32 ^ 4 (l / 32)),
  // clamped to the prompt), 24..39 from the value tile.
  const int T = (p.P + kTile - 1) / kTile;
  const char* kbase = (const char*)(p.k_nope + ((int64_t)b * p.H + h) * T * (kTile * 128));
  const char* vbase = (const char*)(p.v + ((int64_t)b * p.H + h) * T * (kTile * 128));
  const char* rbase = (const char*)(p.ckr + tok0 * (p.DCK + 64) + p.DCK);
  const uint32_t rec = (uint32_t)(p.DCK + 64) * 2;
  const uint32_t tiles_lds = lds_offset(tiles);
  const int dl = opaque_lane();
  const int rope_tok = (dl & 31) ^ (4 * (dl >> 5));
  auto issue = [&](int kt, int s) {
    const uint32_t dst = tiles_lds + s * TB;
    const uint32_t roff = (uint32_t)min(kt * kTile + rope_tok, L - 1) * rec + 16u * (dl >> 5);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int c = 4 * q + w;  // q 0, 1: key rows; 2: RoPE rows; 3, 4: value rows
      if (q < 2) {
        lds_dma16(kbase + (int64_t)kt * 8192 + c * 1024, 16u * dl, dst + c * 1024);
      } else if (q == 2) {
        lds_dma16(rbase + 32 * (c - 8), roff, dst + c * 1024);
      } else {
        lds_dma16(vbase + (int64_t)kt * 8192 + (c - 12) * 1024, 16u * dl, dst + c * 1024);
      }
    }
  };

  // This wave's 32 query positions.
  const int lane = opaque_lane();
  const int col = lane & 31;
  const int pos = q0 + 32 * w + col;
  bf16x8 qf[Gm::KS];
  {
    const int64_t row = (tok0 + min(pos, L - 1)) * p.H + h;
    const bf16x8* ql = (const bf16x8*)(p.q_nope + row * 128 + 8 * (lane >> 5));
    const bf16x8* qr = (const bf16x8*)(p.q_rope + row * 64 + 8 * (lane >> 5));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
    for (int ks = 8; ks < Gm::KS; ++ks) qf[ks] = qr[2 * (ks - 8)];
  }
  const int limit = min(pos + 1, L);  // causal: this row sees positions < limit

  // The queries have to be in registers before the ring copies start (the
  // compiler counts only its own loads, and would otherwise wait for every
  // copy in flight at their first use).
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  for (int i = 0; i < kPfBuf - 1 && i < nkt; ++i) issue(i, i);

  f32x16 O[Gm::NB];
  float m_run = -__builtin_inff(), l_run = 0.0f;
  bf16x8 pf0, pf1;
  float alpha;
  auto tile = [&](int kt, auto first_tag, auto full_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // FULL: the tile lies wholly below the group's first position, so every
    // row sees all of it (no causal mask, and the softmax takes its
    // branch-free form); a compile-time choice.
    constexpr bool FULL = decltype(full_tag)::value;
    // tile kt has landed (for every wave) and slot (kt - 1) % NBUF is free
    if (kt + kPfBuf - 2 < nkt) vm_wait<(kPfBuf - 2) * NI>(); else vm_wait<0>();
    block_sync();
    if (kt + kPfBuf - 1 < nkt) issue(kt + kPfBuf - 1, (kt + kPfBuf - 1) % kPfBuf);
    const char* tb = tiles + (kt % kPfBuf) * TB;
    score_tile<128, false, 0>(tb, nullptr, qf, m_run, l_run, kt * kTile, limit, FULL, p.scale_log2, pf0, pf1,
                              alpha, NoDma{});
    if constexpr (!FIRST) {
      if (__any(alpha != 1.0f)) rescale<128>(O, alpha);
    }
    pv_tile<128, kPvAhead, FIRST>(tb + KROWS * kRow, pf0, pf1, O);
  };
  // Key tiles 0 .. kfull - 1 lie below the group's first position q0.
  const int kfull = min(nkt, q0 / kTile);
  int kt = 1;
  if (kfull > 0) {
    tile(0, std::true_type{}, std::true_type{});
    for (; kt < kfull; ++kt) tile(kt, std::false_type{}, std::true_type{});
  } else {
    tile(0, std::true_type{}, std::false_type{});
  }
  for (; kt < nkt; ++kt) tile(kt, std::false_type{}, std::false_type{});

  // Normalise and write this wave's rows: lane (col, half) holds row `col`,
  // columns 32 nb + 8 (i / 4) + 4 half + i % 4 of block nb.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (pos < L) {
    const int half = opaque_lane() >> 5;
    const int64_t row = (tok0 + pos) * p.H + h;
    if (half == 0) p.lse[row] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
    uint16_t* dst = p.out + row * 128 + 4 * half;
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 a = {(__bf16)(O[nb][4 * q] * inv), (__bf16)(O[nb][4 * q + 1] * inv)};
        const bf16x2 c = {(__bf16)(O[nb][4 * q + 2] * inv), (__bf16)(O[nb][4 * q + 3] * inv)};
        *(uint2*)(dst + 32 * nb + 8 * q) = uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)};
      }
    }
  }
}

}  // namespace

int decode_waves(int R) { return R <= 32 ? 1 : (R <= 64 ? 2 : 4); }
int decode_row_groups(int R) {
  const int rows = 32 * decode_waves(R);
  return (R + rows - 1) / rows;
}
int decode_wgs_per_cu(int R, int d_latent) {
  (void)d_latent;
  return decode_waves(R) == 4 ? 1 : 2;
}

hipError_t launch_decode(const DecodeParams& p, int d_latent, bool fp8, hipStream_t stream) {
  const int nw = decode_waves(p.R);
  if (d_latent == 512) return fp8 ? launch_dc<512, true>(p, nw, stream) : launch_dc<512, false>(p, nw, stream);
  return fp8 ? launch_dc<256, true>(p, nw, stream) : launch_dc<256, false>(p, nw, stream);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.B <= 0 || p.P <= 0) return hipSuccess;
  const int64_t items = (int64_t)((p.P + kPfRows - 1) / kPfRows) * p.H * p.B;
  const dim3 grid((unsigned)((items + 7) / 8 * 8));
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
