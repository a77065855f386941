// Split-K decode of absorbed MLA for 128 query rows per work-group over a
// latent-split shard (d_c = 256), two 32-token tiles per step (gfx950).
//
// The method and the division of a tile's work between the four waves are
// those of decode_wide.hip (MQA form of MLA after the absorb, GQLA abstract on
// the "GQA-to-MLA" Daily Papers listing; one shard of the latent split, TPLA
// abstract): wave w scores query rows 32w .. 32w+31 against the tile from
// LDS and runs their online softmax, then accumulates latent columns
// 64w .. 64w+63 of O^T for all 128 rows from P shared through LDS, one step
// late.  At d_c = 256 a tile carries half the MFMA work of d_c = 512 while the
// costs paid once per step stay the same (the barrier, the softmax's
// cross-lane reductions and its rebase test, the publication of P, the copy
// set-up), so a step here takes two tiles:
//
//   * the two tiles' score chains are interleaved, so that no MFMA waits for
//     the accumulation of the one before it;
//   * one online-softmax update covers both tiles' 64 positions;
//   * one publication of P (16 KiB) and one barrier per pair.
//
// The registers that d_c = 256 leaves free (O^T is 128 accumulators per lane
// instead of 256, the query 80 VGPRs instead of 144) hold the second score
// accumulator and the doubled P operands.  The LDS ring holds three pairs:
// the one scored, the one whose P . V is pending, the copy in flight.
//
// A part with an odd number of tiles ends on a pair whose second tile is not
// the part's: its slot is filled with copies of the first tile's first record
// (finite data, never read past the part's pages) and every one of its
// positions is masked, so its weights are 0.
#include "decode_common.h"
#include "mla_device.h"
#include "mla_kernels.h"
#include "split_plan.h"
#include "tile_ops.h"
#include "wide_common.h"

namespace mla {
namespace {

template <int DC>
struct Pair {
  using Gm = Geo<DC>;
  static constexpr int NW = 4;                   // waves
  static constexpr int ROWS = 32 * NW;           // query rows of a work-group
  static constexpr int NBW = Gm::NB / NW;        // 32-column blocks of O per wave
  static constexpr int TB = Gm::TILE_BYTES;      // one tile image
  static constexpr int NSLOT = 3;                // pair slots: scored, P . V pending, copy in flight
  static constexpr int NI = Gm::GPT / (2 * NW);  // copy instructions per wave per tile
  static constexpr int PB = NW * 4 * 1024;       // P of a pair: [row block][k-step 0..3][lane] x 16 B
  static_assert(Gm::GPT % (2 * NW) == 0, "tile rows must split evenly over the waves");
  static_assert(Gm::NB % NW == 0, "latent blocks must split evenly over the waves");
};

// The copy of one pair, one instruction at a time (issue(q), q < 2 NI: the
// first tile's NI instructions, then the second's), for the score chains to
// spread over their MFMAs; inactive when there is no pair left to copy.
template <int DC>
struct PairDma {
  static constexpr int NW = 4, NI = Geo<DC>::GPT / (2 * NW);
  const char* run0;
  const char* run1;
  int64_t rope_off;
  uint32_t lane_off0, lane_off1, buf_lds;
  int w;
  bool active;
  __device__ __forceinline__ void issue(int q) const {
    if (!active) return;
    const int s = q / NI, qq = q % NI;
    const int g0 = 2 * (qq * NW + w);
    const int64_t off = g0 < Geo<DC>::GC ? (int64_t)g0 * 16 : rope_off + (int64_t)(g0 - Geo<DC>::GC) * 16;
    lds_dma16((s ? run1 : run0) + off, s ? lane_off1 : lane_off0,
              uniform(buf_lds + s * Geo<DC>::TILE_BYTES + (qq * NW + w) * 1024));
  }
};

template <int DC>
__device__ __forceinline__ PairDma<DC> pair_dma(const DecodeParams& p, const TileSrc& a, const TileSrc& b,
                                                uint32_t slot_lds, int w, bool active) {
  const int ol = opaque_lane();
  const int tok = load_token(ol);
  const uint32_t hoff = 16u * (ol >> 5);
  PairDma<DC> d;
  d.run0 = a.run;
  d.run1 = b.run;
  d.rope_off = p.rope_off;
  d.lane_off0 = (uint32_t)(tok < a.nv ? tok : 0) * (uint32_t)p.token_stride + hoff;
  d.lane_off1 = (uint32_t)(tok < b.nv ? tok : 0) * (uint32_t)p.token_stride + hoff;
  d.buf_lds = slot_lds;
  d.w = w;
  d.active = active;
  return d;
}

// The sources of pair j's two tiles (t = ta, ta + 1).  A second tile past the
// part re-reads the first tile's run with no valid token.
__device__ __forceinline__ void pair_srcs(const DecodeParams& p, int page_a, int page_b, int ta, bool has_b, int L,
                                          TileSrc& a, TileSrc& b) {
  a = tile_src(p, page_a, ta, L);
  if (has_b) {
    b = tile_src(p, page_b, ta + 1, L);
  } else {
    b = a;
    b.nv = 0;
  }
}

// S^T of both tiles of a pair against the wave's 32 query rows: two
// accumulator chains, interleaved MFMA by MFMA.  K fragments of both tiles
// are read kScoreAhead k-steps ahead; dma.issue spreads the next pair's copy
// over the MFMAs; pre.load() runs before the MFMAs of k-step Pre::AT.
template <int DC, int NDMA, class Dma, class Pre>
__device__ __forceinline__ void score_pair(const char* ta, const bf16x8 (&qf)[Geo<DC>::KS], const Dma& dma,
                                           Pre& pre, f32x16& sa, f32x16& sb) {
  using Gm = Geo<DC>;
  constexpr int PD = kScoreAhead;
  constexpr int TB = Gm::TILE_BYTES;
  static_assert(Gm::KS % NDMA == 0, "copy instructions must divide the k-steps");
  const int lane = opaque_lane();
  const int half = lane >> 5, col = lane & 31;
  const char* ka = ta + half * kRow + ((col ^ (half << 2)) << 4);
  bf16x8 fa[Gm::KS], fb[Gm::KS];
#pragma unroll
  for (int ks = 0; ks < PD; ++ks) {
    fa[ks] = *(const bf16x8*)(ka + ks * 2 * kRow);
    fb[ks] = *(const bf16x8*)(ka + TB + ks * 2 * kRow);
  }
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    if (ks + PD < Gm::KS) {
      fa[ks + PD] = *(const bf16x8*)(ka + (ks + PD) * 2 * kRow);
      fb[ks + PD] = *(const bf16x8*)(ka + TB + (ks + PD) * 2 * kRow);
    }
    if (ks % (Gm::KS / NDMA) == 0) dma.issue(ks / (Gm::KS / NDMA));
    if (ks == Pre::AT) pre.load();
    if (ks == 0) {
      mfma_v_first(sa, fa[ks], qf[ks]);
      mfma_v_first(sb, fb[ks], qf[ks]);
    } else if (ks + 1 < Gm::KS) {
      mfma_v_acc(sa, fa[ks], qf[ks]);
      mfma_v_acc(sb, fb[ks], qf[ks]);
    } else {
      // sa's result is read only after sb's last MFMA and its wait states
      mfma_v_acc(sa, fa[ks], qf[ks]);
      mfma_v_last(sb, fb[ks], qf[ks]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Online softmax of a pair's scores for the wave's 32 rows, in steps that
// pv_pair spreads over its MFMAs.  Lane (col, half) holds row col; value i of
// va (vb) is the first (second) tile's token 8(i/4) + 4 half + i%4, visible
// iff 8(i/4) + i%4 < rel (relb), rel = (first position the row may not see)
// - (pair start) - 4 half, relb = rel - 32, or -32 (nothing visible) when the
// part has no second tile: the positions past the part's last tile may lie
// inside the sequence, but they belong to the next part.  The same arithmetic as WideSoftmax over 64
// positions: maximum of the raw scores, lazy re-base, weights by one fused
// multiply-add and exp2, P packed to bf16 as [tile][k-step] operands.
struct PairSoftmax {
  static constexpr int STEPS = 20;
  f32x16 va, vb;
  int rel, relb;
  float slog2;
  float& m_run;
  float& l_run;
  float m_new, mu, alpha;
  bf16x8 pf[4];

  __device__ __forceinline__ void step(int j) {
    if (j < 8) {  // mask four entries
      const int r = j < 4 ? rel : relb;
      const int q = j & 3;
      f32x16& v = j < 4 ? va : vb;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * q + c] = (8 * q + c < r) ? v[4 * q + c] : -__builtin_inff();
    } else if (j == 8) {
      float m8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        m8[i] = fmaxf(fmaxf(va[2 * i], va[2 * i + 1]), fmaxf(vb[2 * i], vb[2 * i + 1]));
      m_new = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])), fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
    } else if (j == 9) {
      const float mt = pair_max(m_new) * slog2;
      const bool rebase = mt > m_run + kRebase;  // never for a pair this row sees nothing of (mt = -inf)
      m_new = rebase ? mt : m_run;
      alpha = rebase ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 on the first visible pair
      l_run *= alpha;
      m_run = m_new;
      // A row that has seen no position yet keeps m = -inf with every entry
      // at -inf: exp2(-inf - 0) gives the weights 0 instead of NaN.
      mu = m_new == -__builtin_inff() ? 0.0f : m_new;
    } else if (j < 18) {  // weights, four at a time
      const int q = (j - 10) & 3;
      f32x16& v = j < 14 ? va : vb;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * q + c] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[4 * q + c], slog2, -mu));
    } else if (j == 18) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = (va[2 * i] + va[2 * i + 1]) + (vb[2 * i] + vb[2 * i + 1]);
      l_run += ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    } else if (j == 19) {
      float w8[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x16& v = k < 2 ? va : vb;
#pragma unroll
        for (int i = 0; i < 8; ++i) w8[i] = v[8 * (k & 1) + i];
        pf[k] = pack_bf16x8(w8);
      }
    }
  }
  __device__ __forceinline__ void all() {
#pragma unroll
    for (int j = 0; j < STEPS; ++j) step(j);
  }
};

// Operands of the lagged P . V of a pair for this wave's column blocks over
// all four row blocks: P from LDS (`pb`: [row block][k-step 0..3][lane] x
// 16 B; k-steps 0, 1 the first tile's, 2, 3 the second's), V^T through
// transposing reads of the two tile images of the slot at `tb` (the lane
// pattern of pv_tile in tile_ops.h).  load() reads P and the first column
// block's V; the score chains call it before their last k-steps.
template <int DC>
struct PairPv {
  static constexpr int AT = Geo<DC>::KS - 6;
  struct VF { s16x4 x0, x1, y0, y1; };
  const char* vb;
  const char* pb;
  bf16x8 pf[4][4];
  VF v0[2];
  __device__ __forceinline__ PairPv(const char* tb, const char* pb_, int w) : pb(pb_) {
    const int lane = opaque_lane();
    const int half = lane >> 5;
    const int i16 = lane & 15, grp = lane >> 4;
    const int jj = i16 >> 2, qq = i16 & 3, ch = grp & 1;
    const int godd = qq >> 1;
    vb = tb + (2 * ch + godd) * kRow + (((4 * half + jj) ^ (godd << 2)) << 4) + ((qq & 1) << 3) +
         w * (Geo<DC>::NB / 4) * 4 * kRow;
  }
  __device__ __forceinline__ VF vread(int s, int cb) const {
    const char* a = vb + s * Geo<DC>::TILE_BYTES + cb * 4 * kRow;
    VF f;
    f.x0 = lds_read_tr16(a);
    f.x1 = lds_read_tr16(a + 8 * 16);
    f.y0 = lds_read_tr16(a + 16 * 16);
    f.y1 = lds_read_tr16(a + 24 * 16);
    return f;
  }
  __device__ __forceinline__ void load() {
    const int lane = opaque_lane();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int k = 0; k < 4; ++k) pf[rb][k] = *(const bf16x8*)(pb + (rb * 4 + k) * 1024 + lane * 16);
    v0[0] = vread(0, 0);
    v0[1] = vread(1, 0);
  }
};

// The no-op publication hook of pv_pair.
struct NoPublishPair {
  __device__ __forceinline__ void operator()() const {}
};

// P . V of a pair (operands already loaded) with the softmax steps of the
// next pair placed between the column blocks, front-loaded, and pub() right
// after the last step.
template <int DC, bool STEPS, class SM, class Pub = NoPublishPair>
__device__ __forceinline__ void pv_pair(const PairPv<DC>& op, f32x16 (&O)[4][Geo<DC>::NB / 4], SM& sm,
                                        const Pub& pub = Pub{}) {
  constexpr int NBW = Geo<DC>::NB / 4;
  using VF = typename PairPv<DC>::VF;
  // softmax steps per column block: ceil(2 STEPS / (2 NBW - 1))
  constexpr int SPB = (2 * SM::STEPS + 2 * NBW - 2) / (2 * NBW - 1);
  VF cur[2] = {op.v0[0], op.v0[1]};
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    VF nxt[2];
    if (cb + 1 < NBW) {
      nxt[0] = op.vread(0, cb + 1);
      nxt[1] = op.vread(1, cb + 1);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const VF& c = cur[s];
      const s16x8 a0 = {c.x0[0], c.x0[1], c.x0[2], c.x0[3], c.x1[0], c.x1[1], c.x1[2], c.x1[3]};
      const s16x8 a1 = {c.y0[0], c.y0[1], c.y0[2], c.y0[3], c.y1[0], c.y1[1], c.y1[2], c.y1[3]};
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        O[rb][cb] = mfma32((bf16x8)a0, op.pf[rb][2 * s], O[rb][cb]);
        O[rb][cb] = mfma32((bf16x8)a1, op.pf[rb][2 * s + 1], O[rb][cb]);
      }
    }
    if constexpr (STEPS) {
#pragma unroll
      for (int j = 0; j < SPB; ++j)
        if (cb * SPB + j < SM::STEPS) sm.step(cb * SPB + j);
      if (cb * SPB < SM::STEPS && (cb + 1) * SPB >= SM::STEPS) pub();
    }
    if (cb + 1 < NBW) {
      cur[0] = nxt[0];
      cur[1] = nxt[1];
    }
  }
}

template <int DC>
__global__ void __launch_bounds__(256)
    decode_wide_pair_kernel(DecodeParams p, const int32_t* __restrict__ seq_lens,
                            const int32_t* __restrict__ block_table) {
  using Pr = Pair<DC>;
  using Gm = Geo<DC>;
  constexpr int NW = Pr::NW, ROWS = Pr::ROWS, NBW = Pr::NBW, TB = Pr::TB, NSLOT = Pr::NSLOT, PB = Pr::PB;
  constexpr int NI = Pr::NI;

  __shared__ __attribute__((aligned(1024))) char tiles[NSLOT * 2 * TB];
  __shared__ __attribute__((aligned(1024))) char pbuf[2 * PB];
  __shared__ __attribute__((aligned(16))) float alph[2][ROWS];
  __shared__ __attribute__((aligned(16))) int rflag[2][NW];
  __shared__ float fin_l[ROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware placement, as in decode_wide_kernel.
  int u = blockIdx.x;
  if ((gridDim.x & 7) == 0) u = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int g = u / p.RG, rg = u % p.RG;

  // The split plan, in every wave.
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
  const int np = (n + 1) >> 1;     // pairs
  L = uniform(L);
  const int32_t* bt = block_table + (int64_t)b * p.bt_stride;
  const int rowbase = rg * ROWS;
  const uint32_t tiles_lds = lds_offset(tiles);

  // ---- prologue (as in decode_wide_kernel): the page reads, the query block
  // (the first half of its k-steps staged row-contiguous through LDS slot 1,
  // the rest loaded directly), then the first pair's copies.
  constexpr int KST = DC / 32;
  constexpr int CPR = 2 * KST;
  constexpr int SROW = CPR * 16;
  constexpr int RPI = 1024 / SROW;
  static_assert(NW * 32 * SROW <= (NSLOT - 1) * 2 * TB, "the staged query fits the free slots");
  char* stg = tiles + 2 * TB + w * 32 * SROW;
  const int qrow0 = rowbase + 32 * w;
  const char* qseq = (const char*)(p.q_lat + (int64_t)b * p.R * DC);
  const int pga = tile_page_load(p, bt, t0);
  const int pgb = n > 1 ? tile_page_load(p, bt, t0 + 1) : 0;
  // pages of the next pair to copy (pair 1)
  int pfa = n > 2 ? tile_page_load(p, bt, t0 + 2) : 0;
  int pfb = n > 3 ? tile_page_load(p, bt, t0 + 3) : 0;
  {
    const int ol = opaque_lane();
    const int rr = ol / CPR, cs = ol % CPR;
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int r = j * RPI + rr;
      const int rg_ = min(qrow0 + r, p.R - 1);  // rows past R re-read row R-1 (discarded)
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
    TileSrc sa, sb;
    pair_srcs(p, uniform(pga), uniform(pgb), t0, n > 1, L, sa, sb);
    copy_tile<DC>(p, sa, tiles_lds, w);
    copy_tile<DC>(p, sb, tiles_lds + TB, w);
  }
#pragma unroll
  for (int ks = KST; ks < Gm::KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  vm_wait<0>();
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
  const int my_row = rowbase + 32 * w + col;
  const int limit = min(L - p.S + 1 + my_row / p.H, L);  // first position this lane's row may not see
  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x16 O[4][NBW];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) O[rb][cb] = f32x16{};

  // One pair step: (a) pair j is in LDS, P of pair j - 1 is visible, the slot
  // the next copy overwrites is free; (b) the copy of pair j + 1 spread over
  // the score chains; (c) the scores and softmax of pair j with, from the
  // second pair on (PV), the P . V of pair j - 1.
  auto pair_step = [&](int j, auto pv_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    const int ta = t0 + 2 * j;
    const int slot = j % NSLOT;
    vm_wait<0>();  // pair j and the page indices read with it
    block_sync();
    int4 fl = int4{0, 0, 0, 0};
    if constexpr (PV) fl = *(const int4*)rflag[(j - 1) & 1];
    TileSrc na, nb;
    pair_srcs(p, uniform(pfa), uniform(pfb), ta + 2, 2 * j + 3 < n, L, na, nb);
    const PairDma<DC> dma = pair_dma<DC>(p, na, nb, tiles_lds + ((j + 1) % NSLOT) * 2 * TB, w, j + 1 < np);
    if (2 * j + 4 < n) pfa = tile_page_load(p, bt, ta + 4);
    if (2 * j + 5 < n) pfb = tile_page_load(p, bt, ta + 5);
    const int pos0 = ta * kTile;
    PairPv<DC> pv(tiles + ((j + NSLOT - 1) % NSLOT) * 2 * TB, pbuf + ((j - 1) & 1) * PB, w);
    const int rel = limit - pos0 - 4 * half;
    PairSoftmax sm{{}, {}, rel, 2 * j + 1 < n ? rel - kTile : -kTile, p.scale_log2, m_run, l_run};
    if constexpr (PV) {
      score_pair<DC, 2 * NI>(tiles + slot * 2 * TB, qf, dma, pv, sm.va, sm.vb);
    } else {
      NoPre none;
      score_pair<DC, 2 * NI>(tiles + slot * 2 * TB, qf, dma, none, sm.va, sm.vb);
    }
    if constexpr (PV) {
      if (fl.x | fl.y | fl.z | fl.w) {
        const int pbi = (j - 1) & 1;
        float a[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[rb] = alph[pbi][32 * rb + col];
        rescale_rows<NBW>(O, a);
      }
    }
    // Publish P and the rescale factor of pair j; their buffers [j & 1] were
    // last read in iteration j - 1, before this iteration's barrier.
    auto publish = [&]() {
      char* pw = pbuf + (j & 1) * PB + (w * 4) * 1024 + lane * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) *(bf16x8*)(pw + k * 1024) = sm.pf[k];
      if (half == 0) alph[j & 1][32 * w + col] = sm.alpha;
      const bool any = PV && __any(sm.alpha != 1.0f);
      if (lane == 0) rflag[j & 1][w] = any;
    };
    if constexpr (PV) {
      pv_pair<DC, true>(pv, O, sm, publish);
    } else {
      sm.all();
      publish();
    }
  };
  pair_step(0, std::false_type{});
#pragma nounroll
  for (int j = 1; j < np; ++j) pair_step(j, std::true_type{});
  // ---- drain: P . V of the last pair
  block_sync();
  {
    const int pbi = (np - 1) & 1;
    if (rflag[pbi][0] | rflag[pbi][1] | rflag[pbi][2] | rflag[pbi][3]) {
      float a[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[rb] = alph[pbi][32 * rb + col];
      rescale_rows<NBW>(O, a);
    }
    NoSteps none;
    PairPv<DC> pv(tiles + ((np - 1) % NSLOT) * 2 * TB, pbuf + pbi * PB, w);
    pv.load();
    pv_pair<DC, false>(pv, O, none);
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

}  // namespace

hipError_t launch_decode_wide_pair(const DecodeParams& p, int d_latent, hipStream_t stream) {
  if (d_latent != 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_wide_pair_kernel<256>), dim3(p.P * p.RG), dim3(256), 0, stream, p, p.seq_lens,
                     p.block_table);
  return hipGetLastError();
}

}  // namespace mla
