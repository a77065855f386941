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
// max m, the running sum l and O^T[512 or 256, 32] in accumulators (with at
// most 32 rows and a latency-bound launch, the two waves of a work-group may
// own the same rows instead: both compute the scores and the softmax, and
// each accumulates half of O^T's latent columns).  The softmax is online
// (BLASST abstract on the same listing relies on the same running state),
// with the max only re-based when it grows by more than 2^8 so the
// accumulator rescale is rare.  A work-group of NW waves shares each
// tile; tiles stream through an LDS ring (direct global->LDS DMA for bf16;
// for fp8 the same DMA into a staging slot, then an exact e4m3->bf16 decode
// in LDS).  Each sequence's token axis is cut into parts of W tiles (the
// split plan of split_plan.h); each part writes one normalised partial and
// its log-sum-exp.
//
// The tile products, the online softmax and the LDS tile layout are in
// tile_ops.h (shared with the prefill).
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "tile_ops.h"
#include "decode_common.h"
#include "split_plan.h"

namespace mla {
namespace {

constexpr int kTab = 128;  // tiles per LDS source-table fill

__device__ __forceinline__ int seq_of_tile(const int* cu, int B, int k) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= k) lo = mid; else hi = mid - 1;
  }
  return lo;
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

// Zero the slots of tokens nv..31 of a tile (the last, partial tile of a
// sequence): their DMA'd contents are whatever the page held past the length.
template <int DC, int NW>
__device__ __forceinline__ void zero_tail(char* tb, int nv, int tid) {
  for (int i = tid; i < Geo<DC>::GPT * kTile; i += NW * kWave) {
    const int g = i >> 5, slot = i & 31;
    if ((slot ^ ((g & 1) << 2)) >= nv) *(uint4*)(tb + g * kRow + slot * 16) = uint4{0, 0, 0, 0};
  }
}

// Pitch of one row of NBK staged fp16 column blocks: the row plus 16 bytes,
// so that the rows of one LDS write instruction start in different banks.
template <int NBK>
constexpr int stage_pitch() { return NBK * 64 + 16; }

// The same write as store_partial<NB> for fp16 partials, through LDS: the
// wave puts its 32 normalised rows of NB column blocks (latent columns col0 ..
// col0 + 32 NB) into `stage` (row = lane % 32), then writes them back out
// with every store instruction covering whole rows (NB * 64 contiguous
// bytes), instead of 32 rows x 32 bytes per instruction.  `stage` is this
// wave's own region; nothing else may use it meanwhile.
template <int DC, int NB>
__device__ __forceinline__ void store_partial_staged(const DecodeParams& p, const f32x16* O, float inv, int64_t slot,
                                                     int rowbase, int col0, char* stage) {
  constexpr int PITCH = stage_pitch<NB>();
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
  constexpr int LPR = NB * 4;       // lanes per row (16 bytes each)
  constexpr int RPI = kWave / LPR;  // rows per store instruction
  const int sub = lane / LPR, gi = lane % LPR;
#pragma unroll 4
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + sub;
    const uint4 x = *(const uint4*)(stage + r * PITCH + 16 * gi);
    if (rowbase + r < p.R) *(uint4*)((_Float16*)p.o_part + (slot * p.R + rowbase + r) * DC + col0 + 8 * gi) = x;
  }
}

// CS: waves that share each query row, each accumulating NB / CS of the
// latent column blocks (1, or 2 for at most 32 rows per work-group).
template <int DC, bool FP8, int NW, int NBUF, int CS>
__global__ void __launch_bounds__(NW * kWave)
    decode_kernel(DecodeParams p, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table,
                  const float* __restrict__ kv_scale) {
  using Gm = Geo<DC>;
  constexpr int TB = Gm::TILE_BYTES;
  constexpr int NI = Gm::GPT / (2 * NW);
  constexpr int AHEAD = NBUF - 1;  // tiles in flight ahead of the one computed
  constexpr int RW = 32 * NW / CS;  // query rows per work-group
  constexpr int NBW = Gm::NB / CS;  // accumulator blocks per wave
  static_assert(NW % CS == 0 && Gm::NB % CS == 0, "column slices must divide the waves and the blocks");
  static_assert(Gm::GPT % (2 * NW) == 0, "tile rows must split evenly over the waves");
  static_assert(AHEAD >= 1, "ring too small");
  static_assert(FP8 || NI * AHEAD <= 63, "DMA groups must fit vmcnt");
  static_assert(!FP8 || AHEAD == 1, "fp8 tiles are staged one ahead");

  __shared__ __attribute__((aligned(1024))) char tiles[NBUF * TB];
  __shared__ __attribute__((aligned(16))) float tscale[FP8 ? NBUF * kTile : 4];
  __shared__ __attribute__((aligned(1024))) char f8stage[FP8 ? Fp8Geo<DC>::BYTES : 16];
  __shared__ int cu[kMaxBatch + 1];
  __shared__ int4 tab[kTab];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int wr = w / CS, wc = w % CS;  // this wave's row slot and column slice
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware placement: consecutive work items (the row groups of one token
  // part, then neighbouring parts) land on the same XCD, whose L2 they share.
  int u = blockIdx.x;
  if ((gridDim.x & 7) == 0) u = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int g = u / p.RG, rg = u % p.RG;

  // The split plan: part g is tiles [j W, min((j + 1) W, n_b)) of one
  // sequence b; k0 .. k1 are those tiles in the batch-wide tile numbering.
  __shared__ int plan[3];
  if (w == 0) {
    build_tile_prefix(seq_lens, p.B, cu, lane);
    with_plan(seq_lens, p.B, p.P, lane, [&](const auto& pl) {
      int b = -1, s_b = 0;
      if (g < pl.total) pl.locate_slot(g, lane, b, s_b);
      if (lane == 0) {
        plan[0] = b;
        plan[1] = (g - s_b) * pl.W;
        plan[2] = pl.W;
      }
    });
  }
  block_sync();
  const int pb = uniform(plan[0]);
  if (pb < 0) return;
  const int k0 = uniform(cu[pb]) + uniform(plan[1]);
  const int k1 = min(k0 + uniform(plan[2]), uniform(cu[pb + 1]));

  const int row = rg * RW + 32 * wr + col;  // this lane's query row (S^T column)
  const uint32_t tiles_lds = lds_offset(tiles);

  // The first segment's query rows are touched (one dword per 128-byte line)
  // while the tile-table reads are in flight, so that the wave's own query
  // loads below hit L2 instead of making a further trip to HBM.
  int bc = uniform(seq_of_tile(cu, p.B, k0));
  uint32_t touch = 0;
  {
    const char* qa = (const char*)(p.q_lat + ((int64_t)bc * p.R + rg * RW) * DC);
    const char* qb = (const char*)(p.q_rope + ((int64_t)bc * p.R + rg * RW) * 64);
    const int rows = min(RW, p.R - rg * RW);
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

  // fp8: tile kl's bytes are copied into the staging slot (and its tokens'
  // scales loaded) one tile ahead; stage_finish decodes them into its ring slot.
  float f8_scale = 0.0f;
  auto stage_start = [&]() {
    issue_fp8_dma<DC, NW>(p, src, lds_offset(f8stage), w);
    if (w == 0 && lane < kTile) f8_scale = kv_scale[(int64_t)spage * p.block_size + (spos & (p.block_size - 1)) + lane];
  };
  auto stage_finish = [&]() {
    const int nbuf = (kl - k0) % NBUF;
    vm_wait<0>();
    block_sync();  // every wave's copies have landed
    convert_fp8_tile<DC, NW>(f8stage, tiles + nbuf * TB, snv, tid);
    if (w == 0 && lane < kTile) tscale[nbuf * kTile + lane] = lane < snv ? f8_scale : 0.0f;
    ++kl;
    if (kl < k1) locate();
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
      const int qrow = rg * RW + 32 * wr + (ln & 31);
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
    f32x16 O[NBW];
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
        if (__any(alpha != 1.0f)) rescale(O, alpha);
      }
      pv_tile<DC, kPvAhead, FIRST>(tiles + buf * TB + wc * NBW * 4 * kRow, pf0, pf1, O);
      tile_end();
      ++k;
    };
    // The segment's first tile starts the sums (general path); then the tiles
    // every row sees in full run branch-free; then the masked tail.
    one_tile(std::true_type{}, std::false_type{});
    const int kfull = min(kend, cub + lim_all / kTile);
    while (k < kfull) one_tile(std::false_type{}, std::true_type{});
    while (k < kend) one_tile(std::false_type{}, std::false_type{});

    // ---- normalise and write this (sequence, part) partial
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
    const int64_t slot = g;
    // The lse goes first: vector stores count in vmcnt, so any wait the
    // compiler places before a later store (a spilled address being reloaded)
    // would otherwise also wait for the whole partial to be written.
    {
      // lane-derived indices recomputed here rather than kept live (and
      // spilled) across the tile loop
      const int ln = opaque_lane();
      const int lhalf = ln >> 5, lcol = ln & 31;
      const int lrow = rg * RW + 32 * wr + lcol;
      if (lrow < p.R && lhalf == 0 && wc == 0) p.lse_part[slot * p.R + lrow] = lse;
      // After the part's last tile the ring is idle (every copy has landed and
      // been consumed), so an fp16 partial is staged through it.
      constexpr bool STAGE_FITS = NW * 32 * stage_pitch<NBW>() <= NBUF * TB;
      if (STAGE_FITS && p.o_half && kend == k1) {
        block_sync();
        store_partial_staged<DC, NBW>(p, O, inv, slot, rg * RW + 32 * wr, wc * NBW * 32,
                                      tiles + w * 32 * stage_pitch<NBW>());
      } else if (lrow < p.R) {
        store_partial<NBW>(p, O, inv, (slot * p.R + lrow) * DC + wc * NBW * 32, lhalf);
      }
    }
    ++bc;
    while (bc < p.B - 1 && uniform(cu[bc + 1]) == uniform(cu[bc])) ++bc;
    if (k >= k1) break;
  }
}

template <int DC, bool FP8, int NW, int NBUF, int CS>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const int grid = p.P * p.RG;
  hipLaunchKernelGGL((decode_kernel<DC, FP8, NW, NBUF, CS>), dim3(grid), dim3(NW * kWave), 0, stream, p,
                     p.seq_lens, p.block_table, p.kv_scale);
  return hipGetLastError();
}

// Work-groups run two per CU on a 2-tile ring; 128-row groups use
// decode_wide.hip.  Up to 64 query rows, two waves own 32 rows each.  Up to
// 32 rows, one wave issues a tile's copies and both products itself, and two
// such work-groups per CU keep the CU's copy path busy (it bounds the tile
// loop, so splitting a tile's work over more waves only adds a barrier per
// tile) -- unless the block table holds at most one tile per two part slots:
// then every part is one tile on an otherwise idle CU, the launch is bound
// by the latency of that one tile, and two waves that split the latent
// columns between them (both computing the scores) finish it sooner.
template <int DC, bool FP8>
hipError_t launch_dc(const DecodeParams& p, int nw, hipStream_t stream) {
  if (nw == 2) return launch_one<DC, FP8, 2, 2, 1>(p, stream);
  const int64_t max_tiles = (int64_t)p.B * p.bt_stride * p.block_size / kTile;
  if (2 * max_tiles <= p.P) return launch_one<DC, FP8, 2, 2, 2>(p, stream);
  return launch_one<DC, FP8, 1, 2, 1>(p, stream);
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
  if (nw == 4) return launch_decode_wide(p, d_latent, fp8, stream);
  if (d_latent == 512) return fp8 ? launch_dc<512, true>(p, nw, stream) : launch_dc<512, false>(p, nw, stream);
  return fp8 ? launch_dc<256, true>(p, nw, stream) : launch_dc<256, false>(p, nw, stream);
}

}  // namespace mla
