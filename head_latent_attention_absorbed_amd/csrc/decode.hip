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
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRebase = 8.0f;  // log2 of the largest unnormalised weight kept between re-bases

__device__ __forceinline__ void block_sync() {
  // Work-group barrier for LDS hand-offs: waits for this wave's LDS traffic,
  // leaves its global loads in flight.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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
  static constexpr int GPT = GC + GR;            // granules per token in LDS
  static constexpr int TILE_BYTES = kTile * GPT * 16;
  static constexpr int KS = (DC + 64) / 16;      // k-steps of the score product
  static constexpr int NB = DC / 32;             // 32-column blocks of O^T
};

// bf16 tile: direct DMA of the 16-byte granules into the swizzled LDS layout.
// Slot s of the tile (LDS byte 16*s) holds granule (s % GPT) ^ swz(t) of token
// t = s / GPT; a lane's NI slots are fixed, so their byte offsets inside a
// 32-token run of a page are computed once.  A tile always copies all 32
// slots of its run (they lie inside one allocated page); rows past the
// sequence length are zeroed in LDS afterwards (zero_tail), so stale or NaN
// slot contents never reach the P.V product.
template <int DC, int NW>
struct DmaPlan {
  using Gm = Geo<DC>;
  static constexpr int NI = kTile * Gm::GPT / (kWave * NW);
  uint32_t off[NI];

  __device__ __forceinline__ void init(const DecodeParams& p, int w, int lane) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int s = (q * NW + w) * kWave + lane;
      const int t = s / Gm::GPT;
      const int gr = (s % Gm::GPT) ^ swz(t);
      off[q] = (uint32_t)t * (uint32_t)p.token_stride +
               (gr < Gm::GC ? (uint32_t)gr * 16u : (uint32_t)p.rope_off + (uint32_t)(gr - Gm::GC) * 16u);
    }
  }
  // Issue this wave's NI loads of tile j of sequence b into the LDS buffer at buf_lds.
  __device__ __forceinline__ void issue(const DecodeParams& p, const int32_t* __restrict__ block_table, int b, int j,
                                        uint32_t buf_lds, int w) const {
    b = uniform(b);
    j = uniform(j);
    const int pos0 = j * kTile;
    const int page = block_table[(int64_t)b * p.bt_stride + pos0 / p.block_size];
    const char* base = p.c_kv + (int64_t)page * p.block_stride + (int64_t)(pos0 % p.block_size) * p.token_stride;
#pragma unroll
    for (int q = 0; q < NI; ++q) lds_dma16(base, off[q], uniform(buf_lds + (q * NW + w) * 1024));
  }
};

// Zero the LDS rows of tokens nv..31 of a tile (the last, partial tile of a sequence).
template <int DC, int NW>
__device__ __forceinline__ void zero_tail(char* tb, int nv, int tid) {
  constexpr int ROW = Geo<DC>::GPT * 16;
  for (int o = nv * ROW + tid * 16; o < kTile * ROW; o += NW * kWave * 16) *(uint4*)(tb + o) = uint4{0, 0, 0, 0};
}

// fp8 tile: 8 e4m3 bytes per bf16 granule, loaded into registers, decoded
// exactly (every e4m3 value is a bf16 value) and written to the same layout.
template <int DC, int NW>
struct Fp8Stage {
  using Gm = Geo<DC>;
  static constexpr int NI = kTile * Gm::GPT / (kWave * NW);  // granules per lane
  static constexpr int CH = NI < 9 ? NI : 9;                 // granules kept in flight
  uint2 v[CH];
  float sc;

  __device__ __forceinline__ void load_chunk(const DecodeParams& p, const char* pbase, int nv, int c0, int w,
                                             int lane) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int qq = c0 + q;
      if (qq < NI) {
        const int s = (qq * NW + w) * kWave + lane;
        const int t = s / Gm::GPT;
        const int gr = (s % Gm::GPT) ^ swz(t);
        const int ts = min(t, nv - 1);
        const int64_t off = (int64_t)ts * p.token_stride + (gr < Gm::GC ? gr * 8 : p.rope_off + (gr - Gm::GC) * 8);
        v[q] = *(const uint2*)(pbase + off);
      }
    }
  }
  __device__ __forceinline__ void store_chunk(char* buf, int c0, int w, int lane) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int qq = c0 + q;
      if (qq < NI) {
        const int s = (qq * NW + w) * kWave + lane;
        bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].x, 1.0f, false);
        bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].x, 1.0f, true);
        bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].y, 1.0f, false);
        bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[q].y, 1.0f, true);
        bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        *(bf16x8*)(buf + s * 16) = r;
      }
    }
  }
};

// One 32-token tile of one wave: scores, online-softmax update, P.V.
template <int DC, bool FP8>
__device__ __forceinline__ void tile_step(const char* tb, const float* tsc, const bf16x8 (&qf)[Geo<DC>::KS],
                                          f32x16 (&O)[Geo<DC>::NB], float& m_run, float& l_run, int pos0, int limit,
                                          float slog2, const int (&koff)[4], int voff0, int voff1, int half) {
  using Gm = Geo<DC>;
  // ---- S^T = K . Q^T  (32 tokens x 32 rows)
  f32x16 sacc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    const bf16x8 a = *(const bf16x8*)(tb + koff[ks & 3] + 128 * (ks >> 2));
    sacc = mfma32(a, qf[ks], sacc);
    // Bound the scheduler's read-ahead (registers are the scarce resource).
    if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }

  // ---- online softmax; this lane holds row (lane % 32), tokens 8(i/4) + 4*half + i%4
  float tsv[16];
  if constexpr (FP8) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x4 s4 = *(const f32x4*)(tsc + 8 * a4 + 4 * half);
#pragma unroll
      for (int c = 0; c < 4; ++c) tsv[4 * a4 + c] = s4[c];
    }
  }
  float z[16];
  float mt = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tau = 8 * (i >> 2) + 4 * half + (i & 3);
    float zi = sacc[i] * slog2;
    if constexpr (FP8) zi *= tsv[i];
    z[i] = (pos0 + tau < limit) ? zi : -__builtin_inff();
    mt = fmaxf(mt, z[i]);
  }
  mt = wave_max_pair(mt);
  if (__any(mt > m_run + kRebase)) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
    // Element-wise through an AGPR-constrained block: the accumulators stay
    // in AGPRs and the rescale needs a single temporary VGPR.
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb) {
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
    m_run = m_new;
  }
  float pv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pi = (z[i] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(z[i] - m_run);
    l_run += pi;
    if constexpr (FP8) pv[i] = pi * tsv[i]; else pv[i] = pi;
  }
  const bf16x8 pf0 = pack_bf16x8(pv);
  const bf16x8 pf1 = pack_bf16x8(pv + 8);

  // ---- O^T += V^T . P^T
#pragma unroll
  for (int nb = 0; nb < Gm::NB; ++nb) {
    const char* vb = tb + 128 * (nb >> 1) + ((nb & 1) ? voff1 : voff0);
    const s16x4 x0 = lds_read_tr16(vb);
    const s16x4 x1 = lds_read_tr16(vb + 8 * Gm::GPT * 16);
    const s16x8 a0 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    O[nb] = mfma32((bf16x8)a0, pf0, O[nb]);
    const s16x4 y0 = lds_read_tr16(vb + 16 * Gm::GPT * 16);
    const s16x4 y1 = lds_read_tr16(vb + 24 * Gm::GPT * 16);
    const s16x8 a1 = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    O[nb] = mfma32((bf16x8)a1, pf1, O[nb]);
    if (nb & 1) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int DC, bool FP8, int NW, int NBUF>
__global__ void __launch_bounds__(NW * kWave)
    decode_kernel(DecodeParams p, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table,
                  const float* __restrict__ kv_scale) {
  using Gm = Geo<DC>;
  constexpr int TB = Gm::TILE_BYTES;
  constexpr int NI = kTile * Gm::GPT / (kWave * NW);
  static_assert(kTile * Gm::GPT % (kWave * NW) == 0, "tile must split evenly over the waves");
  static_assert(FP8 ? NBUF == 2 : (NI * (NBUF - 2) <= 63), "DMA groups must fit vmcnt");

  __shared__ __attribute__((aligned(1024))) char tiles[NBUF * TB];
  __shared__ __attribute__((aligned(16))) float tscale[FP8 ? NBUF * kTile : 4];
  __shared__ int cu[kMaxBatch + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

  // Lane-constant LDS offsets of the score A-operand (token `col`, granule 2ks+half).
  const int swz_k = swz(col);
  int koff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) koff[m] = col * Gm::GPT * 16 + (((2 * m + half) ^ swz_k) * 16);
  // ... and of the transposing V^T reads.
  const int i16 = lane & 15, grp = lane >> 4;
  const int jj = i16 >> 2, qq = i16 & 3, ch = grp & 1;
  const int sv = (jj << 1) | half;
  const int e = 2 * ch + (qq >> 1);
  const int vbase = (4 * half + jj) * Gm::GPT * 16 + (qq & 1) * 8;
  const int voff0 = vbase + ((e ^ sv) * 16);
  const int voff1 = vbase + (((4 + e) ^ sv) * 16);

  const uint32_t tiles_lds = lds_offset(tiles);

  // ---- tile loader state: next tile to load (kl) and its sequence (bl)
  int kl = k0;
  int bl = uniform(seq_of_tile(cu, p.B, k0));
  Fp8Stage<DC, NW> stage;

  auto page_base = [&](int b, int j, int& nv) -> const char* {
    const int pos0 = j * kTile;
    nv = min(kTile, seq_lens[b] - pos0);
    const int page = block_table[(int64_t)b * p.bt_stride + pos0 / p.block_size];
    return p.c_kv + (int64_t)page * p.block_stride + (int64_t)(pos0 % p.block_size) * p.token_stride;
  };
  auto stage_scales = [&](int b, int j, int sbuf) {
    if (w == 0 && lane < kTile) {
      const int pos0 = j * kTile;
      const int nv = min(kTile, seq_lens[b] - pos0);
      const int pos = pos0 + min(lane, nv - 1);
      const int page = block_table[(int64_t)b * p.bt_stride + pos / p.block_size];
      tscale[sbuf * kTile + lane] = kv_scale[(int64_t)page * p.block_size + pos % p.block_size];
    }
  };

  DmaPlan<DC, NW> dma;
  if constexpr (!FP8) {
    dma.init(p, w, lane);
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) {
      if (kl < k1) {
        dma.issue(p, block_table, bl, kl - uniform(cu[bl]), tiles_lds + ((kl - k0) % NBUF) * TB, w);
        ++kl;
        while (bl < p.B - 1 && kl >= uniform(cu[bl + 1])) ++bl;
      }
    }
  } else {
    int nv;
    const char* pb = page_base(bl, kl - uniform(cu[bl]), nv);
    for (int c0 = 0; c0 < Fp8Stage<DC, NW>::NI; c0 += Fp8Stage<DC, NW>::CH) {
      stage.load_chunk(p, pb, nv, c0, w, lane);
      stage.store_chunk(tiles, c0, w, lane);
    }
    stage_scales(bl, kl - uniform(cu[bl]), 0);
    ++kl;
    while (bl < p.B - 1 && kl >= uniform(cu[bl + 1])) ++bl;
    block_sync();
  }

  // ---- segments: maximal runs of this part's tiles inside one sequence
  int k = k0;
  int bc = uniform(seq_of_tile(cu, p.B, k0));
  while (k < k1) {
    const int cub = uniform(cu[bc]);
    const int kend = min(uniform(cu[bc + 1]), k1);
    const int L = seq_lens[bc];
    const int limit = min(L - p.S + 1 + row / p.H, L);

    bf16x8 qf[Gm::KS];
    if (row < p.R) {
      const bf16x8* ql = (const bf16x8*)(p.q_lat + ((int64_t)bc * p.R + row) * DC + 8 * half);
      const bf16x8* qr = (const bf16x8*)(p.q_rope + ((int64_t)bc * p.R + row) * 64 + 8 * half);
#pragma unroll
      for (int ks = 0; ks < DC / 16; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
      for (int ks = DC / 16; ks < Gm::KS; ++ks) qf[ks] = qr[2 * (ks - DC / 16)];
      // Let the compiler see the query loads complete here (vmcnt(0)), so it
      // places no waits for them inside the tile loop, where they would also
      // drain the in-flight tile DMA.
      __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks) qf[ks] = bf16x8{};
    }
    f32x16 O[Gm::NB];
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb) O[nb] = f32x16{};
    float m_run = -__builtin_inff(), l_run = 0.0f;

    for (; k < kend; ++k) {
      const int buf = (k - k0) % NBUF;
      if constexpr (!FP8) {
        wait_dma_groups<NI, NBUF - 2>(kl - 1 - k);
        block_sync();
        if ((k - cub + 1) * kTile > L) {  // last tile of the sequence, partially filled
          zero_tail<DC, NW>(tiles + buf * TB, L - (k - cub) * kTile, tid);
          block_sync();
        }
        if (kl < k1) {
          dma.issue(p, block_table, bl, kl - uniform(cu[bl]), tiles_lds + ((kl - k0) % NBUF) * TB, w);
          ++kl;
          while (bl < p.B - 1 && kl >= uniform(cu[bl + 1])) ++bl;
        }
      } else {
        if (kl < k1) {
          int nv;
          const char* pb = page_base(bl, kl - uniform(cu[bl]), nv);
          stage.load_chunk(p, pb, nv, 0, w, lane);
        }
      }

      tile_step<DC, FP8>(tiles + buf * TB, tscale + buf * kTile, qf, O, m_run, l_run, (k - cub) * kTile, limit,
                         p.scale_log2, koff, voff0, voff1, half);

      if constexpr (FP8) {
        if (kl < k1) {
          const int nbuf = (kl - k0) % NBUF;
          int nv;
          const char* pb = page_base(bl, kl - uniform(cu[bl]), nv);
          stage.store_chunk(tiles + nbuf * TB, 0, w, lane);
          for (int c0 = Fp8Stage<DC, NW>::CH; c0 < Fp8Stage<DC, NW>::NI; c0 += Fp8Stage<DC, NW>::CH) {
            stage.load_chunk(p, pb, nv, c0, w, lane);
            stage.store_chunk(tiles + nbuf * TB, c0, w, lane);
          }
          stage_scales(bl, kl - uniform(cu[bl]), nbuf);
          ++kl;
          while (bl < p.B - 1 && kl >= uniform(cu[bl + 1])) ++bl;
        }
        block_sync();
      }
    }

    // ---- normalise and write this (sequence, part) partial
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
    const int64_t slot = (int64_t)bc + g;
    if (row < p.R) {
      float* dst = p.o_part + (slot * p.R + row) * DC + 4 * half;
#pragma unroll
      for (int nb = 0; nb < Gm::NB; ++nb) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const f32x4 v = {O[nb][4 * ig] * inv, O[nb][4 * ig + 1] * inv, O[nb][4 * ig + 2] * inv,
                           O[nb][4 * ig + 3] * inv};
          *(f32x4*)(dst + 32 * nb + 8 * ig) = v;
        }
        __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time
      }
      if (half == 0) p.lse_part[slot * p.R + row] = lse;
    }
    ++bc;
    while (bc < p.B - 1 && uniform(cu[bc + 1]) == uniform(cu[bc])) ++bc;
  }
}

template <int DC, bool FP8, int NW, int NBUF>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const int grid = p.G * p.RG;
  hipLaunchKernelGGL((decode_kernel<DC, FP8, NW, NBUF>), dim3(grid), dim3(NW * kWave), 0, stream, p, p.seq_lens,
                     p.block_table, p.kv_scale);
  return hipGetLastError();
}

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

}  // namespace mla
