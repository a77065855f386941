// Log-sum-exp merge of the decode splits (gfx950).
//
// The online softmax carries (max, sum) so that attention over disjoint token
// ranges can be merged exactly (the running-softmax state the BLASST abstract
// on the "GQA-to-MLA" Daily Papers listing builds on): with per-split
// normalised outputs o_k and log-sum-exps lse_k,
//   lse = log sum_k e^{lse_k},  o = sum_k e^{lse_k - lse} o_k.
#include "mla_device.h"
#include "mla_kernels.h"
#include "split_plan.h"

namespace mla {
namespace {

template <int E, bool HALF>
struct PartRow;  // E consecutive columns of one partial row, loaded as one or two 16-byte words

template <>
struct PartRow<8, true> {
  uint4 v;
  __device__ void load(const void* base, int64_t off) { v = *(const uint4*)((const _Float16*)base + off); }
  __device__ float at(int i) const {
    const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (float)__builtin_bit_cast(f16x2, w)[i & 1];
  }
};
template <>
struct PartRow<4, true> {
  uint2 v;
  __device__ void load(const void* base, int64_t off) { v = *(const uint2*)((const _Float16*)base + off); }
  __device__ float at(int i) const { return (float)__builtin_bit_cast(f16x2, i < 2 ? v.x : v.y)[i & 1]; }
};
template <>
struct PartRow<8, false> {
  f32x4 a, b;
  __device__ void load(const void* base, int64_t off) {
    a = *(const f32x4*)((const float*)base + off);
    b = *(const f32x4*)((const float*)base + off + 4);
  }
  __device__ float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};
template <>
struct PartRow<4, false> {
  f32x4 a;
  __device__ void load(const void* base, int64_t off) { a = *(const f32x4*)((const float*)base + off); }
  __device__ float at(int i) const { return a[i]; }
};

// The value of x in lane j (j wave-uniform).
__device__ __forceinline__ float lane_value(float x, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

// Merge one query row (row r) over its sequence's slots s0 .. s0 + ns - 1
// (the split plan of split_plan.h): this lane's E consecutive columns
// E*lane .. E*lane + E-1 of
//   o = sum_k e^{lse_k - lse} o_k,  lse = log sum_k e^{lse_k}
// into acc (zeros and lse = -inf when the row sees no position).  The splits
// are visited U at a time: lane j requests the lse of split j of the batch
// while every lane requests its columns of all U partial rows, so one memory
// latency covers the whole batch (indices past the last split repeat it with
// weight 0).
template <int DC, bool HALF, int U = 16>
__device__ __forceinline__ float merge_row(const void* o_part, const float* lse_part, int R, int r, int s0, int ns,
                                           int lane, float (&acc)[DC / 64]) {
  constexpr int E = DC / 64;
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  float m = -__builtin_inff(), tot = 0.0f;
  for (int gb = 0; gb < ns; gb += U) {
    const int n = min(U, ns - gb);
    const float lk = lane < n ? lse_part[((int64_t)s0 + gb + lane) * R + r] : -__builtin_inff();
    PartRow<E, HALF> part[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t slot = (int64_t)s0 + gb + min(j, n - 1);
      part[j].load(o_part, (slot * R + r) * DC + E * lane);
    }
    // Keep every load above this point: the lse is waited for while the
    // partial rows are still in flight.
    asm volatile("" ::: "memory");
    // Running maximum over the batches; earlier sums are rescaled when it grows.
    float mb = m;
#pragma unroll
    for (int j = 0; j < U; ++j) mb = fmaxf(mb, lane_value(lk, j));
    if (mb == -__builtin_inff()) continue;  // nothing visible so far
    const float sc = __expf(m - mb);         // 0 when m = -inf
    tot *= sc;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= sc;
    m = mb;
    const float wl = __expf(lk - m);         // this lane's split weight (0 for -inf)
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float wj = lane_value(wl, j);  // 0 past the batch's last split
      tot += wj;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] += wj * part[j].at(i);
    }
  }
  if (m == -__builtin_inff()) return -__builtin_inff();  // the row sees no position
  const float inv = 1.0f / tot;
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] *= inv;
  return m + __logf(tot);
}

// One wave per (sequence, query row); lane i owns columns E*i .. E*i + E-1.
template <int DC, bool HALF>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p, const int32_t* __restrict__ seq_lens) {
  constexpr int E = DC / 64;
  __shared__ int slots[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  if (w == 0) {
    with_plan(seq_lens, p.B, p.P, lane, [&](const auto& pl) {
      int s_b, p_b;
      pl.slots_of(b, lane, s_b, p_b);
      if (lane == 0) {
        slots[0] = s_b;
        slots[1] = p_b;
      }
    });
  }
  __syncthreads();
  const int row = blockIdx.y * 4 + w;
  if (row >= p.R) return;
  float acc[E];
  const float lse = merge_row<DC, HALF>(p.o_part, p.lse_part, p.R, row, slots[0], slots[1], lane, acc);
  float* out = p.o_lat + ((int64_t)b * p.R + row) * DC + E * lane;
#pragma unroll
  for (int i = 0; i < E; i += 4) *(f32x4*)(out + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  if (lane == 0) p.lse[(int64_t)b * p.R + row] = lse;
}

// ---------------------------------------------------------------------------
// Merge fused with the value up-projection.
//
// out[m, h, :] = o[m, h, :] . W_UV[h], o the merged row above.  A work-group
// takes one head h and 16 query rows m0 .. m0+15 (m = b*S + s; the M extent
// of one 16x16x32 MFMA) with sixteen waves:
//  1. W_UV[h] is copied into LDS by DMA at the start (four slices of
//     KW = d_c/4 rows, 16-byte granules XOR-swizzled per row) and stays in
//     flight while the rows are merged.
//  2. Wave w merges row w exactly as the stand-alone merge does (contiguous
//     row loads, all of a row's splits in flight at once); the fp32 row goes
//     to an LDS tile (granules XOR-swizzled by row).
//  3. Wave w = 4 nq + kr multiplies the tile's columns kr*KW .. kr*KW + KW-1
//     (A operand, split into bf16 high and low parts: two MFMAs per step for
//     near-fp32 accuracy) by output columns nq*NV/4 .. of W_UV slice kr
//     (B operand, transposing LDS reads).
//  4. The four K parts of each output are summed through LDS (in the W_UV
//     slices' place) into 16-byte row stores.
// The grid is (row tile, head) with the head fastest, so for H a multiple of
// 8 every row tile of a head lands on the same XCD and shares its L2.

constexpr int kUpRows = 16;  // query rows per work-group, one per wave

template <int DC, int NV>
struct UpGeometry {
  static constexpr int KW = DC / 4;             // latent columns of one K part
  static constexpr int KSW = KW / 32;           // 32-deep k-steps of one K part
  static constexpr int NQ = NV / 4;             // output columns of one wave
  static constexpr int NTW = NQ / 16;           // 16-column output tiles of one wave
  static constexpr int ROWB = NV * 2;           // bytes of one W_UV row in LDS
  static constexpr int GR = NV / 8;             // 16-byte granules of one W_UV row
  static constexpr int SLICE = KW * ROWB;       // bytes of one K part's W_UV slice
  static constexpr int PIECES = SLICE / 1024;   // 1 KiB DMA pieces of one slice
  static constexpr int AROW = DC * 4;           // bytes of one merged fp32 row
  static constexpr int ATILE = kUpRows * AROW;  // the merged tile
  static constexpr int PITCH = NV + 4;          // fp32 row pitch of the reduction buffer
  static constexpr size_t LDS = 4 * (size_t)SLICE + ATILE;
  static_assert(GR >= 8, "the swizzle permutes eight granules");
  static_assert(NTW >= 1, "a wave takes whole 16-column tiles");
  static_assert(SLICE % 4096 == 0, "four waves issue equal shares of 1 KiB DMAs per slice");
  static_assert(4 * kUpRows * PITCH * 4 <= 4 * SLICE, "the reduction buffer reuses the W_UV slices");
  static_assert((kMaxBatch + 1) * sizeof(int) <= (size_t)ATILE, "the slot prefix lives in the merged tile first");
};

// Byte offset of fp32 column c of merged row r: 16-byte granule c/4 at
// position (c/4) ^ (r & 7), so that the sixteen rows of an A-fragment read
// spread over the banks.
__device__ __forceinline__ int arow_off(int r, int c, int arow) {
  return r * arow + ((((c >> 2) ^ (r & 7)) << 4) | ((c & 3) << 2));
}

template <int DC, int NV, bool HALF, bool CF32>
__global__ void __launch_bounds__(1024) combine_up_kernel(CombineUpParams p) {
  using Geo = UpGeometry<DC, NV>;
  constexpr int KW = Geo::KW, KSW = Geo::KSW, NQ = Geo::NQ, NTW = Geo::NTW, ROWB = Geo::ROWB, GR = Geo::GR;
  constexpr int SLICE = Geo::SLICE, PIECES = Geo::PIECES, AROW = Geo::AROW, PITCH = Geo::PITCH;
  constexpr int E = DC / 64;  // merged columns per lane
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* atile = smem + 4 * SLICE;
  int* sb = (int*)atile;  // the slot prefix of the split plan, until the merged rows overwrite it

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kr = w & 3, nq = w >> 2;  // K part and output-column quarter of the product
  const int H = p.H, M = p.B * p.S, R = p.S * H;
  const int h = blockIdx.x % H;
  const int m0 = (blockIdx.x / H) * kUpRows;

  // Split plan first (wave 0), so that its loads are not queued behind the DMA.
  if (w == 0) with_plan(p.seq_lens, p.B, p.P, lane, [&](const auto& pl) { pl.write_slot_prefix(sb, lane); });

  // W_UV[h] rows kr*KW .. kr*KW + KW-1 into slice kr: LDS granule position q
  // of row k holds global granule q ^ swz(k).  Wave (kr, nq) copies pieces
  // nq*PIECES/4 .. of the slice.
  {
    const uint16_t* wsrc = p.w + ((int64_t)h * DC + kr * KW) * NV;
#pragma unroll
    for (int j = 0; j < PIECES / 4; ++j) {
      const int i = nq * (PIECES / 4) + j;
      const int pos = 64 * i + lane;
      const int k = pos / GR, q = pos % GR;
      lds_dma16(wsrc, (uint32_t)((k * NV + 8 * (q ^ swz(k))) * 2), lds_offset(smem + kr * SLICE + 1024 * i));
    }
  }
  block_sync();

  // ---- merge row w of the tile.
  const int m = m0 + w;
  const int mc = min(m, M - 1);
  const int b = mc / p.S, r = (mc % p.S) * H + h;
  const int s0 = sb[b];
  const int ns = m < M ? sb[b + 1] - s0 : 0;  // rows past M merge nothing
  block_sync();  // every read of the slot prefix is done before the merged rows overwrite it
  float acc[E];
  // 16 splits in flight per batch; 8 for fp32 rows of 512, which would not
  // fit the 128 registers a lane has at 16 waves per work-group.
  const float lse = merge_row<DC, HALF, (HALF || DC < 512) ? 16 : 8>(p.o_part, p.lse_part, R, r, s0, ns, lane, acc);
  if (lane == 0 && m < M) p.lse[(int64_t)m * H + h] = lse;
#pragma unroll
  for (int e = 0; e < E; e += 4)
    *(f32x4*)(atile + arow_off(w, E * lane + e, AROW)) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  vm_wait<0>();  // this wave's pieces of the W_UV copy have landed ...
  block_sync();  // ... and everyone's, and the merged tile is complete

  // ---- A fragments (bf16 high and low parts) of K part kr.
  const int mr = lane & 15, cg = lane >> 4;
  bf16x8 ahi[KSW], alo[KSW];
#pragma unroll
  for (int ks = 0; ks < KSW; ++ks) {
    const int c = kr * KW + 32 * ks + 8 * cg;
    const f32x4 x0 = *(const f32x4*)(atile + arow_off(mr, c, AROW));
    const f32x4 x1 = *(const f32x4*)(atile + arow_off(mr, c + 4, AROW));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? x0[e] : x1[e - 4];
      const __bf16 hi = (__bf16)x;
      ahi[ks][e] = hi;
      alo[ks][e] = (__bf16)(x - (float)hi);
    }
  }

  // ---- C[16 x NQ] (output columns nq*NQ ..) over K part kr.
  const char* ws = smem + kr * SLICE;
  const int i16 = lane & 15, jj = i16 >> 2, qq = i16 & 3;
  f32x4 c[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) c[t] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < KSW; ++ks) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int nt = nq * NTW + t;
      s16x4 rr[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int k = 32 * ks + 8 * cg + 4 * h2 + jj;
        const int q = 2 * nt + (qq >> 1);
        rr[h2] = lds_read_tr16(ws + k * ROWB + ((q ^ swz(k)) * 16) + (qq & 1) * 8);
      }
      const s16x8 bv = {rr[0][0], rr[0][1], rr[0][2], rr[0][3], rr[1][0], rr[1][1], rr[1][2], rr[1][3]};
      c[t] = mfma16(ahi[ks], (bf16x8)bv, c[t]);
      c[t] = mfma16(alo[ks], (bf16x8)bv, c[t]);
    }
  }
  block_sync();  // every wave is done with W_UV
  // Partial products red[kr][row][col] in the W_UV slices' place.
  float* red = (float*)smem;
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(kr * kUpRows + 4 * cg + i) * PITCH + nq * NQ + 16 * t + i16] = c[t][i];
  block_sync();

  // ---- sum the four K parts; 8 consecutive output columns per thread.
  for (int e = tid; e < kUpRows * (NV / 8); e += 1024) {
    const int row = e / (NV / 8), nc = (e % (NV / 8)) * 8;
    const int mm = m0 + row;
    if (mm >= M) continue;
    float s[8] = {};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* src = red + (q * kUpRows + row) * PITCH + nc;
      const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] += x0[i];
        s[4 + i] += x1[i];
      }
    }
    const int64_t off = ((int64_t)mm * H + h) * NV + nc;
    if constexpr (CF32) {
      float* o = (float*)p.out + off;
      *(f32x4*)o = f32x4{s[0], s[1], s[2], s[3]};
      *(f32x4*)(o + 4) = f32x4{s[4], s[5], s[6], s[7]};
    } else {
      *(bf16x8*)((uint16_t*)p.out + off) = pack_bf16x8(s);
    }
  }
}

template <int DC, int NV, bool HALF, bool CF32>
hipError_t launch_up_variant(const CombineUpParams& p, hipStream_t stream) {
  constexpr size_t smem = UpGeometry<DC, NV>::LDS;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(combine_up_kernel<DC, NV, HALF, CF32>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  const int tiles = (p.B * p.S + kUpRows - 1) / kUpRows;
  hipLaunchKernelGGL((combine_up_kernel<DC, NV, HALF, CF32>), dim3(tiles * p.H), dim3(1024), smem, stream, p);
  return hipGetLastError();
}

template <int DC, int NV>
hipError_t launch_up_dtypes(const CombineUpParams& p, hipStream_t stream) {
  if (p.o_half) {
    return p.out_f32 ? launch_up_variant<DC, NV, true, true>(p, stream)
                     : launch_up_variant<DC, NV, true, false>(p, stream);
  }
  return p.out_f32 ? launch_up_variant<DC, NV, false, true>(p, stream)
                   : launch_up_variant<DC, NV, false, false>(p, stream);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  dim3 grid(p.B, (p.R + 3) / 4);
  if (p.DC == 512) {
    if (p.o_half) hipLaunchKernelGGL((combine_kernel<512, true>), grid, dim3(256), 0, stream, p, p.seq_lens);
    else hipLaunchKernelGGL((combine_kernel<512, false>), grid, dim3(256), 0, stream, p, p.seq_lens);
  } else {
    if (p.o_half) hipLaunchKernelGGL((combine_kernel<256, true>), grid, dim3(256), 0, stream, p, p.seq_lens);
    else hipLaunchKernelGGL((combine_kernel<256, false>), grid, dim3(256), 0, stream, p, p.seq_lens);
  }
  return hipGetLastError();
}

bool combine_up_supported(int d_latent, int d_v) {
  return (d_latent == 512 || d_latent == 256) && (d_v == 64 || d_v == 128);
}

hipError_t launch_combine_up(const CombineUpParams& p, hipStream_t stream) {
  if (p.DC == 512 && p.NV == 128) return launch_up_dtypes<512, 128>(p, stream);
  if (p.DC == 512 && p.NV == 64) return launch_up_dtypes<512, 64>(p, stream);
  if (p.DC == 256 && p.NV == 128) return launch_up_dtypes<256, 128>(p, stream);
  if (p.DC == 256 && p.NV == 64) return launch_up_dtypes<256, 64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
