// Log-sum-exp merge of the decode splits (gfx950).
//
// The online softmax carries (max, sum) so that attention over disjoint token
// ranges can be merged exactly (the running-softmax state the BLASST abstract
// on the "GQA-to-MLA" Daily Papers listing builds on): with per-split
// normalised outputs o_k and log-sum-exps lse_k,
//   lse = log sum_k e^{lse_k},  o = sum_k e^{lse_k - lse} o_k.
#include "mla_device.h"
#include "mla_kernels.h"

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

// The split range of sequence b: parts g0..g1 (slots b + g); empty (g1 < g0)
// for an idle sequence.  cu is the tile prefix of the batch.
__device__ __forceinline__ void split_range(const int* cu, int B, int G, int b, int& g0, int& g1) {
  const int N = cu[B], cb = cu[b], ce = cu[b + 1];
  g0 = 0;
  g1 = -1;
  if (ce > cb) {
    const int Wt = (N + G - 1) / G;
    g0 = cb / Wt;
    g1 = (ce - 1) / Wt;
  }
}

// Merge one query row (row r of sequence b) over its splits g0..g1: this
// lane's E consecutive columns E*lane .. E*lane + E-1 of
//   o = sum_k e^{lse_k - lse} o_k,  lse = log sum_k e^{lse_k}
// into acc (zeros and lse = -inf when the row sees no position).  The splits
// are visited U at a time: lane j requests the lse of split j of the batch
// while every lane requests its columns of all U partial rows, so one memory
// latency covers the whole batch (indices past the last split repeat it with
// weight 0).
template <int DC, bool HALF>
__device__ __forceinline__ float merge_row(const void* o_part, const float* lse_part, int R, int b, int r, int g0,
                                           int g1, int lane, float (&acc)[DC / 64]) {
  constexpr int E = DC / 64;
  constexpr int U = 16;
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  float m = -__builtin_inff(), tot = 0.0f;
  for (int gb = g0; gb <= g1; gb += U) {
    const int n = min(U, g1 - gb + 1);
    const float lk = lane < n ? lse_part[((int64_t)b + gb + lane) * R + r] : -__builtin_inff();
    PartRow<E, HALF> part[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t slot = (int64_t)b + gb + min(j, n - 1);
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
  __shared__ int cu[kMaxBatch + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  if (w == 0) build_tile_prefix(seq_lens, p.B, cu, lane);
  __syncthreads();
  const int row = blockIdx.y * 4 + w;
  if (row >= p.R) return;
  int g0, g1;
  split_range(cu, p.B, p.G, b, g0, g1);
  float acc[E];
  const float lse = merge_row<DC, HALF>(p.o_part, p.lse_part, p.R, b, row, g0, g1, lane, acc);
  float* out = p.o_lat + ((int64_t)b * p.R + row) * DC + E * lane;
#pragma unroll
  for (int i = 0; i < E; i += 4) *(f32x4*)(out + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  if (lane == 0) p.lse[(int64_t)b * p.R + row] = lse;
}

// ---------------------------------------------------------------------------
// Merge fused with the value up-projection.
//
// out[m, h, :] = o[m, h, :] . W_UV[h], o the merged row above.  A work-group
// takes one head h and 16 query rows m0 .. m0+15 (m = b*S + s); its four waves
// split d_c into four column ranges of KW = d_c / 4.  A wave merges, for all
// 16 rows, only its own KW columns, in exactly the layout of the A operand of
// the 16x16x32 MFMA (lane l: row l % 16, columns 32 ks + 8 (l / 16) .. +7 of
// k-step ks), so the merged rows never leave registers.  The wave's KW rows of
// W_UV[h] are copied into its own LDS slice by DMA at the start (16-byte
// granules XOR-swizzled per row) and read transposed as the B operand.  The
// four partial products are summed through LDS (each wave reuses its own
// slice) into 16-byte row stores.  The merged row is fp32, split into bf16
// high and low parts (two MFMAs per step) for near-fp32 accuracy.
//
// The grid is (row tile, head) with the head fastest, so for H a multiple of 8
// every row tile of a head lands on the same XCD and W_UV[h] is fetched from
// HBM about once.

constexpr int kUpRows = 16;  // query rows per work-group (the M extent of one 16x16 MFMA)

template <int DC, int NV>
struct UpGeometry {
  static constexpr int KW = DC / 4;             // latent columns of one wave
  static constexpr int KSW = KW / 32;           // 32-deep k-steps of one wave
  static constexpr int NT = NV / 16;            // 16-column output tiles
  static constexpr int ROWB = NV * 2;           // bytes of one W_UV row in LDS
  static constexpr int GR = NV / 8;             // 16-byte granules of one W_UV row
  static constexpr int SLICE = KW * ROWB;       // bytes of one wave's W_UV slice
  static constexpr int PITCH = NV + 4;          // fp32 row pitch of the reduction buffer
  static constexpr size_t LDS = 4 * (size_t)SLICE + (kMaxBatch + 1) * sizeof(int);
  static_assert(GR >= 8, "the swizzle permutes eight granules");
  static_assert(SLICE % 1024 == 0, "one DMA instruction fills 1 KiB");
  static_assert(kUpRows * PITCH * 4 <= SLICE, "the reduction buffer reuses the wave's slice");
};

template <int DC, int NV, bool HALF, bool CF32>
__global__ void __launch_bounds__(256) combine_up_kernel(CombineUpParams p) {
  using Geo = UpGeometry<DC, NV>;
  constexpr int KW = Geo::KW, KSW = Geo::KSW, NT = Geo::NT, ROWB = Geo::ROWB, GR = Geo::GR;
  constexpr int SLICE = Geo::SLICE, PITCH = Geo::PITCH;
  constexpr int U = HALF ? 8 : 4;  // splits per batch: 8 (fp16) or 4 (fp32) x KSW 16-byte words in flight
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int* cu = (int*)(smem + 4 * SLICE);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = p.H, M = p.B * p.S, R = p.S * H;
  const int h = blockIdx.x % H;
  const int m0 = (blockIdx.x / H) * kUpRows;
  char* ws = smem + w * SLICE;

  // Tile prefix first (wave 0), so that its loads are not queued behind the DMA.
  if (w == 0) build_tile_prefix(p.seq_lens, p.B, cu, lane);

  // W_UV[h] rows w*KW .. w*KW + KW-1 into this wave's slice: LDS granule
  // position q of row k holds global granule q ^ swz(k).
  {
    const uint16_t* wsrc = p.w + ((int64_t)h * DC + w * KW) * NV;
#pragma unroll
    for (int i = 0; i < SLICE / 1024; ++i) {
      const int pos = 64 * i + lane;
      const int k = pos / GR, q = pos % GR;
      lds_dma16(wsrc, (uint32_t)((k * NV + 8 * (q ^ swz(k))) * 2), lds_offset(ws + 1024 * i));
    }
  }
  block_sync();

  // ---- merge: this lane's row and its 8-column group of every k-step.
  const int mr = lane & 15, cg = lane >> 4;
  const int m = m0 + mr;
  const int mc = min(m, M - 1);  // address row (rows past M merge nothing)
  const int b = mc / p.S, r = (mc % p.S) * H + h;
  int g0, g1;
  split_range(cu, p.B, p.G, b, g0, g1);
  const int n = m < M ? g1 - g0 + 1 : 0;  // splits of this row (0: sees no position)
  const int64_t row0 = ((int64_t)b + g0) * R + r;  // partial row of split 0
  const int col0 = w * KW + 8 * cg;

  float acc[KSW][8];
#pragma unroll
  for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[ks][e] = 0.0f;
  float m_run = -__builtin_inff(), tot = 0.0f;
  for (int jb = 0; __ballot(jb < n) != 0; jb += U) {
    float lk[U];
    PartRow<8, HALF> part[U][KSW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = max(0, min(jb + u, n - 1));  // past the row's last split: repeat it, weight 0
      const int64_t rw = row0 + (int64_t)j * R;
      lk[u] = p.lse_part[rw];
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) part[u][ks].load(p.o_part, rw * DC + col0 + 32 * ks);
    }
    asm volatile("" ::: "memory");  // every load of the batch is issued before the first use
    float mb = m_run;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jb + u >= n) lk[u] = -__builtin_inff();
      mb = fmaxf(mb, lk[u]);
    }
    const float sc = m_run == mb ? 1.0f : __expf(m_run - mb);  // rescale of the earlier sum
    tot *= sc;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[ks][e] *= sc;
    m_run = mb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wu = lk[u] == -__builtin_inff() ? 0.0f : __expf(lk[u] - mb);
      tot += wu;
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[ks][e] += wu * part[u][ks].at(e);
    }
  }
  // A row that sees nothing has read whatever its (unwritten) address held
  // with weight 0; select zeros rather than scale, so NaN there cannot leak.
  const bool seen = tot > 0.0f;
  const float inv = seen ? 1.0f / tot : 0.0f;
  if (w == 0 && cg == 0 && m < M) p.lse[(int64_t)m * H + h] = seen ? m_run + __logf(tot) : -__builtin_inff();

  // ---- A fragments (bf16 high and low parts) of the merged row.
  bf16x8 ahi[KSW], alo[KSW];
#pragma unroll
  for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = seen ? acc[ks][e] * inv : 0.0f;
      const __bf16 hi = (__bf16)x;
      ahi[ks][e] = hi;
      alo[ks][e] = (__bf16)(x - (float)hi);
    }

  // ---- this wave's share of the product: C[16 x NV] over its KW columns.
  vm_wait<0>();  // the wave's W_UV slice has landed (only this wave reads it)
  const int i16 = lane & 15, jj = i16 >> 2, qq = i16 & 3;
  f32x4 c[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) c[nt] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < KSW; ++ks) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s16x4 rr[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int k = 32 * ks + 8 * cg + 4 * h2 + jj;
        const int q = 2 * nt + (qq >> 1);
        rr[h2] = lds_read_tr16(ws + k * ROWB + ((q ^ swz(k)) * 16) + (qq & 1) * 8);
      }
      const s16x8 bv = {rr[0][0], rr[0][1], rr[0][2], rr[0][3], rr[1][0], rr[1][1], rr[1][2], rr[1][3]};
      c[nt] = mfma16(ahi[ks], (bf16x8)bv, c[nt]);
      c[nt] = mfma16(alo[ks], (bf16x8)bv, c[nt]);
    }
  }
  // Partial product into the wave's own slice (its last reads of the slice
  // precede these writes in the wave's LDS queue).
  float* red = (float*)ws;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(4 * cg + i) * PITCH + 16 * nt + i16] = c[nt][i];
  block_sync();

  // ---- sum the four K parts; 8 consecutive columns per thread.
  for (int e = tid; e < kUpRows * (NV / 8); e += 256) {
    const int row = e / (NV / 8), nc = (e % (NV / 8)) * 8;
    const int mm = m0 + row;
    if (mm >= M) continue;
    float s[8] = {};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* src = (const float*)(smem + q * SLICE) + row * PITCH + nc;
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
  hipLaunchKernelGGL((combine_up_kernel<DC, NV, HALF, CF32>), dim3(tiles * p.H), dim3(256), smem, stream, p);
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
