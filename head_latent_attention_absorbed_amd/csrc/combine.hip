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

// One wave per (sequence, query row); lane i owns columns E*i .. E*i + E-1.
// The splits are visited U at a time: lane j requests the lse of split j of
// the batch while every lane requests its columns of all U partial rows, so
// one memory latency covers the whole batch (indices past the last split
// repeat it with weight 0).
template <int DC, bool HALF>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p, const int32_t* __restrict__ seq_lens) {
  constexpr int E = DC / 64;
  constexpr int U = 16;
  __shared__ int cu[kMaxBatch + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  if (w == 0) build_tile_prefix(seq_lens, p.B, cu, lane);
  __syncthreads();
  const int row = blockIdx.y * 4 + w;
  if (row >= p.R) return;

  float* out = p.o_lat + ((int64_t)b * p.R + row) * DC + E * lane;
  const int N = cu[p.B], cb = cu[b], ce = cu[b + 1];
  int g0 = 0, g1 = -1;
  if (ce > cb) {
    const int Wt = (N + p.G - 1) / p.G;
    g0 = cb / Wt;
    g1 = (ce - 1) / Wt;
  }
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  float m = -__builtin_inff(), tot = 0.0f;
  for (int gb = g0; gb <= g1; gb += U) {
    const int n = min(U, g1 - gb + 1);
    const float lk = lane < n ? p.lse_part[((int64_t)b + gb + lane) * p.R + row] : -__builtin_inff();
    PartRow<E, HALF> part[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t slot = (int64_t)b + gb + min(j, n - 1);
      part[j].load(p.o_part, (slot * p.R + row) * DC + E * lane);
    }
    // Keep every load above this point: the lse is waited for while the
    // partial rows are still in flight.
    asm volatile("" ::: "memory");
    // Running maximum over the batches; earlier sums are rescaled when it grows.
    float mb = m;
#pragma unroll
    for (int j = 0; j < U; ++j) mb = fmaxf(mb, lane_value(lk, j));
    if (mb == -__builtin_inff()) continue;  // nothing visible so far
    const float r = __expf(m - mb);          // 0 when m = -inf
    tot *= r;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= r;
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
  if (m == -__builtin_inff()) {  // the row sees no position
#pragma unroll
    for (int i = 0; i < E; i += 4) *(f32x4*)(out + i) = f32x4{};
    if (lane == 0) p.lse[(int64_t)b * p.R + row] = -__builtin_inff();
    return;
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int i = 0; i < E; i += 4) *(f32x4*)(out + i) = f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
  if (lane == 0) p.lse[(int64_t)b * p.R + row] = m + __logf(tot);
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

}  // namespace mla
