// Log-sum-exp merge of the decode splits (gfx950).
//
// The online softmax carries (max, sum) so that attention over disjoint token
// ranges can be merged exactly (the running-softmax state the BLASST abstract
// on the "GQA-to-MLA" Daily Papers listing builds on): with per-split
// normalised outputs o_k and log-sum-exps lse_k,
//   lse = log sum_k e^{lse_k},  o = sum_k e^{lse_k - lse} o_k.
// One wave per (sequence, query row); each lane owns DC/64 latent columns.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

template <int DC>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p, const int32_t* __restrict__ seq_lens) {
  __shared__ int cu[kMaxBatch + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  if (w == 0) build_tile_prefix(seq_lens, p.B, cu, lane);
  __syncthreads();
  const int row = blockIdx.y * 4 + w;
  if (row >= p.R) return;

  constexpr int V4 = DC / 256;  // float4 groups per lane
  float* out = p.o_lat + ((int64_t)b * p.R + row) * DC + 4 * lane;
  float* lse_out = p.lse + (int64_t)b * p.R + row;
  const int N = cu[p.B], cb = cu[b], ce = cu[b + 1];

  float m = -__builtin_inff();
  int g0 = 0, g1 = -1;
  if (ce > cb) {
    const int Wt = (N + p.G - 1) / p.G;
    g0 = cb / Wt;
    g1 = (ce - 1) / Wt;
    for (int g = g0; g <= g1; ++g) m = fmaxf(m, p.lse_part[((int64_t)b + g) * p.R + row]);
  }
  if (m == -__builtin_inff()) {
#pragma unroll
    for (int i = 0; i < V4; ++i) *(f32x4*)(out + 256 * i) = f32x4{};
    if (lane == 0) *lse_out = -__builtin_inff();
    return;
  }
  f32x4 acc[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) acc[i] = f32x4{};
  float tot = 0.0f;
  for (int g = g0; g <= g1; ++g) {
    const int64_t slot = (int64_t)b + g;
    const float lk = p.lse_part[slot * p.R + row];
    if (lk == -__builtin_inff()) continue;
    const float wk = expf(lk - m);
    tot += wk;
    const float* src = p.o_part + (slot * p.R + row) * DC + 4 * lane;
#pragma unroll
    for (int i = 0; i < V4; ++i) acc[i] += wk * *(const f32x4*)(src + 256 * i);
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int i = 0; i < V4; ++i) *(f32x4*)(out + 256 * i) = acc[i] * inv;
  if (lane == 0) *lse_out = m + logf(tot);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  dim3 grid(p.B, (p.R + 3) / 4);
  if (p.DC == 512)
    hipLaunchKernelGGL(combine_kernel<512>, grid, dim3(256), 0, stream, p, p.seq_lens);
  else
    hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(256), 0, stream, p, p.seq_lens);
  return hipGetLastError();
}

}  // namespace mla
