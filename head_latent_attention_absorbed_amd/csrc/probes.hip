// Calibration probes of the device (gfx950): the measured reference points
// the decode's roofline fractions are also given against.  Not part of the
// decode path.
//
//   hbm_read_kernel   streams a buffer through registers: each work-group
//                     reads one contiguous chunk, sixteen non-temporal
//                     16-byte loads in flight per lane: the achievable HBM
//                     read rate.
//   mfma_peak_kernel  four independent chains of v_mfma_f32_32x32x16_bf16 in
//                     two waves per SIMD on every CU: the achievable bf16
//                     MFMA rate.
// (The decode's own copy pattern alone is tile_copy_probe_kernel in
// decode_wide.hip, which shares that kernel's plan and copy code.)
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr uint32_t kNever = 0x9e3779b9u;  // a value the probes' sinks are written only if they produce

// Work-group g streams the g-th contiguous chunk of the buffer; each lane
// keeps 16 non-temporal 16-byte loads in flight (256 lanes x 16 B apart).
// Contiguous chunks per work-group stream faster than a grid-stride walk,
// which scatters each work-group's loads over the whole buffer.
__global__ void __launch_bounds__(256) hbm_read_kernel(const uint4* __restrict__ p, int64_t n16, uint32_t* sink) {
  constexpr int U = 16;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = beg + threadIdx.x;
  for (; i + (U - 1) * 256 < end; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(q + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < end; i += 256) acc ^= q[i];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == kNever) sink[0] = v;  // the loads feed a possible store, so they stay
}

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + 3 * e) % 17));
    b[e] = (__bf16)(0.002f * (float)((lane + 5 * e) % 13));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (blockIdx.x == 0 && threadIdx.x == 0) sink[0] = s;
}

}  // namespace

hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(cus * 8), dim3(256), 0, stream, static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError();
}

int64_t probe_mfma_flops(int iters, int cus) {
  // two work-groups of four waves per CU, four 32x32x16 MFMAs per iteration each
  return (int64_t)cus * 2 * 4 * 4 * (int64_t)iters * (2LL * 32 * 32 * 16);
}

hipError_t launch_probe_mfma(int iters, float* sink, int cus, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(cus * 2), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace mla
