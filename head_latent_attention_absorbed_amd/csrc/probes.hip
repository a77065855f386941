// Calibration probes of the device (gfx950): the measured reference points
// the decode's roofline fractions are also given against.  Not part of the
// decode path.
//
//   hbm_read_kernel   streams a buffer through registers with 16-byte loads
//                     from every CU, four loads in flight per lane (a
//                     grid-stride loop): the achievable HBM read rate.
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

__global__ void __launch_bounds__(256) hbm_read_kernel(const uint4* __restrict__ p, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc.x ^= a.x ^ b.x ^ c.x ^ d.x;
    acc.y ^= a.y ^ b.y ^ c.y ^ d.y;
    acc.z ^= a.z ^ b.z ^ c.z ^ d.z;
    acc.w ^= a.w ^ b.w ^ c.w ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc.x ^= a.x;
    acc.y ^= a.y;
    acc.z ^= a.z;
    acc.w ^= a.w;
  }
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
