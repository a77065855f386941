// TPLA latent split on one device (gfx950): the Hadamard change of basis of
// the latent, the per-shard weight slices, and the sum of the shards' outputs.
//
// TPLA splits the latent, and each head's input dimension with it, over the
// devices; each shard attends on its slice and an all-reduce adds the
// results.  An orthogonal (Hadamard) change of basis applied before the
// split evens out the shards (TPLA abstract on the taxoreview pages for
// dblp:408/6122 and dblp:256/5536-3).  The decode of one shard is the
// ordinary latent decode at d_latent / n over a strided view of the records,
// so only these three pieces are new.
//
// The transform is the fast Walsh-Hadamard transform in Sylvester order,
// x H / sqrt(D): one wave per vector, lane l holding elements E l .. E l + E - 1
// (E = D / 64).  The butterflies over the low log2(E) index bits stay in the
// lane; the other six run across lanes with a lane-xor exchange.  Every
// vector is read once and written once (bound by memory traffic), in fp32
// with one bf16 rounding at the end.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

template <int D, bool CIN, bool COUT>
__global__ void __launch_bounds__(256) hadamard_kernel(HadamardParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  const float norm = 1.0f / __builtin_sqrtf((float)D);
  const int dsub = D / p.n_shards;
  for (int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); v < p.n_vec; v += nw) {
    const int64_t vo = v / p.inner, vi = v % p.inner;
    const uint16_t* src = p.in + vo * p.in_outer + vi * p.in_inner;
    float x[E];
    if constexpr (CIN) {
      if constexpr (E == 8) {
        const uint4 r = *(const uint4*)(src + E * lane);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16);
          x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        const uint2 r = *(const uint2*)(src + E * lane);
        const uint32_t w[2] = {r.x, r.y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16);
          x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __uint_as_float((uint32_t)src[(int64_t)(E * lane + e) * p.in_elem] << 16);
    }
    if (p.rotate) {
#pragma unroll
      for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & h) continue;
          const float a = x[e], b = x[e + h];
          x[e] = a + b;
          x[e + h] = a - b;
        }
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const bool upper = lane & m;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float y = __shfl_xor(x[e], m);
          x[e] = upper ? y - x[e] : x[e] + y;
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] *= norm;
    }
    // Element k = E lane + e goes to shard k / dsub at position k % dsub; the
    // E elements of a lane never straddle two shards (dsub is a multiple of E).
    const int k0 = E * lane;
    uint16_t* dst = p.out + vo * p.out_outer + vi * p.out_inner + (int64_t)(k0 / dsub) * p.out_shard;
    const int kk = k0 % dsub;
    if constexpr (COUT) {
      uint32_t w[E / 2];
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const bf16x2 t = {(__bf16)x[2 * i], (__bf16)x[2 * i + 1]};
        w[i] = __builtin_bit_cast(uint32_t, t);
      }
      if constexpr (E == 8) {
        *(uint4*)(dst + kk) = uint4{w[0], w[1], w[2], w[3]};
      } else {
        *(uint2*)(dst + kk) = uint2{w[0], w[1]};
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) dst[(int64_t)(kk + e) * p.out_elem] = __builtin_bit_cast(uint16_t, (__bf16)x[e]);
    }
  }
}

template <int D>
hipError_t launch_d(const HadamardParams& p, hipStream_t stream) {
  const int64_t wgs = (p.n_vec + 3) / 4;
  const dim3 grid((unsigned)(wgs < 8192 ? wgs : 8192));
  const bool cin = p.in_elem == 1, cout = p.out_elem == 1;
  if (cin && cout) hipLaunchKernelGGL((hadamard_kernel<D, true, true>), grid, dim3(256), 0, stream, p);
  else if (cin) hipLaunchKernelGGL((hadamard_kernel<D, true, false>), grid, dim3(256), 0, stream, p);
  else if (cout) hipLaunchKernelGGL((hadamard_kernel<D, false, true>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((hadamard_kernel<D, false, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// out[m] = sum_i parts[i][m], four elements per thread (m counts multiples of 4).
template <bool F32>
__global__ void __launch_bounds__(256) shard_sum_kernel(const float* __restrict__ parts, int n, int64_t count,
                                                        void* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * q >= count) return;
  f32x4 s = *(const f32x4*)(parts + 4 * q);
  for (int i = 1; i < n; ++i) {
    const f32x4 t = *(const f32x4*)(parts + (int64_t)i * count + 4 * q);
    s = f32x4{s[0] + t[0], s[1] + t[1], s[2] + t[2], s[3] + t[3]};
  }
  if constexpr (F32) {
    *((f32x4*)out + q) = s;
  } else {
    const bf16x2 a = {(__bf16)s[0], (__bf16)s[1]}, b = {(__bf16)s[2], (__bf16)s[3]};
    *((uint2*)out + q) = uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  }
}

}  // namespace

hipError_t launch_hadamard(const HadamardParams& p, hipStream_t stream) {
  if (p.n_vec <= 0) return hipSuccess;
  if (p.d == 512) return launch_d<512>(p, stream);
  if (p.d == 256) return launch_d<256>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_shard_sum(const float* parts, int n, int64_t count, void* out, bool out_f32, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  if (count % 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((count / 4 + 255) / 256));
  if (out_f32) hipLaunchKernelGGL((shard_sum_kernel<true>), grid, dim3(256), 0, stream, parts, n, count, out);
  else hipLaunchKernelGGL((shard_sum_kernel<false>), grid, dim3(256), 0, stream, parts, n, count, out);
  return hipGetLastError();
}

}  // namespace mla
