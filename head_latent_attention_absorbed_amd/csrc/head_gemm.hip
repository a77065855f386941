// Per-head products of the absorb and the value up-projection (gfx950).
//
//   absorb:  q_lat[m, h, :] = q_nope[m, h, :] . W_UK[h]   (K = d_nope, N = d_latent)
//   up-proj: out[m, h, :]   = o_lat[m, h, :]  . W_UV[h]   (K = d_latent, N = d_v)
//
// Folding W_UK into the query is what lets attention run on the cached latent
// without expanding it (TransMLA abstracts on the taxoreview pages; TransMLA
// review page, key_machinery), and W_UV maps the latent output back to value
// space (early TransMLA abstract on the "GQA-to-MLA" Daily Papers listing).
//
// Both are small per-head GEMMs bound by reading W (M = B*S_q rows only), so a
// work-group takes one head and 64 output columns: it stages W[h][:, n0:n0+64]
// in LDS (16-byte granules XOR-swizzled per row), its four waves each reduce a
// quarter of K with 32x32x16 bf16 MFMAs (W^T operand through the transposing
// LDS read), and the quarters are summed through LDS.  An fp32 A operand is
// split into bf16 high and low parts, two MFMAs, for near-fp32 accuracy.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kNB = 64;  // output columns per work-group
// LDS for K <= 512: the W tile (K x 64 bf16) plus the 4-wave reduction buffer.
constexpr int kMaxGemmLds = 512 * kNB * 2 + 4 * 32 * kNB * 4;

__device__ __forceinline__ int swzw(int k) { return ((k & 3) << 1) | ((k >> 2) & 1); }

template <bool AF32, bool CF32>
__global__ void __launch_bounds__(256) head_gemm_kernel(HeadGemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* wt = smem;                                          // [K][64] bf16, swizzled granules
  float* red = (float*)(smem + (size_t)p.K * kNB * 2);     // [4][32][64] fp32

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int nblocks = p.N / kNB;
  const int h = blockIdx.x / nblocks;
  const int n0 = (blockIdx.x % nblocks) * kNB;
  const int K = p.K, H = p.H, N = p.N;

  // Stage W[h][:, n0:n0+64].
  const uint16_t* wsrc = p.w + (int64_t)h * K * N + n0;
  for (int idx = tid; idx < K * 8; idx += 256) {
    const int k = idx >> 3, gc = idx & 7;
    const uint4 v = *(const uint4*)(wsrc + (int64_t)k * N + 8 * gc);
    *(uint4*)(wt + k * 128 + ((gc ^ swzw(k)) * 16)) = v;
  }
  __syncthreads();

  // Lane constants of the transposing W^T reads.
  const int i16 = lane & 15, grp = lane >> 4;
  const int jj = i16 >> 2, qq = i16 & 3, ch = grp & 1;
  const int kq = K / 4;           // K range of this wave
  const int kbeg = w * kq;

  for (int m0 = 0; m0 < p.M; m0 += 32) {
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    const int m = m0 + col;
    for (int ks = 0; ks < kq / 16; ++ks) {
      const int kk = kbeg + 16 * ks + 8 * half;  // first k of this lane's A fragment
      bf16x8 ahi, alo;
      if (m < p.M) {
        if constexpr (AF32) {
          const float* ap = (const float*)p.a + ((int64_t)m * H + h) * K + kk;
          const f32x4 x0 = *(const f32x4*)ap;
          const f32x4 x1 = *(const f32x4*)(ap + 4);
          float v[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const __bf16 hi = (__bf16)v[i];
            ahi[i] = hi;
            alo[i] = (__bf16)(v[i] - (float)hi);
          }
        } else {
          ahi = *(const bf16x8*)((const uint16_t*)p.a + ((int64_t)m * H + h) * K + kk);
        }
      } else {
        ahi = bf16x8{};
        alo = bf16x8{};
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int e = 4 * nt + 2 * ch + (qq >> 1);
        s16x4 r[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int k = kbeg + 16 * ks + 8 * half + 4 * h2 + jj;
          const int sw = (jj << 1) | h2;
          r[h2] = lds_read_tr16(wt + k * 128 + ((e ^ sw) * 16) + (qq & 1) * 8);
        }
        const s16x8 bv = {r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
        acc[nt] = mfma32(ahi, (bf16x8)bv, acc[nt]);
        if constexpr (AF32) acc[nt] = mfma32(alo, (bf16x8)bv, acc[nt]);
      }
    }
    // Reduce the four K quarters.
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ml = 8 * (i >> 2) + 4 * half + (i & 3);
        red[(w * 32 + ml) * kNB + 32 * nt + col] = acc[nt][i];
      }
    }
    __syncthreads();
    {
      const int ml = tid >> 3, nc = (tid & 7) * 8;
      const int mm = m0 + ml;
      if (mm < p.M) {
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          s[i] = red[(0 * 32 + ml) * kNB + nc + i] + red[(1 * 32 + ml) * kNB + nc + i] +
                 red[(2 * 32 + ml) * kNB + nc + i] + red[(3 * 32 + ml) * kNB + nc + i];
        const int64_t off = ((int64_t)mm * H + h) * N + n0 + nc;
        if constexpr (CF32) {
          float* c = (float*)p.c + off;
          *(f32x4*)c = f32x4{s[0], s[1], s[2], s[3]};
          *(f32x4*)(c + 4) = f32x4{s[4], s[5], s[6], s[7]};
        } else {
          *(bf16x8*)((uint16_t*)p.c + off) = pack_bf16x8(s);
        }
      }
    }
    __syncthreads();
  }
}

template <bool AF32, bool CF32>
hipError_t launch_variant(const HeadGemmParams& p, size_t smem, hipStream_t stream) {
  // The W tile plus the reduction buffer exceed the default dynamic-LDS limit
  // when K = 512 (96 KiB); allow that once per instantiation.
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(head_gemm_kernel<AF32, CF32>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kMaxGemmLds);
  if (attr != hipSuccess) return attr;
  if (smem > (size_t)kMaxGemmLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL((head_gemm_kernel<AF32, CF32>), dim3(p.H * (p.N / kNB)), dim3(256), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_head_gemm(const HeadGemmParams& p, bool a_fp32, bool c_fp32, hipStream_t stream) {
  const size_t smem = (size_t)p.K * kNB * 2 + 4 * 32 * kNB * sizeof(float);
  if (a_fp32) return c_fp32 ? launch_variant<true, true>(p, smem, stream) : launch_variant<true, false>(p, smem, stream);
  return c_fp32 ? launch_variant<false, true>(p, smem, stream) : launch_variant<false, false>(p, smem, stream);
}

}  // namespace mla
