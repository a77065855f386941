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
// Both are small per-head GEMMs bound by reading W (M = B*S_q rows only).  A
// work-group takes one head and NSUB*64 output columns and stages that slice
// of W in LDS as NSUB sub-tiles of [K][64] (16-byte granules XOR-swizzled per
// row), read transposed as the MFMA B operand.  Its four waves split the work
// NSUB ways over the sub-tiles and KS = 4 / NSUB ways over K; the K parts are
// summed through LDS, which also turns the accumulator layout into 16-byte
// row-contiguous stores.  Every global load of the W slice and of the wave's
// A fragments is issued before the first is waited for, so a work-group costs
// about one memory latency plus its bytes.  An fp32 A operand is split into
// bf16 high and low parts, two MFMAs, for near-fp32 accuracy.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kSub = 64;          // columns of one W sub-tile
constexpr int kMaxKSteps = 8;     // 16-deep k-steps per wave (K / KS <= 128)
constexpr int kStageBatch = 8;    // W granules per thread loaded before they are stored
constexpr size_t kMaxGemmLds = 96 * 1024;  // 64 KiB W slice + 32 KiB reduction buffer

__device__ __forceinline__ int swzw(int k) { return ((k & 3) << 1) | ((k >> 2) & 1); }

// This lane's A fragments of rows m0..m0+31 for every k-step of its K range:
// row m0 + col, columns kbeg + 16 ks + 8 half .. +7 (zeros past the last
// row).  The row is clamped and the value selected, not branched on, so all
// NKS loads are issued back to back.
template <bool AF32, int NKS>
__device__ __forceinline__ void load_a(const HeadGemmParams& p, int m0, int col, int half, int h, int kbeg,
                                       bf16x8 (&ahi)[NKS], f32x4 (&af)[2 * NKS]) {
  const int m = m0 + col;
  const bool valid = m < p.M;
  const int64_t ar = p.a_row ? p.a_row : (int64_t)p.H * p.K;
  const int64_t ah = p.a_row ? p.a_head : (int64_t)p.K;
  const int64_t rowoff = (int64_t)min(m, p.M - 1) * ar + h * ah + kbeg + 8 * half;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (AF32) {
      const float* ap = (const float*)p.a + rowoff + 16 * ks;
      af[2 * ks] = *(const f32x4*)ap;
      af[2 * ks + 1] = *(const f32x4*)(ap + 4);
    } else {
      ahi[ks] = *(const bf16x8*)((const uint16_t*)p.a + rowoff + 16 * ks);
    }
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (AF32) {
      af[2 * ks] = valid ? af[2 * ks] : f32x4{};
      af[2 * ks + 1] = valid ? af[2 * ks + 1] : f32x4{};
    } else {
      ahi[ks] = valid ? ahi[ks] : bf16x8{};
    }
  }
}

template <int NSUB>
constexpr size_t gemm_lds_bytes(int K) {
  constexpr int KS = 4 / NSUB;
  return (size_t)K * NSUB * kSub * 2 + (size_t)KS * 32 * NSUB * kSub * 4;
}

// NKS: 16-deep k-steps of each wave (K = 16 * NKS * KS).
template <bool AF32, bool CF32, int NSUB, int NKS>
__global__ void __launch_bounds__(256) head_gemm_kernel(HeadGemmParams p) {
  constexpr int KS = 4 / NSUB;
  constexpr int NB = NSUB * kSub;  // columns per work-group
  constexpr int K = 16 * NKS * KS;
  constexpr int GPT = K * NB / 8 / 256;  // W granules per thread
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int H = p.H, N = p.N;
  char* wt = smem;                                     // NSUB x [K][64] bf16, swizzled granules
  float* red = (float*)(smem + (size_t)K * NB * 2);    // [KS][32][NB] fp32

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int nblocks = N / NB;
  const int h = blockIdx.x / nblocks;
  const int n0 = (blockIdx.x % nblocks) * NB;
  const int sub = w % NSUB, kp = w / NSUB;
  const int kbeg = kp * (K / KS);  // K range of this wave

  // A fragments of the first row tile, requested before the W slice so that
  // both are in flight together.
  bf16x8 a_bf[NKS];
  f32x4 a_f[2 * NKS];
  load_a<AF32, NKS>(p, 0, col, half, h, kbeg, a_bf, a_f);

  // Stage W[h][:, n0:n0+NB]: granule i = (sub-tile, k, 16-byte column group),
  // all of this thread's loads first, then all of its LDS stores.
  const uint16_t* wsrc = p.w + (int64_t)h * K * N + n0;
  uint4 v[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int idx = 256 * j + tid;
    const int s = idx / (K * 8), r = idx % (K * 8);
    v[j] = *(const uint4*)(wsrc + (int64_t)(r >> 3) * N + s * kSub + 8 * (r & 7));
  }
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int idx = 256 * j + tid;
    const int s = idx / (K * 8), r = idx % (K * 8);
    const int k = r >> 3;
    *(uint4*)(wt + (size_t)s * K * 128 + k * 128 + (((r & 7) ^ swzw(k)) * 16)) = v[j];
  }
  __syncthreads();

  // Lane constants of the transposing W^T reads.
  const int i16 = lane & 15, grp = lane >> 4;
  const int jj = i16 >> 2, qq = i16 & 3, ch = grp & 1;
  const char* wsub = wt + (size_t)sub * K * 128;

  for (int m0 = 0; m0 < p.M; m0 += 32) {
    if (m0 > 0) load_a<AF32, NKS>(p, m0, col, half, h, kbeg, a_bf, a_f);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      {
        bf16x8 ahi, alo;
        if constexpr (AF32) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = i < 4 ? a_f[2 * ks][i] : a_f[2 * ks + 1][i - 4];
            const __bf16 hi = (__bf16)x;
            ahi[i] = hi;
            alo[i] = (__bf16)(x - (float)hi);
          }
        } else {
          ahi = a_bf[ks];
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int e = 4 * nt + 2 * ch + (qq >> 1);
          s16x4 r[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int k = kbeg + 16 * ks + 8 * half + 4 * h2 + jj;
            const int sw = (jj << 1) | h2;
            r[h2] = lds_read_tr16(wsub + k * 128 + ((e ^ sw) * 16) + (qq & 1) * 8);
          }
          const s16x8 bv = {r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
          acc[nt] = mfma32(ahi, (bf16x8)bv, acc[nt]);
          if constexpr (AF32) acc[nt] = mfma32(alo, (bf16x8)bv, acc[nt]);
        }
      }
    }
    // Partial sums to LDS: rows of the tile, the wave's 64 columns.
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ml = 8 * (i >> 2) + 4 * half + (i & 3);
        red[(kp * 32 + ml) * NB + sub * kSub + 32 * nt + col] = acc[nt][i];
      }
    }
    __syncthreads();
    // Sum the K parts and write 8 consecutive columns per thread.
    for (int e = tid; e < 32 * NB / 8; e += 256) {
      const int ml = e / (NB / 8), nc = (e % (NB / 8)) * 8;
      const int mm = m0 + ml;
      if (mm < p.M) {
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float t = 0.0f;
#pragma unroll
          for (int q = 0; q < KS; ++q) t += red[(q * 32 + ml) * NB + nc + i];
          s[i] = t;
        }
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

template <bool AF32, bool CF32, int NSUB, int NKS>
hipError_t launch_variant(const HeadGemmParams& p, hipStream_t stream) {
  const size_t smem = gemm_lds_bytes<NSUB>(p.K);
  // The W slice plus the reduction buffer exceed the default dynamic-LDS
  // limit; raise it once per instantiation to the largest size used.
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(head_gemm_kernel<AF32, CF32, NSUB, NKS>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxGemmLds);
  if (attr != hipSuccess) return attr;
  if (smem > kMaxGemmLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL((head_gemm_kernel<AF32, CF32, NSUB, NKS>), dim3(p.H * (p.N / (NSUB * kSub))), dim3(256), smem,
                     stream, p);
  return hipGetLastError();
}

template <bool AF32, bool CF32, int NSUB, int NKS, int... MORE>
hipError_t launch_nks(const HeadGemmParams& p, int nks, hipStream_t stream) {
  if (nks == NKS) return launch_variant<AF32, CF32, NSUB, NKS>(p, stream);
  if constexpr (sizeof...(MORE) > 0) return launch_nks<AF32, CF32, NSUB, MORE...>(p, nks, stream);
  return hipErrorInvalidValue;
}

// Absorb (bf16 A and C): K = d_nope, a multiple of 64 up to 512.  Four
// 64-column sub-tiles per work-group (no K split) for K <= 128, else one
// sub-tile with K split four ways.
hipError_t launch_absorb(const HeadGemmParams& p, hipStream_t stream) {
  if (p.N % (4 * kSub) == 0 && p.K <= 128) return launch_nks<false, false, 4, 4, 8>(p, p.K / 16, stream);
  return launch_nks<false, false, 1, 3, 4, 5, 6, 7, 8>(p, p.K / 64, stream);
}

// Up-projection (fp32 A): K = d_latent (256 or 512), one sub-tile, K split four ways.
template <bool CF32>
hipError_t launch_up(const HeadGemmParams& p, hipStream_t stream) {
  return launch_nks<true, CF32, 1, 4, 8>(p, p.K / 64, stream);
}

}  // namespace

// Split-K partial products of a product too deep for one work-group (the
// cache append's x . [W_DKV | W_KR]): bf16 A and W, fp32 C, one K slice of
// K = 128 or 256 per "head".
hipError_t launch_head_gemm_partials(const HeadGemmParams& p, hipStream_t stream) {
  if (p.N % kSub != 0 || (p.K != 128 && p.K != 256)) return hipErrorInvalidValue;
  return launch_nks<false, true, 1, 2, 4>(p, p.K / 64, stream);
}

namespace {

// W [H, R, C] -> [H, C, R], one 64 x 64 tile per work-group through LDS (rows
// padded by 8 elements so that the transposed reads spread over the banks).
__global__ void __launch_bounds__(256) transpose_heads_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                              int R, int C) {
  __shared__ uint16_t t[64][64 + 8];
  const int h = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const uint16_t* src = w + ((int64_t)h * R + r0) * C + c0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = tid + 256 * j;
    t[i / 64][i % 64] = src[(int64_t)(i / 64) * C + i % 64];
  }
  __syncthreads();
  uint16_t* dst = wt + ((int64_t)h * C + c0) * R + r0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = tid + 256 * j;
    dst[(int64_t)(i / 64) * R + i % 64] = t[i % 64][i / 64];
  }
}

}  // namespace

hipError_t launch_transpose_heads(const uint16_t* w, uint16_t* wt, int H, int R, int C, hipStream_t stream) {
  if (R % 64 || C % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_heads_kernel, dim3(C / 64, R / 64, H), dim3(256), 0, stream, w, wt, R, C);
  return hipGetLastError();
}

bool head_gemm_supported(int K, int N) {
  // K = 64 or 128 with N a multiple of 256 (four sub-tiles), or K a multiple
  // of 64 in [192, 512] with N a multiple of 64 (K split four ways).
  if (K % 64 != 0 || K > 512 || N % kSub != 0) return false;
  return K > 128 || N % (4 * kSub) == 0;
}

hipError_t launch_head_gemm(const HeadGemmParams& p, bool a_fp32, bool c_fp32, hipStream_t stream) {
  if (!head_gemm_supported(p.K, p.N)) return hipErrorInvalidValue;
  if (a_fp32) {
    if (p.K != 256 && p.K != 512) return hipErrorInvalidValue;
    return c_fp32 ? launch_up<true>(p, stream) : launch_up<false>(p, stream);
  }
  if (c_fp32) return hipErrorInvalidValue;
  return launch_absorb(p, stream);
}

}  // namespace mla
