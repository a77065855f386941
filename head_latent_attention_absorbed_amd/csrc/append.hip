// Paged cache append: the records of the new tokens (gfx950).
//
// A token's latent is the down-projection of its hidden state, c_KV = x W_DKV
// (the W_DKV of Eq. (11) on the TransMLA review page, named in
// referee_report.minor_comments), and next to it the cache keeps one RoPE
// key shared by every head (core_discovery on the same page), the projection
// x W_KR turned by the token's position.  The two projections are one matrix
// [W_DKV | W_KR] of d_model x (d_c + 64).
//
// The product (M = B*S_q rows, bound by reading the matrix) runs as the
// per-head product with d_model cut into slices of 256: "head" k multiplies
// x[:, 256k .. 256k+255] by rows 256k .. of the matrix into fp32 partials.
// Then one work-group per new token sums its partials (eight waves split the
// slices, LDS adds the eight sums), turns the RoPE pairs (2i, 2i+1) by
// pos * base^(-2i/64) with the angle taken in fp64, and writes the record to
// page block_table[b][pos / block_size], slot pos % block_size, as bf16
// (nearest even) or as e4m3 bytes of v / scale with one fp32 scale per token,
// scale = max|v| / 448 over the record.  The new tokens are the last S_q
// positions of each sequence; an idle slot (length 0) is left alone.
#include <atomic>

#include "mla_absorbed.h"
#include "mla_device.h"
#include "mla_kernels.h"

// Device memory of mla_append_kv_noalloc: the split-K partial products live
// here instead of in a caller workspace.  Every GPU that loads the library
// holds its own copy until the process ends; in host code this name is only a
// stand-in for the symbol, so its device address is looked up once per device
// (append_scratch) and only that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[MLA_APPEND_NOALLOC_MAX_BYTES];

namespace mla {

hipError_t append_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Resolved with the device current; two threads racing here both get
    // the same address, so a plain store suffices.
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

constexpr int kFinishWaves = 8;
constexpr float kE4m3Max = 448.0f;

// OCP E4M3 (bias 7, 3 mantissa bits, no infinity) of |x| <= 448, nearest
// with ties to even, built from the format: below 2^-6 the values are
// multiples of 2^-9 (m = 8 is 2^-6 itself, which the same code denotes);
// above, a binade 2^E holds 1 + m/8.  A negative value keeps its sign even
// when it rounds to zero.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  const int E = ilogbf(a);                       // a in [2^E, 2^(E+1))
  int r = (int)rintf(ldexpf(a, 3 - E));          // 8 .. 16
  int e = E;
  if (r == 16) {
    r = 8;
    ++e;
  }
  const uint32_t code = (uint32_t)(((e + 7) << 3) | (r - 8));
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

template <int DC>
__global__ void __launch_bounds__(kFinishWaves * 64) append_finish_kernel(AppendParams p) {
  constexpr int NR = DC + 64;  // record values
  constexpr int J = NR / 64;   // values per lane: columns lane + 64 j
  __shared__ float red[kFinishWaves][NR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = blockIdx.x;
  const int b = m / p.S, s = m % p.S;
  const int L = p.seq_lens[b];
  const int pos = L - p.S + s;
  if (L <= 0 || pos < 0) return;  // idle slot: nothing to append

  // Wave w sums slices w, w + 8, ...; all of a wave's loads are issued first.
  float v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = 0.0f;
  const float* base = p.part + (int64_t)m * p.KS * NR + lane;
  for (int k0 = w; k0 < p.KS; k0 += 4 * kFinishWaves) {
    float t[4][J];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * kFinishWaves;
#pragma unroll
      for (int j = 0; j < J; ++j) t[u][j] = k < p.KS ? base[(int64_t)k * NR + 64 * j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < J; ++j) v[j] += t[u][j];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) red[w][lane + 64 * j] = v[j];
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float x = 0.0f;
#pragma unroll
    for (int q = 0; q < kFinishWaves; ++q) x += red[q][lane + 64 * j];
    v[j] = x;
  }

  // RoPE on the last 64 values: lane pair (2i, 2i+1) holds pair i.
  {
    const int i = lane >> 1;
    const double th = exp2(-(double)(2 * i) / 64.0 * p.log2_base);
    double sn, cs;
    sincos((double)pos * th, &sn, &cs);
    const float own = v[J - 1];
    const float other = __shfl_xor(own, 1);
    const float x0 = (lane & 1) ? other : own, x1 = (lane & 1) ? own : other;
    v[J - 1] = (lane & 1) ? x0 * (float)sn + x1 * (float)cs : x0 * (float)cs - x1 * (float)sn;
  }

  const int page = p.block_table[(int64_t)b * p.bt_stride + pos / p.block_size];
  const int slot = pos % p.block_size;
  char* rec = p.c_kv + (int64_t)page * p.block_stride + (int64_t)slot * p.token_stride;
  if (!p.fp8) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const __bf16 h = (__bf16)v[j];
      const int64_t off = j < J - 1 ? (int64_t)(lane + 64 * j) * 2 : p.rope_off + (int64_t)lane * 2;
      *(uint16_t*)(rec + off) = __builtin_bit_cast(uint16_t, h);
    }
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax > 0.0f ? amax / kE4m3Max : 1.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float q = fminf(fmaxf(v[j] / scale, -kE4m3Max), kE4m3Max);
      const int64_t off = j < J - 1 ? (int64_t)(lane + 64 * j) : p.rope_off + (int64_t)lane;
      *(uint8_t*)(rec + off) = (uint8_t)e4m3_code(q);
    }
    if (lane == 0) p.kv_scale[(int64_t)page * p.block_size + slot] = scale;
  }
}

}  // namespace

hipError_t launch_append_finish(const AppendParams& p, hipStream_t stream) {
  if (p.M <= 0) return hipSuccess;
  if (p.DC == 512)
    hipLaunchKernelGGL(append_finish_kernel<512>, dim3(p.M), dim3(kFinishWaves * 64), 0, stream, p);
  else if (p.DC == 256)
    hipLaunchKernelGGL(append_finish_kernel<256>, dim3(p.M), dim3(kFinishWaves * 64), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
