// Pieces shared by the two decode kernels (gfx950): waits on the tile
// copies, the record's granule addressing, the e4m3 staging and decode, and
// the store of a normalised partial.
#pragma once
#include "mla_device.h"
#include "mla_kernels.h"
#include "tile_ops.h"

namespace mla {
namespace {

template <int NI, int MAXLATER>
__device__ __forceinline__ void wait_dma_groups(int later) {
  // Tiles complete in issue order; `later` (<= MAXLATER) DMA groups of NI
  // loads were issued after the one being waited for.
  static_assert(NI * MAXLATER <= 63, "vmcnt range");
  if constexpr (MAXLATER == 0) {
    vm_wait<0>();
  } else if constexpr (MAXLATER == 1) {
    if (later <= 0) vm_wait<0>(); else vm_wait<NI>();
  } else {
    static_assert(MAXLATER == 2, "ring depth");
    if (later <= 0) vm_wait<0>();
    else if (later == 1) vm_wait<NI>();
    else vm_wait<NI * 2>();
  }
}



// The token a lane moves in every tile-load instruction: slot lane % 32 of
// row 2m + lane / 32 holds token (lane % 32) ^ (4 * (lane / 32)).
__device__ __forceinline__ int load_token(int lane) { return (lane & 31) ^ ((lane >> 5) << 2); }

// Byte offset of granule row pair (g0, g0+1) inside a cache record (GB-byte
// granules: 16 for bf16, 8 for e4m3).  g0 is even, so a pair never straddles
// the latent and the RoPE key.
template <int DC, int GB>
__device__ __forceinline__ int64_t granule_offset(const DecodeParams& p, int g0) {
  return g0 < Geo<DC>::GC ? (int64_t)g0 * GB : p.rope_off + (int64_t)(g0 - Geo<DC>::GC) * GB;
}

// fp8 tile: the records' e4m3 bytes are copied with global->LDS DMA into a
// staging slot (row pair m = bytes 16m..16m+15 of the latent, then of the
// RoPE key, of token t at byte (32 m + t) * 16), so nothing is held in
// registers while the previous tile is computed; then every thread decodes
// its share exactly (every e4m3 value is a bf16 value) into the bf16 tile
// layout, tokens past the length as zeros.
template <int DC>
struct Fp8Geo {
  static constexpr int NP = Geo<DC>::GPT / 2;      // row pairs of a tile
  static constexpr int NINS = NP / 2;              // DMA instructions (two pairs each)
  static constexpr int BYTES = NP * kTile * 16;    // staging slot
};

template <int DC, int NW>
__device__ __forceinline__ void issue_fp8_dma(const DecodeParams& p, const char* run, uint32_t stage_lds, int w) {
  using F = Fp8Geo<DC>;
  const int ol = opaque_lane();
  const uint32_t lane_off = (uint32_t)(ol & 31) * (uint32_t)p.token_stride + 16u * (ol >> 5);
#pragma unroll
  for (int q = 0; q < (F::NINS + NW - 1) / NW; ++q) {
    const int ins = q * NW + w;
    if (ins < F::NINS) {
      const int m0 = 2 * ins;  // pairs m0, m0 + 1 never straddle the latent and the RoPE key
      const int64_t off = m0 < Geo<DC>::GC / 2 ? (int64_t)m0 * 16 : p.rope_off + (int64_t)(m0 - Geo<DC>::GC / 2) * 16;
      lds_dma16(run + off, lane_off, uniform(stage_lds + ins * 1024));
    }
  }
}

template <int DC, int NW>
__device__ __forceinline__ void convert_fp8_tile(const char* stage, char* tb, int nv, int tid) {
  using F = Fp8Geo<DC>;
  for (int i = tid; i < F::NP * kTile; i += NW * kWave) {
    const int m = i >> 5, t = i & 31;
    const uint4 x = *(const uint4*)(stage + i * 16);
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true);
    const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.z, 1.0f, false);
    const bf16x2 f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.z, 1.0f, true);
    const bf16x2 g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.w, 1.0f, false);
    const bf16x2 h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.w, 1.0f, true);
    bf16x8 lo = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};  // granule row 2m
    bf16x8 hi = {e[0], e[1], f[0], f[1], g[0], g[1], h[0], h[1]};  // granule row 2m + 1
    if (t >= nv) {
      lo = bf16x8{};
      hi = bf16x8{};
    }
    *(bf16x8*)(tb + (2 * m) * kRow + (t << 4)) = lo;            // even row: slot t
    *(bf16x8*)(tb + (2 * m + 1) * kRow + ((t ^ 4) << 4)) = hi;  // odd row: slot t ^ 4
  }
}

// Write NBK accumulator blocks (32 latent columns each, starting at element
// offset `base` of o_part) scaled by inv, as fp16 or fp32.
template <int NBK>
__device__ __forceinline__ void store_partial(const DecodeParams& p, const f32x16* O, float inv, int64_t base,
                                              int half) {
  if (p.o_half) {
    // Lane pair (l, l + 32) swaps packed halves so that each lane stores 8
    // consecutive columns: with column quarters q0..q3 of an 8-column group
    // split 4 + 4 over the pair, the swap gives the lower lane the odd group
    // and the upper lane the even one.
    _Float16* dst = (_Float16*)p.o_part + base + 8 * (1 - half);
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x2 v = {(_Float16)(O[nb][2 * j] * inv), (_Float16)(O[nb][2 * j + 1] * inv)};
        h[j] = __builtin_bit_cast(uint32_t, v);
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {  // 8-column groups (2pr, 2pr + 1)
        const auto r0 = __builtin_amdgcn_permlane32_swap(h[4 * pr + 2], h[4 * pr], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(h[4 * pr + 3], h[4 * pr + 1], false, false);
        const uint4 v = {r0[0], r1[0], r0[1], r1[1]};
        *(uint4*)(dst + 32 * nb + 16 * pr) = v;
      }
      __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time
    }
  } else {
    float* dst = (float*)p.o_part + base + 4 * half;
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const f32x4 v = {O[nb][4 * ig] * inv, O[nb][4 * ig + 1] * inv, O[nb][4 * ig + 2] * inv,
                         O[nb][4 * ig + 3] * inv};
        *(f32x4*)(dst + 32 * nb + 8 * ig) = v;
      }
      __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time
    }
  }
}

}  // namespace
}  // namespace mla
