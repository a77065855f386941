// Pieces shared by the 128-row decode kernels (gfx950): the tile source of
// a part, the bf16 tile copy, the rare rescale of accumulator rows, the
// online softmax of one tile in steps, and the step-less stand-in.
#pragma once
#include "decode_common.h"
#include "mla_device.h"
#include "mla_kernels.h"
#include "tile_ops.h"

namespace mla {
namespace {

// Address of tile t (sequence-local, 32 tokens) of the part's sequence and
// its number of cached tokens.
struct TileSrc {
  const char* run;
  int nv;
  int page_slot;  // page * block_size + first slot (fp8 scales)
};

// The physical page of tile t, read one iteration before the copy that
// needs it.  The read is made a vector load (the lane-dependent zero), so
// that it is counted with the copies (vmcnt) and waited for together with
// them at the next tile barrier; a scalar load would share its counter with
// the LDS reads, whose waits would then also wait for it.
__device__ __forceinline__ int tile_page_load(const DecodeParams& p, const int32_t* bt, int t) {
  return bt[((t * kTile) >> p.block_shift) + (opaque_lane() >> 6)];
}

__device__ __forceinline__ TileSrc tile_src(const DecodeParams& p, int page, int t, int L) {
  const int pos0 = t * kTile;
  const int slot0 = pos0 & (p.block_size - 1);
  TileSrc s;
  s.run = p.c_kv + (int64_t)page * p.block_stride + (int64_t)slot0 * p.token_stride;
  s.nv = min(L - pos0, kTile);
  s.page_slot = page * p.block_size + slot0;
  return s;
}

// bf16 tile copy by four waves: this wave's NI granule-row pairs.  Lanes
// whose token is past the sequence's length copy token 0 instead (finite data
// the softmax weighs 0), so every instruction runs with all lanes.
template <int DC>
__device__ __forceinline__ void copy_tile(const DecodeParams& p, const TileSrc& s, uint32_t buf_lds, int w) {
  constexpr int NW = 4, NI = Geo<DC>::GPT / (2 * NW);
  const int ol = opaque_lane();
  int tok = load_token(ol);
  tok = tok < s.nv ? tok : 0;
  const uint32_t lane_off = (uint32_t)tok * (uint32_t)p.token_stride + 16u * (ol >> 5);
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int g0 = 2 * (q * NW + w);
    lds_dma16(s.run + granule_offset<DC, 16>(p, g0), lane_off, uniform(buf_lds + (q * NW + w) * 1024));
  }
}

// Multiply rows of the accumulators by their factors (rare; see rescale in
// tile_ops.h for the AGPR-constrained form and the wait states).
template <int NBW>
__device__ __forceinline__ void rescale_rows(f32x16 (&O)[4][NBW], const float (&a)[4]) {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = O[rb][cb][i];
        float tmp;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32_e32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(tmp)
                     : "v"(a[rb]));
        O[rb][cb][i] = x;
      }
    }
  }
  asm volatile("s_nop 1" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Online softmax of one tile's scores for the wave's 32 rows (one code path
// for full and partly visible tiles), in steps that pv_rows spreads over its
// MFMAs.  Lane (col, half) holds row col and tokens 8(i/4) + 4 half + i%4 in
// value i; entry i is visible iff 8(i/4) + i%4 < rel, rel = (first position
// the row may not see) - (tile start) - 4 half.  The maximum is taken over
// the raw scores and scaled afterwards (the scale is positive); weights are
// exp2(s * scale - m) with one fused multiply-add.  For an e4m3 tile the raw
// scores are first multiplied by their tokens' scales (the keys' scale) and
// the weights by them again after the sum (the values' scale, carried by P).
template <bool FP8>
struct WideSoftmax {
  static constexpr int STEPS = 12;
  f32x16 v;
  const float* tsc;  // fp8: the tile's per-token scales (LDS)
  int rel;
  float slog2;
  float& m_run;
  float& l_run;
  int half;
  float m_new, mu, alpha;
  bf16x8 pf0, pf1;

  __device__ __forceinline__ void step(int j) {
    if (j < 4) {  // scale (e4m3) and mask four entries
      f32x4 s4 = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (FP8) s4 = *(const f32x4*)(tsc + 8 * j + 4 * half);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = v[4 * j + c];
        if constexpr (FP8) x *= s4[c];
        v[4 * j + c] = (8 * j + c < rel) ? x : -__builtin_inff();
      }
    } else if (j == 4) {
      float a = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      float b = fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7]));
      float c = fmaxf(fmaxf(v[8], v[9]), fmaxf(v[10], v[11]));
      float d = fmaxf(fmaxf(v[12], v[13]), fmaxf(v[14], v[15]));
      m_new = fmaxf(fmaxf(a, b), fmaxf(c, d));
    } else if (j == 5) {
      const float mt = pair_max(m_new) * slog2;
      const bool rebase = mt > m_run + kRebase;  // never for a tile this row sees nothing of (mt = -inf)
      m_new = rebase ? mt : m_run;
      alpha = rebase ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 on the first visible tile
      l_run *= alpha;
      m_run = m_new;
      // A row that has seen no position yet keeps m = -inf with every entry
      // at -inf: exp2(-inf - 0) gives the weights 0 instead of NaN.
      mu = m_new == -__builtin_inff() ? 0.0f : m_new;
    } else if (j < 10) {  // weights, four at a time
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * (j - 6) + c;
        v[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], slog2, -mu));
      }
    } else if (j == 10) {
      float t0 = v[0] + v[1], t1 = v[2] + v[3], t2 = v[4] + v[5], t3 = v[6] + v[7];
      float t4 = v[8] + v[9], t5 = v[10] + v[11], t6 = v[12] + v[13], t7 = v[14] + v[15];
      l_run += ((t0 + t1) + (t2 + t3)) + ((t4 + t5) + (t6 + t7));
      if constexpr (FP8) {  // the scales again (re-read rather than kept in registers)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 s4 = *(const f32x4*)(tsc + 8 * q + 4 * half);
#pragma unroll
          for (int c = 0; c < 4; ++c) v[4 * q + c] *= s4[c];
        }
      }
    } else if (j == 11) {
      float w8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = v[i];
      pf0 = pack_bf16x8(w8);
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = v[8 + i];
      pf1 = pack_bf16x8(w8);
    }
  }
  __device__ __forceinline__ void all() {
#pragma unroll
    for (int j = 0; j < STEPS; ++j) step(j);
  }
};

// The step-less stand-in for pv_rows when no softmax rides along.
struct NoSteps {
  static constexpr int STEPS = 0;
  __device__ __forceinline__ void step(int) {}
};

}  // namespace
}  // namespace mla
