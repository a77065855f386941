// GQLA's GQA decoding path on the latent decode kernel (gfx950).
//
// GQLA weights expose two equivalent decoding paths: MLA's absorbed MQA path
// over the latent, and a GQA path over a cache expanded per head group, run
// with two query tokens per step (GQLA abstract on the "GQA-to-MLA" Daily
// Papers listing).  The GQA path needs no kernel of its own: a group's record
// [K_nope | V | k_rope] is read as a latent record of width d_nope + d_v, and
// the query [q_nope | 0] scores it exactly as q_nope . K_nope + q_rope . k_rope;
// the attention output's last d_v columns are then sum_t p_t V_t.  Each
// (sequence, group) pair is one sequence of that decode, its H / G heads the
// rows.  These two launches only regroup: queries into the per-stream rows
// (with the zero half), and the value columns of the merged rows back into
// [B, S_q, H, d_v].  Both are plain copies bound by memory traffic.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

// One thread per 16-byte granule of the regrouped query rows.
__global__ void __launch_bounds__(256) gqa_queries_kernel(GqaParams p) {
  const int DQ = p.dn + p.dv;                 // width of the query row against the record
  const int gq = DQ / 8, gr = p.dr / 8;       // granules per row
  const int64_t rows = (int64_t)p.B * p.S * p.H;
  const int64_t total = rows * (gq + gr);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / (gq + gr);
    const int c = (int)(i % (gq + gr));
    // destination row r = ((b G + g) S + s) hpg + j
    const int hpg = p.H / p.G;
    const int j = (int)(r % hpg);
    const int64_t t = r / hpg;
    const int s = (int)(t % p.S);
    const int64_t bg = t / p.S;
    const int g = (int)(bg % p.G);
    const int64_t b = bg / p.G;
    const int64_t src = (b * p.S + s) * p.H + (int64_t)g * hpg + j;  // row of q_nope / q_rope
    if (c < gq) {
      const uint4 v = 8 * c < p.dn ? *(const uint4*)(p.q_nope + src * p.dn + 8 * c) : uint4{0, 0, 0, 0};
      *(uint4*)(p.q_cat + r * DQ + 8 * c) = v;
    } else {
      const int cr = c - gq;
      *(uint4*)(p.q_rope_g + r * p.dr + 8 * cr) = *(const uint4*)(p.q_rope + src * p.dr + 8 * cr);
    }
  }
}

// One thread per four output values (and the row's lse with the first four).
template <bool F32>
__global__ void __launch_bounds__(256) gqa_output_kernel(GqaParams p) {
  const int DQ = p.dn + p.dv;
  const int q4 = p.dv / 4;
  const int64_t rows = (int64_t)p.B * p.S * p.H;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * q4; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / q4;  // output row (b S + s) H + h
    const int c = (int)(i % q4);
    const int h = (int)(r % p.H);
    const int64_t bs = r / p.H;
    const int s = (int)(bs % p.S);
    const int64_t b = bs / p.S;
    const int hpg = p.H / p.G;
    const int g = h / hpg, j = h % hpg;
    const int64_t src = ((b * p.G + g) * p.S + s) * hpg + j;  // merged row of stream (b, g)
    const f32x4 v = *(const f32x4*)(p.o_lat + src * DQ + p.dn + 4 * c);
    if constexpr (F32) {
      *(f32x4*)((float*)p.out + r * p.dv + 4 * c) = v;
    } else {
      const bf16x2 a = {(__bf16)v[0], (__bf16)v[1]}, d = {(__bf16)v[2], (__bf16)v[3]};
      *(uint2*)((uint16_t*)p.out + r * p.dv + 4 * c) =
          uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, d)};
    }
    if (c == 0) p.lse[r] = p.lse_g[src];
  }
}

dim3 grid_for(int64_t work) {
  const int64_t wgs = (work + 255) / 256;
  return dim3((unsigned)(wgs < 16384 ? wgs : 16384));
}

}  // namespace

hipError_t launch_gqa_queries(const GqaParams& p, hipStream_t stream) {
  const int64_t work = (int64_t)p.B * p.S * p.H * ((p.dn + p.dv) / 8 + p.dr / 8);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(gqa_queries_kernel, grid_for(work), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gqa_output(const GqaParams& p, bool out_f32, hipStream_t stream) {
  const int64_t work = (int64_t)p.B * p.S * p.H * (p.dv / 4);
  if (work == 0) return hipSuccess;
  if (out_f32) hipLaunchKernelGGL((gqa_output_kernel<true>), grid_for(work), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((gqa_output_kernel<false>), grid_for(work), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
