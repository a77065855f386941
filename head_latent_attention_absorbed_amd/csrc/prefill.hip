// MLA-form prefill attention over tile-native keys and values (gfx950).
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "tile_ops.h"

namespace mla {
namespace {

// Prefill in the MLA form (keys and values reconstructed per head, as the
// prefill-decode separation of the TPLA abstract keeps for the compute-bound
// prefill): every position of a prompt attends causally to the positions up
// to it, per head, over K = [W_UK c ; k_rope] (128 + 64) and V = c W_UV (128)
// made by mla_prefill_kv.  The tile products, the online softmax and P.V
// are the decode's, at latent width 128: a 32-token tile of K (24 granule
// rows) and of V (16 rows) in the same granule-major LDS layout, one wave per
// 32 query positions of one head, four waves per work-group.  The keys and
// values are stored in that layout already (tile-native), so a tile is two
// contiguous 8 KiB copies plus the shared RoPE keys gathered from the
// records, all global->LDS DMA into a two-slot ring.
constexpr int kPfRows = 128;  // query positions per work-group
constexpr int kPfBuf = 2;     // ring slots: one tile computed while the next lands

// Three work-groups per CU (registers held to 168 per lane, a 40 KiB ring
// each): the tile loop is a chain of dependent MFMA and softmax steps, so
// more waves per SIMD pay more than a deeper ring (measured on the 2 x 4096
// DeepSeek-V3 prompt batch: 2252 us with a 4-slot ring at two groups per CU,
// 2018 us like this).
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
prefill_kernel(PrefillParams p) {
  using Gm = Geo<128>;
  constexpr int KROWS = Gm::GPT;   // 24 granule rows of K
  constexpr int VROWS = 16;        // 16 granule rows of V
  constexpr int TB = (KROWS + VROWS) * kRow;
  constexpr int NI = (KROWS + VROWS) / 8;  // DMA instructions per wave per tile (2 rows each, 4 waves)
  __shared__ __attribute__((aligned(1024))) char tiles[kPfBuf * TB];

  const int w = uniform(threadIdx.x >> 6);
  // XCD-aware placement: work item u = (sequence, head, query tile), longest
  // rows first; the grid (a multiple of 8) is dealt so that consecutive work
  // items land on the same XCD, which keeps each head's keys and values in
  // one L2 while its query tiles, all starting from key tile 0, re-read them.
  const int ntile = (p.P + kPfRows - 1) / kPfRows;
  const int u = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
  if (u >= ntile * p.H * p.B) return;
  const int pair = u / ntile;
  const int b = pair / p.H, h = pair % p.H;
  const int qt = ntile - 1 - u % ntile;  // longest rows first
  const int L = min(p.seq_lens[b], p.P);
  const int q0 = qt * kPfRows;
  if (q0 >= L) return;
  const int nkt = (min(L, q0 + kPfRows) + kTile - 1) / kTile;  // key tiles this group needs
  const int64_t tok0 = (int64_t)b * p.P;

  // Tile kt into ring slot s.  Instruction q of wave w fills granule rows
  // 2c, 2c + 1 with c = 4 q + w: rows 0..15 from the key tile, 16..23 from
  // the records' RoPE keys (lane l brings position 32 kt + (l % 32 ^ 4 (l / 32)),
  // clamped to the prompt), 24..39 from the value tile.
  const int T = (p.P + kTile - 1) / kTile;
  const char* kbase = (const char*)(p.k_nope + ((int64_t)b * p.H + h) * T * (kTile * 128));
  const char* vbase = (const char*)(p.v + ((int64_t)b * p.H + h) * T * (kTile * 128));
  const char* rbase = (const char*)(p.ckr + tok0 * (p.DCK + 64) + p.DCK);
  const uint32_t rec = (uint32_t)(p.DCK + 64) * 2;
  const uint32_t tiles_lds = lds_offset(tiles);
  const int dl = opaque_lane();
  const int rope_tok = (dl & 31) ^ (4 * (dl >> 5));
  auto issue = [&](int kt, int s) {
    const uint32_t dst = tiles_lds + s * TB;
    const uint32_t roff = (uint32_t)min(kt * kTile + rope_tok, L - 1) * rec + 16u * (dl >> 5);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int c = 4 * q + w;  // q 0, 1: key rows; 2: RoPE rows; 3, 4: value rows
      if (q < 2) {
        lds_dma16(kbase + (int64_t)kt * 8192 + c * 1024, 16u * dl, dst + c * 1024);
      } else if (q == 2) {
        lds_dma16(rbase + 32 * (c - 8), roff, dst + c * 1024);
      } else {
        lds_dma16(vbase + (int64_t)kt * 8192 + (c - 12) * 1024, 16u * dl, dst + c * 1024);
      }
    }
  };

  // This wave's 32 query positions.
  const int lane = opaque_lane();
  const int col = lane & 31;
  const int pos = q0 + 32 * w + col;
  bf16x8 qf[Gm::KS];
  {
    const int64_t row = (tok0 + min(pos, L - 1)) * p.H + h;
    const bf16x8* ql = (const bf16x8*)(p.q_nope + row * 128 + 8 * (lane >> 5));
    const bf16x8* qr = (const bf16x8*)(p.q_rope + row * 64 + 8 * (lane >> 5));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
    for (int ks = 8; ks < Gm::KS; ++ks) qf[ks] = qr[2 * (ks - 8)];
  }
  const int limit = min(pos + 1, L);  // causal: this row sees positions < limit

  // The queries have to be in registers before the ring copies start (the
  // compiler counts only its own loads, and would otherwise wait for every
  // copy in flight at their first use).
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  for (int i = 0; i < kPfBuf - 1 && i < nkt; ++i) issue(i, i);

  f32x16 O[Gm::NB];
  float m_run = -__builtin_inff(), l_run = 0.0f;
  bf16x8 pf0, pf1;
  float alpha;
  auto tile = [&](int kt, auto first_tag, auto full_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // FULL: the tile lies wholly below the group's first position, so every
    // row sees all of it (no causal mask, and the softmax takes its
    // branch-free form); a compile-time choice.
    constexpr bool FULL = decltype(full_tag)::value;
    // tile kt has landed (for every wave) and slot (kt - 1) % NBUF is free
    if (kt + kPfBuf - 2 < nkt) vm_wait<(kPfBuf - 2) * NI>(); else vm_wait<0>();
    block_sync();
    if (kt + kPfBuf - 1 < nkt) issue(kt + kPfBuf - 1, (kt + kPfBuf - 1) % kPfBuf);
    const char* tb = tiles + (kt % kPfBuf) * TB;
    score_tile<128, false, 0>(tb, nullptr, qf, m_run, l_run, kt * kTile, limit, FULL, p.scale_log2, pf0, pf1,
                              alpha, NoDma{});
    if constexpr (!FIRST) {
      if (__any(alpha != 1.0f)) rescale(O, alpha);
    }
    pv_tile<128, kPvAhead, FIRST>(tb + KROWS * kRow, pf0, pf1, O);
  };
  // Key tiles 0 .. kfull - 1 lie below the group's first position q0.
  const int kfull = min(nkt, q0 / kTile);
  int kt = 1;
  if (kfull > 0) {
    tile(0, std::true_type{}, std::true_type{});
    for (; kt < kfull; ++kt) tile(kt, std::false_type{}, std::true_type{});
  } else {
    tile(0, std::true_type{}, std::false_type{});
  }
  for (; kt < nkt; ++kt) tile(kt, std::false_type{}, std::false_type{});

  // Normalise and write this wave's rows: lane (col, half) holds row `col`,
  // columns 32 nb + 8 (i / 4) + 4 half + i % 4 of block nb.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (pos < L) {
    const int half = opaque_lane() >> 5;
    const int64_t row = (tok0 + pos) * p.H + h;
    if (half == 0) p.lse[row] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
    uint16_t* dst = p.out + row * 128 + 4 * half;
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 a = {(__bf16)(O[nb][4 * q] * inv), (__bf16)(O[nb][4 * q + 1] * inv)};
        const bf16x2 c = {(__bf16)(O[nb][4 * q + 2] * inv), (__bf16)(O[nb][4 * q + 3] * inv)};
        *(uint2*)(dst + 32 * nb + 8 * q) = uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)};
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.B <= 0 || p.P <= 0) return hipSuccess;
  const int64_t items = (int64_t)((p.P + kPfRows - 1) / kPfRows) * p.H * p.B;
  const dim3 grid((unsigned)((items + 7) / 8 * 8));
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
