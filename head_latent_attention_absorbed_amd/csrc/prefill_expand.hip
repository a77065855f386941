// Per-head keys and values of a prompt, from its latent records (gfx950).
//
//   k_nope[b, h, t, :] = W_UK[h] . c[b, t]      v[b, h, t, :] = W_UV[h]^T . c[b, t]
//
// In the MLA form the prefill attends over keys and values reconstructed per
// head from the cached latent (prefill-decode separation of the TPLA
// abstract; up-projections as in the TransMLA review page, core_discovery).
//
// Both products are one shape: D^T[128 dims][32 positions] = W^T[128][d_c] .
// C^T[d_c][32], with W^T = W_UK[h] for keys and the transposed W_UV[h] for
// values.  Written this way the MFMA output holds four consecutive dims of
// one position per lane, which is the granule order of the tile-native layout
// the prefill attention copies straight into LDS, so every store is a
// contiguous 512-byte run per wave.
//
// A work-group owns one head, keys and values: each of its eight waves (two
// per SIMD) keeps its 32 rows of one W^T in registers for the whole launch
// and streams 32-position tiles of records, which are copied into a
// four-slot LDS ring with global->LDS DMA (three tiles in flight) in the
// decode's granule-major layout, so the B-operand reads are conflict-free.
// Serving keys and values from one copy halves the re-reads of the records.  Only the tiles that hold
// positions < L_b are computed; positions L_b..end of the last one are
// written as zeros, and tiles past it are not written.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kXBuf = 4;  // ring slots

constexpr int kXWaves = 8;  // four for keys, four for values

template <int DC>
__global__ void __launch_bounds__(kXWaves * 64) expand_kernel(ExpandParams p) {
  constexpr int KS = DC / 16;        // 16-deep k-steps
  constexpr int ROWS = DC / 8;       // granule rows of a record tile
  constexpr int TBX = ROWS * kRow;   // bytes of one ring slot
  constexpr int NI = ROWS / (2 * kXWaves);  // DMA instructions per wave per tile (2 rows each)
  __shared__ __attribute__((aligned(1024))) char ring[kXBuf * TBX];
  // Lengths clamped to [0, P], read from LDS inside the loop: a global load
  // there would make the compiler wait for every ring copy in flight.
  __shared__ int lens[kMaxBatch];

  const int wv = uniform(threadIdx.x >> 6);
  const int lane = opaque_lane();
  const int h = blockIdx.x % p.H;
  const int split = blockIdx.x / p.H;
  const int kind = wv >> 2, w = wv & 3;  // keys or values; this wave's 32 of the 128 rows
  const int T = (p.P + kTile - 1) / kTile;

  // This wave's rows of W^T: dim 32 w + lane % 32, k = 16 ks + 8 (lane / 32).
  bf16x8 wf[KS];
  {
    const uint16_t* wsrc =
        (kind ? p.wvt : p.wuk) + ((int64_t)h * 128 + 32 * w + (lane & 31)) * DC + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wf[ks] = *(const bf16x8*)(wsrc + 16 * ks);
  }

  for (int b = threadIdx.x; b < p.B; b += kXWaves * 64) lens[b] = min(max(p.seq_lens[b], 0), p.P);
  __syncthreads();

  // The tiles to compute, over all sequences: tile j of sequence b while
  // 32 j < L_b.  This work-group takes a contiguous share of them.
  int ntot = 0;
  for (int b = 0; b < p.B; ++b) ntot += (lens[b] + kTile - 1) / kTile;
  const int ns = gridDim.x / p.H;
  const int f0 = (int)((int64_t)ntot * split / ns), f1 = (int)((int64_t)ntot * (split + 1) / ns);
  if (f0 >= f1) return;

  // Cursor over (b, j) for the DMA (runs NBUF - 1 tiles ahead) and for the compute.
  struct Cursor {
    int b, j, L;
  };
  auto seek = [&](int f) {
    Cursor c{0, 0, 0};
    for (;;) {
      const int L = lens[c.b];
      const int n = (L + kTile - 1) / kTile;
      if (f < n) {
        c.j = f;
        c.L = L;
        return c;
      }
      f -= n;
      ++c.b;
    }
  };
  auto advance = [&](Cursor& c) {
    if (++c.j * kTile >= c.L) {
      c.j = 0;
      do {
        ++c.b;
      } while (c.b < p.B && lens[c.b] == 0);
      if (c.b < p.B) c.L = lens[c.b];
    }
  };

  const uint32_t rec = (uint32_t)(DC + 64) * 2;
  const uint32_t ring_lds = lds_offset(ring);
  // Tile (b, j) into ring slot s: instruction q of wave wv fills granule rows
  // 2 (8 q + wv) and +1; lane l brings position 32 j + (l % 32 ^ 4 (l / 32)).
  const int slot_tok = (lane & 31) ^ (4 * (lane >> 5));
  auto issue = [&](const Cursor& c, int s) {
    const char* base = (const char*)(p.ckr + (int64_t)c.b * p.P * (DC + 64));
    const uint32_t voff = (uint32_t)min(c.j * kTile + slot_tok, c.L - 1) * rec + 16u * (lane >> 5);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int g0 = 2 * (kXWaves * q + wv);
      lds_dma16(base + 16 * g0, voff, ring_lds + s * TBX + g0 * kRow);
    }
  };

  // The W^T rows must have arrived before the ring copies start: the
  // compiler counts only its own loads, and would otherwise wait for every
  // copy in flight at the first use of wf.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(wf[ks]));

  Cursor cd = seek(f0);
  for (int i = 0; i < kXBuf - 1 && f0 + i < f1; ++i) {
    issue(cd, i);
    advance(cd);
  }

  uint16_t* const out = kind ? p.v : p.k_nope;
  Cursor cc = seek(f0);
  // B-operand read of this lane: row 2 ks + lane / 32, its position's slot.
  const int rd = (lane >> 5) * kRow + (((lane & 31) ^ (4 * (lane >> 5))) << 4);
  for (int f = f0; f < f1; ++f) {
    const int i = f - f0;
    if (f + kXBuf - 2 < f1) vm_wait<(kXBuf - 2) * NI>(); else vm_wait<0>();
    block_sync();
    if (f + kXBuf - 1 < f1) {
      issue(cd, (i + kXBuf - 1) % kXBuf);
      advance(cd);
    }
    const char* tb = ring + (i % kXBuf) * TBX + rd;
    f32x16 acc{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bv = *(const bf16x8*)(tb + 2 * ks * kRow);
      acc = mfma32(wf[ks], bv, acc);
    }
    // acc[4 i + r] = D[dim 8 i + 4 (lane / 32) + r][position lane % 32]:
    // granule 4 w + i of the position, its half lane / 32.
    const int t = lane & 31;
    const bool valid = cc.j * kTile + t < cc.L;
    uint16_t* dst = out + (((int64_t)cc.b * p.H + h) * T + cc.j) * (kTile * 128) + 4 * (lane >> 5);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * w + gi;
      const int slot = t ^ (4 * (g & 1));
      const bf16x2 a = {(__bf16)acc[4 * gi], (__bf16)acc[4 * gi + 1]};
      const bf16x2 c = {(__bf16)acc[4 * gi + 2], (__bf16)acc[4 * gi + 3]};
      const uint2 v = valid ? uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)} : uint2{0, 0};
      *(uint2*)(dst + (g * kTile + slot) * 8) = v;
    }
    advance(cc);
  }
}

template <int DC>
hipError_t launch_dc(const ExpandParams& p, hipStream_t stream) {
  // Enough (head, share) work-groups to give every CU one.
  const int ns = (256 + p.H - 1) / p.H;
  hipLaunchKernelGGL(expand_kernel<DC>, dim3(p.H * ns), dim3(kXWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expand(const ExpandParams& p, int d_latent, hipStream_t stream) {
  if (d_latent == 512) return launch_dc<512>(p, stream);
  if (d_latent == 256) return launch_dc<256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
