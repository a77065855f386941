// The batch's split plan of the decode and merge kernels (gfx950).
//
// Every work-group of the decode and of the merge computes the same plan from
// seq_lens, so the host needs no lengths.  With n_b = ceil(L_b / 32) tiles in
// sequence b and P partial slots:
//   W   = min { W >= 1 : sum_b ceil(n_b / W) <= P }   (tiles per part)
//   p_b = ceil(n_b / W)                                (parts of sequence b)
//   sequence b owns slots s_b .. s_b + p_b - 1, s_b = sum_{b' < b} p_{b'};
//   its part j covers tiles [j W, min((j + 1) W, n_b)).
// A part never crosses a sequence, so each part is one (sequence, token
// range) and writes one partial.  W exists whenever P >= B (W = max n_b
// gives one part per sequence).
#pragma once
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

// The plan as one wave sees it: lane l holds the tile counts of sequences
// l, l + 64, ... (at most CH * 64 of them; WavePlanFor picks CH = 1 when
// the batch fits one wave, which keeps the search short).
template <int CH>
struct WavePlanN {
  int n[CH], len[CH];
  int B, nch, W, total;

  // Loads the lengths and finds W for P slots (P >= B).  All lanes of one wave.
  __device__ void build(const int32_t* __restrict__ seq_lens, int B_, int P, int lane) {
    B = B_;
    nch = (B + kWave - 1) / kWave;
    int N = 0, nmax = 0, nz = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      n[c] = 0;
      len[c] = 0;
      if (c < nch) {
        const int b = c * kWave + lane;
        const int L = b < B ? seq_lens[b] : 0;
        len[c] = L;
        n[c] = L > 0 ? (L + kTile - 1) / kTile : 0;
        N += n[c];
        nmax = max(nmax, n[c]);
        nz += n[c] > 0;
      }
    }
    N = wave_sum(N);
    nmax = wave_max(nmax);
    nz = wave_sum(nz);
    if (N == 0) {
      W = 1;
      total = 0;
      return;
    }
    // f(W) = sum_b ceil(n_b / W) is non-increasing, f(W) >= N / W and
    // f(W) <= N / W + nz, so W lies in [ceil(N / P), ceil(N / (P - nz))]
    // (or max n_b when P == nz).
    int lo = max(1, (N + P - 1) / P);
    int hi = P > nz ? min(nmax, (N + (P - nz) - 1) / (P - nz)) : nmax;
    hi = max(hi, lo);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (count(mid) <= P) hi = mid;
      else lo = mid + 1;
    }
    W = lo;
    total = count(W);
  }

  __device__ int count(int w) const {
    int s = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nch) s += (n[c] + w - 1) / w;
    return wave_sum(s);
  }

  // The sequence owning slot g (< total) and its first slot; all lanes.
  __device__ void locate_slot(int g, int lane, int& b, int& s_b) const {
    int run = 0;
    b = -1;
    s_b = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < nch && b < 0) {
        const int pc = (n[c] + W - 1) / W;
        const int x = wave_incl_sum(pc);
        const int start = run + x - pc;
        const unsigned long long hit = __ballot(pc > 0 && g >= start && g < start + pc);
        if (hit) {
          const int l = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
          b = c * kWave + l;
          s_b = lane_value(start, l);
        }
        run += lane_value(x, kWave - 1);
      }
    }
  }

  // First slot and part count of sequence b; all lanes.
  __device__ void slots_of(int b, int lane, int& s_b, int& p_b) const {
    int run = 0;
    s_b = 0;
    p_b = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < nch) {
        const int pc = (n[c] + W - 1) / W;
        const int x = wave_incl_sum(pc);
        if (b >= c * kWave && b < (c + 1) * kWave) {
          const int l = b - c * kWave;
          s_b = run + lane_value(x, l) - lane_value(pc, l);
          p_b = lane_value(pc, l);
        }
        run += lane_value(x, kWave - 1);
      }
    }
  }

  // sb[b] = s_b for b = 0 .. B (sb[B] = total) into LDS; all lanes.
  __device__ void write_slot_prefix(int* sb, int lane) const {
    int run = 0;
    if (lane == 0) sb[0] = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < nch) {
        const int x = wave_incl_sum((n[c] + W - 1) / W);
        const int b = c * kWave + lane;
        if (b < B) sb[b + 1] = run + x;
        run += lane_value(x, kWave - 1);
      }
    }
  }

  // Length of sequence b (wave-uniform b).
  __device__ int length(int b) const {
    int v = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nch && b >= c * kWave && b < (c + 1) * kWave) v = lane_value(len[c], b - c * kWave);
    return v;
  }

  // Tiles of sequence b (wave-uniform b).
  __device__ int tiles(int b, int lane) const {
    int v = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nch && b >= c * kWave && b < (c + 1) * kWave) v = lane_value(n[c], b - c * kWave);
    (void)lane;
    return v;
  }
};

using WavePlan = WavePlanN<kMaxBatch / kWave>;

// Runs f(plan) with the plan of the batch built by the calling wave.
template <class F>
__device__ __forceinline__ void with_plan(const int32_t* __restrict__ seq_lens, int B, int P, int lane, F&& f) {
  if (B <= kWave) {
    WavePlanN<1> pl;
    pl.build(seq_lens, B, P, lane);
    f(pl);
  } else {
    WavePlan pl;
    pl.build(seq_lens, B, P, lane);
    f(pl);
  }
}

}  // namespace mla
