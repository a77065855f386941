// Device-side helpers shared by the gfx950 kernels of the absorbed-MLA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

constexpr int kWave = 64;

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
constexpr int kTile = 32;  // tokens per decode tile (the M extent of one 32x32 MFMA)
constexpr int kRow = kTile * 16;  // bytes of one granule row of a tile

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A[l%32][8*(l/32) .. +8], B[8*(l/32) .. +8][l%32] and
// D[8*(i/4) + 4*(l/32) + i%4][l%32] in accumulator register i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16] and
// D[4*(l/16) + i][l%16] in accumulator register i.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read of 4 bf16: within each 16-lane group, lane i receives
// element (i % 4) of the 8-byte words addressed by lanes 4*j + i/4, j = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(lds_void_ptr)(p));
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

// 16-byte global -> LDS copy without passing through VGPRs: lane i reads
// base + voff_i (base wave-uniform, voff_i a 32-bit byte offset) and the 64
// lanes write consecutive 16-byte slots starting at LDS offset `lds`
// (wave-uniform).  Issued from inline asm so that the compiler does not put a
// full vmcnt(0) wait in front of every LDS read; completion is tracked by
// hand with vm_wait<N>().  M0 (the LDS destination) is declared clobbered.
__device__ __forceinline__ void lds_dma16(const void* base_any, uint32_t voff, uint32_t lds) {
  // Make the base provably wave-uniform.  readfirstlane returns int: widen
  // each half through uint32_t so the low half is zero-, not sign-, extended.
  const uint64_t b = reinterpret_cast<uint64_t>(base_any);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(dst)
      : "memory", "m0");
}

// One 32-bit value at a wave-uniform address, read through the scalar path
// and waited for in the same statement.  Its counter is the one the LDS
// instructions use, not the vector-memory one, so this read can complete
// while LDS copies issued before it are still in flight (a vector load
// could only be waited for together with them).
__device__ __forceinline__ int scalar_read_now(const int32_t* addr) {
  const uint64_t a = reinterpret_cast<uint64_t>(addr);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint64_t sa = ((uint64_t)hi << 32) | (uint64_t)lo;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sa) : "memory");
  return v;
}

// A lane id the compiler cannot see through, so that lane-derived constants
// are recomputed where they are used instead of being kept live (and spilled)
// across the whole kernel.
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Work-group barrier for LDS hand-offs: waits for this wave's LDS traffic,
// leaves its global loads in flight.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}



__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[i];
  return r;
}

// Reductions over the lane pair (l, l ^ 32) without going through LDS:
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, so with x in both, the two results hold x[l % 32]
// and x[l % 32 + 32] in every lane (in some order).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// XOR swizzle of the 16-byte granules of one cache record in LDS: token t's
// granule g is stored at position g ^ swz(t).  Eight consecutive tokens map a
// granule to eight distinct bank groups (the K-operand reads), and four
// consecutive aligned tokens map an even/odd granule pair to eight distinct
// bank groups (the transposing V-operand reads).
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// Wave-wide scans through DPP row shifts and row broadcasts (a few VALU
// cycles each, where a shuffle through ds_bpermute waits on LDS): lane l gets
// the inclusive scan of x over lanes 0..l.  Disabled lanes and sources past a
// row's start keep the 0 passed as `old`, the identity of both operations
// (the values scanned here are non-negative).
template <class Op>
__device__ __forceinline__ int wave_scan(int x, Op op) {
  int v = x;
  v = op(v, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(0, x, 0x113, 0xf, 0xf, false));  // row_shr:3
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, false));  // row_shr:4, banks 1-3
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, false));  // row_shr:8, banks 2-3
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15, rows 1, 3
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31, rows 2, 3
  return v;
}
struct AddOp {
  __device__ __forceinline__ int operator()(int a, int b) const { return a + b; }
};
struct MaxOp {
  __device__ __forceinline__ int operator()(int a, int b) const { return max(a, b); }
};
__device__ __forceinline__ int wave_incl_sum(int x) { return wave_scan(x, AddOp{}); }
// Lane l's value of x, l wave-uniform (a scalar read, no LDS).
__device__ __forceinline__ int lane_value(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ int wave_sum(int x) { return lane_value(wave_scan(x, AddOp{}), kWave - 1); }
__device__ __forceinline__ int wave_max(int x) { return lane_value(wave_scan(x, MaxOp{}), kWave - 1); }

// Sequence tile bookkeeping shared by the decode and combine kernels: the
// prefix sum cu[0..B] of ceil(seq_len / kTile) over the batch, built in LDS by
// one wave.  Returns cu[B].
__device__ inline int build_tile_prefix(const int32_t* __restrict__ seq_lens, int B, int* cu, int lane) {
  int run = 0;
  if (lane == 0) cu[0] = 0;
  for (int base = 0; base < B; base += kWave) {
    int i = base + lane;
    int n = 0;
    if (i < B) {
      int L = seq_lens[i];
      n = L > 0 ? (L + kTile - 1) / kTile : 0;
    }
    const int x = wave_incl_sum(n);
    if (i < B) cu[i + 1] = run + x;
    run += lane_value(x, kWave - 1);
  }
  return run;
}

}  // namespace mla
