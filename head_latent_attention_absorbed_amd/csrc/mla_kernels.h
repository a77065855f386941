// Host-visible parameter blocks and launchers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Largest batch the decode/combine kernels accept (their tile prefix sums live in LDS).
constexpr int kMaxBatch = 1024;

struct DecodeParams {
  const uint16_t* q_lat;     // bf16 [B, S, H, DC]
  const uint16_t* q_rope;    // bf16 [B, S, H, 64]
  const char* c_kv;          // page 0 slot 0 of the latent part
  int64_t rope_off;          // bytes from a token's latent to its RoPE key
  int64_t token_stride;      // bytes between consecutive slots of a page
  int64_t block_stride;      // bytes between consecutive pages
  const float* kv_scale;     // fp8 only: [pages][block_size]
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t bt_stride;         // entries per block_table row
  int32_t B, H, S, R;        // batch, heads, query tokens, rows = S * H
  int32_t RG;                // row groups (work-groups sharing one token range)
  int32_t P;                 // partial slots (the split plan's budget of parts)
  int32_t block_size;        // tokens per page: 32 * 2^k
  int32_t block_shift;       // log2(block_size)
  float scale_log2;          // softmax_scale * log2(e)
  void* o_part;              // fp32 or fp16 [parts, R, DC]
  int32_t o_half;            // o_part holds fp16
  float* lse_part;           // fp32 [parts, R]
};

// Waves per work-group and row groups the decode uses for R rows.
int decode_waves(int R);
int decode_row_groups(int R);
// Work-groups of one row group the device runs at once (token parts).
int decode_wgs_per_cu(int R, int d_latent);

hipError_t launch_decode(const DecodeParams& p, int d_latent, bool fp8, hipStream_t stream);
// The 128-row work-group form (decode_wide.hip), used when R > 64.
hipError_t launch_decode_wide(const DecodeParams& p, int d_latent, bool fp8, hipStream_t stream);
// Its e4m3 form (decode_wide_fp8.hip).
hipError_t launch_decode_wide_fp8(const DecodeParams& p, int d_latent, hipStream_t stream);
// Its bf16 form at d_c = 256 with two tiles per step (decode_wide_pair.hip).
hipError_t launch_decode_wide_pair(const DecodeParams& p, int d_latent, hipStream_t stream);
// The bf16 128-row decode's tile copies alone (same plan, grid and copy
// instructions, one tile in flight, no products): a calibration probe.
hipError_t launch_probe_tile_copy(const DecodeParams& p, int d_latent, uint32_t* sink, hipStream_t stream);

// Calibration probes (probes.hip).
hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t stream);
int64_t probe_mfma_flops(int iters, int cus);
hipError_t launch_probe_mfma(int iters, float* sink, int cus, hipStream_t stream);

// Input validation (validate.hip).
struct ValidateParams {
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t num_pages;
  int B, S, MB, block_size;
  int32_t* out;
};
hipError_t launch_validate(const ValidateParams& p, hipStream_t stream);

// Tile-native layout of the prefill's per-head keys and values: for
// sequence b, head h and 32-position tile j, 16 granule rows g (elements
// 8g..8g+7) of 32 slots; position 32 j + t sits in slot t ^ (4 (g & 1)).
// One tile is 4096 bf16 (8 KiB) at element ((b H + h) T + j) 4096,
// T = ceil(P / 32): the LDS image of the attention's key/value tiles.
struct ExpandParams {
  const uint16_t* ckr;       // bf16 [B, P, DC + 64] records
  const uint16_t* wuk;       // bf16 [H, 128, DC] (W_UK)
  const uint16_t* wvt;       // bf16 [H, 128, DC] (W_UV transposed)
  const int32_t* seq_lens;
  int32_t B, P, H;
  uint16_t* k_nope;          // tile-native, bf16
  uint16_t* v;               // tile-native, bf16
};
hipError_t launch_expand(const ExpandParams& p, int d_latent, hipStream_t stream);

// MLA-form prefill attention (d_nope 128, d_rope 64, d_v 128).
struct PrefillParams {
  const uint16_t* q_nope;    // bf16 [B, P, H, 128]
  const uint16_t* q_rope;    // bf16 [B, P, H, 64]
  const uint16_t* k_nope;    // tile-native (ExpandParams)
  const uint16_t* ckr;       // bf16 [B, P, DCK + 64]: k_rope at element DCK of each record
  const uint16_t* v;         // tile-native (ExpandParams)
  const int32_t* seq_lens;
  int32_t B, P, H, DCK;
  float scale_log2;          // softmax_scale * log2(e)
  uint16_t* out;             // bf16 [B, P, H, 128]
  float* lse;                // fp32 [B, P, H]
};
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
// Hadamard change of basis (x H / sqrt(d), Sylvester order) of bf16 vectors
// of length d (256 or 512), or a plain copy when !rotate, with the result's
// elements split over n_shards outputs.  Vector v starts at element
// (v / inner) in_outer + (v % inner) in_inner of `in`, element k at + k in_elem;
// its element k goes to (v / inner) out_outer + (v % inner) out_inner
// + (k / (d / n_shards)) out_shard + (k % (d / n_shards)) out_elem of `out`.
// in == out is allowed when both layouts are the same.
struct HadamardParams {
  const uint16_t* in;
  uint16_t* out;
  int64_t n_vec;
  int64_t inner;
  int64_t in_outer, in_inner, in_elem;
  int64_t out_outer, out_inner, out_elem, out_shard;
  int32_t d, n_shards;
  bool rotate;
};
hipError_t launch_hadamard(const HadamardParams& p, hipStream_t stream);
// out[m] = sum over i < n of parts[i * count + m] (fp32 in; bf16 RNE or fp32 out).
hipError_t launch_shard_sum(const float* parts, int n, int64_t count, void* out, bool out_f32, hipStream_t stream);

// Regrouping around the GQA decoding path (GQLA), run as the latent decode
// over per-group records [K_nope (dn) | V (dv) | k_rope (dr)] with streams
// (b, g) as sequences and the group's H / G heads as rows.
struct GqaParams {
  int32_t B, S, H, G, dn, dv, dr;
  const uint16_t* q_nope;    // bf16 [B, S, H, dn]
  const uint16_t* q_rope;    // bf16 [B, S, H, dr]
  uint16_t* q_cat;           // bf16 [B G, S, H / G, dn + dv]: [q_nope | 0]
  uint16_t* q_rope_g;        // bf16 [B G, S, H / G, dr]
  const float* o_lat;        // fp32 [B G, S, H / G, dn + dv]: merged rows
  const float* lse_g;        // fp32 [B G, S, H / G]
  void* out;                 // [B, S, H, dv], bf16 or fp32
  float* lse;                // fp32 [B, S, H]
};
hipError_t launch_gqa_queries(const GqaParams& p, hipStream_t stream);
hipError_t launch_gqa_output(const GqaParams& p, bool out_f32, hipStream_t stream);

// W [H, R, C] bf16 -> its transpose [H, C, R] (R, C multiples of 64).
hipError_t launch_transpose_heads(const uint16_t* w, uint16_t* wt, int H, int R, int C, hipStream_t stream);

struct CombineParams {
  const void* o_part;        // fp32 or fp16 [parts, R, DC]
  int32_t o_half;
  const float* lse_part;
  const int32_t* seq_lens;
  int32_t B, R, P, DC;       // P: partial slots, as given to the decode
  float* o_lat;              // fp32 [B, R, DC]
  float* lse;                // fp32 [B, R]
};

hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

// The merge fused with the value up-projection: out[m, h, :] = o[m, h, :] . W[h]
// for the merged row o of query row m = b*S + s, head h.
struct CombineUpParams {
  const void* o_part;        // fp32 or fp16 [parts, R, DC]
  int32_t o_half;
  const float* lse_part;
  const int32_t* seq_lens;
  const uint16_t* w;         // bf16 W_UV [H, DC, NV]
  void* out;                 // bf16 or fp32 [B*S, H, NV]
  int32_t out_f32;
  float* lse;                // fp32 [B*S, H]
  int32_t B, S, H, P, DC, NV;  // P: partial slots, as given to the decode
};

// Whether the fused kernel exists for this latent rank and value width.
bool combine_up_supported(int d_latent, int d_v);
hipError_t launch_combine_up(const CombineUpParams& p, hipStream_t stream);

// Per-head product C[m, h, :] = A[m, h, :] . W[h]  (A: [M, H, K], W: [H, K, N], C: [M, H, N]).
struct HeadGemmParams {
  const void* a;             // bf16 or fp32
  const uint16_t* w;         // bf16
  void* c;                   // bf16 or fp32
  int32_t M, H, K, N;
  // Element strides of A between rows and between heads; both 0 = dense
  // [M, H, K].  a_head = 0 multiplies one row by every head's matrix.
  int64_t a_row, a_head;
};

// Whether a kernel exists for reduction depth K and N output columns per head.
bool head_gemm_supported(int K, int N);
hipError_t launch_head_gemm(const HeadGemmParams& p, bool a_fp32, bool c_fp32, hipStream_t stream);
// bf16 A, fp32 C, K = 128 or 256 per head, N a multiple of 64.
hipError_t launch_head_gemm_partials(const HeadGemmParams& p, hipStream_t stream);

// Cache append: the records of the S_q new tokens of every sequence from the
// split-K partial products of x . [W_DKV | W_KR].
constexpr int kAppendSlice = 256;  // d_model columns per partial product
struct AppendParams {
  const float* part;         // fp32 [M, KS, DC + 64]: row m's partial products
  int32_t KS, M, S;          // K slices, rows (B * S_q), S_q
  int32_t DC;                // latent width; the record is DC + 64 values
  char* c_kv;                // latent of page 0, slot 0
  int64_t rope_off;          // bytes from a record's latent to its RoPE key
  int64_t token_stride, block_stride;
  float* kv_scale;           // e4m3 only: [pages][block_size]
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t bt_stride, block_size;
  double log2_base;          // log2 of the RoPE base
  int32_t fp8;
};
hipError_t launch_append_finish(const AppendParams& p, hipStream_t stream);
// Device address, on the current device, of the fixed scratch array of
// mla_append_kv_noalloc (MLA_APPEND_NOALLOC_MAX_BYTES bytes, 256-byte aligned).
hipError_t append_scratch(void** ptr);

}  // namespace mla
