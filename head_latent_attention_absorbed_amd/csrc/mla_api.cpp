// C ABI of libmla_absorbed.so: argument checks, plan sizing and launches.
// Declarations and the meaning of every argument are in include/mla_absorbed.h.
#include "mla_absorbed.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "mla_kernels.h"

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mla_status_t ok() {
  g_last_error.clear();
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

mla_status_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return MLA_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n <= 0) return fail(MLA_ERR_HIP, "CU count query failed: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return MLA_OK;
}

mla_status_t check_shape(const mla_shape_t* s) {
  if (!s) return fail(MLA_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->num_heads < 1 || s->q_len < 1 || s->d_nope < 1 || s->d_rope < 1 || s->d_latent < 1 ||
      s->d_v < 1 || s->block_size < 1 || s->max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARG, "shape has a non-positive size");
  if (!std::isfinite(s->softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale is not finite");
  // The kernels take a tile's maximum over the raw scores and scale it
  // afterwards, which is the maximum of the scaled scores only for a
  // positive scale.
  if (!(s->softmax_scale > 0.0f)) return fail(MLA_ERR_UNSUPPORTED, "softmax_scale %g (must be > 0)", s->softmax_scale);
  if (s->cache_dtype != MLA_BF16 && s->cache_dtype != MLA_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARG, "cache_dtype must be MLA_BF16 or MLA_FP8_E4M3");
  if (s->out_dtype != MLA_BF16 && s->out_dtype != MLA_FP32)
    return fail(MLA_ERR_INVALID_ARG, "out_dtype must be MLA_BF16 or MLA_FP32");
  if (s->partial_dtype != MLA_FP32 && s->partial_dtype != MLA_FP16)
    return fail(MLA_ERR_INVALID_ARG, "partial_dtype must be MLA_FP32 or MLA_FP16");
  if (s->batch > mla::kMaxBatch) return fail(MLA_ERR_UNSUPPORTED, "batch %d > %d", s->batch, mla::kMaxBatch);
  if (s->q_len > 8) return fail(MLA_ERR_UNSUPPORTED, "q_len %d > 8", s->q_len);
  if (s->d_latent != 512 && s->d_latent != 256)
    return fail(MLA_ERR_UNSUPPORTED, "d_latent %d (kernels exist for 512 and 256)", s->d_latent);
  if (s->d_rope != 64) return fail(MLA_ERR_UNSUPPORTED, "d_rope %d (kernels exist for 64)", s->d_rope);
  if (s->d_nope % 64 != 0 || s->d_nope > 512)
    return fail(MLA_ERR_UNSUPPORTED, "d_nope %d (multiple of 64 up to 512)", s->d_nope);
  if (s->d_v % 64 != 0) return fail(MLA_ERR_UNSUPPORTED, "d_v %d (multiple of 64)", s->d_v);
  if (s->block_size < MLA_TILE_TOKENS || (s->block_size & (s->block_size - 1)) != 0)
    return fail(MLA_ERR_UNSUPPORTED, "block_size %d (a power of two >= %d)", s->block_size, MLA_TILE_TOKENS);
  if ((int64_t)s->batch * s->q_len > (1 << 20)) return fail(MLA_ERR_UNSUPPORTED, "batch * q_len too large");
  return MLA_OK;
}

mla_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// The record layout checks shared by the decode and its copy probe: strides,
// and the RoPE key inside the record after the latent (rope_off = its offset).
mla_status_t check_cache_layout(const char* who, const mla_shape_t* shape, const void* c_kv, const void* k_rope,
                                int64_t token_stride, int64_t block_stride, int64_t* rope_off) {
  const int elem = shape->cache_dtype == MLA_FP8_E4M3 ? 1 : 2;
  const int64_t off = static_cast<const char*>(k_rope) - static_cast<const char*>(c_kv);
  if (token_stride <= 0 || token_stride % 16 || block_stride % 16 ||
      block_stride < (int64_t)shape->block_size * token_stride || (int64_t)shape->block_size * token_stride > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG,
                "%s: token_stride/block_stride must be positive multiples of 16 with "
                "block_stride >= block_size * token_stride",
                who);
  if (off < (int64_t)shape->d_latent * elem || off + (int64_t)shape->d_rope * elem > token_stride)
    return fail(MLA_ERR_INVALID_ARG, "%s: k_rope must follow the latent inside the record (k_rope - c_kv = %lld bytes)",
                who, (long long)off);
  *rope_off = off;
  return MLA_OK;
}


}  // namespace

extern "C" {

mla_status_t mla_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return fail(MLA_ERR_INVALID_ARG, "mla_probe_hbm_read: NULL pointer");
  if (!aligned16(buf) || bytes <= 0 || bytes % 16)
    return fail(MLA_ERR_INVALID_ARG, "mla_probe_hbm_read: buf must be 16-byte aligned and bytes a positive multiple of 16");
  int cus = 0;
  mla_status_t st = device_cus(&cus);
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_probe_hbm_read(buf, bytes, sink, cus, stream), "mla_probe_hbm_read launch");
}

mla_status_t mla_probe_mfma(int32_t iters, float* sink, int64_t* flops, hipStream_t stream) {
  if (!sink || !flops) return fail(MLA_ERR_INVALID_ARG, "mla_probe_mfma: NULL pointer");
  if (iters <= 0) return fail(MLA_ERR_INVALID_ARG, "mla_probe_mfma: iters %d must be positive", iters);
  int cus = 0;
  mla_status_t st = device_cus(&cus);
  if (st != MLA_OK) return st;
  *flops = mla::probe_mfma_flops(iters, cus);
  return hip_status(mla::launch_probe_mfma(iters, sink, cus, stream), "mla_probe_mfma launch");
}

mla_status_t mla_probe_tile_copy(const mla_shape_t* shape, const void* c_kv, const void* k_rope, int64_t token_stride,
                                 int64_t block_stride, const int32_t* block_table, const int32_t* seq_lens,
                                 int32_t num_parts, uint32_t* sink, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_rope || !block_table || !seq_lens || !sink)
    return fail(MLA_ERR_INVALID_ARG, "mla_probe_tile_copy: NULL pointer");
  if (shape->cache_dtype != MLA_BF16 || shape->q_len * shape->num_heads <= 64)
    return fail(MLA_ERR_UNSUPPORTED, "mla_probe_tile_copy: only the bf16 cache with more than 64 query rows");
  if (!aligned16(c_kv) || !aligned16(k_rope))
    return fail(MLA_ERR_INVALID_ARG, "mla_probe_tile_copy: c_kv and k_rope must be 16-byte aligned");
  int64_t rope_off = 0;
  st = check_cache_layout("mla_probe_tile_copy", shape, c_kv, k_rope, token_stride, block_stride, &rope_off);
  if (st != MLA_OK) return st;
  if (num_parts < shape->batch)
    return fail(MLA_ERR_INVALID_ARG, "mla_probe_tile_copy: num_parts %d < batch %d", num_parts, shape->batch);
  mla::DecodeParams p{};
  p.c_kv = static_cast<const char*>(c_kv);
  p.rope_off = rope_off;
  p.token_stride = token_stride;
  p.block_stride = block_stride;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.bt_stride = shape->max_blocks_per_seq;
  p.B = shape->batch;
  p.H = shape->num_heads;
  p.S = shape->q_len;
  p.R = shape->q_len * shape->num_heads;
  p.RG = mla::decode_row_groups(p.R);
  p.P = num_parts;
  p.block_size = shape->block_size;
  p.block_shift = __builtin_ctz((unsigned)shape->block_size);
  if ((int64_t)p.P * p.RG > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "too many work-groups");
  return hip_status(mla::launch_probe_tile_copy(p, shape->d_latent, sink, stream), "mla_probe_tile_copy launch");
}

mla_status_t mla_validate_decode_inputs(const mla_shape_t* shape, const int32_t* block_table, const int32_t* seq_lens,
                                        int64_t num_pages, int32_t* violations, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!block_table || !seq_lens || !violations)
    return fail(MLA_ERR_INVALID_ARG, "mla_validate_decode_inputs: NULL pointer");
  if (num_pages <= 0)
    return fail(MLA_ERR_INVALID_ARG, "mla_validate_decode_inputs: num_pages %lld must be positive",
                (long long)num_pages);
  if (reinterpret_cast<uintptr_t>(violations) % 4)
    return fail(MLA_ERR_INVALID_ARG, "mla_validate_decode_inputs: violations must be 4-byte aligned");
  mla::ValidateParams p{};
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.num_pages = num_pages;
  p.B = shape->batch;
  p.S = shape->q_len;
  p.MB = shape->max_blocks_per_seq;
  p.block_size = shape->block_size;
  p.out = violations;
  return hip_status(mla::launch_validate(p, stream), "mla_validate_decode_inputs launch");
}

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this request";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "unknown mla_status_t";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status_t mla_absorb_q(const mla_shape_t* shape, const void* q_nope, const void* w_uk, void* q_lat,
                          hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_nope || !w_uk || !q_lat) return fail(MLA_ERR_INVALID_ARG, "mla_absorb_q: NULL tensor");
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat))
    return fail(MLA_ERR_INVALID_ARG, "mla_absorb_q: tensors must be 16-byte aligned");
  if (!mla::head_gemm_supported(shape->d_nope, shape->d_latent))
    return fail(MLA_ERR_UNSUPPORTED, "mla_absorb_q: no kernel for d_nope %d, d_latent %d", shape->d_nope,
                shape->d_latent);
  mla::HeadGemmParams p{};
  p.a = q_nope;
  p.w = static_cast<const uint16_t*>(w_uk);
  p.c = q_lat;
  p.M = shape->batch * shape->q_len;
  p.H = shape->num_heads;
  p.K = shape->d_nope;
  p.N = shape->d_latent;
  return hip_status(mla::launch_head_gemm(p, false, false, stream), "mla_absorb_q launch");
}

mla_status_t mla_decode_num_parts(const mla_shape_t* shape, int32_t* num_parts) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!num_parts) return fail(MLA_ERR_INVALID_ARG, "num_parts is NULL");
  int cus = 0;
  st = device_cus(&cus);
  if (st != MLA_OK) return st;
  const int R = shape->q_len * shape->num_heads;
  const int wgs = cus * mla::decode_wgs_per_cu(R, shape->d_latent);
  const int G = std::max(1, wgs / mla::decode_row_groups(R));
  *num_parts = std::max(G, shape->batch);
  return ok();
}

mla_status_t mla_decode_paged(const mla_shape_t* shape, const void* q_lat, const void* q_rope, const void* c_kv,
                              const void* k_rope, int64_t token_stride, int64_t block_stride, const float* kv_scale,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t num_parts, void* o_part,
                              float* lse_part, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_lat || !q_rope || !c_kv || !k_rope || !block_table || !seq_lens || !o_part || !lse_part)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_paged: NULL tensor");
  const bool fp8 = shape->cache_dtype == MLA_FP8_E4M3;
  if (fp8 && !kv_scale) return fail(MLA_ERR_INVALID_ARG, "mla_decode_paged: fp8 cache needs kv_scale");
  if (!fp8 && kv_scale) return fail(MLA_ERR_INVALID_ARG, "mla_decode_paged: kv_scale given for a bf16 cache");
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(o_part))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_paged: tensors must be 16-byte aligned");
  int64_t rope_off = 0;
  st = check_cache_layout("mla_decode_paged", shape, c_kv, k_rope, token_stride, block_stride, &rope_off);
  if (st != MLA_OK) return st;
  if (num_parts < shape->batch)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_paged: num_parts %d < batch %d", num_parts, shape->batch);
  mla::DecodeParams p{};
  p.q_lat = static_cast<const uint16_t*>(q_lat);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.c_kv = static_cast<const char*>(c_kv);
  p.rope_off = rope_off;
  p.token_stride = token_stride;
  p.block_stride = block_stride;
  p.kv_scale = kv_scale;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.bt_stride = shape->max_blocks_per_seq;
  p.B = shape->batch;
  p.H = shape->num_heads;
  p.S = shape->q_len;
  p.R = shape->q_len * shape->num_heads;
  p.RG = mla::decode_row_groups(p.R);
  p.P = num_parts;
  p.block_size = shape->block_size;
  p.block_shift = __builtin_ctz((unsigned)shape->block_size);
  p.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
  p.o_part = o_part;
  p.o_half = shape->partial_dtype == MLA_FP16;
  p.lse_part = lse_part;
  if ((int64_t)p.P * p.RG > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "too many decode work-groups");
  return hip_status(mla::launch_decode(p, shape->d_latent, fp8, stream), "mla_decode_paged launch");
}

mla_status_t mla_combine_lse(const mla_shape_t* shape, int32_t num_parts, const void* o_part, const float* lse_part,
                             const int32_t* seq_lens, float* o_lat, float* lse, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!o_part || !lse_part || !seq_lens || !o_lat || !lse)
    return fail(MLA_ERR_INVALID_ARG, "mla_combine_lse: NULL tensor");
  if (!aligned16(o_part) || !aligned16(o_lat))
    return fail(MLA_ERR_INVALID_ARG, "mla_combine_lse: o_part and o_lat must be 16-byte aligned");
  if (num_parts < shape->batch)
    return fail(MLA_ERR_INVALID_ARG, "mla_combine_lse: num_parts %d < batch %d", num_parts, shape->batch);
  mla::CombineParams p{};
  p.o_part = o_part;
  p.o_half = shape->partial_dtype == MLA_FP16;
  p.lse_part = lse_part;
  p.seq_lens = seq_lens;
  p.B = shape->batch;
  p.R = shape->q_len * shape->num_heads;
  p.P = num_parts;
  p.DC = shape->d_latent;
  p.o_lat = o_lat;
  p.lse = lse;
  return hip_status(mla::launch_combine(p, stream), "mla_combine_lse launch");
}

mla_status_t mla_up_v(const mla_shape_t* shape, const float* o_lat, const void* w_uv, void* out,
                      hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!o_lat || !w_uv || !out) return fail(MLA_ERR_INVALID_ARG, "mla_up_v: NULL tensor");
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "mla_up_v: tensors must be 16-byte aligned");
  if (!mla::head_gemm_supported(shape->d_latent, shape->d_v))
    return fail(MLA_ERR_UNSUPPORTED, "mla_up_v: no kernel for d_latent %d, d_v %d", shape->d_latent, shape->d_v);
  mla::HeadGemmParams p{};
  p.a = o_lat;
  p.w = static_cast<const uint16_t*>(w_uv);
  p.c = out;
  p.M = shape->batch * shape->q_len;
  p.H = shape->num_heads;
  p.K = shape->d_latent;
  p.N = shape->d_v;
  return hip_status(mla::launch_head_gemm(p, true, shape->out_dtype == MLA_FP32, stream), "mla_up_v launch");
}

mla_status_t mla_combine_up_v(const mla_shape_t* shape, int32_t num_parts, const void* o_part,
                              const float* lse_part, const int32_t* seq_lens, const void* w_uv, void* out,
                              float* lse, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!o_part || !lse_part || !seq_lens || !w_uv || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "mla_combine_up_v: NULL tensor");
  if (!aligned16(o_part) || !aligned16(w_uv) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "mla_combine_up_v: o_part, w_uv and out must be 16-byte aligned");
  if (num_parts < shape->batch)
    return fail(MLA_ERR_INVALID_ARG, "mla_combine_up_v: num_parts %d < batch %d", num_parts, shape->batch);
  if (!mla::combine_up_supported(shape->d_latent, shape->d_v))
    return fail(MLA_ERR_UNSUPPORTED, "mla_combine_up_v: no kernel for d_latent %d, d_v %d", shape->d_latent,
                shape->d_v);
  mla::CombineUpParams p{};
  p.o_part = o_part;
  p.o_half = shape->partial_dtype == MLA_FP16;
  p.lse_part = lse_part;
  p.seq_lens = seq_lens;
  p.w = static_cast<const uint16_t*>(w_uv);
  p.out = out;
  p.out_f32 = shape->out_dtype == MLA_FP32;
  p.lse = lse;
  p.B = shape->batch;
  p.S = shape->q_len;
  p.H = shape->num_heads;
  p.P = num_parts;
  p.DC = shape->d_latent;
  p.NV = shape->d_v;
  return hip_status(mla::launch_combine_up(p, stream), "mla_combine_up_v launch");
}

namespace {

mla_status_t append_slices(const mla_shape_t* shape, int32_t d_model, int* ks) {
  if (d_model < mla::kAppendSlice || d_model % mla::kAppendSlice != 0 || d_model > (1 << 16))
    return fail(MLA_ERR_UNSUPPORTED, "d_model %d (a multiple of %d up to 65536)", d_model, mla::kAppendSlice);
  *ks = d_model / mla::kAppendSlice;
  (void)shape;
  return MLA_OK;
}

}  // namespace

mla_status_t mla_append_kv_workspace_bytes(const mla_shape_t* shape, int32_t d_model, size_t* bytes) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  int ks = 0;
  st = append_slices(shape, d_model, &ks);
  if (st != MLA_OK) return st;
  *bytes = (size_t)shape->batch * shape->q_len * ks * (shape->d_latent + shape->d_rope) * sizeof(float);
  return ok();
}

namespace {

// Checks and launches of mla_append_kv; `workspace == nullptr` asks for the
// library's own scratch array (mla_append_kv_noalloc), which is looked up
// only after every argument check has passed.
mla_status_t append_impl(const char* who, const mla_shape_t* shape, int32_t d_model, const void* x,
                         const void* w_dkv, float rope_base, void* c_kv, void* k_rope, int64_t token_stride,
                         int64_t block_stride, float* kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool own_scratch = workspace == nullptr;
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  int ks = 0;
  st = append_slices(shape, d_model, &ks);
  if (st != MLA_OK) return st;
  if (!x || !w_dkv || !c_kv || !k_rope || !block_table || !seq_lens)
    return fail(MLA_ERR_INVALID_ARG, "%s: NULL tensor", who);
  if (!std::isfinite(rope_base) || rope_base <= 1.0f)
    return fail(MLA_ERR_INVALID_ARG, "%s: rope_base must be finite and > 1", who);
  const bool fp8 = shape->cache_dtype == MLA_FP8_E4M3;
  if (fp8 && !kv_scale) return fail(MLA_ERR_INVALID_ARG, "%s: fp8 cache needs kv_scale", who);
  if (!fp8 && kv_scale) return fail(MLA_ERR_INVALID_ARG, "%s: kv_scale given for a bf16 cache", who);
  if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(workspace) || !aligned16(c_kv) || !aligned16(k_rope))
    return fail(MLA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", who);
  const int elem = fp8 ? 1 : 2;
  const int64_t rope_off = static_cast<const char*>(k_rope) - static_cast<const char*>(c_kv);
  if (token_stride <= 0 || token_stride % 16 || block_stride % 16 ||
      block_stride < (int64_t)shape->block_size * token_stride)
    return fail(MLA_ERR_INVALID_ARG,
                "%s: token_stride/block_stride must be positive multiples of 16 with "
                "block_stride >= block_size * token_stride", who);
  if (rope_off < (int64_t)shape->d_latent * elem || rope_off + (int64_t)shape->d_rope * elem > token_stride)
    return fail(MLA_ERR_INVALID_ARG, "%s: k_rope must follow the latent inside the record", who);
  size_t need = 0;
  st = mla_append_kv_workspace_bytes(shape, d_model, &need);
  if (st != MLA_OK) return st;
  if (own_scratch) {
    if (need > (size_t)MLA_APPEND_NOALLOC_MAX_BYTES)
      return fail(MLA_ERR_UNSUPPORTED,
                  "%s: needs %zu bytes of partial products, more than the library's fixed %zu-byte scratch "
                  "(use mla_append_kv with a workspace)", who, need, (size_t)MLA_APPEND_NOALLOC_MAX_BYTES);
    hipError_t e = mla::append_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e, "mla_append_kv_noalloc scratch lookup");
    workspace_bytes = MLA_APPEND_NOALLOC_MAX_BYTES;
  } else if (workspace_bytes < need) {
    return fail(MLA_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes, need);
  }
  const int M = shape->batch * shape->q_len;
  mla::HeadGemmParams g{};
  g.a = x;
  g.w = static_cast<const uint16_t*>(w_dkv);
  g.c = workspace;
  g.M = M;
  g.H = ks;
  g.K = mla::kAppendSlice;
  g.N = shape->d_latent + shape->d_rope;
  hipError_t e = mla::launch_head_gemm_partials(g, stream);
  if (e != hipSuccess) return hip_status(e, own_scratch ? "mla_append_kv_noalloc product launch"
                                                        : "mla_append_kv product launch");
  mla::AppendParams p{};
  p.part = static_cast<const float*>(workspace);
  p.KS = ks;
  p.M = M;
  p.S = shape->q_len;
  p.DC = shape->d_latent;
  p.c_kv = static_cast<char*>(c_kv);
  p.rope_off = rope_off;
  p.token_stride = token_stride;
  p.block_stride = block_stride;
  p.kv_scale = kv_scale;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.bt_stride = shape->max_blocks_per_seq;
  p.block_size = shape->block_size;
  p.log2_base = std::log2((double)rope_base);
  p.fp8 = fp8;
  return hip_status(mla::launch_append_finish(p, stream),
                    own_scratch ? "mla_append_kv_noalloc launch" : "mla_append_kv launch");
}

}  // namespace

mla_status_t mla_append_kv(const mla_shape_t* shape, int32_t d_model, const void* x, const void* w_dkv,
                           float rope_base, void* c_kv, void* k_rope, int64_t token_stride, int64_t block_stride,
                           float* kv_scale, const int32_t* block_table, const int32_t* seq_lens, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return fail(MLA_ERR_INVALID_ARG, "mla_append_kv: NULL tensor (workspace)");
  return append_impl("mla_append_kv", shape, d_model, x, w_dkv, rope_base, c_kv, k_rope, token_stride, block_stride,
                     kv_scale, block_table, seq_lens, workspace, workspace_bytes, stream);
}

mla_status_t mla_append_kv_noalloc(const mla_shape_t* shape, int32_t d_model, const void* x, const void* w_dkv,
                                   float rope_base, void* c_kv, void* k_rope, int64_t token_stride,
                                   int64_t block_stride, float* kv_scale, const int32_t* block_table,
                                   const int32_t* seq_lens, hipStream_t stream) {
  return append_impl("mla_append_kv_noalloc", shape, d_model, x, w_dkv, rope_base, c_kv, k_rope, token_stride,
                     block_stride, kv_scale, block_table, seq_lens, nullptr, 0, stream);
}

namespace {

mla_status_t check_prefill(const mla_shape_t* shape, int32_t prompt_len) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (shape->d_nope != 128 || shape->d_v != 128)
    return fail(MLA_ERR_UNSUPPORTED, "prefill: d_nope %d, d_v %d (kernels exist for 128, 128)", shape->d_nope,
                shape->d_v);
  // The prompt's records and the outputs are bf16 only: a shape that says
  // otherwise would have its buffers read or written in the wrong type.
  if (shape->cache_dtype != MLA_BF16 || shape->out_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "prefill: records and outputs are bf16 (cache_dtype and out_dtype MLA_BF16)");
  if (prompt_len < 1 || prompt_len > (1 << 20) || (int64_t)shape->batch * prompt_len > (1 << 24))
    return fail(MLA_ERR_INVALID_ARG, "prefill: prompt_len %d out of range", prompt_len);
  return MLA_OK;
}

}  // namespace

mla_status_t mla_prefill_workspace_bytes(const mla_shape_t* shape, size_t* bytes) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (size_t)shape->num_heads * shape->d_latent * shape->d_v * 2;  // W_UV transposed
  return ok();
}

mla_status_t mla_prefill_kv_elems(const mla_shape_t* shape, int32_t prompt_len, int64_t* elems) {
  mla_status_t st = check_prefill(shape, prompt_len);
  if (st != MLA_OK) return st;
  if (!elems) return fail(MLA_ERR_INVALID_ARG, "elems is NULL");
  *elems = (int64_t)shape->batch * shape->num_heads * ((prompt_len + 31) / 32) * 32 * 128;
  return ok();
}

mla_status_t mla_prefill_kv(const mla_shape_t* shape, int32_t prompt_len, const void* ckr, const void* w_uk,
                            const void* w_uv, const int32_t* seq_lens, void* k_nope, void* v, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  mla_status_t st = check_prefill(shape, prompt_len);
  if (st != MLA_OK) return st;
  if (!ckr || !w_uk || !w_uv || !seq_lens || !k_nope || !v || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_kv: NULL tensor");
  if (!aligned16(ckr) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(k_nope) || !aligned16(v) ||
      !aligned16(workspace))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_kv: tensors must be 16-byte aligned");
  size_t need = 0;
  st = mla_prefill_workspace_bytes(shape, &need);
  if (st != MLA_OK) return st;
  if (workspace_bytes < need)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_kv: workspace of %zu bytes, %zu needed", workspace_bytes, need);
  uint16_t* wvt = static_cast<uint16_t*>(workspace);
  hipError_t e = mla::launch_transpose_heads(static_cast<const uint16_t*>(w_uv), wvt, shape->num_heads,
                                             shape->d_latent, shape->d_v, stream);
  if (e != hipSuccess) return hip_status(e, "mla_prefill_kv transpose launch");
  mla::ExpandParams x{};
  x.ckr = static_cast<const uint16_t*>(ckr);
  x.wuk = static_cast<const uint16_t*>(w_uk);
  x.wvt = wvt;
  x.seq_lens = seq_lens;
  x.B = shape->batch;
  x.P = prompt_len;
  x.H = shape->num_heads;
  x.k_nope = static_cast<uint16_t*>(k_nope);
  x.v = static_cast<uint16_t*>(v);
  return hip_status(mla::launch_expand(x, shape->d_latent, stream), "mla_prefill_kv launch");
}

mla_status_t mla_prefill_attention(const mla_shape_t* shape, int32_t prompt_len, const void* q_nope,
                                   const void* q_rope, const void* k_nope, const void* ckr, const void* v,
                                   const int32_t* seq_lens, void* out, float* lse, hipStream_t stream) {
  mla_status_t st = check_prefill(shape, prompt_len);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_rope || !k_nope || !ckr || !v || !seq_lens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_attention: NULL tensor");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(k_nope) || !aligned16(ckr) || !aligned16(v) ||
      !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "mla_prefill_attention: tensors must be 16-byte aligned");
  mla::PrefillParams p{};
  p.q_nope = static_cast<const uint16_t*>(q_nope);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.k_nope = static_cast<const uint16_t*>(k_nope);
  p.ckr = static_cast<const uint16_t*>(ckr);
  p.v = static_cast<const uint16_t*>(v);
  p.seq_lens = seq_lens;
  p.B = shape->batch;
  p.P = prompt_len;
  p.H = shape->num_heads;
  p.DCK = shape->d_latent;
  p.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  return hip_status(mla::launch_prefill(p, stream), "mla_prefill_attention launch");
}

mla_status_t mla_tpla_split_weights(const mla_shape_t* shape, int32_t n_shards, int32_t hadamard, const void* w_uk,
                                    const void* w_uv, void* w_uk_shards, void* w_uv_shards, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (n_shards != 1 && n_shards != 2 && n_shards != 4)
    return fail(MLA_ERR_UNSUPPORTED, "mla_tpla_split_weights: n_shards %d (1, 2 or 4)", n_shards);
  if (!w_uk || !w_uv || !w_uk_shards || !w_uv_shards)
    return fail(MLA_ERR_INVALID_ARG, "mla_tpla_split_weights: NULL tensor");
  if (!aligned16(w_uk) || !aligned16(w_uk_shards) || !aligned16(w_uv) || !aligned16(w_uv_shards))
    return fail(MLA_ERR_INVALID_ARG, "mla_tpla_split_weights: tensors must be 16-byte aligned");
  const int64_t H = shape->num_heads, dn = shape->d_nope, dc = shape->d_latent, dv = shape->d_v;
  const int64_t dcs = dc / n_shards;
  mla::HadamardParams k{};
  k.in = static_cast<const uint16_t*>(w_uk);
  k.out = static_cast<uint16_t*>(w_uk_shards);
  k.n_vec = H * dn;  // the rows of every W_UK[h]
  k.inner = 1;
  k.in_outer = dc;
  k.in_elem = 1;
  k.out_outer = dcs;
  k.out_elem = 1;
  k.out_shard = H * dn * dcs;
  k.d = (int32_t)dc;
  k.n_shards = n_shards;
  k.rotate = hadamard != 0;
  hipError_t e = mla::launch_hadamard(k, stream);
  if (e != hipSuccess) return hip_status(e, "mla_tpla_split_weights key launch");
  mla::HadamardParams v{};
  v.in = static_cast<const uint16_t*>(w_uv);
  v.out = static_cast<uint16_t*>(w_uv_shards);
  v.n_vec = H * dv;  // the columns of every W_UV[h]
  v.inner = dv;
  v.in_outer = dc * dv;
  v.in_inner = 1;
  v.in_elem = dv;
  v.out_outer = dcs * dv;
  v.out_inner = 1;
  v.out_elem = dv;
  v.out_shard = H * dcs * dv;
  v.d = (int32_t)dc;
  v.n_shards = n_shards;
  v.rotate = hadamard != 0;
  return hip_status(mla::launch_hadamard(v, stream), "mla_tpla_split_weights value launch");
}

mla_status_t mla_tpla_rotate_cache(const mla_shape_t* shape, void* c_kv, int64_t token_stride, int64_t block_stride,
                                   int32_t num_pages, hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (shape->cache_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "mla_tpla_rotate_cache: bf16 caches only");
  if (!c_kv) return fail(MLA_ERR_INVALID_ARG, "mla_tpla_rotate_cache: NULL cache");
  if (num_pages < 0) return fail(MLA_ERR_INVALID_ARG, "mla_tpla_rotate_cache: num_pages %d", num_pages);
  if (!aligned16(c_kv) || token_stride % 16 || block_stride % 16 ||
      token_stride < (int64_t)shape->d_latent * 2 || block_stride < (int64_t)shape->block_size * token_stride)
    return fail(MLA_ERR_INVALID_ARG, "mla_tpla_rotate_cache: bad alignment or strides");
  mla::HadamardParams k{};
  k.in = static_cast<const uint16_t*>(c_kv);
  k.out = static_cast<uint16_t*>(c_kv);
  k.n_vec = (int64_t)num_pages * shape->block_size;
  k.inner = shape->block_size;
  k.in_outer = k.out_outer = block_stride / 2;
  k.in_inner = k.out_inner = token_stride / 2;
  k.in_elem = k.out_elem = 1;
  k.out_shard = 0;
  k.d = shape->d_latent;
  k.n_shards = 1;
  k.rotate = true;
  return hip_status(mla::launch_hadamard(k, stream), "mla_tpla_rotate_cache launch");
}

mla_status_t mla_tpla_reduce(const mla_shape_t* shape, int32_t n_shards, const float* parts, void* out,
                             hipStream_t stream) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (n_shards < 1 || n_shards > 64) return fail(MLA_ERR_INVALID_ARG, "mla_tpla_reduce: n_shards %d", n_shards);
  if (!parts || !out) return fail(MLA_ERR_INVALID_ARG, "mla_tpla_reduce: NULL tensor");
  if (!aligned16(parts) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "mla_tpla_reduce: tensors must be 16-byte aligned");
  const int64_t count = (int64_t)shape->batch * shape->q_len * shape->num_heads * shape->d_v;
  if (count % 4) return fail(MLA_ERR_UNSUPPORTED, "mla_tpla_reduce: output size not a multiple of 4");
  return hip_status(mla::launch_shard_sum(parts, n_shards, count, out, shape->out_dtype == MLA_FP32, stream),
                    "mla_tpla_reduce launch");
}

namespace {

mla_status_t check_gqa(const mla_shape_t* shape, int32_t groups) {
  mla_status_t st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (groups < 1 || shape->num_heads % groups)
    return fail(MLA_ERR_INVALID_ARG, "gqa: %d heads do not split into %d groups", shape->num_heads, groups);
  const int dq = shape->d_nope + shape->d_v;
  if (dq != 256 && dq != 512)
    return fail(MLA_ERR_UNSUPPORTED, "gqa: d_nope + d_v = %d (the decode reads 256- or 512-wide records)", dq);
  if ((int64_t)shape->batch * groups > mla::kMaxBatch)
    return fail(MLA_ERR_UNSUPPORTED, "gqa: batch * groups %d > %d", shape->batch * groups, mla::kMaxBatch);
  return MLA_OK;
}

mla::GqaParams gqa_params(const mla_shape_t* shape, int32_t groups) {
  mla::GqaParams p{};
  p.B = shape->batch;
  p.S = shape->q_len;
  p.H = shape->num_heads;
  p.G = groups;
  p.dn = shape->d_nope;
  p.dv = shape->d_v;
  p.dr = shape->d_rope;
  return p;
}

}  // namespace

mla_status_t mla_gqa_queries(const mla_shape_t* shape, int32_t groups, const void* q_nope, const void* q_rope,
                             void* q_cat, void* q_rope_g, hipStream_t stream) {
  mla_status_t st = check_gqa(shape, groups);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_rope || !q_cat || !q_rope_g) return fail(MLA_ERR_INVALID_ARG, "mla_gqa_queries: NULL tensor");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(q_cat) || !aligned16(q_rope_g))
    return fail(MLA_ERR_INVALID_ARG, "mla_gqa_queries: tensors must be 16-byte aligned");
  mla::GqaParams p = gqa_params(shape, groups);
  p.q_nope = static_cast<const uint16_t*>(q_nope);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.q_cat = static_cast<uint16_t*>(q_cat);
  p.q_rope_g = static_cast<uint16_t*>(q_rope_g);
  return hip_status(mla::launch_gqa_queries(p, stream), "mla_gqa_queries launch");
}

mla_status_t mla_gqa_output(const mla_shape_t* shape, int32_t groups, const float* o_lat, const float* lse_g,
                            void* out, float* lse, hipStream_t stream) {
  mla_status_t st = check_gqa(shape, groups);
  if (st != MLA_OK) return st;
  if (!o_lat || !lse_g || !out || !lse) return fail(MLA_ERR_INVALID_ARG, "mla_gqa_output: NULL tensor");
  if (!aligned16(o_lat) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "mla_gqa_output: o_lat and out must be 16-byte aligned");
  mla::GqaParams p = gqa_params(shape, groups);
  p.o_lat = o_lat;
  p.lse_g = lse_g;
  p.out = out;
  p.lse = lse;
  return hip_status(mla::launch_gqa_output(p, shape->out_dtype == MLA_FP32, stream), "mla_gqa_output launch");
}

}  // extern "C"
