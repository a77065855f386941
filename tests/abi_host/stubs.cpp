// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// the C ABI layer (mla_api.cpp) uses, so that the layer's argument checks,
// plan sizing and parameter marshalling can run under the address and
// undefined-behaviour sanitizers on a machine without a GPU.  Launchers only
// count their calls and check a few fields of the parameter block.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "mla_kernels.h"

int g_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev) {
  (void)dev;
  *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "hip error"; }
}

namespace {
hipError_t launched(bool ok) {
  ++g_launches;
  if (!ok) {
    std::fprintf(stderr, "launcher received an inconsistent parameter block\n");
    std::abort();
  }
  return hipSuccess;
}
}  // namespace

namespace mla {
int decode_waves(int R) { return R <= 32 ? 1 : (R <= 64 ? 2 : 4); }
int decode_row_groups(int R) { return (R + 32 * decode_waves(R) - 1) / (32 * decode_waves(R)); }
int decode_wgs_per_cu(int R, int) { return decode_waves(R) == 4 ? 1 : 2; }
hipError_t launch_decode(const DecodeParams& p, int, bool, hipStream_t) {
  return launched(p.P >= p.B && p.R == p.S * p.H && p.RG >= 1 && p.q_lat && p.o_part && p.lse_part);
}
hipError_t launch_decode_wide(const DecodeParams& p, int d, bool f, hipStream_t s) { return launch_decode(p, d, f, s); }
hipError_t launch_expand(const ExpandParams& p, int, hipStream_t) { return launched(p.k_nope && p.v); }
hipError_t launch_prefill(const PrefillParams& p, hipStream_t) { return launched(p.out && p.lse); }
hipError_t launch_hadamard(const HadamardParams& p, hipStream_t) { return launched(p.in && p.out && p.d > 0); }
hipError_t launch_shard_sum(const float* parts, int n, int64_t count, void* out, bool, hipStream_t) {
  return launched(parts && out && n > 0 && count > 0);
}
hipError_t launch_gqa_queries(const GqaParams& p, hipStream_t) { return launched(p.q_cat && p.q_rope_g); }
hipError_t launch_gqa_output(const GqaParams& p, bool, hipStream_t) { return launched(p.out && p.lse); }
hipError_t launch_transpose_heads(const uint16_t* w, uint16_t* wt, int, int, int, hipStream_t) {
  return launched(w && wt);
}
hipError_t launch_combine(const CombineParams& p, hipStream_t) { return launched(p.o_lat && p.P >= p.B); }
bool combine_up_supported(int d_latent, int d_v) {
  return (d_latent == 512 || d_latent == 256) && (d_v == 64 || d_v == 128);
}
hipError_t launch_combine_up(const CombineUpParams& p, hipStream_t) { return launched(p.out && p.P >= p.B); }
bool head_gemm_supported(int K, int N) { return K % 64 == 0 && K <= 512 && N % 64 == 0; }
hipError_t launch_head_gemm(const HeadGemmParams& p, bool, bool, hipStream_t) { return launched(p.a && p.w && p.c); }
hipError_t launch_head_gemm_partials(const HeadGemmParams& p, hipStream_t) { return launched(p.c != nullptr); }
hipError_t launch_append_finish(const AppendParams& p, hipStream_t) { return launched(p.part && p.KS > 0); }
hipError_t launch_probe_tile_copy(const DecodeParams& p, int, uint32_t* sink, hipStream_t) {
  return launched(sink && p.P >= p.B && p.RG >= 1);
}
hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t) {
  return launched(buf && sink && bytes >= 16 && cus > 0);
}
int64_t probe_mfma_flops(int iters, int cus) { return (int64_t)cus * 2 * 4 * 4 * iters * 32768; }
hipError_t launch_probe_mfma(int iters, float* sink, int cus, hipStream_t) { return launched(sink && iters > 0 && cus > 0); }
hipError_t launch_validate(const ValidateParams& p, hipStream_t) {
  return launched(p.block_table && p.seq_lens && p.out && p.num_pages > 0 && p.B > 0);
}
hipError_t append_scratch(void** ptr) {
  alignas(256) static char fake[16];
  *ptr = fake;
  return hipSuccess;
}
}  // namespace mla
