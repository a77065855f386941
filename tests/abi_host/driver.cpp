// Calls every entry point of the C ABI with valid and invalid arguments (fake,
// never dereferenced device addresses; the launchers are host stand-ins) and
// checks the returned statuses.  Built with the address and undefined-
// behaviour sanitizers by the CPU test suite; exits non-zero on any mismatch.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "mla_absorbed.h"

extern int g_launches;

namespace {
int g_fail = 0;
void expect(mla_status_t got, mla_status_t want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d %s: status %d, expected %d (%s)\n", line, what, (int)got, (int)want,
                 mla_last_error());
    ++g_fail;
  }
  if (want != MLA_OK && std::strlen(mla_last_error()) == 0) {
    std::fprintf(stderr, "line %d %s: failure without a message\n", line, what);
    ++g_fail;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

void* A(uintptr_t k) { return reinterpret_cast<void*>((uintptr_t)1 << 40 | (k << 12)); }  // 16-byte aligned

mla_shape_t shape(int B = 2, int H = 128, int S = 1, int dc = 512, mla_dtype_t cache = MLA_BF16) {
  mla_shape_t s{};
  s.batch = B;
  s.num_heads = H;
  s.q_len = S;
  s.d_nope = 128;
  s.d_rope = 64;
  s.d_latent = dc;
  s.d_v = 128;
  s.block_size = 64;
  s.max_blocks_per_seq = 128;
  s.softmax_scale = 1.0f / std::sqrt(192.0f);
  s.cache_dtype = cache;
  s.out_dtype = MLA_BF16;
  s.partial_dtype = MLA_FP16;
  return s;
}
}  // namespace

int main() {
  hipStream_t st = nullptr;
  mla_shape_t s = shape();
  const int64_t ts = 1152, bs = 64 * 1152;
  char* ckv = static_cast<char*>(A(1));

  // valid calls reach their launchers
  int before = g_launches;
  EXPECT(mla_absorb_q(&s, A(2), A(3), A(4), st), MLA_OK);
  int32_t parts = 0;
  EXPECT(mla_decode_num_parts(&s, &parts), MLA_OK);
  if (parts < s.batch) { std::fprintf(stderr, "num_parts %d < batch\n", parts); ++g_fail; }
  EXPECT(mla_decode_paged(&s, A(5), A(6), ckv, ckv + 1024, ts, bs, nullptr, (int32_t*)A(7), (int32_t*)A(8), parts,
                          A(9), (float*)A(10), st), MLA_OK);
  EXPECT(mla_combine_lse(&s, parts, A(9), (float*)A(10), (int32_t*)A(8), (float*)A(11), (float*)A(12), st), MLA_OK);
  EXPECT(mla_up_v(&s, (float*)A(11), A(13), A(14), st), MLA_OK);
  EXPECT(mla_combine_up_v(&s, parts, A(9), (float*)A(10), (int32_t*)A(8), A(13), A(14), (float*)A(12), st), MLA_OK);
  size_t ws = 0;
  EXPECT(mla_append_kv_workspace_bytes(&s, 4096, &ws), MLA_OK);
  EXPECT(mla_append_kv(&s, 4096, A(15), A(16), 10000.0f, ckv, ckv + 1024, ts, bs, nullptr, (int32_t*)A(7),
                       (int32_t*)A(8), A(17), ws, st), MLA_OK);
  EXPECT(mla_append_kv_noalloc(&s, 4096, A(15), A(16), 10000.0f, ckv, ckv + 1024, ts, bs, nullptr, (int32_t*)A(7),
                               (int32_t*)A(8), st), MLA_OK);
  size_t pws = 0;
  int64_t elems = 0;
  EXPECT(mla_prefill_workspace_bytes(&s, &pws), MLA_OK);
  EXPECT(mla_prefill_kv_elems(&s, 4096, &elems), MLA_OK);
  EXPECT(mla_prefill_kv(&s, 4096, A(18), A(3), A(13), (int32_t*)A(8), A(19), A(20), A(21), pws, st), MLA_OK);
  EXPECT(mla_prefill_attention(&s, 4096, A(22), A(23), A(19), A(18), A(20), (int32_t*)A(8), A(24), (float*)A(25), st),
         MLA_OK);
  EXPECT(mla_tpla_split_weights(&s, 2, 1, A(3), A(13), A(26), A(27), st), MLA_OK);
  EXPECT(mla_tpla_rotate_cache(&s, ckv, ts, bs, 100, st), MLA_OK);
  EXPECT(mla_tpla_reduce(&s, 2, (float*)A(28), A(29), st), MLA_OK);
  mla_shape_t g = shape(4, 32, 2, 512);
  EXPECT(mla_gqa_queries(&g, 8, A(30), A(31), A(32), A(33), st), MLA_OK);
  EXPECT(mla_gqa_output(&g, 8, (float*)A(34), (float*)A(35), A(36), (float*)A(37), st), MLA_OK);
  int64_t flops = 0;
  EXPECT(mla_probe_hbm_read(A(39), 1 << 20, (uint32_t*)A(40), st), MLA_OK);
  EXPECT(mla_probe_mfma(100, (float*)A(40), &flops, st), MLA_OK);
  if (flops <= 0) { std::fprintf(stderr, "mfma probe reported %lld flops\n", (long long)flops); ++g_fail; }
  EXPECT(mla_probe_tile_copy(&s, ckv, ckv + 1024, ts, bs, (int32_t*)A(7), (int32_t*)A(8), parts, (uint32_t*)A(40),
                             st), MLA_OK);
  EXPECT(mla_validate_decode_inputs(&s, (int32_t*)A(7), (int32_t*)A(8), 1000, (int32_t*)A(41), st), MLA_OK);
  if (g_launches <= before) { std::fprintf(stderr, "valid calls launched nothing\n"); ++g_fail; }

  // invalid arguments are refused before anything is launched
  before = g_launches;
  EXPECT(mla_absorb_q(nullptr, A(2), A(3), A(4), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_absorb_q(&s, nullptr, A(3), A(4), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_absorb_q(&s, (char*)A(2) + 2, A(3), A(4), st), MLA_ERR_INVALID_ARG);
  mla_shape_t bad = s;
  bad.softmax_scale = -1.0f;
  EXPECT(mla_absorb_q(&bad, A(2), A(3), A(4), st), MLA_ERR_UNSUPPORTED);
  bad = s;
  bad.softmax_scale = NAN;
  EXPECT(mla_absorb_q(&bad, A(2), A(3), A(4), st), MLA_ERR_INVALID_ARG);
  bad = s;
  bad.d_latent = 384;
  EXPECT(mla_absorb_q(&bad, A(2), A(3), A(4), st), MLA_ERR_UNSUPPORTED);
  bad = s;
  bad.batch = 5000;
  EXPECT(mla_decode_num_parts(&bad, &parts), MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_paged(&s, A(5), A(6), ckv, ckv + 1024, ts, bs, nullptr, (int32_t*)A(7), (int32_t*)A(8), 1,
                          A(9), (float*)A(10), st), MLA_ERR_INVALID_ARG);  // num_parts < batch
  EXPECT(mla_decode_paged(&s, A(5), A(6), ckv, ckv + 512, ts, bs, nullptr, (int32_t*)A(7), (int32_t*)A(8), parts,
                          A(9), (float*)A(10), st), MLA_ERR_INVALID_ARG);  // RoPE key overlaps the latent
  EXPECT(mla_decode_paged(&s, A(5), A(6), ckv, ckv + 1024, ts, bs, (float*)A(38), (int32_t*)A(7), (int32_t*)A(8),
                          parts, A(9), (float*)A(10), st), MLA_ERR_INVALID_ARG);  // scale with a bf16 cache
  mla_shape_t f8 = shape(2, 64, 4, 512, MLA_FP8_E4M3);
  EXPECT(mla_decode_paged(&f8, A(5), A(6), ckv, ckv + 512, 576, 64 * 576, nullptr, (int32_t*)A(7), (int32_t*)A(8),
                          16, A(9), (float*)A(10), st), MLA_ERR_INVALID_ARG);  // e4m3 without scales
  EXPECT(mla_append_kv(&s, 4096, A(15), A(16), 10000.0f, ckv, ckv + 1024, ts, bs, nullptr, (int32_t*)A(7),
                       (int32_t*)A(8), A(17), ws - 4, st), MLA_ERR_INVALID_ARG);
  mla_shape_t big = shape(228);
  EXPECT(mla_append_kv_noalloc(&big, 4096, A(15), A(16), 10000.0f, ckv, ckv + 1024, ts, bs, nullptr, (int32_t*)A(7),
                               (int32_t*)A(8), st), MLA_ERR_UNSUPPORTED);
  EXPECT(mla_prefill_kv(&s, 0, A(18), A(3), A(13), (int32_t*)A(8), A(19), A(20), A(21), pws, st),
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_tpla_split_weights(&s, 3, 1, A(3), A(13), A(26), A(27), st), MLA_ERR_UNSUPPORTED);
  EXPECT(mla_gqa_queries(&g, 5, A(30), A(31), A(32), A(33), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_probe_hbm_read(A(39), 24, (uint32_t*)A(40), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_probe_hbm_read((char*)A(39) + 8, 1 << 20, (uint32_t*)A(40), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_probe_mfma(0, (float*)A(40), &flops, st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_validate_decode_inputs(&s, (int32_t*)A(7), (int32_t*)A(8), 0, (int32_t*)A(41), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_validate_decode_inputs(&s, nullptr, (int32_t*)A(8), 10, (int32_t*)A(41), st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_validate_decode_inputs(&s, (int32_t*)A(7), (int32_t*)A(8), 10, (int32_t*)((char*)A(41) + 2), st),
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_probe_mfma(100, (float*)A(40), nullptr, st), MLA_ERR_INVALID_ARG);
  EXPECT(mla_probe_tile_copy(&f8, ckv, ckv + 512, 576, 64 * 576, (int32_t*)A(7), (int32_t*)A(8), 16, (uint32_t*)A(40),
                             st), MLA_ERR_UNSUPPORTED);
  if (g_launches != before) { std::fprintf(stderr, "an invalid call launched a kernel\n"); ++g_fail; }

  // every status has a name; messages are per thread
  for (int k = 0; k < 4; ++k)
    if (!mla_status_string((mla_status_t)k) || !*mla_status_string((mla_status_t)k)) ++g_fail;
  std::vector<std::thread> th;
  std::vector<int> ok(8, 0);
  for (int t = 0; t < 8; ++t)
    th.emplace_back([&, t] {
      mla_shape_t q = shape(2 + t);
      q.d_latent = 100 + t;
      for (int r = 0; r < 200; ++r) {
        if (mla_absorb_q(&q, A(2), A(3), A(4), st) != MLA_ERR_UNSUPPORTED) return;
        char want[32];
        std::snprintf(want, sizeof want, "d_latent %d", 100 + t);
        if (!std::strstr(mla_last_error(), want)) return;
      }
      ok[t] = 1;
    });
  for (auto& x : th) x.join();
  for (int t = 0; t < 8; ++t)
    if (!ok[t]) { std::fprintf(stderr, "thread %d saw another thread's message\n", t); ++g_fail; }

  if (g_fail) std::fprintf(stderr, "%d failures\n", g_fail);
  else std::printf("abi host checks passed (%d launches)\n", g_launches);
  return g_fail ? 1 : 0;
}
