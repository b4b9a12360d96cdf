// Host-side logic of the C ABI, exercised without a GPU: page layout, split
// plan, the device-metadata contract check and the argument checks of every
// call (which fill the kernels' launch arguments).  Built together with
// host_checks.cpp by tests/test_host_sanitized.py under AddressSanitizer and
// UndefinedBehaviorSanitizer; exits non-zero on the first failed expectation.
// Device pointers are stand-ins (host buffers): nothing here dereferences
// them, which is what is being checked.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "host_checks.h"
#include "mla_args.h"

using namespace mla_host;

static int g_checks = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    ++g_checks;                                                           \
    if (!(cond)) {                                                        \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      exit(1);                                                            \
    }                                                                     \
  } while (0)

alignas(256) static char g_buf[1 << 16];
static void* dev(int i) { return g_buf + 256 * i; }           // 16-byte aligned stand-ins
static void* misaligned(int i) { return g_buf + 256 * i + 8; }

static mla_config v2(int cache = MLA_BF16) {
  mla_config c{128, 512, 64, 128, 128, MLA_PAGE_TOKENS, 1.0f / sqrtf(192.f), cache, MLA_BF16};
  return c;
}
static mla_config tiny() {
  mla_config c{4, 16, 8, 8, 8, MLA_PAGE_TOKENS, 0.25f, MLA_F32, MLA_F32};
  return c;
}

static void test_status_and_version() {
  EXPECT(mla_abi_version() == MLA_ABI_VERSION);
  for (int s = 0; s <= 4; ++s) EXPECT(strcmp(mla_status_string((mla_status)s), "unknown status") != 0);
  EXPECT(strcmp(mla_status_string((mla_status)99), "unknown status") == 0);
}

static void test_config_and_layout() {
  size_t pb, ro, so;
  mla_config c = v2();
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_OK && pb == 73728 && ro == 65536 && so == 73728);
  c = v2(MLA_FP8_E4M3);
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_OK && pb == 41216 && pb / 64 == 644);
  c = v2(MLA_FP8_E4M3_G128);
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_OK && pb == 41984 && pb / 64 == 656);
  c = tiny();
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_OK && pb == 64 * 24 * 4);
  EXPECT(mla_page_layout(nullptr, &pb, &ro, &so) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_page_layout(&c, nullptr, &ro, &so) == MLA_ERR_INVALID_ARG);
  c = v2();
  c.block_size = 32;
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_INVALID_ARG);
  c = v2();
  c.softmax_scale = NAN;
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_INVALID_ARG);
  c.softmax_scale = -1.f;
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_INVALID_ARG);
  c = v2();
  c.num_heads = 64;
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_UNSUPPORTED);
  c = v2();
  c.act_dtype = MLA_FP8_E4M3;  // activations are F32 or BF16
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_INVALID_ARG);
  c = v2();
  c.act_dtype = MLA_F32;  // BF16 cache with float32 activations: no kernel
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_UNSUPPORTED);
  c = v2();
  c.cache_dtype = 9;
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_INVALID_ARG);
  c = tiny();
  c.d_latent = 4096;  // too large for the float32 kernel
  EXPECT(mla_page_layout(&c, &pb, &ro, &so) == MLA_ERR_UNSUPPORTED);
}

static void test_plan() {
  mla_config c = v2();
  mla_plan p;
  const int32_t lens[3] = {16384, 32768, 20000};
  EXPECT(mla_decode_plan(&c, 3, lens, 0, 0, 256, &p) == MLA_OK);
  EXPECT(p.num_workers == 256 && p.num_slots == 258);
  EXPECT(p.workspace_bytes == workspace_bytes(&c, 258));
  const int32_t one[1] = {100};
  EXPECT(mla_decode_plan(&c, 1, one, 0, 0, 256, &p) == MLA_OK && p.num_workers == 2);
  EXPECT(mla_decode_plan(&c, 32, nullptr, 0, 2048, 256, &p) == MLA_OK && p.num_workers == 256);
  EXPECT(mla_decode_plan(&c, 32, nullptr, 0, 2048, 100, &p) == MLA_OK && p.num_workers == 96);
  EXPECT(mla_decode_plan(&c, 3, nullptr, 0, 300, 256, &p) == MLA_OK && p.num_workers == 15);
  EXPECT(mla_decode_plan(&c, 1, nullptr, 0, 0, 256, &p) == MLA_ERR_INVALID_ARG);  // no lengths at all
  EXPECT(mla_decode_plan(&c, 0, lens, 0, 0, 256, &p) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode_plan(&c, 3, lens, 0, 0, 256, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode_plan(&c, 3, lens, 0, -1, 256, &p) == MLA_ERR_INVALID_ARG);
  const int32_t neg[2] = {10, -5};
  EXPECT(mla_decode_plan(&c, 2, neg, 0, 0, 256, &p) == MLA_ERR_INVALID_ARG);
  // a large ragged batch: one worker per CU, the slots it needs
  std::vector<int32_t> many(4096, 1);
  EXPECT(mla_decode_plan(&c, 4096, many.data(), 0, 0, 256, &p) == MLA_OK);
  EXPECT(p.num_workers == 256 && p.num_slots == 256 + 4095);
}

static void test_metadata_check() {
  mla_config c = v2();
  const int32_t lens[2] = {100, 64};
  const int32_t table[2 * 3] = {0, 1, -1, 2, -1, -1};
  int32_t err = 7;
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, nullptr, 0, &err) == MLA_OK && err == -1);
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 2, nullptr, 0, &err) == MLA_ERR_INVALID_ARG &&
         err == 1);  // page 2 out of range
  const int32_t zero[2] = {100, 0};
  EXPECT(mla_check_decode_inputs_host(&c, 2, zero, table, 3, 3, nullptr, 0, &err) == MLA_ERR_INVALID_ARG &&
         err == 1);
  const int32_t longer[2] = {200, 64};  // needs 4 columns
  EXPECT(mla_check_decode_inputs_host(&c, 2, longer, table, 3, 3, nullptr, 0, &err) == MLA_ERR_INVALID_ARG &&
         err == 0);
  const int32_t idx_ok[2 * 4] = {0, 5, 99, -1, 1, 2, 3, 63};
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, idx_ok, 4, &err) == MLA_OK);
  const int32_t idx_unsorted[2 * 4] = {5, 0, 99, -1, 1, 2, 3, 63};
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, idx_unsorted, 4, &err) == MLA_ERR_INVALID_ARG &&
         err == 0);
  const int32_t idx_gap[2 * 4] = {0, 5, 99, -1, 1, -1, 3, 63};  // a value after padding
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, idx_gap, 4, &err) == MLA_ERR_INVALID_ARG &&
         err == 1);
  const int32_t idx_range[2 * 4] = {0, 5, 100, -1, 1, 2, 3, 63};  // 100 >= seq_len
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, idx_range, 4, &err) == MLA_ERR_INVALID_ARG &&
         err == 0);
  const int32_t idx_dup[2 * 4] = {0, 5, 5, -1, 1, 2, 3, 63};
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, idx_dup, 4, &err) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, nullptr, 4, &err) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_check_decode_inputs_host(&c, 2, lens, table, 3, 3, idx_ok, 4, nullptr) == MLA_OK);
}

static void test_prepare_decode() {
  mla_config c = v2();
  mla::DecodeArgs a;
  Path path;
  const int32_t* table = (const int32_t*)dev(3);
  const int32_t* lens = (const int32_t*)dev(4);
  // direct mode
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, nullptr, nullptr, 0, dev(5),
                        (float*)dev(6), &a, &path) == MLA_OK);
  EXPECT(path == Path::kMfmaBf16 && a.num_workers == 0 && a.o_lat == dev(5) && a.page_bytes == 73728 &&
         a.rope_off == 65536 && a.topk_idx == nullptr && a.batch == 2 && a.bt_stride == 4);
  // split mode
  mla_plan p{7, 8, 0};
  const size_t need = workspace_bytes(&c, 8);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, &p, dev(7), need, nullptr,
                        nullptr, &a, &path) == MLA_OK);
  EXPECT(a.num_workers == 7 && a.part_o == dev(7) && a.part_bf16 == 1 &&
         (char*)a.part_lse == (char*)dev(7) + 8 * 128 * 512 * 4);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, &p, dev(7), need - 1,
                        nullptr, nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, nullptr, dev(7), need,
                        nullptr, nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  mla_plan big{70000, 70001, 0};
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, &big, dev(7), SIZE_MAX,
                        nullptr, nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  // nulls, misalignment, index list without length and the reverse
  EXPECT(prepare_decode(&c, nullptr, dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, nullptr, nullptr, 0, dev(5),
                        nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_decode(&c, misaligned(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, nullptr, nullptr, 0,
                        dev(5), nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, (const int32_t*)dev(8), 0, 2, nullptr,
                        nullptr, 0, dev(5), nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 16, 2, nullptr, nullptr, 0, dev(5),
                        nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), (int64_t)1 << 24, table, 4, lens, nullptr, 0, 2, nullptr,
                        nullptr, 0, dev(5), nullptr, &a, &path) == MLA_ERR_UNSUPPORTED);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 0, nullptr, nullptr, 0, dev(5),
                        nullptr, &a, &path) == MLA_ERR_INVALID_ARG);
  // FP8 with an index list: the MFMA kernel with per-token scales
  c = v2(MLA_FP8_E4M3);
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, (const int32_t*)dev(8), 2048, 2, nullptr,
                        nullptr, 0, dev(5), nullptr, &a, &path) == MLA_OK);
  EXPECT(path == Path::kMfmaFp8 && cache_kind(path) == mla::CacheKind::kFp8Token && a.scale_off == 32768 + 8192 &&
         a.topk == 2048);
  // float32 partials on the float32 path
  c = tiny();
  EXPECT(prepare_decode(&c, dev(0), dev(1), dev(2), 10, table, 4, lens, nullptr, 0, 2, &p,
                        dev(7), workspace_bytes(&c, 8), nullptr, nullptr, &a, &path) == MLA_OK);
  EXPECT(path == Path::kF32 && a.part_bf16 == 0);
}

static void test_prepare_merges_and_gemms() {
  mla_config c = v2();
  mla_plan p{7, 9, 0};
  const size_t need = workspace_bytes(&c, 9);
  const int32_t* lens = (const int32_t*)dev(4);
  mla::CombineArgs a;
  EXPECT(prepare_combine(&c, dev(7), need, lens, 0, 3, &p, dev(5), (float*)dev(6), &a) == MLA_OK);
  EXPECT(a.num_workers == 7 && a.o_lat == dev(5) && a.out_bf16 == 1 && a.part_bf16 == 1);
  EXPECT(prepare_combine(&c, dev(7), need, lens, 0, 3, &p, nullptr, nullptr, &a) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_combine(&c, dev(7), need - 16, lens, 0, 3, &p, dev(5), nullptr, &a) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_combine(&c, dev(7), need, lens, 0, 70000, &p, dev(5), nullptr, &a) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_combine(&c, dev(7), need, lens, 0, 3, &p, misaligned(5), nullptr, &a) == MLA_ERR_INVALID_ARG);
  mla::CombineUpArgs u;
  EXPECT(prepare_combine_up(&c, dev(7), need, lens, 0, 3, &p, dev(8), dev(9), nullptr, &u) == MLA_OK);
  EXPECT(u.w_uv == dev(8) && u.out == dev(9) && u.c.o_lat == nullptr);
  EXPECT(prepare_combine_up(&c, dev(7), need, lens, 0, 3, &p, nullptr, dev(9), nullptr, &u) == MLA_ERR_INVALID_ARG);
  mla_config t = tiny();
  EXPECT(prepare_combine_up(&t, dev(7), workspace_bytes(&t, 9), lens, 0, 3, &p, dev(8), dev(9), nullptr, &u) ==
         MLA_ERR_UNSUPPORTED);
  mla::HeadGemmArgs g;
  Path path;
  EXPECT(prepare_head_gemm(&c, dev(0), dev(1), dev(2), 64, true, &g, &path) == MLA_OK);
  EXPECT(g.M == 512 && g.K == 128 && g.batch == 64);
  EXPECT(prepare_head_gemm(&c, dev(0), dev(1), dev(2), 64, false, &g, &path) == MLA_OK);
  EXPECT(g.M == 128 && g.K == 512);
  EXPECT(prepare_head_gemm(&c, dev(0), misaligned(1), dev(2), 64, true, &g, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(prepare_head_gemm(&c, dev(0), dev(1), dev(2), 65535 * 32 + 1, true, &g, &path) == MLA_ERR_UNSUPPORTED);
}

static void test_packed_partials() {
  mla_config c = v2();
  void* po;
  float* pl;
  partials_at(&c, Path::kMfmaBf16, dev(0), 319, true, &po, &pl);
  EXPECT((char*)pl - (char*)po == 319 * 128 * 512 * 2);
  EXPECT(packed_partials_bytes(&c, Path::kMfmaBf16, 319) == (size_t)319 * 128 * 512 * 2 + 319 * 128 * 4);
  partials_at(&c, Path::kMfmaBf16, dev(0), 319, false, &po, &pl);
  EXPECT((char*)pl - (char*)po == 319 * 128 * 512 * 4);
  mla_config t = tiny();
  EXPECT(packed_partials_bytes(&t, Path::kF32, 3) == al16(3 * 4 * 16 * 4) + al16(3 * 4 * 4));
}

static void test_side_calls() {
  mla_config c = v2();
  Path path;
  const float* cs = (const float*)dev(3);
  EXPECT(check_cache_append(&c, dev(0), dev(1), cs, cs, 100, (const int32_t*)dev(2), dev(4), 10,
                            (const int32_t*)dev(5), 4, 8, &path) == MLA_OK);
  EXPECT(check_cache_append(&c, dev(0), dev(1), cs, nullptr, 100, (const int32_t*)dev(2), dev(4), 10,
                            (const int32_t*)dev(5), 4, 8, &path) == MLA_ERR_INVALID_ARG);
  EXPECT(check_cache_append(&c, dev(0), dev(1), cs, cs, 0, (const int32_t*)dev(2), dev(4), 10,
                            (const int32_t*)dev(5), 4, 8, &path) == MLA_ERR_INVALID_ARG);
  mla_config odd = tiny();
  odd.d_rope = 7;
  EXPECT(check_cache_append(&odd, dev(0), dev(1), nullptr, nullptr, 0, (const int32_t*)dev(2), dev(4), 10,
                            (const int32_t*)dev(5), 4, 8, &path) == MLA_ERR_UNSUPPORTED);
  EXPECT(check_prepare_w_uk_t(&c, dev(0), dev(1)) == MLA_OK);
  mla_config fp8 = v2(MLA_FP8_E4M3);
  EXPECT(check_prepare_w_uk_t(&fp8, dev(0), dev(1)) == MLA_OK);
  EXPECT(check_prefill_expand(&fp8, dev(0), 10, (const int32_t*)dev(1), 4096, dev(2), dev(3), dev(4), dev(5),
                              dev(6)) == MLA_OK);
  mla_config big32 = v2(MLA_F32);
  big32.act_dtype = MLA_F32;
  EXPECT(check_prepare_w_uk_t(&big32, dev(0), dev(1)) == MLA_ERR_UNSUPPORTED);
  EXPECT(check_prefill_expand(&c, dev(0), 10, (const int32_t*)dev(1), 4096, dev(2), dev(3), dev(4), dev(5),
                              dev(6)) == MLA_OK);
  EXPECT(check_prefill_expand(&c, dev(0), 10, (const int32_t*)dev(1), 0, dev(2), dev(3), dev(4), dev(5),
                              dev(6)) == MLA_ERR_INVALID_ARG);
  EXPECT(check_prefill_attn(&c, dev(0), dev(1), dev(2), dev(3), dev(4), 4096, 4000, 96, dev(5), nullptr) == MLA_OK);
  EXPECT(check_prefill_attn(&c, dev(0), dev(1), dev(2), dev(3), dev(4), 4096, 4000, 97, dev(5), nullptr) ==
         MLA_ERR_INVALID_ARG);
  EXPECT(check_prefill_attn(&c, dev(0), dev(1), dev(2), dev(3), dev(4), 4096, -1, 10, dev(5), nullptr) ==
         MLA_ERR_INVALID_ARG);
  size_t pb, so;
  EXPECT(mla_indexer_page_layout(128, &pb, &so) == MLA_OK && pb == 8448 && so == 8192);
  EXPECT(mla_indexer_page_layout(0, &pb, &so) == MLA_ERR_INVALID_ARG);
  const int32_t* t32 = (const int32_t*)dev(1);
  EXPECT(check_indexer_scores(64, 128, dev(0), (const float*)dev(2), dev(3), 10, t32, 4, t32, 2, (const float*)dev(4),
                              5000) == MLA_OK);
  EXPECT(check_indexer_scores(32, 128, dev(0), (const float*)dev(2), dev(3), 10, t32, 4, t32, 2,
                              (const float*)dev(4), 5000) == MLA_ERR_UNSUPPORTED);
  EXPECT(check_indexer_scores(64, 128, dev(0), (const float*)dev(2), dev(3), 10, t32, 4, t32, 2,
                              (const float*)((char*)dev(4) + 2), 5000) == MLA_ERR_INVALID_ARG);
  EXPECT(check_topk_select((const float*)dev(0), 5001, t32, 2, 2048, (const int32_t*)dev(2), dev(3), 1000, 1000,
                           1 << 20) == MLA_OK);
  EXPECT(check_topk_select((const float*)dev(0), 5001, t32, 2, 2048, (const int32_t*)dev(2), dev(3), 999, 1000,
                           1 << 20) == MLA_ERR_INVALID_ARG);
  EXPECT(check_topk_select((const float*)dev(0), (1 << 20) + 1, t32, 2, 2048, (const int32_t*)dev(2), dev(3), 1000,
                           1000, 1 << 20) == MLA_ERR_UNSUPPORTED);
  EXPECT(check_topk_select((const float*)dev(0), 5001, t32, 2, 0, (const int32_t*)dev(2), dev(3), 1000, 1000,
                           1 << 20) == MLA_ERR_INVALID_ARG);
}

// The split partition shared by the attention and merge kernels
// (mla_args.h): bounds start at 0, end at W and never decrease; worker_of
// inverts worker_lo; dense batches with at least 64 units per worker give
// workers on even XCDs (p / (P / 8) even) the larger shares, by 65 : 63.
static void test_partition() {
  using namespace mla;
  const int64_t Ps[] = {1, 7, 8, 16, 96, 100, 256, 1024};
  const int64_t Ws[] = {1, 5, 255, 256, 1023, 16383, 16384, 16385, 49152 + 64 * 12, 1532221 / 32 + 64 * 12, 4108,
                        (int64_t)1 << 32};
  for (int32_t topk : {0, 2048}) {
    for (int64_t P : Ps) {
      for (int64_t W : Ws) {
        const bool weighted = xcd_weighted(W, P, topk);
        EXPECT(weighted == (topk == 0 && P >= 16 && (P & (P - 1)) == 0 && W >= 64 * P));
        EXPECT(worker_lo(0, W, P, topk) == 0 && worker_lo(P, W, P, topk) == W);
        int64_t even = 0, odd = 0;
        bool monotone = true, inverse = true, no_empty = true;
        for (int64_t q = 0; q < P; ++q) {
          const int64_t a = worker_lo(q, W, P, topk), b = worker_lo(q + 1, W, P, topk);
          monotone = monotone && b >= a;
          if (W >= P) no_empty = no_empty && b > a;
          if (b > a) {
            // the first and last unit of a non-empty share belong to it
            inverse = inverse && worker_of(a, W, P, topk) == q && worker_of(b - 1, W, P, topk) == q;
          }
          if (P % 8 == 0 && (q / (P / 8)) % 2 == 0) even += b - a;
          else odd += b - a;
        }
        EXPECT(monotone);
        EXPECT(inverse);
        if (!weighted) EXPECT(no_empty);
        if (weighted) {
          EXPECT(no_empty);
          // even-XCD workers carry 65/128 of the units, to within one unit each
          const double want = (double)W * 65.0 / 128.0;
          EXPECT(fabs((double)even - want) <= (double)P);
          EXPECT(even > odd);
        }
      }
    }
  }
  // every unit of a small space maps to the worker whose range holds it
  for (int64_t P : {16, 24, 256}) {
    const int64_t W = 64 * P + 37;
    for (int64_t x = 0; x < W; ++x) {
      const int64_t q = worker_of(x, W, P, 0);
      if (!(q >= 0 && q < P && worker_lo(q, W, P, 0) <= x && x < worker_lo(q + 1, W, P, 0))) {
        EXPECT(false);
        break;
      }
    }
  }
  // equal shares, empty workers included: the last worker whose range starts
  // at or before x, (x + 1) P - 1 over W
  for (int64_t P : {7, 16, 100, 256}) {
    for (int64_t W : {1, 3, 15, 16, 17, 99, 255, 1000}) {
      for (int64_t x = 0; x < W; ++x) {
        if (worker_of(x, W, P, 2048) != ((x + 1) * P - 1) / W || worker_of(x, W, P, 0) != ((x + 1) * P - 1) / W) {
          EXPECT(false);
          break;
        }
      }
    }
  }
}

int main() {
  test_status_and_version();
  test_config_and_layout();
  test_plan();
  test_metadata_check();
  test_prepare_decode();
  test_prepare_merges_and_gemms();
  test_packed_partials();
  test_side_calls();
  test_partition();
  printf("host checks: %d expectations met\n", g_checks);
  return 0;
}
