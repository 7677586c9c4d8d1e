// Host sanitizer run of the library's host code (test infrastructure): the
// planners over a wide grid of shapes and options (extreme sizes included),
// the paged-input checker on random tables, the status strings, and every
// forward entry point with arguments that validation must reject before
// any device work.  The launch functions are stubs that abort: no call
// here may reach them.  tests/test_sanitizers.py builds this file and
// attn_api.cpp with AddressSanitizer and UndefinedBehaviorSanitizer (no
// recovery), links the HIP runtime for the symbols only, and expects exit
// status 0.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "attn_decode.h"
#include "internal.h"

namespace skv {
hipError_t launch_append(const AppendParams&, hipStream_t) { std::abort(); }
hipError_t launch_split_mfma(int, bool, const SplitParams&, int, hipStream_t, const AppendParams*,
                             bool*) {
  std::abort();
}
hipError_t launch_combine(int, const CombineParams&, hipStream_t) { std::abort(); }
hipError_t scratch_device_address(void**) { std::abort(); }
}  // namespace skv

static int failures = 0;
#define CHECK(c, msg)                                                          \
  do {                                                                         \
    if (!(c)) {                                                                \
      std::fprintf(stderr, "FAIL: %s (line %d)\n", msg, __LINE__);             \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static uint32_t state = 88172645u;
static uint32_t next_u32() {  // xorshift32
  state ^= state << 13;
  state ^= state >> 17;
  state ^= state << 5;
  return state;
}

static bool valid_status(attn_status s) { return s >= ATTN_OK && s <= ATTN_ERR_DATA; }

static void check_plan(const attn_plan& p, int64_t max_seqlen) {
  CHECK(p.num_splits >= 1 && p.num_splits <= 1024, "plan splits in range");
  CHECK(int64_t(p.grid) == (p.extra_blocks > 0 ? int64_t(p.units) + p.extra_blocks
                                                : int64_t(p.units) * p.num_splits),
        "grid = units * splits, or units + extra blocks");
  CHECK(p.extra_blocks == 0 || (p.num_splits > 1 && p.grid < int64_t(p.units) * p.num_splits),
        "a compact list only for a split call, and only when it is smaller");
  CHECK(p.extra_blocks >= 0 &&
            (p.heads_per_row == 1 || p.heads_per_row == 2 || p.heads_per_row == 4),
        "plan flags");
  CHECK(p.heads_per_row == 1 || (p.pack_gqa == 1 && p.rows_per_unit <= 16 && p.row_blocks == 1 &&
                                 p.kernel == 41128),
        "head groups: packed, one 16-row block, the group kernel");
  CHECK(p.split_keys >= 16 && p.split_keys % 16 == 0, "split keys in granules");
  CHECK(int64_t(p.split_keys) * p.num_splits >= max_seqlen, "splits cover max_seqlen_k");
  CHECK(p.workspace_bytes >= 0, "workspace size");
  // partials and counters only for a split call with work (an empty batch needs none)
  CHECK((p.num_splits > 1 && p.units > 0) == (p.workspace_bytes > 0), "workspace only when split");
}

int main() {
  // status strings and version
  for (int c = -3; c < 20; ++c) CHECK(attn_status_str(attn_status(c)) != nullptr, "status string");
  CHECK(attn_abi_version() == ATTN_ABI_VERSION, "abi version");

  // decode planner over a grid, extreme sizes included
  const int batches[] = {0, 1, 7, 1024, 65536, 1 << 20};
  const int qlens[] = {1, 2, 8, 64, 4096};
  const int heads[][2] = {{1, 1}, {8, 2}, {32, 8}, {64, 1}, {128, 128}, {6, 4}};
  const int dims[] = {1, 8, 32, 64, 96, 128, 255, 256, 257};
  const int pages[] = {16, 48, 17};
  const int lens[] = {0, 1, 1000, 16384, 1 << 20, 1 << 30};
  const int splits[] = {-1, 0, 1, 4, 1024, 1025};
  const int packs[] = {-2, -1, 0, 1, 2};
  const int cus[] = {-1, 0, 1, 256, 304};
  int ok_plans = 0;
  for (int b : batches)
    for (int ql : qlens)
      for (auto& hh : heads)
        for (int d : dims)
          for (int pg : pages)
            for (int L : lens) {
              attn_decode_shape s{};
              s.batch = b; s.q_len = ql; s.num_heads_q = hh[0]; s.num_heads_kv = hh[1];
              s.head_dim = d; s.page_size = pg;
              s.max_pages_per_seq = int((int64_t(L) + pg - 1) / pg > 0 ? (int64_t(L) + pg - 1) / pg : 1);
              s.max_seqlen_k = L; s.dtype = int(next_u32() % 3);  // 2: unsupported dtype
              const uint32_t h = next_u32() % 4;
              s.sum_seqlen_k = h == 0 ? 0 : h == 1 ? int64_t(b) * L : h == 2 ? L : -1;
              attn_plan p;
              const attn_status st = attn_decode_plan(&s, splits[next_u32() % 6],
                                                      packs[next_u32() % 5], cus[next_u32() % 5], &p);
              CHECK(valid_status(st), "decode plan status");
              if (st == ATTN_OK) {
                check_plan(p, L);
                ++ok_plans;
              }
            }
  CHECK(ok_plans > 1000, "enough valid plans exercised");
  CHECK(attn_decode_plan(nullptr, 0, -1, 0, nullptr) == ATTN_ERR_NULL, "null shape");

  // dense planner
  for (int hq : {1, 8, 32, 33})
    for (int hkv : {1, 8, 11})
      for (int ql : {1, 4, 128})
        for (int kv : {-1, 0, 1, 1023, 4096, 1 << 30})
          for (int d : {1, 80, 128, 256, 300}) {
            attn_dense_shape s{hq, hkv, ql, kv, d, int(next_u32() % 2)};
            attn_plan p;
            const attn_status st = attn_dense_plan(&s, splits[next_u32() % 6], cus[next_u32() % 5], &p);
            CHECK(valid_status(st), "dense plan status");
            if (st == ATTN_OK) check_plan(p, kv);
          }

  // paged-input checker on random tables, some entries out of range
  for (int trial = 0; trial < 200; ++trial) {
    attn_decode_shape s{};
    s.batch = 1 + int(next_u32() % 9); s.q_len = 1; s.num_heads_q = 4; s.num_heads_kv = 2;
    s.head_dim = 64; s.page_size = 16; s.max_pages_per_seq = 1 + int(next_u32() % 5);
    s.max_seqlen_k = s.max_pages_per_seq * 16; s.dtype = ATTN_BF16;
    std::vector<int32_t> bt(size_t(s.batch) * s.max_pages_per_seq), sl(size_t(s.batch));
    const int64_t num_pages = 1 + next_u32() % 40;
    for (auto& x : bt) x = int32_t(next_u32() % 50) - 3;
    for (auto& x : sl) x = int32_t(next_u32() % (s.max_seqlen_k + 20)) - 5;
    int32_t bad = -1;  // written only on failure
    const attn_status st = attn_check_paged_inputs(&s, bt.data(), sl.data(), num_pages, &bad);
    CHECK(st == ATTN_OK || st == ATTN_ERR_DATA, "paged check status");
    CHECK(st == ATTN_OK ? bad == -1 : (bad >= 0 && bad < s.batch), "bad batch index reported");
    // with appended keys (lengths near INT32_MAX too: the sum must not wrap)
    const int new_len = int(next_u32() % 24) - 2;
    if (trial % 10 == 0) sl[0] = 0x7FFFFFF0;
    bad = -1;
    const attn_status st2 =
        attn_check_kvcache_inputs(&s, bt.data(), sl.data(), num_pages, new_len, &bad);
    if (new_len < 0) {
      CHECK(st2 == ATTN_ERR_ARG && bad == -1, "kvcache check rejects new_len < 0");
    } else {
      CHECK(st2 == ATTN_OK || st2 == ATTN_ERR_DATA, "kvcache check status");
      CHECK(st2 == ATTN_OK ? bad == -1 : (bad >= 0 && bad < s.batch), "kvcache bad batch index");
      if (trial % 10 == 0) CHECK(st2 == ATTN_ERR_DATA && bad == 0, "huge length rejected");
    }
  }

  // forward entry points: rejected before any device work
  attn_decode_shape good{};
  good.batch = 2; good.q_len = 1; good.num_heads_q = 8; good.num_heads_kv = 2; good.head_dim = 128;
  good.page_size = 16; good.max_pages_per_seq = 4; good.max_seqlen_k = 64; good.dtype = ATTN_BF16;
  alignas(16) static uint8_t buf[4096];
  const int32_t* i32 = reinterpret_cast<const int32_t*>(buf);
  CHECK(attn_decode_fwd(&good, nullptr, buf, buf, i32, i32, 0, -1, 0.f, buf, nullptr, nullptr, 0,
                        nullptr) == ATTN_ERR_NULL, "decode fwd null q");
  CHECK(attn_decode_fwd(&good, buf + 2, buf, buf, i32, i32, 0, -1, 0.f, buf, nullptr, nullptr, 0,
                        nullptr) == ATTN_ERR_ALIGN, "decode fwd misaligned q");
  attn_decode_shape bad_shape = good;
  bad_shape.num_heads_kv = 3;
  CHECK(attn_decode_fwd(&bad_shape, buf, buf, buf, i32, i32, 0, -1, 0.f, buf, nullptr, nullptr, 0,
                        nullptr) == ATTN_ERR_SHAPE, "decode fwd bad heads");
  CHECK(attn_decode_fwd(&good, buf, buf, buf, i32, i32, 0, -1, __builtin_nanf(""), buf, nullptr,
                        nullptr, 0, nullptr) == ATTN_ERR_ARG, "decode fwd NaN scale");
  CHECK(attn_decode_kvcache_fwd(&good, buf, buf, buf, i32, i32, nullptr, buf, 1, 0, 0, -1, 0.f, buf,
                                nullptr, nullptr, 0, nullptr) != ATTN_OK, "kvcache fwd k_new null");
  CHECK(attn_decode_kvcache_fwd(&good, buf, buf, buf, i32, i32, nullptr, nullptr, 0, 2, 0, -1, 0.f,
                                buf, nullptr, nullptr, 0, nullptr) != ATTN_OK, "kvcache fwd causal 2");
  CHECK(attn_decode_varlen_fwd(&good, buf, buf, buf, i32, nullptr, i32, 2, nullptr, nullptr, 0, 0, 0,
                               0.f, buf, nullptr, nullptr, 0, nullptr) == ATTN_ERR_NULL,
        "varlen fwd null seqlens");
  CHECK(attn_decode_varlen_fwd(&good, buf, buf, buf, i32, i32, i32, -1, nullptr, nullptr, 0, 0, 0,
                               0.f, buf, nullptr, nullptr, 0, nullptr) != ATTN_OK,
        "varlen fwd negative total_q");
  attn_dense_shape dgood{8, 2, 4, 100, 128, ATTN_FP16};
  CHECK(attn_dense_fwd(&dgood, buf, buf, nullptr, 0, 0.f, buf, nullptr, nullptr, 0, nullptr) ==
            ATTN_ERR_NULL, "dense fwd null v");
  CHECK(attn_dense_fwd(nullptr, buf, buf, buf, 0, 0.f, buf, nullptr, nullptr, 0, nullptr) ==
            ATTN_ERR_NULL, "dense fwd null shape");
  const float* f32 = reinterpret_cast<const float*>(buf);
  CHECK(attn_combine_fwd(0, 1, 1, 1, 8, ATTN_FP16, f32, f32, buf, nullptr, nullptr) == ATTN_ERR_ARG,
        "combine zero splits");
  CHECK(attn_combine_fwd(4, 1, 1, 1, 513, ATTN_FP16, f32, f32, buf, nullptr, nullptr) ==
            ATTN_ERR_UNSUPPORTED, "combine head_dim 513");
  CHECK(attn_combine_fwd(4, 0, 1, 1, 8, ATTN_FP16, f32, f32, buf, nullptr, nullptr) == ATTN_OK,
        "combine empty batch");
  attn_plan last;
  CHECK(valid_status(attn_last_plan(&last)), "last plan status");
  CHECK(attn_last_plan(nullptr) == ATTN_ERR_NULL, "last plan null");

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host API sanitizer run: ok (%d valid decode plans)\n", ok_plans);
  return 0;
}
