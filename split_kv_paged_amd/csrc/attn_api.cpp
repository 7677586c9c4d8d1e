// attn_api.cpp -- the C ABI (include/attn_decode.h): validation, planning,
// launches.  Host code only; the kernels live in *_kernel.hip.
#include "attn_decode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "internal.h"

namespace {

constexpr int kBlockM = 16;         // M tile of the pack rule (MFMA tile height)
constexpr int kBlockN = 128;        // N tile of the "at most 4 blocks" split rule
constexpr int kGranule = 16;        // split ranges are multiples of 16 keys
// Raising a split count to fill the CUs (with the length sum) stops at 16
// splits (one round of partial loads in the combine) and at kFillKeys keys
// per split (a 16-key tile for each of the 8 waves).
constexpr int kFillSplits = 16;
constexpr int kFillKeys = 128;
constexpr int kMaxSplitsRule = 128; // candidate split counts tried by the rule
constexpr int kMaxSplits = 1024;    // largest split count a caller may ask for
constexpr int kDefaultCus = 256;    // one MI355X
constexpr int kRowsPerBlock = 16;   // packed query rows per workgroup (MFMA tile height)
constexpr int kMaxHeadDim = 256;
constexpr int kMaxDevices = 64;

thread_local attn_plan g_last_plan;
thread_local bool g_have_last = false;
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<void*> g_scratch[kMaxDevices];  // device address of each GPU's scratch array

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// lpnh.cn "pack_gqa 与 num_splits" article, section "pack_gqa 怎么选": row
// efficiency (valid rows over rows rounded up to the M tile) with and without
// packing, single-precision quotients, packing when the unpacked one is below
// 0.9 of the packed one (compared in double, as the page's literal is).
bool should_pack_gqa(bool varlen_q, int seqlen_q, int group, int block_m) {
  if (varlen_q) return true;
  const float nopack = float(seqlen_q) / float(round_up(seqlen_q, block_m));
  const int64_t rows = int64_t(seqlen_q) * group;
  const float pack = float(rows) / float(round_up(rows, block_m));
  return nopack < 0.9 * pack;
}

// Same article, section "num_splits 怎么选": one split when the units fill
// 80% of the compute units or the KV spans at most 4 N tiles; otherwise the
// smallest split count whose last-wave efficiency n_waves / ceil(n_waves) is
// within 85% of the best over 1 .. min(128, N tiles).
int num_splits_rule(int64_t total_mblocks, int num_cus, int64_t num_n_blocks) {
  if (total_mblocks >= 0.8 * num_cus) return 1;
  if (num_n_blocks <= 4) return 1;
  const int max_splits = int(num_n_blocks < kMaxSplitsRule ? num_n_blocks : kMaxSplitsRule);
  float eff[kMaxSplitsRule + 1];
  float best = 0.f;
  for (int s = 1; s <= max_splits; ++s) {
    const float n_waves = float(total_mblocks * s) / float(num_cus);
    eff[s] = n_waves / std::ceil(n_waves);
    if (eff[s] > best) best = eff[s];
  }
  for (int s = 1; s <= max_splits; ++s)
    if (eff[s] >= 0.85 * best) return s;
  return 1;
}

// Packed rows one workgroup carries: 16 (one MFMA row block); where the
// kernels exist (16-byte loads at head dims 64 and 128), 32 for units of
// more than 16 rows and 64 beyond 32, so a workgroup reads its KV once for
// all of them.
int rows_per_block(int64_t rows, int head_dim) {
  if (head_dim != 64 && head_dim != 128) return kRowsPerBlock;
  if (rows > 2 * kRowsPerBlock) return 4 * kRowsPerBlock;
  if (rows > kRowsPerBlock) return 2 * kRowsPerBlock;
  return kRowsPerBlock;
}

// Ragged batches (not from the pages; their rule sees only max_seqlen_k).
// Given the sum of the batch's lengths, a compute unit's fair share of the
// job is streams * sum / num_cus keys, streams being the KV passes per
// sequence (head units x row blocks).  In a ragged batch (longest sequence
// over twice the mean) whose longest sequence also exceeds one and a half
// shares, that sequence would outlast the rest of the batch on one
// workgroup, so it is cut into pieces of at most three fifths of a share;
// shorter sequences keep fewer splits (with the length sum the call
// launches only the splits that hold keys, see the compact list).  Uniform
// batches are left to the pages' rule, which already sizes splits by the
// common length.  Returns the split count this asks for (1 when it does not
// apply), at most kMaxSplitsRule.
// Measured on MI355X with the compact list (paged, 8 KV heads, lengths
// log-uniform), us, two shares and two-thirds pieces -> one and a half
// shares and three-fifths pieces: 128 sequences fp16 d 64 (head pairs,
// 1..8192) 46.8 (S 7) -> 45.4 (S 8); 32 bf16 d 128 (1..8192) 24.8 (S 14)
// -> 24.5 (S 15); 128 bf16 d 128 (1..8192; the longest 1.76 shares) 126.0
// (S 1) -> 100.7 (S 3); 64 up to 4096 and 256 fp16 d 64 up to 4096: the same
// S and time.  Earlier, on a slower kernel, half-share pieces had lost to
// two-thirds ones (128 sequences d 64 54.1 -> 53.6 us; 32 sequences d 128
// 43.0 -> 38.1; 64 up to 4096 31.4 -> 30.0).
int ragged_splits(int64_t batch, int64_t streams, int64_t sum_seqlen_k, int64_t max_seqlen_k,
                  int num_cus) {
  if (sum_seqlen_k <= 0 || streams <= 0 || batch <= 0) return 1;
  const double mean = double(sum_seqlen_k) / double(batch);
  const double share = double(streams) * double(sum_seqlen_k) / double(num_cus);
  if (double(max_seqlen_k) <= 2.0 * mean || double(max_seqlen_k) <= 1.5 * share) return 1;
  const double s = std::ceil(5.0 * double(max_seqlen_k) / (3.0 * share));
  return s >= kMaxSplitsRule ? kMaxSplitsRule : int(s);
}

// Diagnostic kernel id: 10000 (16-byte loads), 20000 (16-byte loads with a
// column mask: head_dim a multiple of 8), 30000 (element loads: any other
// head_dim) or 40000 (head groups) + 1000 if paged + the tile head dim
// (32/64/128/256).  A forward call whose split kernel also wrote the
// appended keys records kAppendedInKernel more.
constexpr int kAppendedInKernel = 100000;
int kernel_id(int head_dim, bool paged, bool grouped) {
  if (grouped) return 40000 + 1000 + 128;
  const bool exact = head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256;
  const int loads = exact ? 10000 : head_dim % 8 == 0 ? 20000 : 30000;
  const int tile = head_dim <= 32 ? 32 : head_dim <= 64 ? 64 : head_dim <= 128 ? 128 : 256;
  return loads + (paged ? 1000 : 0) + tile;
}

// Shared planner.  `dense` always packs (the dense API has no pack switch).
attn_status make_plan(int64_t batch, int q_len, int hq, int hkv, int head_dim, int64_t max_seqlen_k,
                      int num_splits, int pack_gqa, int num_cus, bool dense, attn_plan* out,
                      bool varlen = false, int64_t sum_seqlen_k = 0) {
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
  if (pack_gqa < -1 || pack_gqa > 1) return ATTN_ERR_ARG;
  if (num_cus < 0) return ATTN_ERR_ARG;
  if (num_cus == 0) num_cus = kDefaultCus;
  const int group = hq / hkv;
  bool pack;
  if (dense)
    pack = true;
  else if (pack_gqa < 0)
    pack = should_pack_gqa(varlen, q_len, group, kBlockM);
  else
    pack = pack_gqa == 1;
  // Head groups (paged, head_dim 64 or 32, packed, R = 128 / head_dim
  // dividing the KV heads, all R heads' rows within one 16-row block, and
  // the length sum given): R adjacent KV heads are one 128-wide key row in
  // the cache, so a workgroup reads 256 contiguous bytes per key instead of
  // 128 or 64, and 1/R as many workgroups move the same bytes.  Measured on
  // MI355X: fp16 GQA-4 d 64, 64 sequences of 2048 keys, 53.7 -> 46.8 us;
  // the ragged 128-sequence GQA-2 d-64 batch with its length sum, 54.0 ->
  // 48.7 us; bf16 GQA-4 d 32, 32 sequences of 4096 keys, 46.4 -> 28.0 us
  // (S 4: the quads leave 64 units, so the rule splits them).
  // A group multiplies the bytes of its longest sequence's workgroup, so
  // without the sum (no ragged split) the ragged batch went from 76.4 to
  // 95.9 us: groups wait for the sum, and plans without it stay the pages'
  // rule.
  // With one query head per KV head (G = 1) packing changes no row, so the
  // pack rule's "off" does not keep such heads from a group (fp16 MHA d 64,
  // 32 sequences of 2048 keys: 96.7 -> 87.9 us).
  const int per_row = head_dim == 64 ? 2 : head_dim == 32 ? 4 : 1;
  const bool grouped = !dense && sum_seqlen_k > 0 && per_row > 1 && hkv % per_row == 0 &&
                       (pack || (group == 1 && pack_gqa != 0)) &&
                       int64_t(q_len) * per_row * group <= kBlockM;
  if (grouped) pack = true;
  const int64_t hr = grouped ? per_row : 1;  // KV heads per unit
  int splits = num_splits;
  if (splits == 0) {
    const int64_t heads = grouped ? hkv / hr : pack ? hkv : hq;
    const int64_t rows =
        grouped ? int64_t(q_len) * hr * group : pack ? int64_t(q_len) * group : q_len;
    // The rule's units are workgroups (the page's CTAs): a workgroup carries
    // 16, 32 or 64 packed rows, so the unit count divides the rows by that,
    // not by the 16-row MFMA tile the pack rule uses.  Measured on MI355X
    // (bf16 GQA-8, q_len 8, 4 sequences of 4096 keys, 64-row workgroups):
    // 51.1 us at the S = 4 that 16-row units give, 44.8 at the S = 16 that
    // workgroup units give.
    const int64_t rpb0 = rows_per_block(rows, grouped ? 128 : head_dim);
    const int64_t total = batch * heads * ceil_div(rows, rpb0);
    splits = num_splits_rule(total, num_cus, ceil_div(max_seqlen_k, kBlockN));
    splits = std::max(splits, ragged_splits(batch, heads * ceil_div(rows, rpb0), sum_seqlen_k,
                                            max_seqlen_k, num_cus));
    // With the length sum (a caller that plans on the host), a split count
    // that leaves compute units idle is raised until the workgroups fill
    // them: the rule's 85% slack spares separate combine launches, and the
    // fused combine here costs about the same at any count up to 16 (one
    // round of loads), as long as each split keeps a tile for each of the
    // 8 waves.  Measured on MI355X (bf16 GQA-8, 4 sequences of 16384 keys,
    // 16 units): the rule's S = 14 (224 workgroups) 26.05-26.09 us, S = 16
    // (256) 25.51-25.55.
    if (sum_seqlen_k > 0 && splits > 1 && total * splits < num_cus) {
      const int64_t fill = std::min<int64_t>(
          {int64_t(num_cus) / total, int64_t(kFillSplits), max_seqlen_k / kFillKeys});
      if (fill > splits) splits = int(fill);
    }
  }
  if (splits > 1) pack = true;  // same article, section "常见坑点"

  const int64_t rows_per_unit =
      grouped ? int64_t(q_len) * hr * group : pack ? int64_t(q_len) * group : q_len;
  const int rpb = rows_per_block(rows_per_unit, grouped ? 128 : head_dim);
  const int64_t row_blocks = ceil_div(rows_per_unit, rpb);
  const int64_t unit_heads = grouped ? hkv / hr : pack ? hkv : hq;
  const int64_t units = batch * unit_heads * row_blocks;
  int64_t grid = units * splits;
  if (grid > INT32_MAX || rows_per_unit > INT32_MAX) return ATTN_ERR_SHAPE;
  const int64_t nrows = batch * q_len * int64_t(hq);
  // one split length for the batch: whole 16-key granules, S of them cover max_seqlen_k
  const int64_t split_keys =
      int64_t(kGranule) * std::max<int64_t>(1, ceil_div(ceil_div(max_seqlen_k, kGranule), splits));
  if (split_keys > INT32_MAX) return ATTN_ERR_SHAPE;
  // Compact list (paged splits with a length sum): sequence b needs
  // ceil(L_b / C) - 1 <= floor(L_b / C) splits past the first, and the sum
  // of floors is at most floor(sum / C), so that many extra workgroups per
  // head unit and row block give every extra split one workgroup.  Used
  // when it launches fewer workgroups than the split-major grid.
  int64_t extra = 0;
  if (!dense && splits > 1 && sum_seqlen_k > 0 && batch <= skv::kMaxOrderBatch) {
    const int64_t bound = std::max<int64_t>(1, sum_seqlen_k / split_keys * unit_heads * row_blocks);
    if (units + bound < grid) {
      extra = bound;
      grid = units + extra;
    }
  }
  int64_t ws = 0;
  if (splits > 1) {
    // the fused combine addresses the partials with 32-bit byte offsets
    if (int64_t(splits) * nrows * head_dim * 4 >= (int64_t(1) << 32)) return ATTN_ERR_UNSUPPORTED;
    ws = round_up(int64_t(splits) * nrows * head_dim * 4, 256) +
         round_up(int64_t(splits) * nrows * 4, 256) +
         round_up(units * 4 * skv::kCounterStride, 256);
  }

  std::memset(out, 0, sizeof(*out));
  out->num_splits = splits;
  out->pack_gqa = pack ? 1 : 0;
  out->rows_per_unit = int(rows_per_unit);
  out->rows_per_block = rpb;
  out->row_blocks = int(row_blocks);
  out->units = int(units > INT32_MAX ? INT32_MAX : units);
  out->grid = int(grid);
  out->split_granule = kGranule;
  out->num_cus = num_cus;
  out->combine = splits > 1 ? 2 : 0;
  out->kernel = kernel_id(head_dim, !dense, grouped);
  out->heads_per_row = int(hr);
  out->split_keys = int(split_keys);
  out->extra_blocks = int(extra);
  out->workspace_bytes = ws;
  return ATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

attn_status check_decode_shape(const attn_decode_shape* s) {
  if (!s) return ATTN_ERR_NULL;
  if (s->batch < 0 || s->q_len <= 0 || s->num_heads_q <= 0 || s->num_heads_kv <= 0 ||
      s->head_dim <= 0 || s->page_size <= 0 || s->max_pages_per_seq <= 0 || s->max_seqlen_k < 0)
    return ATTN_ERR_SHAPE;
  if (s->num_heads_q % s->num_heads_kv != 0) return ATTN_ERR_SHAPE;
  if (int64_t(s->max_seqlen_k) > int64_t(s->max_pages_per_seq) * s->page_size) return ATTN_ERR_SHAPE;
  if (s->sum_seqlen_k < 0 || s->sum_seqlen_k > int64_t(s->batch) * s->max_seqlen_k)
    return ATTN_ERR_SHAPE;
  if (s->dtype != ATTN_FP16 && s->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (s->head_dim > kMaxHeadDim) return ATTN_ERR_UNSUPPORTED;
  if (s->page_size % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status check_dense_shape(const attn_dense_shape* s) {
  if (!s) return ATTN_ERR_NULL;
  if (s->num_heads_q <= 0 || s->num_heads_kv <= 0 || s->q_len <= 0 || s->kv_len < 0 ||
      s->head_dim <= 0)
    return ATTN_ERR_SHAPE;
  if (s->num_heads_q % s->num_heads_kv != 0) return ATTN_ERR_SHAPE;
  if (s->dtype != ATTN_FP16 && s->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (s->head_dim > kMaxHeadDim) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status check_scale(float scale) {
  if (std::isnan(scale) || std::isinf(scale)) return ATTN_ERR_ARG;
  return ATTN_OK;
}

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 0;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

attn_status check_workspace(const attn_plan& plan, void* ws, size_t ws_bytes) {
  if (plan.workspace_bytes == 0) return ATTN_OK;
  if (!ws || ws_bytes < size_t(plan.workspace_bytes)) return ATTN_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Where a split call keeps its float32 partials and arrival counters.
struct WsView {
  float* o_part = nullptr;
  float* lse_part = nullptr;
  int* counters = nullptr;
};

// The caller's workspace: partial outputs, partial LSEs, then the counters,
// each at a 256-byte boundary (include/attn_decode.h).
WsView caller_workspace(const attn_plan& plan, int64_t nrows, int head_dim, void* ws) {
  WsView v;
  if (plan.num_splits <= 1) return v;
  const int64_t o_bytes = round_up(int64_t(plan.num_splits) * nrows * head_dim * 4, 256);
  const int64_t l_bytes = round_up(int64_t(plan.num_splits) * nrows * 4, 256);
  v.o_part = static_cast<float*>(ws);
  v.lse_part = reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes);
  v.counters = reinterpret_cast<int*>(static_cast<char*>(ws) + o_bytes + l_bytes);
  return v;
}

// Launch the split kernel (which merges the splits itself when S > 1).
attn_status run(const attn_plan& plan, skv::SplitParams prm, bool paged, int dtype, int head_dim,
                void* out, float* lse, const WsView& ws, hipStream_t stream,
                int64_t max_seqlen_k = 0, int64_t sum_seqlen_k = 0,
                const skv::AppendParams* append = nullptr) {
  const int S = plan.num_splits;
  prm.num_splits = S;
  prm.split_keys = plan.split_keys;
  prm.rows = plan.rows_per_unit;
  prm.row_blocks = plan.row_blocks;
  prm.nrb = plan.rows_per_block / kRowsPerBlock;
  if (plan.heads_per_row > 1) {  // a unit is a group of adjacent KV heads
    prm.head_group = plan.heads_per_row;
    prm.hkv /= plan.heads_per_row;
    prm.group *= plan.heads_per_row;
  }
  prm.heads_per_unit = plan.pack_gqa ? prm.group : 1;
  prm.unit_heads = plan.pack_gqa ? prm.hkv : prm.hq;
  prm.head_dim = head_dim;
  prm.out = out;
  prm.lse = lse;
  prm.o_part = ws.o_part;
  prm.lse_part = ws.lse_part;
  prm.counters = ws.counters;
  // Paged calls whose grid needs more than one round run the first split's
  // sequences longest first (ranked inside its workgroups).  max_seqlen_k is
  // only a bound; when the length sum is given, a batch of short sequences
  // (mean under kMinRankMean keys) is not ranked either, since each
  // workgroup's round trip for the lengths then outweighs the order.
  prm.by_length = paged && prm.batch <= skv::kMaxRankBatch && plan.grid > plan.num_cus &&
                  max_seqlen_k >= skv::kMinRankKeys &&
                  (sum_seqlen_k <= 0 || sum_seqlen_k >= int64_t(skv::kMinRankMean) * prm.batch);
  prm.extra_blocks = paged ? plan.extra_blocks : 0;
  bool in_kernel = false;
  if (skv::launch_split_mfma(dtype, paged, prm, plan.grid, stream, append, &in_kernel) !=
      hipSuccess)
    return ATTN_ERR_HIP;
  g_last_plan = plan;
  if (in_kernel) g_last_plan.kernel += kAppendedInKernel;
  g_have_last = true;
  return ATTN_OK;
}

// The scratch of attn_decode_fwd_noalloc: counters at its start (a fixed
// place, so they stay zero from call to call), then the partials.  The
// device address is looked up once per device, with that device current.
attn_status scratch_workspace(const attn_plan& plan, int64_t nrows, int head_dim, WsView* v) {
  *v = WsView{};
  if (plan.num_splits <= 1) return ATTN_OK;
  const int64_t c_bytes = int64_t(plan.units) * 4 * skv::kCounterStride;
  const int64_t o_bytes = round_up(int64_t(plan.num_splits) * nrows * head_dim * 4, 256);
  const int64_t l_bytes = round_up(int64_t(plan.num_splits) * nrows * 4, 256);
  if (c_bytes > skv::kScratchCounterBytes ||
      skv::kScratchCounterBytes + o_bytes + l_bytes > skv::kScratchBytes)
    return ATTN_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  void* base = g_scratch[dev].load(std::memory_order_acquire);
  if (!base) {
    if (skv::scratch_device_address(&base) != hipSuccess || !base) return ATTN_ERR_HIP;
    g_scratch[dev].store(base, std::memory_order_release);
  }
  char* b = static_cast<char*>(base);
  v->counters = reinterpret_cast<int*>(b);
  v->o_part = reinterpret_cast<float*>(b + skv::kScratchCounterBytes);
  v->lse_part = reinterpret_cast<float*>(b + skv::kScratchCounterBytes + o_bytes);
  return ATTN_OK;
}

// Paged forward shared by attn_decode_fwd and attn_decode_kvcache_fwd.
attn_status decode_common(const attn_decode_shape* shape, const void* q, void* k_cache,
                          void* v_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                          const void* k_new, const void* v_new, int new_len, int causal,
                          int num_splits, int pack_gqa, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const int32_t* cu_q = nullptr, int total_q = 0,
                          bool use_scratch = false) {
  attn_status st = check_decode_shape(shape);
  if (st != ATTN_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !cache_seqlens || !out) return ATTN_ERR_NULL;
  if (new_len < 0 || (causal != 0 && causal != 1)) return ATTN_ERR_ARG;
  if (new_len > 0 && (!k_new || !v_new)) return ATTN_ERR_NULL;
  if (new_len > 0 && (!aligned(k_new, 16) || !aligned(v_new, 16))) return ATTN_ERR_ALIGN;
  if (cu_q) {  // varlen queries: packed, at most q_len (= max_seqlen_q) per sequence
    if (!aligned(cu_q, 4)) return ATTN_ERR_ALIGN;
    if (total_q < 0 || int64_t(total_q) > int64_t(shape->batch) * shape->q_len)
      return ATTN_ERR_SHAPE;
    if (pack_gqa == 0) return ATTN_ERR_ARG;
    pack_gqa = 1;
  }
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(cache_seqlens, 4) || (lse && !aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != ATTN_OK) return st;
  attn_plan plan;
  const int cus = device_cus();
  if (cus <= 0) return ATTN_ERR_HIP;
  st = make_plan(shape->batch, shape->q_len, shape->num_heads_q, shape->num_heads_kv,
                 shape->head_dim, shape->max_seqlen_k, num_splits, pack_gqa, cus, false, &plan,
                 cu_q != nullptr, shape->sum_seqlen_k);
  if (st != ATTN_OK) return st;
  const int64_t nrows = int64_t(shape->batch) * shape->q_len * shape->num_heads_q;
  WsView wsv;
  if (use_scratch) {
    if ((st = scratch_workspace(plan, nrows, shape->head_dim, &wsv)) != ATTN_OK) return st;
  } else {
    if ((st = check_workspace(plan, workspace, workspace_bytes)) != ATTN_OK) return st;
    wsv = caller_workspace(plan, nrows, shape->head_dim, workspace);
  }
  if (shape->batch == 0) {
    g_last_plan = plan;
    g_have_last = true;
    return ATTN_OK;
  }
  const int D = shape->head_dim;
  skv::SplitParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.batch = shape->batch;
  p.q_len = shape->q_len;
  p.hq = shape->num_heads_q;
  p.hkv = shape->num_heads_kv;
  p.group = p.hq / p.hkv;
  p.page_size = shape->page_size;
  p.max_pages = shape->max_pages_per_seq;
  p.kv_len = 0;
  p.nrows = shape->batch * shape->q_len * shape->num_heads_q;
  p.n_si = shape->num_heads_q;
  p.n_sh = 1;
  p.seq_add = new_len;
  p.causal = causal;
  p.cu_q = cu_q;
  p.total_q = total_q;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(D));
  p.scale_log2 = scale * 1.4426950408889634074f;
  // The new keys go into the cache before attention reads them: written by
  // the split kernel itself where it can, else by the append kernel first on
  // the same stream.
  skv::AppendParams a{};
  if (new_len > 0) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seqlens = cache_seqlens;
    a.batch = shape->batch;
    a.new_len = new_len;
    a.hkv = shape->num_heads_kv;
    a.head_dim = D;
    a.page_size = shape->page_size;
    a.max_pages = shape->max_pages_per_seq;
    a.num_cus = cus;
  }
  return run(plan, p, true, shape->dtype, D, out, lse, wsv, static_cast<hipStream_t>(stream),
             shape->max_seqlen_k, shape->sum_seqlen_k, new_len > 0 ? &a : nullptr);
}

}  // namespace

extern "C" {

attn_status attn_decode_plan(const attn_decode_shape* shape, int num_splits, int pack_gqa,
                             int num_cus, attn_plan* plan) {
  if (!plan) return ATTN_ERR_NULL;
  attn_status st = check_decode_shape(shape);
  if (st != ATTN_OK) return st;
  return make_plan(shape->batch, shape->q_len, shape->num_heads_q, shape->num_heads_kv,
                   shape->head_dim, shape->max_seqlen_k, num_splits, pack_gqa, num_cus, false,
                   plan, false, shape->sum_seqlen_k);
}

attn_status attn_dense_plan(const attn_dense_shape* shape, int num_splits, int num_cus,
                            attn_plan* plan) {
  if (!plan) return ATTN_ERR_NULL;
  attn_status st = check_dense_shape(shape);
  if (st != ATTN_OK) return st;
  return make_plan(1, shape->q_len, shape->num_heads_q, shape->num_heads_kv, shape->head_dim,
                   shape->kv_len, num_splits, -1, num_cus, true, plan);
}

attn_status attn_decode_fwd(const attn_decode_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* cache_seqlens, int num_splits, int pack_gqa,
                            float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_common(shape, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                       block_table, cache_seqlens, nullptr, nullptr, 0, 0, num_splits, pack_gqa,
                       softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_decode_fwd_noalloc(const attn_decode_shape* shape, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* cache_seqlens,
                                    int num_splits, int pack_gqa, float softmax_scale, void* out,
                                    float* lse, void* stream) {
  return decode_common(shape, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                       block_table, cache_seqlens, nullptr, nullptr, 0, 0, num_splits, pack_gqa,
                       softmax_scale, out, lse, nullptr, 0, stream, nullptr, 0, true);
}

attn_status attn_decode_varlen_fwd(const attn_decode_shape* shape, const void* q, void* k_cache,
                                   void* v_cache, const int32_t* block_table,
                                   const int32_t* cache_seqlens, const int32_t* cu_seqlens_q,
                                   int total_q, const void* k_new, const void* v_new, int new_len,
                                   int causal, int num_splits, float softmax_scale, void* out,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!cu_seqlens_q) return ATTN_ERR_NULL;
  return decode_common(shape, q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new,
                       new_len, causal, num_splits, -1, softmax_scale, out, lse, workspace,
                       workspace_bytes, stream, cu_seqlens_q, total_q);
}

attn_status attn_decode_kvcache_fwd(const attn_decode_shape* shape, const void* q, void* k_cache,
                                    void* v_cache, const int32_t* block_table,
                                    const int32_t* cache_seqlens, const void* k_new,
                                    const void* v_new, int new_len, int causal, int num_splits,
                                    int pack_gqa, float softmax_scale, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(shape, q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new,
                       new_len, causal, num_splits, pack_gqa, softmax_scale, out, lse, workspace,
                       workspace_bytes, stream);
}

attn_status attn_dense_fwd(const attn_dense_shape* shape, const void* q, const void* k,
                           const void* v, int num_splits, float softmax_scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_dense_shape(shape);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != ATTN_OK) return st;
  attn_plan plan;
  const int cus = device_cus();
  if (cus <= 0) return ATTN_ERR_HIP;
  st = make_plan(1, shape->q_len, shape->num_heads_q, shape->num_heads_kv, shape->head_dim,
                 shape->kv_len, num_splits, -1, cus, true, &plan);
  if (st != ATTN_OK) return st;
  if ((st = check_workspace(plan, workspace, workspace_bytes)) != ATTN_OK) return st;
  const int D = shape->head_dim;
  skv::SplitParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.batch = 1;
  p.q_len = shape->q_len;
  p.hq = shape->num_heads_q;
  p.hkv = shape->num_heads_kv;
  p.group = p.hq / p.hkv;
  p.page_size = 16;
  p.max_pages = 0;
  p.kv_len = shape->kv_len;
  p.nrows = shape->num_heads_q * shape->q_len;
  p.n_si = 1;
  p.n_sh = shape->q_len;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(D));
  p.scale_log2 = scale * 1.4426950408889634074f;
  return run(plan, p, false, shape->dtype, D, out, lse,
             caller_workspace(plan, int64_t(shape->num_heads_q) * shape->q_len, D, workspace),
             static_cast<hipStream_t>(stream));
}

attn_status attn_combine_fwd(int num_splits, int batch, int q_len, int num_heads, int head_dim,
                             int dtype, const float* o_part, const float* lse_part, void* out,
                             float* lse, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
  if (batch < 0 || q_len <= 0 || num_heads <= 0 || head_dim <= 0) return ATTN_ERR_SHAPE;
  if (head_dim > 512) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_FP16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!o_part || !lse_part || !out) return ATTN_ERR_NULL;
  if (!aligned(o_part, 4) || !aligned(lse_part, 4) || !aligned(out, 2) || (lse && !aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  const int64_t nrows = int64_t(batch) * q_len * num_heads;
  if (nrows > INT32_MAX / 4) return ATTN_ERR_SHAPE;
  if (nrows == 0) return ATTN_OK;
  skv::CombineParams c{};
  c.o_part = o_part;
  c.lse_part = lse_part;
  c.out = out;
  c.lse = lse;
  c.num_splits = num_splits;
  c.nrows = int(nrows);
  c.head_dim = head_dim;
  c.q_len = q_len;
  c.heads = num_heads;
  if (skv::launch_combine(dtype, c, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status attn_check_kvcache_inputs(const attn_decode_shape* shape,
                                      const int32_t* block_table_host,
                                      const int32_t* cache_seqlens_host, int64_t num_pages,
                                      int new_len, int32_t* bad_batch) {
  attn_status st = check_decode_shape(shape);
  if (st != ATTN_OK) return st;
  if (new_len < 0) return ATTN_ERR_ARG;
  if (!block_table_host || !cache_seqlens_host) return ATTN_ERR_NULL;
  for (int b = 0; b < shape->batch; ++b) {
    // keys the call covers: the cached ones plus those it appends
    const int64_t L = int64_t(cache_seqlens_host[b]) + new_len;
    bool bad = cache_seqlens_host[b] < 0 || L > shape->max_seqlen_k;
    const int64_t used = bad ? 0 : ceil_div(L, shape->page_size);
    for (int64_t t = 0; t < used && !bad; ++t) {
      const int32_t pg = block_table_host[int64_t(b) * shape->max_pages_per_seq + t];
      bad = pg < 0 || pg >= num_pages;
    }
    if (bad) {
      if (bad_batch) *bad_batch = b;
      return ATTN_ERR_DATA;
    }
  }
  return ATTN_OK;
}

attn_status attn_check_paged_inputs(const attn_decode_shape* shape,
                                    const int32_t* block_table_host,
                                    const int32_t* cache_seqlens_host, int64_t num_pages,
                                    int32_t* bad_batch) {
  return attn_check_kvcache_inputs(shape, block_table_host, cache_seqlens_host, num_pages, 0,
                                   bad_batch);
}

attn_status attn_last_plan(attn_plan* plan) {
  if (!plan) return ATTN_ERR_NULL;
  if (!g_have_last) return ATTN_ERR_ARG;
  *plan = g_last_plan;
  return ATTN_OK;
}

const char* attn_status_str(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "inconsistent sizes";
    case ATTN_ERR_UNSUPPORTED: return "outside the supported envelope";
    case ATTN_ERR_ARG: return "argument out of range";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_DATA: return "block_table or cache_seqlens entry out of range";
  }
  return "unknown status";
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
