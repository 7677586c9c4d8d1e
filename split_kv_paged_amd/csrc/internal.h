// internal.h -- launch parameters shared by the host API and the HIP kernels.
// Not part of the public ABI (include/attn_decode.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

// Division of a non-negative 32-bit integer by a divisor fixed for the
// launch, as a multiply-high, a subtract and two shifts (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994:
// the round-up method, exact for every 32-bit dividend):
//   l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
//   t = (n * m) >> 32, n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0).
struct FastDiv {
  uint32_t m;
  int s1, s2;
};

// One split-kernel launch.  Rows: a "row" is one (b, i, hq) query vector.
//   first query of sequence b: qb = cu_q ? cu_q[b] : b * q_len
//   row index n(b, i, hq) = (qb + i) * n_si + hq * n_sh
//   q / out element offset = n * head_dim          (all layouts)
//   lse index              = (b * Hq + hq) * q_len + i, varlen: hq * total_q + qb + i
// KV addressing of key t, KV head h:
//   paged: page = block_table[b * max_pages + t / page_size],
//          elem = ((page * page_size + t % page_size) * Hkv + h) * head_dim
//   dense: elem = (h * kv_len + t) * head_dim
struct SplitParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;  // paged only
  const int32_t* seqlens;      // paged only
  void* out;                   // final output (num_splits == 1)
  float* lse;                  // final LSE, may be null (num_splits == 1)
  float* o_part;               // [S][nrows][D] (num_splits > 1)
  float* lse_part;             // [S][nrows]    (num_splits > 1)
  int* counters;               // [units] arrival counters (kCounterStride apart), zero between
                               // calls (fused combine)
  int batch, q_len, hq, hkv, group;  // group = Hq / Hkv
  int page_size, max_pages, kv_len;
  int head_dim;        // elements per row of q, k, v and out
  int num_splits;
  int split_keys;      // keys per split (multiple of 16); split s = [s*C, (s+1)*C)
  int rows;            // valid rows per unit (q_len * heads_per_unit)
  int row_blocks;      // ceil(rows / (16 * nrb))
  int nrb;             // 16-row blocks per workgroup (1, 2 or 4)
  int heads_per_unit;  // group (packed) or 1
  int unit_heads;      // Hkv (packed) or Hq
  int nrows;           // batch * q_len * Hq
  int n_si, n_sh;
  float scale_log2;    // softmax scale * log2(e)
  int by_length;       // paged: run sequences longest first (see kMaxRankBatch)
  int head_group;      // paged, head_dim 64 or 32, > 1: a unit is head_group adjacent KV
                       // heads read as one 128-wide key row (hkv, group and
                       // heads_per_unit count such groups)
  int extra_blocks;    // paged, 0: split-major grid of units * num_splits workgroups;
                       // > 0: extra_blocks workgroups take the splits >= 1 from a
                       // device-built list, then one workgroup per unit runs split 0
                       // (batch <= kMaxOrderBatch)
  int seq_add;         // paged: keys attended = seqlens[b] + seq_add (appended keys)
  int causal;          // query i of q_len sees keys j <= L - q_len + i
  const int32_t* cu_q; // varlen: queries of sequence b are rows cu_q[b] .. cu_q[b+1]-1
  int total_q;         // varlen: cu_q[batch]; lse is [Hq, total_q]
  // Filled by launch_split_mfma from the fields above: division by
  // batch * unit_heads * row_blocks, unit_heads, group, heads_per_unit,
  // page_size, split_keys and (head groups) the query heads per KV head,
  // heads_per_unit * head_dim / 128.
  FastDiv fd_units, fd_unit_heads, fd_group, fd_hpu, fd_page, fd_split_keys, fd_gq;
  // Set by launch_split_mfma for an appending launch (paged, direct-to-LDS
  // tiles), else null: the seq_add keys [batch, seq_add, Hkv, head_dim] that
  // the split kernel itself writes into the cache.
  const void* k_new;
  const void* v_new;
};

// Append new_len keys per sequence to the paged cache (before attention):
// k_new/v_new [batch, new_len, Hkv, head_dim] go to key positions
// seqlens[b] .. seqlens[b] + new_len - 1.
// At most this many keys per sequence are appended by the split kernel
// itself; longer appends (and the register-ring kernels, and varlen calls)
// run the append kernel first.
constexpr int kMaxFusedNew = 4;
struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* seqlens;
  int batch, new_len, hkv, head_dim, page_size, max_pages;
  int num_cus;  // of the device (whether the split kernel's appending copy fits)
};
hipError_t launch_append(const AppendParams& p, hipStream_t s);

// Arrival counters of the fused combine sit one per 128-byte line: the
// atomics of different units then never queue on one line.
constexpr int kCounterStride = 32;  // int32 elements between two units' counters
// Library-held scratch of attn_decode_fwd_noalloc (scratch.hip): arrival
// counters first (kScratchCounterBytes, zero between calls: the kernel
// rearms them), then the float32 partial outputs and LSEs.
constexpr long kScratchBytes = 16l << 20;
constexpr long kScratchCounterBytes = 512l << 10;  // 4096 units at kCounterStride
// Device address of this device's scratch (hipGetSymbolAddress; call with the
// device current).
hipError_t scratch_device_address(void** ptr);
constexpr int kMaxOrderBatch = 1024;  // largest batch of the compact split list (its LDS list)
// Split-0 workgroups rank the sequences by length (longest first) for
// batches of at most kMaxRankBatch sequences whose longest has at least
// kMinRankKeys keys.  Each workgroup pays a round trip for the lengths and
// an O(batch^2 / threads) count, which only pays where the order matters.
// Measured on MI355X (paged, 8 KV heads; ranked / unranked, us): 128
// sequences of 100..300 keys 26.3 / 24.2 and of 500..1500 keys 88.2 / 94.9;
// 128 ragged sequences (1..8192 keys) 75.0 / 91.4, with their length sum
// 48.7 / 57.7; 64 ragged ones (1..4096) 29.7 / 35.8; 256 ragged ones with
// their sum 97.9 / 106.5; 256 of 100..300 keys 64.8 / 43.0; 512 ragged ones
// (1..4096) 189 / 125.
constexpr int kMaxRankBatch = 256;
constexpr int kMinRankKeys = 1024;
constexpr int kMinRankMean = 256;  // with the length sum: mean keys per sequence to rank
static_assert(kMaxRankBatch % 16 == 0 && kMaxRankBatch <= kMaxOrderBatch, "rank list size");

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse;          // may be null
  int num_splits;
  int nrows;
  int head_dim;
  // row n = (b * q_len + i) * heads + h  ->  lse index (b * heads + h) * q_len + i
  int q_len, heads;
};

// Split kernel (split_mfma.hip): 16 packed rows per workgroup, fused
// combine when num_splits > 1; p.head_dim in [1, 256].
// append (may be null): keys to write into the paged cache before attention
// reads it, either by the split kernel itself (then *in_kernel = true) or by
// the append kernel first.
hipError_t launch_split_mfma(int dtype, bool paged, const SplitParams& p, int grid,
                             hipStream_t s, const AppendParams* append = nullptr,
                             bool* in_kernel = nullptr);
hipError_t launch_combine(int dtype, const CombineParams& p, hipStream_t s);

}  // namespace skv
