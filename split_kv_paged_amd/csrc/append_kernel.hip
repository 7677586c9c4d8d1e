// append_kernel.hip -- write new keys and values into the paged KV cache.
//
// The lpnh.cn "pack_gqa 与 num_splits" article's example call passes new
// keys and values with the cache (section "num_splits 怎么选"); they take
// key positions cache_seqlens[b] .. cache_seqlens[b] + new_len - 1 of each
// sequence, in the pages the block table maps there (PA_BBND layout of the
// MixedQuantSparseFlashMla article, section 参数说明), before attention
// reads the cache.  One workgroup per (sequence, new key) copies the Hkv
// rows of K and V, in 16-byte chunks where the row length allows.
// The split kernel writes up to kMaxFusedNew keys a sequence itself where it
// can (split_mfma.hip); this kernel covers the other calls.
#include "internal.h"

namespace skv {
namespace {

__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  const int b = blockIdx.x / p.new_len;
  const int t = blockIdx.x % p.new_len;
  const int pos = p.seqlens[b] + t;
  const int slot_page = pos / p.page_size;
  if (pos < 0 || slot_page >= p.max_pages) return;  // outside the table: nothing to write
  const long page = p.block_table[(long)b * p.max_pages + slot_page];
  const long dst = ((page * p.page_size + pos % p.page_size) * p.hkv) * p.head_dim;
  const long src = ((long)b * p.new_len + t) * p.hkv * p.head_dim;
  const int n = p.hkv * p.head_dim;
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + src;
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + src;
  uint16_t* kc = static_cast<uint16_t*>(p.k_cache) + dst;
  uint16_t* vc = static_cast<uint16_t*>(p.v_cache) + dst;
  if (n % 8 == 0) {
    // 16-byte chunks: the rows start 16-byte aligned (aligned bases, rows of
    // a multiple of 8 elements); each thread loads before it stores, so its
    // loads are in flight together
    const uint4* __restrict__ kn4 = reinterpret_cast<const uint4*>(kn);
    const uint4* __restrict__ vn4 = reinterpret_cast<const uint4*>(vn);
    uint4* __restrict__ kc4 = reinterpret_cast<uint4*>(kc);
    uint4* __restrict__ vc4 = reinterpret_cast<uint4*>(vc);
    for (int e = threadIdx.x; e < n / 8; e += blockDim.x) {
      const uint4 kv = kn4[e], vv = vn4[e];
      kc4[e] = kv;
      vc4[e] = vv;
    }
    return;
  }
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const uint16_t kv = kn[e], vv = vn[e];
    kc[e] = kv;
    vc[e] = vv;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  const long grid = (long)p.batch * p.new_len;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(grid)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace skv
