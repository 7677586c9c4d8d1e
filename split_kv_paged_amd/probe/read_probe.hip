// read_probe.hip -- read-only bandwidth probes (include/attn_probe.h).
//
// Two kernels that read KV bytes and only fold them into checksums: a plain
// grid-stride stream over contiguous memory, and the decode kernel's page
// walk (one workgroup of 8 waves per (sequence, KV head), 16-key tiles
// dealt round-robin to the waves, page ids from the block table 64 tiles at
// a time).  Their launch times are the empirical ceiling for a call that
// moves the same bytes.  All loads are 16-byte and non-temporal, as in the
// decode kernel.
#include "attn_probe.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves

__device__ __forceinline__ u32x4_t ld_nt(const u32x4_t* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ uint32_t words(u32x4_t v) { return (v.x + v.y) + (v.z + v.w); }

// Sum of s over the workgroup (every thread gets it).
__device__ __forceinline__ uint32_t block_sum(uint32_t s) {
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) atomicAdd(&red, s);
  __syncthreads();
  return red;
}

// a[0, na) then b[0, nb) in 16-byte units; four loads in flight per thread.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* a, long na,
                                                               const u32x4_t* b, long nb,
                                                               uint32_t* sums) {
  const long n = na + nb;
  const long stride = (long)gridDim.x * kThreads;
  long i = (long)blockIdx.x * kThreads + threadIdx.x;
  auto at = [&](long j) { return j < na ? a + j : b + (j - na); };
  uint32_t s = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t v0 = ld_nt(at(i));
    const u32x4_t v1 = ld_nt(at(i + stride));
    const u32x4_t v2 = ld_nt(at(i + 2 * stride));
    const u32x4_t v3 = ld_nt(at(i + 3 * stride));
    s += (words(v0) + words(v1)) + (words(v2) + words(v3));
  }
  for (; i < n; i += stride) s += words(ld_nt(at(i)));
  const uint32_t t = block_sum(s);
  if (threadIdx.x == 0) sums[blockIdx.x] = t;
}

struct PageProbe {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* seqlens;
  uint32_t* sums;
  int batch, hkv, page_size, max_pages;
  int split_keys;  // keys per split (a multiple of 16)
};

constexpr int kPageWaves = 16;

// Buffer descriptor over [base, base + bytes): a load past the end returns
// zero and moves no data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4_t ld_buf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2 /* nt */));
}

// One workgroup of 16 waves per (split s, sequence b, KV head h), split-major
// like the decode kernel's grid; wave w takes the 16-key tiles w, w + 16, ...
// of the split's keys [s C, min((s + 1) C, L_b)) with one tile in flight.
// The decode kernel's XCD order too: in each full group of 8 (b, h) units,
// XCD x (workgroup index mod 8) reads the slice whose byte offset in the
// key row has bit 9 equal to bit 0 of x (and, 256-byte slices, bit 10 equal
// to bit 1 of x).
// CPR: 16-byte chunks per key row (head_dim / 8).  Chunk j = lane + 64 u of
// a tile is row j / CPR, column chunk j % CPR, so one load instruction
// covers 64 / CPR whole rows.  A tile's descriptors end after its last
// valid key, so rows past the range read as zero without traffic.
template <int CPR>
__global__ __launch_bounds__(kPageWaves * 64) void page_read_kernel(const PageProbe p) {
  constexpr int kPer = 16 * CPR / 64;  // chunks of a tile per lane, per cache
  static_assert(kPer >= 1, "head_dim >= 32");
  const int units = p.batch * p.hkv;
  const int split = int(blockIdx.x) / units;
  int u = int(blockIdx.x) % units;
  constexpr int kSlice = CPR * 16;  // bytes of one head's slice of a key row
  if constexpr (kSlice == 256 || kSlice == 128) {
    constexpr int kSlices = 1024 / kSlice;
    if (p.hkv % kSlices == 0 && (u | 7) < units) {
      const int x = int(blockIdx.x) & 7;
      u = (u & ~7) | (kSlice == 256 ? 2 * (x & 3) + (x >> 2) : 4 * (x & 1) + (x >> 1));
    }
  }
  const int b = u / p.hkv;
  const int h = u % p.hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = split * p.split_keys;
  const int t1 = min(t0 + p.split_keys, p.seqlens[b]);
  const int n_tiles = t1 > t0 ? (t1 - t0 + 15) / 16 : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + kPageWaves - 1) / kPageWaves : 0;
  const int row_bytes = p.hkv * CPR * 16;  // from one key row to the next
  int off[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = lane + 64 * u;
    off[u] = (j / CPR) * row_bytes + (j % CPR) * 16;
  }
  uint32_t s = 0;
  for (int cb = 0; cb < my_tiles; cb += 64) {
    int pages;
    {
      const int key = t0 + (wave + kPageWaves * (cb + lane)) * 16;
      pages = p.block_table[(long)b * p.max_pages + min(key / p.page_size, p.max_pages - 1)];
    }
    const int n = min(64, my_tiles - cb);
    for (int i = 0; i < n; ++i) {
      const int page = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(pages, i));
      const int key0 = t0 + (wave + kPageWaves * (cb + i)) * 16;
      const long e0 = ((long)page * p.page_size + key0 % p.page_size) * p.hkv * (CPR * 8) +
                      (long)h * (CPR * 8);
      const uint32_t bytes = uint32_t(min(16, t1 - key0) * row_bytes);
      const __amdgpu_buffer_rsrc_t rk = rsrc(p.k + e0, bytes);
      const __amdgpu_buffer_rsrc_t rv = rsrc(p.v + e0, bytes);
      u32x4_t kk[kPer], vv[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        kk[u] = ld_buf(rk, off[u]);
        vv[u] = ld_buf(rv, off[u]);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) s += words(kk[u]) + words(vv[u]);
    }
  }
  const uint32_t t = block_sum(s);
  if (threadIdx.x == 0) p.sums[(long)split * units + u] = t;  // [s, b, h]
}

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

attn_status launched() { return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" attn_status attn_probe_stream_read(const void* a, size_t a_bytes, const void* b,
                                              size_t b_bytes, uint32_t* sums, int num_blocks,
                                              void* stream) {
  if (!sums || (a_bytes && !a) || (b_bytes && !b)) return ATTN_ERR_NULL;
  if (a_bytes % 16 || b_bytes % 16 || num_blocks < 1 || num_blocks > 65536) return ATTN_ERR_ARG;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sums, 4)) return ATTN_ERR_ALIGN;
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(a),
                     long(a_bytes / 16), static_cast<const u32x4_t*>(b), long(b_bytes / 16), sums);
  return launched();
}

extern "C" attn_status attn_probe_page_read(const attn_decode_shape* s, const void* k_cache,
                                            const void* v_cache, const int32_t* block_table,
                                            const int32_t* cache_seqlens, int split_keys,
                                            uint32_t* sums, void* stream) {
  if (!s || !k_cache || !v_cache || !block_table || !cache_seqlens || !sums) return ATTN_ERR_NULL;
  if (s->batch < 0 || s->num_heads_kv <= 0 || s->head_dim <= 0 || s->page_size <= 0 ||
      s->max_pages_per_seq <= 0 || s->max_seqlen_k < 0 ||
      int64_t(s->max_seqlen_k) > int64_t(s->max_pages_per_seq) * s->page_size)
    return ATTN_ERR_SHAPE;
  if (split_keys < 0 || split_keys % 16 != 0) return ATTN_ERR_ARG;
  if (s->page_size % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
      !aligned(cache_seqlens, 4) || !aligned(sums, 4))
    return ATTN_ERR_ALIGN;
  const int C = split_keys > 0 ? split_keys : (s->max_seqlen_k > 0 ? s->max_seqlen_k : 16);
  const long splits = split_keys > 0 && s->max_seqlen_k > 0 ? (s->max_seqlen_k + C - 1) / C : 1;
  const PageProbe p{static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                    block_table, cache_seqlens, sums, s->batch, s->num_heads_kv, s->page_size,
                    s->max_pages_per_seq, C};
  const long grid = splits * s->batch * s->num_heads_kv;
  if (grid > 0x7FFFFFFFl) return ATTN_ERR_SHAPE;
  if (grid == 0) return ATTN_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 block(kPageWaves * 64);
  switch (s->head_dim) {
    case 32: hipLaunchKernelGGL(page_read_kernel<4>, dim3(grid), block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(page_read_kernel<8>, dim3(grid), block, 0, st, p); break;
    case 128: hipLaunchKernelGGL(page_read_kernel<16>, dim3(grid), block, 0, st, p); break;
    case 256: hipLaunchKernelGGL(page_read_kernel<32>, dim3(grid), block, 0, st, p); break;
    default: return ATTN_ERR_UNSUPPORTED;
  }
  return launched();
}
