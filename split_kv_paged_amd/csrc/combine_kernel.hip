// combine_kernel.hip -- merge of per-split partial outputs (gfx950).
//
// The split kernel leaves, per query row and split s, a normalised partial
// output O_s and its logsumexp LSE_s (natural log, -inf for an empty split).
// The lpnh.cn "pack_gqa 与 num_splits" article (section
// "两个开关在 kernel 层面各做了什么") describes merging them at the end; the
// merge is the max-shifted log-sum-exp rule, evaluated here in base 2:
//   M = max_s LSE_s,  w_s = 2^((LSE_s - M) log2 e),
//   O = sum_s w_s O_s / sum_s w_s,  LSE = M + ln(sum_s w_s).
// A row whose partials are all empty gets O = 0 and LSE = -inf.
//
// One wave per row; each lane streams head_dim/64 columns of every partial
// (coalesced fp32 loads), so the pass reads S*(head_dim+1)*4 bytes per row
// once.  Any head_dim in [1, 512].
#include "internal.h"

namespace skv {
namespace {

constexpr float kLog2e = 1.4426950408889634074f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kWaves = 4;

template <int DT>
__device__ __forceinline__ uint16_t round16(float x);
template <>
__device__ __forceinline__ uint16_t round16<0>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <>
__device__ __forceinline__ uint16_t round16<1>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int DT>
__global__ __launch_bounds__(kWaves * 64) void combine_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (n >= p.nrows) return;
  const int S = p.num_splits;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, p.lse_part[(long)s * p.nrows + n]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    const float o = __builtin_bit_cast(
        float, __builtin_amdgcn_ds_bpermute((lane ^ x) << 2, __builtin_bit_cast(int, M)));
    M = fmaxf(M, o);
  }
  const int D = p.head_dim;
  uint16_t* out = static_cast<uint16_t*>(p.out);
  if (M == -INFINITY) {
    for (int d = lane; d < D; d += 64) out[(long)n * D + d] = round16<DT>(0.f);
    if (lane == 0 && p.lse) {
      const int h = n % p.heads, i = (n / p.heads) % p.q_len, b = n / (p.heads * p.q_len);
      p.lse[((long)b * p.heads + h) * p.q_len + i] = -INFINITY;
    }
    return;
  }
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ls = p.lse_part[(long)s * p.nrows + n];
    const float w = (ls == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ls - M) * kLog2e);
    wsum += w;
    const float* os = p.o_part + ((long)s * p.nrows + n) * D;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = lane + 64 * k;
      if (d < D) acc[k] = fmaf(w, os[d], acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = lane + 64 * k;
    if (d < D) out[(long)n * D + d] = round16<DT>(acc[k] / wsum);
  }
  if (lane == 0 && p.lse) {
    const int h = n % p.heads, i = (n / p.heads) % p.q_len, b = n / (p.heads * p.q_len);
    p.lse[((long)b * p.heads + h) * p.q_len + i] = M + log2f(wsum) * kLn2;
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const CombineParams& p, hipStream_t s) {
  if (p.nrows <= 0) return hipSuccess;
  const int grid = (p.nrows + kWaves - 1) / kWaves;
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<1>, dim3(grid), dim3(kWaves * 64), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<0>, dim3(grid), dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace skv
