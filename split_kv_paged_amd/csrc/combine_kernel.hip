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
// once, kBatch splits per round of loads.  Any head_dim in [1, 512].
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

// KD = columns per lane / 1 (head_dim <= 64 * KD).  The partials of kBatch
// splits are loaded in one round of independent loads, then folded in.
constexpr int kBatch = 8;

template <int DT, int KD>
__global__ __launch_bounds__(kWaves * 64) void combine_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (n >= p.nrows) return;
  const int S = p.num_splits;
  const int D = p.head_dim;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, p.lse_part[(long)s * p.nrows + n]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    const float o = __builtin_bit_cast(
        float, __builtin_amdgcn_ds_bpermute((lane ^ x) << 2, __builtin_bit_cast(int, M)));
    M = fmaxf(M, o);
  }
  uint16_t* out = static_cast<uint16_t*>(p.out);
  if (M == -INFINITY) {
    for (int d = lane; d < D; d += 64) out[(long)n * D + d] = round16<DT>(0.f);
    if (lane == 0 && p.lse) {
      const int h = n % p.heads, i = (n / p.heads) % p.q_len, b = n / (p.heads * p.q_len);
      p.lse[((long)b * p.heads + h) * p.q_len + i] = -INFINITY;
    }
    return;
  }
  float acc[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float ls[kBatch], ov[kBatch][KD];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {  // clamped indices: no branches between the loads
      const long row = (long)min(s0 + j, S - 1) * p.nrows + n;
      ls[j] = p.lse_part[row];
#pragma unroll
      for (int k = 0; k < KD; ++k) ov[j][k] = p.o_part[row * D + min(lane + 64 * k, D - 1)];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = (s0 + j >= S || ls[j] == -INFINITY)
                          ? 0.f
                          : __builtin_amdgcn_exp2f((ls[j] - M) * kLog2e);
      wsum += w;
#pragma unroll
      for (int k = 0; k < KD; ++k) acc[k] = fmaf(w, ov[j][k], acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    const int d = lane + 64 * k;
    if (d < D) out[(long)n * D + d] = round16<DT>(acc[k] / wsum);
  }
  if (lane == 0 && p.lse) {
    const int h = n % p.heads, i = (n / p.heads) % p.q_len, b = n / (p.heads * p.q_len);
    p.lse[((long)b * p.heads + h) * p.q_len + i] = M + log2f(wsum) * kLn2;
  }
}

template <int DT>
void launch_kd(const CombineParams& p, int grid, hipStream_t s) {
  const int kd = (p.head_dim + 63) / 64;
  if (kd <= 1)
    hipLaunchKernelGGL((combine_kernel<DT, 1>), dim3(grid), dim3(kWaves * 64), 0, s, p);
  else if (kd <= 2)
    hipLaunchKernelGGL((combine_kernel<DT, 2>), dim3(grid), dim3(kWaves * 64), 0, s, p);
  else if (kd <= 4)
    hipLaunchKernelGGL((combine_kernel<DT, 4>), dim3(grid), dim3(kWaves * 64), 0, s, p);
  else
    hipLaunchKernelGGL((combine_kernel<DT, 8>), dim3(grid), dim3(kWaves * 64), 0, s, p);
}

}  // namespace

hipError_t launch_combine(int dtype, const CombineParams& p, hipStream_t s) {
  if (p.nrows <= 0) return hipSuccess;
  const int grid = (p.nrows + kWaves - 1) / kWaves;
  if (dtype == 1)
    launch_kd<1>(p, grid, s);
  else
    launch_kd<0>(p, grid, s);
  return hipGetLastError();
}

}  // namespace skv
