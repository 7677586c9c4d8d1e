// split_kernel.hip -- split-KV decode / small-query attention kernel for gfx950.
//
// One workgroup owns one work unit (sequence b, head unit, row block, KV
// split s) and computes, for up to R packed query rows, the attention of
// those rows over the keys of split s:
//   * packing (lpnh.cn "pack_gqa 与 num_splits" article, section
//     "两个开关在 kernel 层面各做了什么"): the G query heads of one KV head
//     (times q_len) are the rows of one unit, so each K/V byte is read once
//     for all of them;
//   * split s covers keys [s*C, (s+1)*C) clipped to L, with one split length
//     C = 16*ceil(ceil(max_seqlen_k/16)/S) for the whole batch, so a split's
//     first key does not depend on the sequence's length; a split emits its
//     partial output and LSE, and a separate combine pass merges them (same
//     article and section);
//   * online softmax with a running max m, running sum l and an fp32
//     accumulator rescaled by 2^(m_old - m_new) (ai6s.net FlashAttention
//     article, section "FlashAttention 的数学细节"), in base 2 with
//     scale*log2(e) folded into the score, so the exponent is one native
//     v_exp_f32 (the MXFlashAttn page, section 已知限制, names software exp2
//     emulation as its decode kernel's remaining gap);
//   * fp32 accumulation of QK^T and PV (SmallQ FlashAttention README,
//     section 精度策略); QK^T uses v_dot2 on the stored 16-bit pairs, whose
//     products are exact in fp32.
//
// Data movement (the part that sets the speed: decode is a stream over the
// KV cache).  Keys are processed in tiles of 16.  A lane owns CPL 16-byte
// chunks of one key row (LPT lanes per key, TPS = 64/LPT keys per step), so
// every global load is a 16-byte dwordx4 and the LPT lanes of a key read one
// contiguous run of the row.  Each lane consumes only the bytes it loaded,
// so tiles are double-buffered in VGPRs: tile n+1 is in flight while tile n
// is computed.  The per-lane partial dot products are summed over the LPT
// lanes of a key with DPP (quad_perm, half-row mirror, row mirror).
//
// Each group of LPT lanes keeps its own (m, l) per row over the keys it saw;
// the references move lazily, only when a tile's max exceeds the reference
// by more than 2^8, so the common tile needs no rescale (results are the same
// softmax: numerator and denominator share the reference).  At the end the
// groups of a wave are merged with shuffles, and the waves of the workgroup
// through LDS, by the log-sum-exp rules.
#include <type_traits>

#include "internal.h"

namespace skv {
namespace {

constexpr int kTile = 16;
constexpr float kRescaleHeadroom = 8.0f;  // log2 units
constexpr float kLn2 = 0.693147180559945309417f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem;

template <>
struct Elem<0> {  // IEEE binary16
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  // (a, b) rounded to nearest-even, a in the low half
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, half2_t));
  }
  static constexpr uint32_t kOnePair = 0x3C003C00u;  // (1.0, 1.0)
};

template <>
struct Elem<1> {  // bfloat16
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), c, false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return __builtin_bit_cast(float, w << 16);
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, bf162_t));
  }
  static constexpr uint32_t kOnePair = 0x3F803F80u;  // (1.0, 1.0)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPT consecutive lanes; every lane gets the sum.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPT >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LPT >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPT >= 8) x += dpp<0x141>(x);  // half-row mirror: the other quad of 8
  if constexpr (LPT >= 16) x += dpp<0x140>(x); // row mirror: the other half of 16
  static_assert(LPT <= 16, "a key spans at most one DPP row");
  return x;
}

// All-reduce over the key groups of a wave: lanes that differ in the bits
// above log2(LPT) (same chunk lane j).  Inside a 16-lane row the groups are
// combined by DPP row rotations; across rows by the gfx950 permlane16/32
// swaps.  Everything stays in VGPRs (no LDS traffic).
template <int LPT, bool MAX>
__device__ __forceinline__ float groups_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (LPT <= 4) x = op(x, dpp<0x124>(x));  // row_ror:4
  if constexpr (LPT <= 8) x = op(x, dpp<0x128>(x));  // row_ror:8
  {
    const auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                      __builtin_bit_cast(unsigned, x), false,
                                                      false);
    x = op(__builtin_bit_cast(float, (unsigned)s16[0]), __builtin_bit_cast(float, (unsigned)s16[1]));
  }
  {
    const auto s32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                      __builtin_bit_cast(unsigned, x), false,
                                                      false);
    x = op(__builtin_bit_cast(float, (unsigned)s32[0]), __builtin_bit_cast(float, (unsigned)s32[1]));
  }
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer descriptor (gfx9 dword3: 32-bit data format, no stride) over
// `bytes` bytes from `base`; loads past the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int voffset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}

template <int DT, int D, int R, int LPT, int NW, int NBUF, bool PAGED>
__global__ __launch_bounds__(NW * 64) void split_kernel(const SplitParams p) {
  using E = Elem<DT>;
  constexpr int TPS = 64 / LPT;     // keys per step
  constexpr int NS = kTile / TPS;   // steps per tile
  constexpr int CPL = D / (8 * LPT);  // 16-byte chunks per lane per key
  static_assert(NS >= 1 && CPL >= 1 && TPS * NS == kTile && CPL * 8 * LPT == D, "tiling");
  static_assert(NBUF >= 2, "at least one tile in flight while one is computed");
  static_assert(NS % 2 == 0, "PV pairs the keys of two steps");

  struct Buf {
    uint4 k[NS][CPL];
    uint4 v[NS][CPL];
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / LPT;  // key within a step
  const int j = lane % LPT;    // chunk lane within the key

  // unit decode: (b, unit head, row block, split), split fastest
  int bid = blockIdx.x;
  const int split = bid % p.num_splits;
  bid /= p.num_splits;
  const int rb = bid % p.row_blocks;
  bid /= p.row_blocks;
  const int uh = bid % p.unit_heads;
  const int b = bid / p.unit_heads;
  const int hq0 = uh * p.heads_per_unit;
  const int h = hq0 / p.group;

  // The split's first key is known without the sequence length, so the
  // page ids of this wave's first tiles, the query rows and the length are
  // all fetched in one round trip.  Lane i of a wave holds the page id of
  // the wave's tile cb + i (tiles are dealt to waves round-robin), for one
  // chunk of 64 tiles at a time; the loop reads it with v_readlane.
  const int t0 = split * p.split_keys;
  auto load_pages = [&](int cb) -> int {
    if constexpr (PAGED) {
      const int tt = t0 + (wave + (cb + lane) * NW) * kTile;
      return p.block_table[(long)b * p.max_pages + min(tt / p.page_size, p.max_pages - 1)];
    } else {
      return 0;
    }
  };
  int pages = load_pages(0);
  const int L = PAGED ? p.seqlens[b] : p.kv_len;
  const int t1 = min(t0 + p.split_keys, L);
  const int n_tiles = t1 > t0 ? (t1 - t0 + kTile - 1) / kTile : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + NW - 1) / NW : 0;

  // ---- query rows (raw 16-bit pairs, in the lane's chunk order) ----------
  uint32_t qv[R][CPL][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int pr = rb * R + r;
    if (pr < p.rows) {
      const int i = pr / p.heads_per_unit;
      const int hq = hq0 + pr % p.heads_per_unit;
      const long n = (long)b * p.n_sb + (long)i * p.n_si + (long)hq * p.n_sh;
      const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + n * D);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint4 t = qp[j + c * LPT];
        qv[r][c][0] = t.x; qv[r][c][1] = t.y; qv[r][c][2] = t.z; qv[r][c][3] = t.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) qv[r][c][w] = 0u;
    }
  }

  float acc[R][CPL * 8];
  float m[R], l[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < CPL * 8; ++e) acc[r][e] = 0.f;
  }

  const long row_stride = PAGED ? (long)p.hkv * D : (long)D;
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(p.v);

  // element offset of key row 0 of tile idx, KV head h
  auto tile_row0 = [&](int idx, int page) -> long {
    const int tt = t0 + (wave + idx * NW) * kTile;
    if constexpr (PAGED) {
      return ((long)page * p.page_size + tt % p.page_size) * p.hkv * D + (long)h * D;
    } else {
      return ((long)h * p.kv_len + tt) * D;
    }
  };

  // Per-lane byte offset of step st inside a tile (the chunk c adds an
  // immediate c*LPT*16).
  int voff[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
    voff[st] = int(((st * TPS + sub) * row_stride + j * 8) * 2);

  // Each tile is read through buffer descriptors whose range ends at the
  // last key of the split inside the tile: rows past it (poisoned or
  // belonging to the next split, or past the end of a dense tensor) read as
  // zero and never fault.
  auto issue = [&](Buf& bf, int idx, int page) {
    // the page id is wave-uniform; say so, so the descriptors stay in SGPRs
    page = __builtin_amdgcn_readfirstlane(page);
    const int tt = t0 + (wave + idx * NW) * kTile;
    const long row0 = tile_row0(idx, page);
    const uint32_t bytes = uint32_t(min(kTile, t1 - tt) * row_stride * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + row0, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + row0, bytes);
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        bf.k[st][c] = load16(rk, voff[st] + c * LPT * 16);
        bf.v[st][c] = load16(rv, voff[st] + c * LPT * 16);
      }
  };

  // One tile: scores, lazy reference update, probabilities rounded to the
  // 16-bit type in pairs of keys, and PV as v_dot2 over those key pairs (the
  // running sum l takes the same rounded values, so numerator and
  // denominator use identical weights).  FULL tiles skip the key mask.
  const float c = p.scale_log2;
  auto process_tile = [&](const Buf& bf, int tt, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    float dr[NS][R];  // raw q.k per key step and row
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float d = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          d = E::dot2(qv[r][cc][0], bf.k[st][cc].x, d);
          d = E::dot2(qv[r][cc][1], bf.k[st][cc].y, d);
          d = E::dot2(qv[r][cc][2], bf.k[st][cc].z, d);
          d = E::dot2(qv[r][cc][3], bf.k[st][cc].w, d);
        }
        dr[st][r] = group_sum<LPT>(d);
      }
      if constexpr (!FULL) {
        const bool valid = tt + st * TPS + sub < t1;
#pragma unroll
        for (int r = 0; r < R; ++r) dr[st][r] = valid ? dr[st][r] : -INFINITY;
      }
    }
    // lazy reference update (scale > 0, so the max commutes with it)
    bool need = false;
    float mnew[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mt = dr[0][r];
#pragma unroll
      for (int st = 1; st < NS; ++st) mt = fmaxf(mt, dr[st][r]);
      mt *= c;
      mnew[r] = (mt > m[r] + kRescaleHeadroom) ? mt : m[r];
      need |= mnew[r] != m[r];
    }
    if (__any(need)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float alpha = (mnew[r] == m[r]) ? 1.f : fast_exp2(m[r] - mnew[r]);
        m[r] = mnew[r];
        l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < CPL * 8; ++e) acc[r][e] *= alpha;
      }
    }
    // probabilities of key steps (2sp, 2sp+1), packed
    uint32_t pp[NS / 2][R];
#pragma unroll
    for (int sp = 0; sp < NS / 2; ++sp)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float p0 = fast_exp2(fmaf(dr[2 * sp][r], c, -m[r]));
        float p1 = fast_exp2(fmaf(dr[2 * sp + 1][r], c, -m[r]));
        if constexpr (!FULL) {  // masked keys; m may still be -inf here
          p0 = (dr[2 * sp][r] == -INFINITY) ? 0.f : p0;
          p1 = (dr[2 * sp + 1][r] == -INFINITY) ? 0.f : p1;
        }
        pp[sp][r] = E::pack(p0, p1);
        l[r] = E::dot2(pp[sp][r], E::kOnePair, l[r]);
      }
    // PV: pair the value rows of keys 2sp and 2sp+1 element by element
#pragma unroll
    for (int sp = 0; sp < NS / 2; ++sp)
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        const uint32_t a4[4] = {bf.v[2 * sp][cc].x, bf.v[2 * sp][cc].y, bf.v[2 * sp][cc].z,
                                bf.v[2 * sp][cc].w};
        const uint32_t b4[4] = {bf.v[2 * sp + 1][cc].x, bf.v[2 * sp + 1][cc].y,
                                bf.v[2 * sp + 1][cc].z, bf.v[2 * sp + 1][cc].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = __builtin_amdgcn_perm(b4[w], a4[w], 0x05040100u);  // elem 2w
          const uint32_t hi = __builtin_amdgcn_perm(b4[w], a4[w], 0x07060302u);  // elem 2w+1
#pragma unroll
          for (int r = 0; r < R; ++r) {
            acc[r][cc * 8 + 2 * w] = E::dot2(lo, pp[sp][r], acc[r][cc * 8 + 2 * w]);
            acc[r][cc * 8 + 2 * w + 1] = E::dot2(hi, pp[sp][r], acc[r][cc * 8 + 2 * w + 1]);
          }
        }
      }
  };
  auto process = [&](const Buf& bf, int idx) {
    const int tt = t0 + (wave + idx * NW) * kTile;
    if (tt + kTile <= t1)
      process_tile(bf, tt, std::true_type{});
    else
      process_tile(bf, tt, std::false_type{});
  };

  // ---- main loop: NBUF tiles in a register ring ----------------------------
  // The loads of tiles n+1 .. n+NBUF-1 are in flight while tile n is
  // computed.  Indices past the chunk's last tile are clamped (a redundant,
  // cached re-read), so every load is unconditional, and nothing but the
  // tile index is carried from one iteration to the next.
  for (int cb = 0; cb < my_tiles; cb += 64) {
    if (cb > 0) pages = load_pages(cb);
    const int n = min(64, my_tiles - cb);
    const int last = n - 1;
    auto page_at = [&](int i) { return __builtin_amdgcn_readlane(pages, i); };
    Buf ring[NBUF];
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k) issue(ring[k], cb + min(k, last), page_at(min(k, last)));
    int i = 0;
    bool more = true;
    while (more) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        if (more) {
          const int nx = min(i + NBUF - 1, last);
          issue(ring[(k + NBUF - 1) % NBUF], cb + nx, page_at(nx));
          process(ring[k], cb + i);
          more = ++i < n;
        }
      }
    }
  }

  // ---- merge the key groups of this wave (lanes differing in `sub`) ------
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float M = groups_reduce<LPT, true>(m[r]);
    const float f = (m[r] == -INFINITY) ? 0.f : fast_exp2(m[r] - M);
    l[r] = groups_reduce<LPT, false>(l[r] * f);
#pragma unroll
    for (int e = 0; e < CPL * 8; ++e) acc[r][e] = groups_reduce<LPT, false>(acc[r][e] * f);
    m[r] = M;
  }

  // ---- merge the waves through LDS and write -----------------------------
  __shared__ float s_acc[NW][R][D];
  __shared__ float s_m[NW][R];
  __shared__ float s_l[NW][R];
  if (sub == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[wave][r][(j + c * LPT) * 8 + e] = acc[r][c * 8 + e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s_m[wave][r] = m[r];
      s_l[wave][r] = l[r];
    }
  }
  __syncthreads();

  for (int t = threadIdx.x; t < R * D; t += NW * 64) {
    const int r = t / D;
    const int d = t % D;
    const int pr = rb * R + r;
    if (pr >= p.rows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][r]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = (s_m[w][r] == -INFINITY) ? 0.f : fast_exp2(s_m[w][r] - M);
        num = fmaf(f, s_acc[w][r][d], num);
        den = fmaf(f, s_l[w][r], den);
      }
    }
    const float o = (M == -INFINITY) ? 0.f : num / den;
    const float lse = (M == -INFINITY) ? -INFINITY : (M + log2f(den)) * kLn2;
    const int i = pr / p.heads_per_unit;
    const int hq = hq0 + pr % p.heads_per_unit;
    const long n = (long)b * p.n_sb + (long)i * p.n_si + (long)hq * p.n_sh;
    if (p.num_splits == 1) {
      static_cast<uint16_t*>(p.out)[n * D + d] = E::round(o);
      if (d == 0 && p.lse) p.lse[((long)b * p.hq + hq) * p.q_len + i] = lse;
    } else {
      p.o_part[((long)split * p.nrows + n) * D + d] = o;
      if (d == 0) p.lse_part[(long)split * p.nrows + n] = lse;
    }
  }
}

// kernel choice per (head_dim, rows per block): lanes per key, waves per
// workgroup and tiles in the register ring
#ifndef SKV_NW
#define SKV_NW 8
#endif
#ifndef SKV_NBUF
#define SKV_NBUF 2
#endif
#ifndef SKV_LPT_R4
#define SKV_LPT_R4 16  // lanes per key (x D/128) when a block carries <= 4 rows
#endif
template <int D, int R>
struct Cfg {
  static constexpr int LPT_R4 = SKV_LPT_R4 * D / 128 < 8 ? 8 : SKV_LPT_R4 * D / 128;
  static constexpr int LPT = (R <= 4) ? LPT_R4 : D / 8;
  static constexpr int NW = SKV_NW;
  static constexpr int NBUF = SKV_NBUF;
};

template <int DT, int D, int R, bool PAGED>
hipError_t launch_one(const SplitParams& p, int grid, hipStream_t s) {
  constexpr int LPT = Cfg<D, R>::LPT;
  constexpr int NW = Cfg<D, R>::NW;
  constexpr int NBUF = Cfg<D, R>::NBUF;
  hipLaunchKernelGGL((split_kernel<DT, D, R, LPT, NW, NBUF, PAGED>), dim3(grid), dim3(NW * 64), 0,
                     s, p);
  return hipGetLastError();
}

template <int DT, int D, bool PAGED>
hipError_t launch_rows(int rows, const SplitParams& p, int grid, hipStream_t s) {
  switch (rows) {
    case 1: return launch_one<DT, D, 1, PAGED>(p, grid, s);
    case 2: return launch_one<DT, D, 2, PAGED>(p, grid, s);
    case 4: return launch_one<DT, D, 4, PAGED>(p, grid, s);
    case 8: return launch_one<DT, D, 8, PAGED>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, bool PAGED>
hipError_t launch_dim(const SplitVariant& v, const SplitParams& p, int grid, hipStream_t s) {
  switch (v.head_dim) {
    case 64: return launch_rows<DT, 64, PAGED>(v.rows_per_block, p, grid, s);
    case 128: return launch_rows<DT, 128, PAGED>(v.rows_per_block, p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool split_variant_supported(const SplitVariant& v) {
  const bool dim = v.head_dim == 64 || v.head_dim == 128;
  const bool rows = v.rows_per_block == 1 || v.rows_per_block == 2 || v.rows_per_block == 4 ||
                    v.rows_per_block == 8;
  return dim && rows && (v.dtype == 0 || v.dtype == 1);
}

int split_variant_id(const SplitVariant& v) {
  return (v.paged ? 1000 : 0) + v.dtype * 100 + (v.head_dim == 128 ? 10 : 0) + v.rows_per_block;
}

hipError_t launch_split(const SplitVariant& v, const SplitParams& p, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (v.paged) {
    return v.dtype == 1 ? launch_dim<1, true>(v, p, grid, s) : launch_dim<0, true>(v, p, grid, s);
  }
  return v.dtype == 1 ? launch_dim<1, false>(v, p, grid, s) : launch_dim<0, false>(v, p, grid, s);
}

}  // namespace skv
