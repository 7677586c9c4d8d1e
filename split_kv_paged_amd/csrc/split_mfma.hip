// split_mfma.hip -- split-KV decode / small-query attention on gfx950 matrix cores.
//
// Work unit: (sequence, head unit, block of 16, 32 or 64 packed query rows,
// split).  A head unit is one KV head with its G query heads packed into the
// rows (pack_gqa), one query head, or (head dims 64 and 32) 2 or 4
// adjacent KV heads read as one 128-wide key row.  One workgroup per unit; its waves take the
// 16-key tiles of the split's key range round-robin, each with its own online
// softmax state, and merge through LDS at the end.  The two contractions run
// on the matrix cores:
//
//   S^T (16 keys x 16 rows) = K (16 x D) . Q^T (D x 16)
//       v_mfma_f32_16x16x32_{bf16,f16}, D/32 instructions per 16-key tile.
//       With K as the A operand, lane l holds the scores of query row l%16
//       for keys 4*(l/16)..+3: one row per lane, so the softmax needs no
//       per-key lane reductions, and the probabilities are already in the
//       A layout of the next product.
//   O (16 rows x D) += P (16 x 16 keys) . V (16 keys x D)
//       v_mfma_f32_16x16x32_{bf16,f16}, D/16 instructions per tile: a
//       lane's 8 k-values are its 4 keys' probabilities rounded to the
//       16-bit type and the 4 rounded residues (A), against its 4 V values
//       twice (B), so P carries 16 (bf16) or 22 (fp16) significant bits.
//       O and the LSE are normalised by a float32 running sum of the
//       unrounded probabilities.
//       The V tile sits in the wave's LDS slot and is read back with
//       ds_read_b64_tr_b16, which delivers the key-major B operand.
//
// Tile loads.  With 16-byte chunks and at least 8 of them a key row (head
// dims 64..256, GEN 0/1/3), K and V go from memory straight into the wave's
// LDS slot with 16-byte buffer loads to LDS: each instruction fills 1 KB,
// whole key rows, so every load touches whole cache lines, and no register
// holds a tile in flight.  A wave reads tile n out of its slot (K in the
// MFMA A layout, V transposed), refills the slot with tile n+1, then
// computes tile n.  The other kernels (head dim 32, or element loads) move
// tiles through a ring of NBUF register buffers and stage V in LDS.  Every
// K/V load is non-temporal: each KV byte is read once per call.
// A buffer descriptor ends at the split's last key, so keys past it (another
// split, the poisoned tail of a page, the end of a dense tensor) read as zero
// without a fault.  The physical page of each tile comes from the block
// table, 64 tiles' worth per vector load, broadcast with readlane.  A launch
// that also appends keys to the cache (APP) ends the descriptors at the
// cached keys and puts the new rows into the slots from k_new / v_new.
//
// Packed query rows beyond the unit's real rows are zero; their lanes do the
// same (SIMD) work and are never written.  A workgroup carries one, two or
// four 16-row blocks (NRB) of one unit.  Units are placed on the XCDs by
// where their slices sit in the key rows (see the work lists below), and
// the launch-invariant integer divisions of the index arithmetic are
// multiply-high-and-shift sequences prepared on the host.
//
// Sources: attention definition (SmallQ FlashAttention README, section 接口);
// online softmax with max offset (ai6s.net FlashAttention article, section
// "FlashAttention 的数学细节"); GQA packing and split partials with their
// logsumexp (lpnh.cn "pack_gqa 与 num_splits" article, section
// "两个开关在 kernel 层面各做了什么"); fp32 accumulation (SmallQ README,
// section 精度策略).
#include <type_traits>

#include "internal.h"

namespace skv {
namespace {

constexpr int kTile = 16;
constexpr float kHeadroom = 8.0f;  // log2 units before the reference moves
constexpr float kLn2 = 0.693147180559945309417f;

typedef float f4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));

template <int DT>
struct Mf;

template <>
struct Mf<1> {  // bfloat16
  static __device__ __forceinline__ f4_t qk(uint4 a, uint4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a),
                                                   __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, bf2_t));
  }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  // the two values of a packed pair, exactly, as floats
  static __device__ __forceinline__ f2_t widen(uint32_t v) {
    return (f2_t){__builtin_bit_cast(float, v << 16), __builtin_bit_cast(float, v & 0xFFFF0000u)};
  }
};

template <>
struct Mf<0> {  // IEEE binary16
  static __device__ __forceinline__ f4_t qk(uint4 a, uint4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, h2_t));
  }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ f2_t widen(uint32_t v) {
    return __builtin_convertvector(__builtin_bit_cast(h2_t, v), f2_t);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Cache policy of every K/V tile load: non-temporal (CPol::NT).  Each KV
// byte is read once per call, so keeping it in L2 only evicts what is worth
// keeping.  Measured (paged GQA-4 bf16 decode / uniform L 4000 / long
// context S = 14 / ragged S = 5, us): 27.5 / 93.0 / 32.0 / 64.0 with the
// default policy, 25.7 / 84.7 / 29.8 / 59.7 with NT.
constexpr int kStream = 2;

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int voffset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, kStream));
}

// a 16-bit element (zero-extended); offsets past the descriptor's range read 0
__device__ __forceinline__ uint32_t load2(__amdgpu_buffer_rsrc_t r, int voffset) {
  return uint32_t(
      __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, voffset, 0, kStream)));
}
constexpr int kPastEnd = 0x7FFFFFF0;  // beyond any tile's range (tiles are < 2 GiB)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// n / d for n >= 0 (d's FastDiv); the same code on scalar or vector values
__device__ __forceinline__ int fdiv(int n, FastDiv d) {
  const uint32_t u = uint32_t(n);
  const uint32_t t = __umulhi(u, d.m);
  return int((t + ((u - t) >> d.s1)) >> d.s2);
}

// Partials shared between workgroups on different XCDs go straight to and
// from memory: stores and loads carry the sc0|sc1 (system coherence) cache
// policy, so they are written through and read past every cache, and no
// cache has to be flushed or invalidated.
constexpr int kSysCoherent = 17;  // CPol::SC0 | CPol::SC1
__device__ __forceinline__ void publish(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, int(byte_off), 0,
                                        kSysCoherent);
}
__device__ __forceinline__ void publish4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), r, int(byte_off), 0,
                                         kSysCoherent);
}
__device__ __forceinline__ f4_t fetch4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, int(byte_off), 0, kSysCoherent));
}
__device__ __forceinline__ float fetch(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r, int(byte_off), 0, kSysCoherent));
}

// max / sum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48)
template <bool MAX>
__device__ __forceinline__ float across_rows(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  const auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
  x = op(__builtin_bit_cast(float, (unsigned)s16[0]), __builtin_bit_cast(float, (unsigned)s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
  return op(__builtin_bit_cast(float, (unsigned)s32[0]), __builtin_bit_cast(float, (unsigned)s32[1]));
}

__device__ __forceinline__ float from_lane(float x, int src_lane) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, x)));
}

// D is the head dimension the tiles are built for (32, 64, 128 or 256); the
// real one, p.head_dim <= D, may be any value.  Columns past p.head_dim read
// as zero, so they add nothing to the scores and produce output columns that
// are never stored (the SmallQ README, section "任意 headDim 支持": pad
// inside, store only the real columns).  GEN selects how K, V and Q move:
//   0  head_dim == D: 16-byte loads;
//   1  head_dim a multiple of 8 (rows stay 16-byte aligned): 16-byte loads,
//      a chunk past the head dim gets an offset past the buffer range;
//   2  any other head_dim: 16-bit element loads;
//   3  head groups (paged, D = 128, head_dim 64 or 32): 16-byte loads of
//      whole 128-wide rows of 2 or 4 adjacent KV heads.
// NRB: 16-row blocks a workgroup carries (1; 2 or 4 when a unit has more
// than 16 or 32 packed rows, so its KV is read once for up to 64 rows).
// tid: the thread index (passed in so that the compact list's loop can
// hide it from loop-invariant hoisting).  APP: this launch also appends
// p.seq_add keys per sequence from p.k_new / p.v_new (see below).
template <int DT, int D, int NW, int NBUF, bool PAGED, int GEN, int NRB, bool APP>
__device__ __forceinline__ void split_unit(const SplitParams& p, const int split, const int b,
                                           const int uh, const int rb, const int tid) {
  using M = Mf<DT>;
  constexpr int KB = D / 32;        // 16x16x32 products per tile (QK)
  constexpr int DB = D / 16;        // 16x16x16 products per tile (PV)
  // Chunk (8 elements, 16 bytes) of a key row that lane group g holds for
  // product kb of S^T = K . Q^T: chunk 4kb + g, so the four lane groups of
  // one load instruction read 64 contiguous bytes of each row (half a
  // 128-byte line; any chunk order gives the same dot products as long as
  // Q uses it too).
  auto chunk = [](int g_, int kb_) { return kb_ * 4 + g_; };
  // LDS bytes per staged key row: unpadded with the 16-byte chunks of row
  // r permuted by XOR with swz(r) (needs 8 chunks a row), else padded by 32
  // bytes against bank clashes.  The K reads (16 rows, one chunk each) and
  // the transposed V reads (rows 4g + i, 32-byte pairs of chunks, a half
  // wave at a time) then repeat no LDS bank whether a cycle serves 128 or
  // 256 bytes (gfx950 serves 256: 64 banks):
  //   16 chunks or more a row: swz(r) = 2(r & 3) + ((r >> 2) & 1)
  //     + 8 ((r >> 2) ^ (r >> 3) & 1)   (16 chunk columns for 16 rows; 8
  //     pairs for rows 0..7 and for rows 8..15);
  //   8 chunks a row (two rows a bank cycle): swz(r) = 2 ((r & 3) ^ (r >> 2
  //     & 1)) + ((r >> 2) ^ (r >> 3) & 1)  (each chunk column once among the
  //     even rows and once among the odd ones; distinct pairs per row parity
  //     in each half wave).
  // Without the (r >> 3) terms rows r and r + 8 (K) and rows i and 4 + i (V)
  // shared banks at 256 bytes a cycle (measured: 0.66 conflicts per LDS
  // access on the paged GQA-4 d 128 workload, 0.003 with them).
  constexpr bool kSwz = D >= 64;
  constexpr int ROWB = kSwz ? D * 2 : D * 2 + 32;
  auto swz = [](int r) {
    if constexpr (D >= 128)
      return 2 * (r & 3) + ((r >> 2) & 1) + 8 * (((r >> 2) ^ (r >> 3)) & 1);
    else
      return 2 * ((r & 3) ^ ((r >> 2) & 1)) + (((r >> 2) ^ (r >> 3)) & 1);
  };
  // NBUF == 0: no register ring; each tile goes from memory straight into
  // the wave's LDS slot, one tile in flight per wave while the previous one
  // is computed
  constexpr bool kDma = NBUF == 0;
  static_assert(!kDma || (kSwz && GEN != 2), "direct-to-LDS tiles need >= 8 16-byte chunks a row");
  static_assert(D % 32 == 0, "head_dim");
  // GEN 3 (paged, head groups): R = D / head_dim adjacent KV heads (2 at
  // head dim 64, 4 at 32) are one D-wide key row (the cache layout puts
  // them side by side), and the unit packs all R heads' query rows.  A
  // row's head_dim query values sit in its own head's slice of the D
  // columns and the rest is zero, so its scores see only its head's keys;
  // its output is the same slice of O.
  constexpr bool kGroup = GEN == 3;
  static_assert(!kGroup || (PAGED && NRB == 1 && D == 128), "head groups: paged, one row block");
  const int hd = GEN == 0 ? D : p.head_dim;              // query / output row
  const int kvd = GEN == 1 || GEN == 2 ? p.head_dim : D;  // key / value row
  // first tile column of packed row pr's head (head groups: slice
  // (pr mod R*G) / G of the row, G = heads_per_unit * head_dim / D)
  auto col0 = [&](int pr) {
    return kGroup ? fdiv(pr - fdiv(pr, p.fd_hpu) * p.heads_per_unit, p.fd_gq) * hd : 0;
  };

  struct Buf {
    uint4 k[KB];
    uint4 v[KB];
  };

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;  // S^T: query row; O: column within a 16-wide d block
  const int g = lane >> 4;    // S^T: key group (keys 4g..4g+3); O: rows 4g..4g+3

  const int hq0 = uh * p.heads_per_unit;
  const int h = p.heads_per_unit == p.group ? uh : fdiv(hq0, p.fd_group);

  // split range and this wave's tiles (round-robin over the waves)
  const int t0 = split * p.split_keys;
  auto load_pages = [&](int cb) -> int {
    if constexpr (PAGED) {
      const int tt = t0 + (wave + (cb + lane) * NW) * kTile;
      return p.block_table[(long)b * p.max_pages + min(fdiv(tt, p.fd_page), p.max_pages - 1)];
    } else {
      return 0;
    }
  };
  // queries of this sequence: rows qbase .. qbase + qlen_b - 1 of q / out
  int qbase = b * p.q_len, qlen_b = p.q_len;
  if (p.cu_q) {
    qbase = p.cu_q[b];
    qlen_b = p.cu_q[b + 1] - qbase;
  }
  const int rows_b = p.cu_q ? qlen_b * p.heads_per_unit : p.rows;  // real packed rows
  const int row0 = rb * 16 * NRB;  // first packed row of this workgroup
  if (row0 >= rows_b) return;      // a row block past this sequence's queries
  // The page ids of the first tiles and the query rows do not depend on the
  // sequence's length: their loads go out together with the length load, so
  // the first tile waits for one round trip instead of two.
  int pages = load_pages(0);
  auto row_of = [&](int i, int hq) -> long {
    return (long)(qbase + i) * p.n_si + (long)hq * p.n_sh;
  };
  auto lse_of = [&](int i, int hq) -> long {
    return p.cu_q ? (long)hq * p.total_q + qbase + i : ((long)b * p.hq + hq) * p.q_len + i;
  };
  // ---- Q^T as the B operand: lane l holds row l%16 of each 16-row block,
  // chunks g*KB + kb ------------------------------------------------------
  // Four row blocks at D = 128 would need 64 more VGPRs than eight waves
  // have next to their accumulators, so there the workgroup stages its 64
  // query rows in LDS and each wave reads a row block's operand per tile.
  // Otherwise each lane loads its rows' operands into registers, after the
  // first tile has gone out (the loads then overlap the tile's flight, and
  // the first tile waits for the page ids alone).
  constexpr bool kQLds = NRB == 4 && D == 128;
  static_assert(!kQLds || GEN == 0, "staged Q rows are whole 16-byte chunks");
  uint4 qb[kQLds ? 1 : NRB][KB];
  const int L = PAGED ? p.seqlens[b] + p.seq_add : p.kv_len;
  // Splits of this sequence that hold keys.  Past the last key a split has
  // nothing to add (its LSE would be -inf, weight zero in the combine), so
  // its workgroup leaves at once; a sequence that fits in one split is
  // finished by split 0 alone, with no partials and no combine.  At most
  // num_splits arrive: a length over max_seqlen_k (outside the contract)
  // loses its keys past the last split instead of leaving a unit's counter
  // waiting for a split that never runs.
  const int nsplit =
      p.num_splits == 1 ? 1
                        : min(p.num_splits, max(1, fdiv(L + p.split_keys - 1, p.fd_split_keys)));
  if (split >= nsplit) return;
  const bool direct = nsplit == 1;
  const int t1 = min(t0 + p.split_keys, L);
  // Keys appended by this call (k_new set; paged calls whose tiles go
  // straight to LDS): the last seq_add keys, [Lc, L), are read from k_new /
  // v_new [batch, seq_add, Hkv, head_dim] rather than from the cache, and
  // one workgroup of the KV head (row block 0, the first query head of its
  // group) writes them into the cache for later calls.  No workgroup of
  // this launch reads those cache rows, so no ordering between workgroups
  // is needed.
  constexpr bool fused = APP;
  static_assert(!APP || (PAGED && kDma), "appending launches: paged, direct-to-LDS tiles");
  const int Lc = fused ? L - p.seq_add : L;  // keys already in the cache
  const int n_tiles = t1 > t0 ? (t1 - t0 + kTile - 1) / kTile : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + NW - 1) / NW : 0;

  // Keys a lane's row may see: [t0, lim[r]).  Causal (bottom-right): query
  // i of q_len sees keys j <= L - q_len + i.  Every tile applies the mask
  // (a few VALU ops); a separate unmasked copy of the tile code would make
  // the compiler keep two copies of the accumulators live.
  int lim[NRB];
#pragma unroll
  for (int r = 0; r < NRB; ++r) lim[r] = t1;
  if (p.causal) {
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int i_row = fdiv(row0 + 16 * r + n16, p.fd_hpu);
      lim[r] = min(t1, max(0, L - qlen_b + 1 + i_row));
    }
  }
  __shared__ __attribute__((aligned(16))) uint8_t s_q[kQLds ? 16 * NRB * D * 2 : 16];
  if constexpr (kQLds) {
    constexpr int kChunks = 16 * NRB * (D / 8);  // 16-byte chunks of the 64 rows
    for (int ci = tid; ci < kChunks; ci += NW * 64) {
      const int rr = ci / (D / 8), cc = ci % (D / 8);
      const int rowq = row0 + rr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rowq < rows_b) {
        const int iq = fdiv(rowq, p.fd_hpu);
        const long n = row_of(iq, hq0 + rowq - iq * p.heads_per_unit);
        v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + n * hd)[cc];
      }
      *reinterpret_cast<uint4*>(s_q + rr * (D * 2) + ((cc ^ swz(rr & 15)) * 16)) = v;
    }
    __syncthreads();
  }

  f4_t acc[NRB][DB];  // O blocks
  float m[NRB];           // reference max of row n16 of block r (S^T layout), log2 units
  float l32[NRB];         // float32 sum of this lane's probabilities (row n16)
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[r][db] = (f4_t){0.f, 0.f, 0.f, 0.f};
    m[r] = -INFINITY;
    l32[r] = 0.f;
  }

  const long row_stride = PAGED ? (long)p.hkv * kvd : (long)kvd;
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(p.v);
  const int voff = int(n16 * row_stride * 2);  // key n16 of the tile

  // Per-wave slots during the loop (V tile, then the K tile when it goes
  // through LDS too); the same bytes hold the waves' partial outputs
  // (NW x 16 rows x D floats) for the merge.
  constexpr int kSlot = kTile * ROWB * (kDma ? 2 : 1);
  constexpr int kStage = NW * kSlot;
  constexpr int kMerge = NW * 16 * D * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kStage > kMerge ? kStage : kMerge];
  // Each wave's K tile sits right after its V tile, so the two share
  // address registers (a 4 KB immediate offset at D = 128).
  uint8_t* const my_v = s_buf + wave * kSlot;
  uint8_t* const my_k = my_v + kTile * ROWB;  // (direct-to-LDS tiles only)
  typedef __attribute__((address_space(3))) s4_t* lds_s4_ptr;
  const uint32_t v_wr = uint32_t(n16 * ROWB);  // row of this lane's V bytes (unswizzled)
  const int f_wr = swz(n16);  // chunk XOR of row n16
  // transposed read of d block db: lane 16g + 4i + q reads key 4g+i, d 16db + 4q .. +3
  const uint32_t v_rd = uint32_t((4 * g + ((lane & 15) >> 2)) * ROWB + (lane & 3) * 8);
  // swizzled: row r = 4g+i, chunk 2db + (q>>1) lands at chunk
  // 2(db ^ (swz(r) >> 1)) + ((q>>1) ^ (swz(r) & 1))
  const int r_rd = 4 * g + ((lane & 15) >> 2);
  const uint32_t v_rd_swz = uint32_t(r_rd * ROWB + (((lane & 3) >> 1) ^ (swz(r_rd) & 1)) * 16 +
                                     (lane & 1) * 8);
  const int i_rd = swz(r_rd) >> 1;

  auto tile_row0 = [&](int idx, int page) -> long {
    const int tt = t0 + (wave + idx * NW) * kTile;
    if constexpr (PAGED) {
      return ((long)page * p.page_size + tt - fdiv(tt, p.fd_page) * p.page_size) * p.hkv * kvd +
             (long)h * kvd;
    } else {
      return ((long)h * p.kv_len + tt) * kvd;
    }
  };

  auto issue = [&](Buf& bf, int idx, int page) {
    page = __builtin_amdgcn_readfirstlane(page);
    const int tt = t0 + (wave + idx * NW) * kTile;
    const long row0 = tile_row0(idx, page);
    const uint32_t bytes = uint32_t(min(kTile, t1 - tt) * row_stride * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + row0, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + row0, bytes);
    if constexpr (GEN == 2) {
      // element loads; a column past the head dim gets an offset past the
      // descriptor's range, which reads as zero
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint32_t wk[4], wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c0 = chunk(g, kb) * 8 + 2 * e;
          const int o0 = c0 < kvd ? int((n16 * row_stride + c0) * 2) : kPastEnd;
          const int o1 = c0 + 1 < kvd ? int((n16 * row_stride + c0 + 1) * 2) : kPastEnd;
          wk[e] = load2(rk, o0) | (load2(rk, o1) << 16);
          wv[e] = load2(rv, o0) | (load2(rv, o1) << 16);
        }
        bf.k[kb] = make_uint4(wk[0], wk[1], wk[2], wk[3]);
        bf.v[kb] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int ck = chunk(g, kb);
        const int off = (GEN == 0 || ck * 8 < kvd) ? voff + ck * 16 : kPastEnd;
        bf.k[kb] = load16(rk, off);
        bf.v[kb] = load16(rv, off);
      }
    }
  };

  auto load_q = [&]() {
#pragma unroll
    for (int r = 0; r < (kQLds ? 0 : NRB); ++r) {
      const int rowq = row0 + 16 * r + n16;  // packed row of this lane in block r of S^T
      const bool real = rowq < rows_b;
      long n = 0;
      if (real) {
        const int i = fdiv(rowq, p.fd_hpu);
        const int hq = hq0 + rowq - i * p.heads_per_unit;
        n = row_of(i, hq);
      }
      if constexpr (GEN == 2) {
        const uint16_t* qr = static_cast<const uint16_t*>(p.q) + n * hd;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c0 = chunk(g, kb) * 8 + 2 * e;
            const uint32_t lo = (real && c0 < hd) ? qr[c0] : 0u;
            const uint32_t hi = (real && c0 + 1 < hd) ? qr[c0 + 1] : 0u;
            w[e] = lo | (hi << 16);
          }
          qb[r][kb] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else {
        const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + n * hd);
        const int c0 = col0(rowq) / 8;  // first 16-byte chunk of this row's slice (head groups)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int c = chunk(g, kb) - c0;
          qb[r][kb] = (real && c >= 0 && (GEN == 0 || c * 8 < hd)) ? qp[c] : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  const float c = p.scale_log2;
  // A 16-bit probability rounded once has a relative error up to 2^-9
  // (bfloat16) or 2^-12 (fp16); times large, cancelling V rows that can
  // exceed the output tolerance (seen at 0.06 in bf16 and 0.015 in fp16
  // with 8x outlier K/V rows).  So P goes into P.V as the rounded value plus
  // the rounding of its residue (16 or 22 significant bits together), in
  // one 16x16x32 product per d block: a lane's 8 k-values are its 4 keys'
  // rounded P and their 4 residues (A), against its 4 V values twice (B).
  // The keys keep the order of the score layout, so no lane exchange.  The
  // row sums then come from the float32 sum of the unrounded P.
  // Scores, online softmax and P.V of one tile: kq holds this lane's K
  // operand chunks, vop(db) returns the V operand of d block db.
  auto tile_math = [&](const uint4 (&kq)[KB], auto vop, int tt) {
    // S^T = K . Q^T for each row block (one K tile, NRB query blocks)
    f4_t s[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      s[r] = (f4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint4 qv;
        if constexpr (kQLds)  // row 16r + n16 has the chunk XOR of row n16
          qv = *reinterpret_cast<const uint4*>(s_q + (16 * r + n16) * (D * 2) +
                                               ((chunk(g, kb) ^ f_wr) * 16));
        else
          qv = qb[r][kb];
        s[r] = M::qk(kq[kb], qv, s[r]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[r][i] = (tt + 4 * g + i < lim[r]) ? s[r][i] : -INFINITY;
    }
    uint2 pa[NRB], pl[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      // row max over the tile, lazy reference update
      float mt = fmaxf(fmaxf(s[r][0], s[r][1]), fmaxf(s[r][2], s[r][3]));
      mt = across_rows<true>(mt) * c;
      const bool need = mt > m[r] + kHeadroom;
      if (__any(need)) {
        const float mnew = need ? mt : m[r];
        const float alpha = (mnew == m[r]) ? 1.f : fast_exp2(m[r] - mnew);  // -inf -> 0
        m[r] = mnew;
        l32[r] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = from_lane(alpha, 4 * g + i);  // O rows 4g+i live in lanes of row 4g+i
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[r][db][i] *= ai;
        }
      }
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = fast_exp2(fmaf(s[r][i], c, -m[r]));
        pr[i] = (s[r][i] == -INFINITY) ? 0.f : pr[i];
      }
      l32[r] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      pa[r] = make_uint2(M::pack(pr[0], pr[1]), M::pack(pr[2], pr[3]));
      const f2_t h01 = M::widen(pa[r].x), h23 = M::widen(pa[r].y);  // the rounding residue
      pl[r] = make_uint2(M::pack(pr[0] - h01[0], pr[1] - h01[1]),
                         M::pack(pr[2] - h23[0], pr[3] - h23[1]));
    }
    // O += P . V for each row block (one V operand per d block)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint2 vt = vop(db);
#pragma unroll
      for (int r = 0; r < NRB; ++r)
        acc[r][db] = M::qk(make_uint4(pa[r].x, pa[r].y, pl[r].x, pl[r].y),
                           make_uint4(vt.x, vt.y, vt.x, vt.y), acc[r][db]);
    }
  };
  // transposed read of d block db of the wave's staged V tile
  auto v_tr = [&](int db) -> uint2 {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4_ptr)(my_v + (kSwz ? v_rd_swz + ((db ^ i_rd) * 32) : v_rd + db * 32))));
  };
  auto process_tile = [&](const Buf& bf, int tt) {
    // stage V (row-major) for the transposed reads
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (kSwz) {
        *reinterpret_cast<uint4*>(my_v + n16 * ROWB + ((chunk(g, kb) ^ f_wr) * 16)) = bf.v[kb];
      } else {
        *reinterpret_cast<uint4*>(my_v + v_wr + chunk(g, kb) * 16) = bf.v[kb];
      }
    }
    tile_math(bf.k, v_tr, tt);
  };
  // Direct-to-LDS issue of tile idx: 1 KB per instruction, lane l landing
  // at byte 16 l of it, so lane l fetches the global chunk that the
  // swizzled layout puts there (row r's chunk c sits at c ^ f(r)).
  constexpr int kCPR = ROWB / 16;    // 16-byte chunks per staged row
  constexpr int kRPI = 1024 / ROWB;  // rows per load instruction
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // The appended keys of a tile (at most kMaxFusedNew rows): lane l holds
  // chunk l % kCPR of new row j * kNewPer + l / kCPR, fetched from k_new /
  // v_new with the tile's cache rows and put into the slot when it lands.
  constexpr int kNewPer = 64 / kCPR;
  constexpr int kNewPass = (kMaxFusedNew + kNewPer - 1) / kNewPer;
  uint4 nk[fused ? kNewPass : 1] = {}, nv[fused ? kNewPass : 1] = {};
  auto new_key = [&](int tt, int j) -> int {  // key of this lane's row j, or -1
    const int key = max(tt, Lc) + j * kNewPer + lane / kCPR;
    return key < min(tt + kTile, t1) && (GEN == 0 || (lane % kCPR) * 8 < kvd) ? key : -1;
  };
  auto fetch_new = [&](int tt) {
    const uint16_t* kn = static_cast<const uint16_t*>(p.k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(p.v_new);
#pragma unroll
    for (int j = 0; j < kNewPass; ++j) {
      const int key = new_key(tt, j);
      if (key >= 0) {
        const long src = ((long)(b * p.seq_add + key - Lc) * p.hkv + h) * kvd + (lane % kCPR) * 8;
        nk[j] = *reinterpret_cast<const uint4*>(kn + src);
        nv[j] = *reinterpret_cast<const uint4*>(vn + src);
      }
    }
  };
  auto put_new = [&](int idx, int page, bool writer) {
    const int tt = t0 + (wave + idx * NW) * kTile;
    // the appending entry point takes a writable cache (k_cache, v_cache)
    uint16_t* kc = static_cast<uint16_t*>(const_cast<void*>(p.k));
    uint16_t* vc = static_cast<uint16_t*>(const_cast<void*>(p.v));
    const long row0 = tile_row0(idx, page);
#pragma unroll
    for (int j = 0; j < kNewPass; ++j) {
      const int key = new_key(tt, j);
      if (key >= 0) {
        const int r = key - tt, c = lane % kCPR;
        const int off = r * ROWB + ((c ^ swz(r)) * 16);
        *reinterpret_cast<uint4*>(my_k + off) = nk[j];
        *reinterpret_cast<uint4*>(my_v + off) = nv[j];
        if (writer && key < p.max_pages * p.page_size) {
          const long dst = row0 + (long)r * row_stride + c * 8;
          *reinterpret_cast<uint4*>(kc + dst) = nk[j];
          *reinterpret_cast<uint4*>(vc + dst) = nv[j];
        }
      }
    }
  };
  auto issue_dma = [&](int idx, int page) {
    page = __builtin_amdgcn_readfirstlane(page);
    const int tt = t0 + (wave + idx * NW) * kTile;
    const long row0 = tile_row0(idx, page);
    // rows past the cached keys read as zero; appended ones come from k_new
    const uint32_t bytes =
        uint32_t((fused ? max(0, min(kTile, min(t1, Lc) - tt)) : min(kTile, t1 - tt)) * row_stride * 2);
    if constexpr (fused) {
      if (tt + kTile > Lc) fetch_new(tt);
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + row0, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + row0, bytes);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int row = j * kRPI + lane / kCPR;
      const int ch = (lane % kCPR) ^ swz(row);
      const int off = (GEN == 0 || ch * 8 < kvd) ? int(row * row_stride * 2) + ch * 16 : kPastEnd;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(my_k + j * 1024), 16, off, 0, 0, kStream);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(my_v + j * 1024), 16, off, 0, 0, kStream);
    }
  };
  auto process = [&](const Buf& bf, int idx) {
    const int tt = t0 + (wave + idx * NW) * kTile;
    process_tile(bf, tt);
  };

  // ---- main loop ----------------------------------------------------------
  if constexpr (kDma) {
    // s_waitcnt immediates: vmcnt(0) alone, lgkmcnt(0) alone
    constexpr int kWaitVm0 = 0x0F70, kWaitLgkm0 = 0xC07F;
    // The first tile goes out before the loop: there the compiler waits for
    // the page ids alone, not for the query rows loaded after them.
    if (my_tiles > 0) issue_dma(0, __builtin_amdgcn_readlane(pages, 0));
    load_q();
    const bool writer = fused && rb == 0 && hq0 % p.group == 0;
    for (int cb = 0; cb < my_tiles; cb += 64) {
      auto page_at = [&](int i) { return __builtin_amdgcn_readlane(pages, i); };
      if (cb > 0) {
        pages = load_pages(cb);
        issue_dma(cb, page_at(0));
      }
      const int n = min(64, my_tiles - cb);
      for (int i = 0; i < n; ++i) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);  // tile i has landed in the slot
        if constexpr (fused) {
          if (t0 + (wave + (cb + i) * NW) * kTile + kTile > Lc) put_new(cb + i, page_at(i), writer);
        }
        uint4 kq[KB];
        uint2 vt[DB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          kq[kb] = *reinterpret_cast<const uint4*>(my_k + n16 * ROWB + ((chunk(g, kb) ^ f_wr) * 16));
#pragma unroll
        for (int db = 0; db < DB; ++db) vt[db] = v_tr(db);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot is read out before it is refilled
        if (i + 1 < n) issue_dma(cb + i + 1, page_at(i + 1));
        tile_math(kq, [&](int db) { return vt[db]; }, t0 + (wave + (cb + i) * NW) * kTile);
      }
    }
  } else {  // NBUF tiles in a register ring
  load_q();
  for (int cb = 0; cb < my_tiles; cb += 64) {
    if (cb > 0) pages = load_pages(cb);
    const int n = min(64, my_tiles - cb);
    const int last = n - 1;
    auto page_at = [&](int i) { return __builtin_amdgcn_readlane(pages, i); };
    Buf ring[NBUF > 0 ? NBUF : 1];
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
  }

  // partial buffers of a split call (the host keeps them below 4 GiB)
  const __amdgpu_buffer_rsrc_t r_opart =
      make_rsrc(p.o_part, uint32_t(min<long>((long)p.num_splits * p.nrows * hd * 4, 0xFFFFFFFFl)));
  const __amdgpu_buffer_rsrc_t r_lpart =
      make_rsrc(p.lse_part, uint32_t(min<long>((long)p.num_splits * p.nrows * 4, 0xFFFFFFFFl)));

  // ---- merge the waves through LDS and write, one 16-row block at a time --
  // O layout: lane l holds rows 4g..4g+3, columns 16db + n16.  m and the
  // probability sum of row r are held by lanes with n16 == r.  Wave w's
  // partial enters row r with weight 2^(m_w - M) / sum_w' 2^(m_w' - M) l_w'
  // (M = max_w m_w), so an output element is a plain weighted sum over the
  // waves, VEC columns per thread.  Each thread derives its row's weights
  // from the waves' m and l (two 16-byte LDS reads per 4 waves) after the
  // one barrier that publishes them: measured against a separate weights
  // pass between two barriers (us): paged GQA-4 bf16 23.50 -> 23.35, long
  // context 25.96 -> 25.77, small-q MHA 15.16 -> 15.07.
  constexpr int RMAX = 16;
  constexpr int VEC = GEN == 2 ? 1 : 4;  // head dims of the 16-byte kernels are multiples of 8
  float* s_acc = reinterpret_cast<float*>(s_buf);  // [NW][16][D]
  // row r's reference maxima and float32 probability sums, one per wave
  __shared__ __attribute__((aligned(16))) float s_m[RMAX][NW];
  __shared__ __attribute__((aligned(16))) float s_l32[RMAX][NW];
#pragma unroll
  for (int blk = 0; blk < NRB; ++blk) {
    const int rows_here = min(RMAX, rows_b - row0 - 16 * blk);
    if (rows_here <= 0) break;
    // The merge rows reuse the tile slots.  With direct-to-LDS tiles, wave
    // w's rows of the first block (16 x D floats) occupy exactly its own
    // slot (16 K and 16 V rows of D 16-bit values), which it has read out,
    // so only a later block (or a register-ring kernel, whose slots are
    // smaller) waits for the other waves first.
    if (!kDma || blk > 0) __syncthreads();
    const float l32b = across_rows<false>(l32[blk]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      if (r < rows_here) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          s_acc[((long)wave * RMAX + r) * D + db * 16 + n16] = acc[blk][db][i];
      }
    }
    if (g == 0 && n16 < rows_here) {
      s_m[n16][wave] = m[blk];
      s_l32[n16][wave] = l32b;
    }
    __syncthreads();
    for (int t = tid * VEC; t < rows_here * hd; t += NW * 64 * VEC) {
      const int r = t / hd;
      const int d = t % hd;  // a multiple of VEC, and VEC divides hd
      const int pr = row0 + 16 * blk + r;
      const int col = col0(pr) + d;
      // Row r's weights, computed by each of its threads from the waves'
      // maxima and sums (16-byte LDS reads): wave w's partial enters with
      // weight 2^(m_w - M) / sum_w' 2^(m_w' - M) l_w', M = max_w m_w.
      float mw[NW], lw[NW];
#pragma unroll
      for (int w = 0; w < NW; w += 4) {
        const f4_t a = *reinterpret_cast<const f4_t*>(&s_m[r][w]);
        const f4_t c4 = *reinterpret_cast<const f4_t*>(&s_l32[r][w]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mw[w + e] = a[e];
          lw[w + e] = c4[e];
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mw[w]);
      float f[NW], fl[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        f[w] = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - mx);
        fl[w] = f[w] * lw[w];
      }
#pragma unroll
      for (int h = 1; h < NW; h <<= 1)
#pragma unroll
        for (int w = 0; w < NW; w += 2 * h) fl[w] += fl[w + h];
      const bool empty = mx == -INFINITY;  // no wave saw a key of this row
      const float inv = empty ? 0.f : 1.f / fl[0];
      const float lse_r = empty ? -INFINITY : (mx + log2f(fl[0])) * kLn2;
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = f[w] * inv;
        const float* a = s_acc + ((long)w * RMAX + r) * D + col;
        if constexpr (VEC == 4) {
          const f4_t v = *reinterpret_cast<const f4_t*>(a);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = fmaf(wt, v[e], o[e]);
        } else {
          o[0] = fmaf(wt, a[0], o[0]);
        }
      }
      const int i = fdiv(pr, p.fd_hpu);
      const int hq = hq0 + pr - i * p.heads_per_unit;
      const long nrow = row_of(i, hq);
      if (direct) {
        uint16_t* dst = static_cast<uint16_t*>(p.out) + nrow * hd + d;
        if constexpr (VEC == 4)
          *reinterpret_cast<uint2*>(dst) = make_uint2(M::pack(o[0], o[1]), M::pack(o[2], o[3]));
        else
          dst[0] = M::round(o[0]);
        if (d == 0 && p.lse) p.lse[lse_of(i, hq)] = lse_r;
      } else {  // write-through stores: the merging workgroup may sit on another XCD
        const uint32_t off = uint32_t(((long)split * p.nrows + nrow) * hd + d) * 4u;
        if constexpr (VEC == 4)
          publish4(r_opart, off, (f4_t){o[0], o[1], o[2], o[3]});
        else
          publish(r_opart, off, o[0]);
        if (d == 0) publish(r_lpart, uint32_t((long)split * p.nrows + nrow) * 4u, lse_r);
      }
    }
  }
  if (direct) return;

  // ---- fused combine: the last split of a unit to finish merges all ------
  // Every split that holds keys writes its partials through to memory
  // (system-coherent stores, no cache maintenance), waits until they are
  // complete, then bumps the unit's arrival counter; the workgroup that sees
  // the other nsplit-1 arrivals before its own reads the partials back with
  // cache-bypassing loads and merges them, writes the output and rearms the
  // counter at zero for the next call.
  // Each thread owns VEC adjacent output columns of a row.  It reads the
  // partial LSE and the VEC partial outputs (one 16-byte load) of kBatch
  // splits in one round of independent loads and folds each batch with the
  // max-shifted log-sum-exp rule (running maximum, rescaled sums); the
  // lanes of a row load the same LSE addresses, which a wave's load
  // coalesces.
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int kBatch = 16;
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();
  const int unit = (b * p.unit_heads + uh) * p.row_blocks + rb;
  int* const counter = p.counters + (long)unit * kCounterStride;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
             nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  const int S = nsplit;
  const int rows_unit = min(16 * NRB, rows_b - row0);
  for (int t = tid * VEC; t < rows_unit * hd; t += NW * 64 * VEC) {
    const int r = t / hd;
    const int d = t % hd;
    const int pr = row0 + r;
    const int i = fdiv(pr, p.fd_hpu);
    const int hq = hq0 + pr - i * p.heads_per_unit;
    const long nrow = row_of(i, hq);
    float mx = -INFINITY, wsum = 0.f;  // log2 units
    float acc_o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc_o[e] = 0.f;
    for (int sp0 = 0; sp0 < S; sp0 += kBatch) {
      float ls[kBatch];
      f4_t o[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {  // unconditional loads (clamped index), no branches
        const int sp = min(sp0 + k, S - 1);
        ls[k] = fetch(r_lpart, uint32_t((long)sp * p.nrows + nrow) * 4u);
        const uint32_t off = uint32_t(((long)sp * p.nrows + nrow) * hd + d) * 4u;
        if constexpr (VEC == 4)
          o[k] = fetch4(r_opart, off);
        else
          o[k][0] = fetch(r_opart, off);
      }
      float bm = -INFINITY;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        ls[k] = sp0 + k < S ? ls[k] * kLog2e : -INFINITY;
        bm = fmaxf(bm, ls[k]);
      }
      const float mn = fmaxf(mx, bm);  // stays -inf while no split had keys
      const float alpha = mx == mn ? 1.f : fast_exp2(mx - mn);
      wsum *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc_o[e] *= alpha;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float w = ls[k] == -INFINITY ? 0.f : fast_exp2(ls[k] - mn);
        wsum += w;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc_o[e] = fmaf(w, o[k][e], acc_o[e]);
      }
      mx = mn;
    }
    const float inv = mx == -INFINITY ? 0.f : 1.f / wsum;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + nrow * hd + d;
    if constexpr (VEC == 4)
      *reinterpret_cast<uint2*>(dst) = make_uint2(M::pack(acc_o[0] * inv, acc_o[1] * inv),
                                                  M::pack(acc_o[2] * inv, acc_o[3] * inv));
    else
      dst[0] = M::round(acc_o[0] * inv);
    if (d == 0 && p.lse)
      p.lse[lse_of(i, hq)] = mx == -INFINITY ? -INFINITY : (mx + log2f(wsum)) * kLn2;
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Work lists.
// Split-major (extra_blocks == 0): workgroups run split-major from the last
// split down.  The last splits exist only for the longest sequences, so
// their work is dispatched first and the short remainder fills in behind
// it; a split past a sequence's last key returns at once.
// Compact (extra_blocks > 0, a ragged batch whose length sum the caller
// gave): the first extra_blocks workgroups take the splits 1 .. n_b - 1 of
// the sequences that need them, from a list each of them builds from the
// lengths; then one workgroup per unit runs split 0.  The empty splits of
// short sequences are never launched.  The host sizes extra_blocks from the
// length sum so that each takes one item; with a smaller count (a wrong
// sum) they loop over the items, which stays correct.
// In both, when the grid takes more than one round of workgroups, the
// batch is small (kMaxRankBatch) and its sequences long (kMinRankKeys),
// split 0 (the one every sequence has) runs its sequences longest first (a
// longest-processing-time order): each of its workgroups ranks the batch
// by length, ties by index.
// The row blocks of one (sequence, head unit) sit 8 workgroups apart:
// workgroups are dealt to the 8 XCDs round-robin, so they land on the same
// XCD, close in time, and the second one to read a KV tile finds it in
// that XCD's L2.  Head units go in groups of 8: workgroup g*8*row_blocks +
// rb*n + i runs a head unit 8g + j, row block rb, where n = 8 except in the
// last, shorter group.  Within a full group the unit follows the XCD
// (paged calls): XCD x reads the units whose slice of each key row starts
// at a byte offset with bit 9 equal to bit 0 of x and, where the slice
// offsets reach it, bit 10 equal to bit 1 of x.  Found by sweeping head ->
// XCD permutations (MI355X, paged GQA-4 bf16 d 128, us): identity (KV
// head h on XCD h) 24.7, the kept map 23.7, the other maps tried 24.1 to
// 24.9; 64 sequences of 2048 keys 87.3 -> 84.0; fp16 d 64 (128-byte
// slices, no head pairs) 51.7 -> 51.2.  Otherwise j = i.
// EXTRA: a kernel built for the compact list (its loop over items costs
// about ten VGPRs, so the split-major kernels are built without it).
template <int DT, int D, int NW, int NBUF, bool PAGED, int GEN, int NRB, bool EXTRA, bool APP>
__global__ __launch_bounds__(NW * 64) void mfma_split_kernel(const SplitParams p) {
  static_assert(PAGED || !EXTRA, "the compact list is for paged calls");
  if constexpr (PAGED && !EXTRA) {
    // One scalar load per 60 bytes of the argument block, all issued before
    // any is used: every cache line of the block arrives in one round trip,
    // and the argument loads that follow hit the scalar cache (the compiler
    // otherwise fetches the lines in three dependent rounds).  Measured
    // (us): paged GQA-4 bf16 23.34 -> 23.07, long context 25.81 -> 25.54;
    // the compact-list and dense kernels, not touched, gained nothing from
    // it (ragged 46.42 -> 46.62, dense decode 4.86 -> 4.91, small-q MHA
    // 15.07 -> 15.00).
    const uint32_t* a = reinterpret_cast<const uint32_t*>(&p);
    static_assert(sizeof(SplitParams) <= 75 * 4, "six loads cover the argument block");
    const uint32_t w0 = a[0], w1 = a[15], w2 = a[30], w3 = a[45], w4 = a[60],
                   w5 = a[sizeof(SplitParams) / 4 - 1];
    asm volatile("" ::"s"(w0), "s"(w1), "s"(w2), "s"(w3), "s"(w4), "s"(w5));
  }
  __shared__ __attribute__((aligned(16))) int s_seq[kMaxOrderBatch + 1];
  if (EXTRA && int(blockIdx.x) < p.extra_blocks) {
    // Extra items of sequence b: (n_b - 1) x head units x row blocks, with
    // n_b = ceil(L_b / split_keys) splits (at most num_splits, as in the
    // split-major grid).  s_seq[b] = items of sequences before b (an
    // exclusive prefix); s_seq[batch] = all items.
    const int per_seq = p.unit_heads * p.row_blocks;
    for (int i = threadIdx.x; i < p.batch; i += NW * 64) {
      const int L = p.seqlens[i] + p.seq_add;
      const int more = L > p.split_keys ? fdiv(L - 1, p.fd_split_keys) : 0;
      s_seq[i + 1] = min(more, p.num_splits - 1) * per_seq;
    }
    if (threadIdx.x == 0) s_seq[0] = 0;
    __syncthreads();
    if (threadIdx.x < 64) {  // wave 0 scans s_seq[1 .. batch] in place, 64 chunks
      const int lane = threadIdx.x;
      const int chunk = (p.batch + 63) / 64;
      const int lo = 1 + min(p.batch, lane * chunk);
      const int hi = 1 + min(p.batch, (lane + 1) * chunk);
      int run = 0;
      for (int i = lo; i < hi; ++i) run += s_seq[i];
      int incl = run;
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      run = incl - run;
      for (int i = lo; i < hi; ++i) {
        run += s_seq[i];
        s_seq[i] = run;
      }
    }
    __syncthreads();
    const int total = s_seq[p.batch];
    for (int item = int(blockIdx.x); item < total; item += p.extra_blocks) {
      int lo = 0, hi = p.batch;  // s_seq[lo] <= item < s_seq[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_seq[mid] <= item) lo = mid; else hi = mid;
      }
      // every lane found the same values: keep them scalar
      const int bs = __builtin_amdgcn_readfirstlane(lo);
      const int r = __builtin_amdgcn_readfirstlane(item - s_seq[lo]);
      // The thread index passes through an empty asm, so that nothing the
      // unit derives from it is hoisted out of this loop and kept live
      // across it (that raised the kernel's VGPR count by a third).
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int rem = r % per_seq;
      split_unit<DT, D, NW, NBUF, PAGED, GEN, NRB, APP>(p, 1 + r / per_seq, bs, rem % p.unit_heads,
                                                  rem / p.unit_heads, tid);
      __syncthreads();  // the unit's LDS is reused by the next one
    }
    return;
  }
  const int units = p.batch * p.unit_heads * p.row_blocks;
  const int id0 = int(blockIdx.x) - (EXTRA ? p.extra_blocks : 0);
  const int sq = EXTRA ? 0 : fdiv(id0, p.fd_units);
  const int split = EXTRA ? 0 : p.num_splits - 1 - sq;
  int rb, bid;
  {
    const int pairs = p.batch * p.unit_heads;
    const int id = id0 - sq * units;
    const int grp = p.row_blocks == 1 ? id >> 3 : id / (8 * p.row_blocks);
    const int rem = id - grp * 8 * p.row_blocks;
    const int n = min(8, pairs - grp * 8);
    rb = n == 8 ? rem >> 3 : rem / n;
    int j = rem - rb * n;
    if constexpr (PAGED && (GEN == 0 || GEN == 3) && (D == 128 || D == 64)) {
      // A unit's slice of a key row is D * 2 bytes (256 or 128) at offset
      // h * D * 2, h the unit's KV head (head group).  Packed, with a
      // multiple of kPer units per sequence (key rows of at least 1 KiB),
      // member m of a full group of 8 has its slice at offset bits 8-10
      // (D 128) or 7-9 (D 64) equal to the bits of m.  XCD x takes the
      // member whose offset bit 9 is bit 0 of x, and (D 128) bit 10 bit 1.
      constexpr int kPer = 1024 / (D * 2);
      if (n == 8 && p.heads_per_unit == p.group && p.unit_heads % kPer == 0) {
        const int x = int(blockIdx.x) & 7;
        j = D == 128 ? 2 * (x & 3) + (x >> 2) : 4 * (x & 1) + (x >> 1);
      }
    }
    bid = grp * 8 + j;
  }
  int b = fdiv(bid, p.fd_unit_heads);
  const int uh = bid - b * p.unit_heads;
  if (PAGED && p.by_length && split == 0) {
    // Rank of sequence i: the sequences longer than it, plus the equally
    // long ones before it.  Four adjacent threads share a sequence, each
    // comparing a quarter of the batch 4 lengths per LDS read (lengths
    // padded to a multiple of 16 with -1, below every real length), and
    // add their counts with two shuffles.
    int* const s_len = s_seq;
    __shared__ int s_pick;
    const int bp = (p.batch + 15) & ~15;  // <= kMaxRankBatch <= kMaxOrderBatch
    for (int i = threadIdx.x; i < bp; i += NW * 64) s_len[i] = i < p.batch ? max(p.seqlens[i], 0) : -1;
    __syncthreads();
    const int q = threadIdx.x & 3;
    const int quarter = bp >> 2;  // a multiple of 4
    for (int i0 = 0; i0 < p.batch; i0 += NW * 16) {
      const int i = i0 + int(threadIdx.x >> 2);
      const int li = s_len[min(i, bp - 1)];
      int rank = 0;
      for (int j = q * quarter; j < (q + 1) * quarter; j += 4) {
        const int4 v = *reinterpret_cast<const int4*>(s_len + j);
        rank += (v.x > li) + (v.x == li && j < i) + (v.y > li) + (v.y == li && j + 1 < i) +
                (v.z > li) + (v.z == li && j + 2 < i) + (v.w > li) + (v.w == li && j + 3 < i);
      }
      rank += __shfl_xor(rank, 1);
      rank += __shfl_xor(rank, 2);
      if (q == 0 && i < p.batch && rank == b) s_pick = i;
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(s_pick);
  }
  split_unit<DT, D, NW, NBUF, PAGED, GEN, NRB, APP>(p, split, b, uh, rb, threadIdx.x);
}

// Waves per workgroup: 8 up to D = 128, 4 at D = 256 (accumulators and
// the merge buffer).  Tiles of 16-byte chunks with at least 8 chunks a row
// go straight to LDS (NBUF = 0).  The others use a register ring: two
// tiles per wave up to D = 64, one above (two would spill).
// Measured, ring against direct-to-LDS (paged bf16 GQA-4 decode, d 128):
// 28.2 vs 27.4 us; with 32 query rows per unit (causal q_len 8): 37.2 vs
// 34.7 us.  Direct-to-LDS with 16 waves, or two tiles per wave step, was
// slower (28.2 and 28.1 us).
// Workgroups of a kernel resident per CU (looked up once per kernel, on the
// first GPU that launches it: every GPU of a process is taken to be alike).
template <auto K>
int resident(int nw) {
  static const int n = [nw] {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(K),
                                                     nw * 64, 0) != hipSuccess)
      return 0;
    return blocks;
  }();
  return n;
}

template <int DT, int D, bool PAGED, int GEN, int NRB>
hipError_t launch_mfma_k(const SplitParams& prm, int grid, hipStream_t s,
                         const AppendParams* append, bool* in_kernel) {
  constexpr bool kDirect = GEN != 2 && D >= 64;
  constexpr int NW = D <= 128 ? 8 : 4;
  constexpr int NBUF = kDirect ? 0 : D >= 128 ? 1 : 2;
  // Appended keys: a direct-to-LDS kernel takes a few per sequence itself
  // (one launch instead of two) where its appending copy keeps the plain
  // one's resident workgroups, or the grid fits in one round of them;
  // otherwise the append kernel runs first.
  if (append && append->new_len > 0) {
    if constexpr (kDirect && PAGED) {
      if (append->new_len <= kMaxFusedNew && !prm.cu_q) {
        const bool ex = prm.extra_blocks > 0;  // the compact list's kernels
        constexpr auto kPlain = mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, false, false>;
        constexpr auto kPlainEx = mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, true, false>;
        constexpr auto kApp = mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, false, true>;
        constexpr auto kAppEx = mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, true, true>;
        const int plain = ex ? resident<kPlainEx>(NW) : resident<kPlain>(NW);
        const int fused = ex ? resident<kAppEx>(NW) : resident<kApp>(NW);
        if (fused > 0 && (fused >= plain || grid <= (long)fused * append->num_cus)) {
          SplitParams p = prm;
          p.k_new = append->k_new;
          p.v_new = append->v_new;
          if (ex)
            hipLaunchKernelGGL((mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, true, true>),
                               dim3(grid), dim3(NW * 64), 0, s, p);
          else
            hipLaunchKernelGGL((mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, false, true>),
                               dim3(grid), dim3(NW * 64), 0, s, p);
          if (in_kernel) *in_kernel = true;
          return hipGetLastError();
        }
      }
    }
    const hipError_t e = launch_append(*append, s);
    if (e != hipSuccess) return e;
  }
  SplitParams p = prm;
  p.k_new = p.v_new = nullptr;
  if (p.extra_blocks > 0) {
    if constexpr (PAGED) {
      hipLaunchKernelGGL((mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, true, false>),
                         dim3(grid), dim3(NW * 64), 0, s, p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((mfma_split_kernel<DT, D, NW, NBUF, PAGED, GEN, NRB, false, false>),
                     dim3(grid), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

// Two or four 16-row blocks per workgroup exist for the 16-byte-load
// kernels at head dims 64 and 128 (the planner asks for them only there);
// four at 128 read Q from LDS.
template <int DT, int D, bool PAGED, int GEN>
hipError_t launch_mfma_d(const SplitParams& p, int grid, hipStream_t s, const AppendParams* a,
                         bool* ik) {
  if constexpr (GEN == 0 && (D == 64 || D == 128)) {
    if (p.nrb == 2) return launch_mfma_k<DT, D, PAGED, GEN, 2>(p, grid, s, a, ik);
  }
  if constexpr (GEN == 0 && (D == 64 || D == 128)) {
    if (p.nrb == 4) return launch_mfma_k<DT, D, PAGED, GEN, 4>(p, grid, s, a, ik);
  }
  if (p.nrb != 1) return hipErrorInvalidValue;
  return launch_mfma_k<DT, D, PAGED, GEN, 1>(p, grid, s, a, ik);
}

template <int DT, bool PAGED>
hipError_t launch_mfma_dt(const SplitParams& p, int grid, hipStream_t s, const AppendParams* a,
                          bool* ik) {
  const int d = p.head_dim;
  if (p.head_group > 1) {  // 2 head-dim-64 or 4 head-dim-32 KV heads per 128-wide row
    if constexpr (PAGED) {
      if (p.head_group * d == 128 && p.nrb == 1)
        return launch_mfma_k<DT, 128, PAGED, 3, 1>(p, grid, s, a, ik);
    }
    return hipErrorInvalidValue;
  }
  switch (d) {
    case 32: return launch_mfma_d<DT, 32, PAGED, 0>(p, grid, s, a, ik);
    case 64: return launch_mfma_d<DT, 64, PAGED, 0>(p, grid, s, a, ik);
    case 128: return launch_mfma_d<DT, 128, PAGED, 0>(p, grid, s, a, ik);
    case 256: return launch_mfma_d<DT, 256, PAGED, 0>(p, grid, s, a, ik);
  }
  if (d % 8 == 0) {  // rows stay 16-byte aligned
    if (d <= 32) return launch_mfma_d<DT, 32, PAGED, 1>(p, grid, s, a, ik);
    if (d <= 64) return launch_mfma_d<DT, 64, PAGED, 1>(p, grid, s, a, ik);
    if (d <= 128) return launch_mfma_d<DT, 128, PAGED, 1>(p, grid, s, a, ik);
    if (d <= 256) return launch_mfma_d<DT, 256, PAGED, 1>(p, grid, s, a, ik);
    return hipErrorInvalidValue;
  }
  if (d <= 32) return launch_mfma_d<DT, 32, PAGED, 2>(p, grid, s, a, ik);
  if (d <= 64) return launch_mfma_d<DT, 64, PAGED, 2>(p, grid, s, a, ik);
  if (d <= 128) return launch_mfma_d<DT, 128, PAGED, 2>(p, grid, s, a, ik);
  if (d <= 256) return launch_mfma_d<DT, 256, PAGED, 2>(p, grid, s, a, ik);
  return hipErrorInvalidValue;
}

}  // namespace

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  const int l = d <= 1 ? 0 : 32 - __builtin_clz(d - 1);  // ceil(log2 d)
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

hipError_t launch_split_mfma(int dtype, bool paged, const SplitParams& prm, int grid,
                             hipStream_t s, const AppendParams* append, bool* in_kernel) {
  if (grid <= 0) return append && append->new_len > 0 ? launch_append(*append, s) : hipSuccess;
  SplitParams p = prm;
  auto pos = [](long v) { return uint32_t(v > 1 ? v : 1); };
  p.fd_units = make_fastdiv(pos((long)p.batch * p.unit_heads * p.row_blocks));
  p.fd_unit_heads = make_fastdiv(pos(p.unit_heads));
  p.fd_group = make_fastdiv(pos(p.group));
  p.fd_hpu = make_fastdiv(pos(p.heads_per_unit));
  p.fd_page = make_fastdiv(pos(p.page_size));
  p.fd_split_keys = make_fastdiv(pos(p.split_keys));
  p.fd_gq = make_fastdiv(pos(p.head_group > 1 ? (long)p.heads_per_unit * p.head_dim / 128 : 1));
  if (paged)
    return dtype == 1 ? launch_mfma_dt<1, true>(p, grid, s, append, in_kernel)
                      : launch_mfma_dt<0, true>(p, grid, s, append, in_kernel);
  return dtype == 1 ? launch_mfma_dt<1, false>(p, grid, s, append, in_kernel)
                    : launch_mfma_dt<0, false>(p, grid, s, append, in_kernel);
}

}  // namespace skv
