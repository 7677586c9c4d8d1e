/*
 * attn_probe.h -- C ABI of the read-only bandwidth probes (libattn_probe.so).
 *
 * Measurement helpers, not attention: they read the same KV bytes as a
 * decode call and do nothing else, so their speed is the empirical ceiling
 * the decode kernel is measured against.  Each probe folds what it read
 * into 32-bit checksums (sums of the little-endian 32-bit words, modulo
 * 2^32) so that no load can be dropped and a test can check that every
 * byte was read exactly once.
 *
 * Conventions: as in attn_decode.h.  Pointers are device pointers owned by
 * the caller; `stream` is a hipStream_t passed as void*; arguments are
 * checked on the host before anything is enqueued, and nothing is launched
 * on error.  Status codes are attn_status values.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "attn_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streams a[0 .. a_bytes) and then b[0 .. b_bytes) once, with 16-byte
 * non-temporal loads, num_blocks workgroups of 512 threads in a grid-stride
 * loop (each thread keeps four loads in flight).
 *   sums  uint32 [num_blocks]: workgroup w's sum of the words it read; the
 *         sum over w is the checksum of both ranges.
 * a_bytes and b_bytes are multiples of 16 (either may be 0, with a NULL
 * pointer); a, b 16-byte aligned, sums 4-byte aligned; 1 <= num_blocks <=
 * 65536.  Errors: ATTN_ERR_NULL, ATTN_ERR_ALIGN, ATTN_ERR_ARG (sizes),
 * ATTN_ERR_HIP (launch). */
attn_status attn_probe_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes,
                                   uint32_t* sums, int num_blocks, void* stream);

/* Reads the valid keys of a paged cache the way the decode kernel walks
 * it: split-major, one workgroup per (split s, sequence b, KV head h), each
 * of 16 waves taking the 16-key tiles w, w + 16, ... of the split's keys
 * [s * split_keys, min((s + 1) * split_keys, cache_seqlens[b])), one tile in
 * flight: per tile the 16 K rows and the 16 V rows of head h, with 16-byte
 * non-temporal loads.  Physical pages come from block_table, 64 tiles per
 * load.  Units go to XCDs as in the decode kernel (in each group of 8
 * consecutive (b, h), XCD x reads the slice whose offset in the key row has
 * bit 9 equal to bit 0 of x).  (Sixteen waves with one tile each read as
 * fast as the best of the deeper per-wave pipelines tried with 8 waves.)
 *   shape        as for attn_decode_fwd (q_len, num_heads_q, dtype and
 *                sum_seqlen_k are not used); head_dim 32, 64, 128 or 256
 *   k_cache,
 *   v_cache      [num_pages, page_size, num_heads_kv, head_dim], 16-bit
 *   split_keys   keys per split, a multiple of 16; 0 = no split
 *   sums         uint32 [S, batch, num_heads_kv] with S = ceil(max_seqlen_k
 *                / split_keys) (1 without split): the checksum of the K and
 *                V rows that split read; the sum over s is the checksum of
 *                keys j < L_b of head h
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE (as attn_decode_fwd), ATTN_ERR_ARG
 * (split_keys), ATTN_ERR_UNSUPPORTED (another head_dim, page_size not a
 * multiple of 16), ATTN_ERR_ALIGN, ATTN_ERR_HIP.  Device data (page ids,
 * lengths <= max_seqlen_k) is the caller's contract, as for
 * attn_decode_fwd. */
attn_status attn_probe_page_read(const attn_decode_shape* shape, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* cache_seqlens, int split_keys, uint32_t* sums,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
