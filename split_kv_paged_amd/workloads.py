"""Seeded synthetic inputs for decode / small-query attention.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic.  Its arrays feed both the GPU library and the CPU
oracle, so both see the same bytes: 16-bit tensors are returned as raw
``uint16`` bit patterns (float32 draws rounded to nearest-even).

Workload shapes follow the decode and small-query settings the pages test:
GQA ratios 2/4/8 and head_dim 64/128 (MXFlashAttn capability matrix), query
lengths 1-8 and KV lengths up to 16384 with 1023/1025-style tails (SmallQ
README, supported shapes), and the paged cache of the MXFlashAttn M1 kernel.

Paged recipe (draw order: lengths, page permutation, Q, K, V, outliers):
  * cache_seqlens from the workload's length rule;
  * the pool has sum(ceil(L_b / page)) live pages plus ``spare_pages`` spare
    pages; live pages get physical ids from a seeded permutation;
  * block_table[b, t] is the physical page of logical page t of sequence b;
    table slots past a sequence's last page point at a spare page;
  * Q, K, V ~ N(0, 1) in float32, rounded to the storage dtype;
  * optional outliers: a Bernoulli(p) mask over (pool slot, KV head) rows
    multiplies those K and V rows by a factor before rounding;
  * slots past L in each last page, and every spare page, hold NaN.
"""
from dataclasses import dataclass, field

import numpy as np

NAN16 = {"fp16": 0x7E00, "bf16": 0x7FC0}


def to_bits(x, dtype):
    """Round float32 values to fp16/bf16 (nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            rounded[nan] = NAN16["bf16"]
        return rounded
    raise ValueError("dtype must be fp16 or bf16")


def from_bits(bits, dtype):
    """float32 view of fp16/bf16 bit patterns (for display and bounds)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class PagedWorkload:
    name: str
    dtype: str
    batch: int
    q_len: int
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    page_size: int
    q: np.ndarray             # uint16 [B, q_len, Hq, d]
    k_cache: np.ndarray       # uint16 [num_pages, page, Hkv, d]
    v_cache: np.ndarray       # uint16 [num_pages, page, Hkv, d]
    block_table: np.ndarray   # int32 [B, max_pages]
    cache_seqlens: np.ndarray  # int32 [B]
    scale: float
    spare_page: int
    meta: dict = field(default_factory=dict)

    @property
    def max_seqlen_k(self):
        return int(self.cache_seqlens.max()) if self.batch else 0

    @property
    def kv_bytes(self):
        """Algorithmic KV bytes: valid tokens x Hkv x d x 2 (K and V) x 2 bytes."""
        return int(self.cache_seqlens.astype(np.int64).sum()) * self.num_heads_kv * \
            self.head_dim * 2 * 2


@dataclass
class DenseWorkload:
    name: str
    dtype: str
    num_heads_q: int
    num_heads_kv: int
    q_len: int
    kv_len: int
    head_dim: int
    q: np.ndarray   # uint16 [Hq, q_len, d]
    k: np.ndarray   # uint16 [Hkv, kv_len, d]
    v: np.ndarray   # uint16 [Hkv, kv_len, d]
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def kv_bytes(self):
        return self.kv_len * self.num_heads_kv * self.head_dim * 2 * 2


def make_paged(seed, dtype, batch, q_len, num_heads_q, num_heads_kv, head_dim, page_size,
               seqlens, outlier_p=0.0, outlier_scale=8.0, spare_pages=1, name="paged",
               scale=None):
    """Paged workload with the given per-sequence lengths (array or callable(rng))."""
    rng = np.random.default_rng(seed)
    if callable(seqlens):
        seqlens = seqlens(rng)
    seqlens = np.asarray(seqlens, dtype=np.int64).reshape(batch)
    n_pages_seq = (seqlens + page_size - 1) // page_size
    live = int(n_pages_seq.sum())
    num_pages = live + spare_pages
    perm = rng.permutation(live)
    spare = live  # first spare page id
    max_pages = max(1, int(n_pages_seq.max()) if batch else 1)
    bt = np.full((batch, max_pages), spare if spare_pages else 0, dtype=np.int32)
    pos = 0
    for b in range(batch):
        n = int(n_pages_seq[b])
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    q = rng.standard_normal((batch, q_len, num_heads_q, head_dim), dtype=np.float32)
    k = rng.standard_normal((num_pages, page_size, num_heads_kv, head_dim), dtype=np.float32)
    v = rng.standard_normal((num_pages, page_size, num_heads_kv, head_dim), dtype=np.float32)
    n_out = 0
    if outlier_p > 0:
        mask = rng.random((num_pages, page_size, num_heads_kv)) < outlier_p
        k[mask] *= outlier_scale
        v[mask] *= outlier_scale
        n_out = int(mask.sum())
    kb, vb = to_bits(k, dtype), to_bits(v, dtype)
    del k, v
    nan = NAN16[dtype]
    # poison: slots past L in each last page, and the spare pages
    for b in range(batch):
        L = int(seqlens[b])
        n = int(n_pages_seq[b])
        if n and L % page_size:
            p = bt[b, n - 1]
            kb[p, L % page_size:] = nan
            vb[p, L % page_size:] = nan
    if spare_pages:
        kb[live:] = nan
        vb[live:] = nan
    return PagedWorkload(
        name=name, dtype=dtype, batch=batch, q_len=q_len, num_heads_q=num_heads_q,
        num_heads_kv=num_heads_kv, head_dim=head_dim, page_size=page_size, q=to_bits(q, dtype),
        k_cache=kb, v_cache=vb, block_table=bt, cache_seqlens=seqlens.astype(np.int32),
        scale=(1.0 / np.sqrt(head_dim)) if scale is None else scale,
        spare_page=spare if spare_pages else -1,
        meta={"seed": seed, "num_pages": num_pages, "live_pages": live, "outlier_rows": n_out})


def make_dense(seed, dtype, num_heads_q, num_heads_kv, q_len, kv_len, head_dim, name="dense",
               scale=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((num_heads_q, q_len, head_dim), dtype=np.float32)
    k = rng.standard_normal((num_heads_kv, kv_len, head_dim), dtype=np.float32)
    v = rng.standard_normal((num_heads_kv, kv_len, head_dim), dtype=np.float32)
    return DenseWorkload(name=name, dtype=dtype, num_heads_q=num_heads_q,
                         num_heads_kv=num_heads_kv, q_len=q_len, kv_len=kv_len,
                         head_dim=head_dim, q=to_bits(q, dtype), k=to_bits(k, dtype),
                         v=to_bits(v, dtype),
                         scale=(1.0 / np.sqrt(head_dim)) if scale is None else scale,
                         meta={"seed": seed})


# ---- the five named workloads ------------------------------------------------

def c1_dense_decode():
    """Dense decode, fp16: Hq 8 / Hkv 2, d 64, qLen 1, kvLen 512, scale 1/8."""
    return make_dense(1001, "fp16", 8, 2, 1, 512, 64, name="dense_decode_fp16_h8g4_d64_L512",
                      scale=1.0 / 8.0)


C2_KV_LENS = (1, 1023, 1025, 3000, 4096)


def c2_smallq(kv_len):
    """Small-q dense MHA, fp16: 32 heads, qLen 4, d 128, given kvLen."""
    return make_dense(1002, "fp16", 32, 32, 4, kv_len, 128,
                      name="smallq_mha_fp16_h32_q4_d128_L%d" % kv_len)


def c3_paged_gqa4(spare_pages=1):
    """Paged GQA decode, bf16: B 32, Hq 32 / Hkv 8, d 128, qLen 1, page 16,
    L_b ~ U{900..1100}."""
    return make_paged(1003, "bf16", 32, 1, 32, 8, 128, 16,
                      lambda rng: rng.integers(900, 1101, size=32), spare_pages=spare_pages,
                      name="paged_decode_bf16_b32_h32g4_d128_L900-1100")


def c4_long(spare_pages=1):
    """Long-context split-KV decode, bf16: B 4, Hq 32 / Hkv 4, d 128, L 16384."""
    return make_paged(1004, "bf16", 4, 1, 32, 4, 128, 16, np.full(4, 16384),
                      spare_pages=spare_pages, name="paged_decode_bf16_b4_h32g8_d128_L16384")


def c5_lengths(rng, batch=128, max_len=8192):
    L = np.floor(np.exp(rng.uniform(0.0, np.log(max_len + 1), size=batch))).astype(np.int64)
    L = np.clip(L, 1, max_len)
    L[0], L[1], L[2] = 1, 1023, 1025
    return L


def c5_ragged(spare_pages=1):
    """Ragged large-batch paged decode, fp16: B 128, Hq 16 / Hkv 8, d 64,
    L log-uniform in [1, 8192] with 1/1023/1025 forced, 1% outlier rows x8."""
    return make_paged(1005, "fp16", 128, 1, 16, 8, 64, 16, c5_lengths, outlier_p=0.01,
                      outlier_scale=8.0, spare_pages=spare_pages,
                      name="paged_decode_fp16_b128_h16g2_d64_Lloguni1-8192")
