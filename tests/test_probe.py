"""The read-only bandwidth probes (include/attn_probe.h): exports and host
argument checks on the CPU; on the GPU, their word-sum checksums against
numpy, which shows each probe read every byte of its range once and
nothing else (a key past a sequence's length would add the NaN bits that
poison the tail of its last page)."""
import ctypes
import os
import re
import sys

import numpy as np
import pytest

from split_kv_paged_amd import lib as L
from split_kv_paged_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_probe.h")


@pytest.fixture(scope="module")
def plib():
    from split_kv_paged_amd import probe
    if not os.path.exists(probe.LIB_PATH):
        from split_kv_paged_amd import build
        build.build()
    return probe.load()


def test_every_declared_probe_is_exported(plib):
    from split_kv_paged_amd import probe
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))
    assert set(declared) == set(probe.EXPORTS), declared
    out = os.popen("nm -D --defined-only %s" % probe.LIB_PATH).read()
    for name in declared:
        assert re.search(r"\bT %s\b" % name, out), name


def test_probe_arguments_rejected_before_launch(plib):
    P = ctypes.c_void_p
    a, s = P(0x10000), P(0x20000)  # never dereferenced: every call below fails validation
    assert plib.attn_probe_stream_read(a, 32, None, 0, None, 4, None) == 1       # NULL sums
    assert plib.attn_probe_stream_read(None, 32, None, 0, s, 4, None) == 1       # NULL a
    assert plib.attn_probe_stream_read(a, 24, None, 0, s, 4, None) == 4          # not 16-byte
    assert plib.attn_probe_stream_read(a, 32, None, 0, s, 0, None) == 4          # no blocks
    assert plib.attn_probe_stream_read(a, 32, None, 0, s, 65537, None) == 4
    assert plib.attn_probe_stream_read(P(0x10008), 32, None, 0, s, 4, None) == 6  # alignment
    shape = L.DecodeShape(2, 1, 8, 8, 128, 16, 4, 64, L.BF16, 0)
    args = [P(0x10000), P(0x20000), P(0x30000), P(0x40000), 0, P(0x50000), None]
    assert plib.attn_probe_page_read(None, *args) == 1
    assert plib.attn_probe_page_read(ctypes.byref(shape), None, *args[1:]) == 1
    bad = L.DecodeShape(2, 1, 8, 8, 128, 16, 4, 65, L.BF16, 0)  # max_seqlen_k > 4 pages
    assert plib.attn_probe_page_read(ctypes.byref(bad), *args) == 2
    odd = L.DecodeShape(2, 1, 8, 8, 96, 16, 4, 64, L.BF16, 0)
    assert plib.attn_probe_page_read(ctypes.byref(odd), *args) == 3
    pg = L.DecodeShape(2, 1, 8, 8, 128, 24, 4, 64, L.BF16, 0)
    assert plib.attn_probe_page_read(ctypes.byref(pg), *args) == 3
    mis = [P(0x10008)] + args[1:]
    assert plib.attn_probe_page_read(ctypes.byref(shape), *mis) == 6
    for split_keys in (-16, 8, 40):
        sk = args[:4] + [split_keys] + args[5:]
        assert plib.attn_probe_page_read(ctypes.byref(shape), *sk) == 4


def word_sum(bits16):
    """Sum mod 2^32 of the little-endian 32-bit words of 16-bit elements."""
    w = np.ascontiguousarray(bits16).view(np.uint32).astype(np.uint64)
    return int(w.sum() % (1 << 32))


def page_sums(wl):
    B, hkv = wl.batch, wl.num_heads_kv
    P = wl.page_size
    out = np.zeros((B, hkv), dtype=np.uint32)
    for b in range(B):
        Lb = int(wl.cache_seqlens[b])
        if Lb == 0:
            continue
        j = np.arange(Lb)
        pages = wl.block_table[b, j // P]
        for h in range(hkv):
            out[b, h] = (word_sum(wl.k_cache[pages, j % P, h, :]) +
                         word_sum(wl.v_cache[pages, j % P, h, :])) % (1 << 32)
    return out


def case(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.mark.gpu
@pytest.mark.parametrize("a_bytes,b_bytes,blocks", [
    (1 << 20, 48, 512), (16, 0, 1), (0, 4096, 3), (3 * 7919 * 16, 5 * 16, 1000)])
def test_stream_read_checksum(plib, a_bytes, b_bytes, blocks):
    import torch
    from split_kv_paged_amd import probe
    case("stream_read a=%d b=%d blocks=%d" % (a_bytes, b_bytes, blocks))
    rng = np.random.default_rng(a_bytes + b_bytes + blocks)
    ha = rng.integers(0, 1 << 16, a_bytes // 2 + 64, dtype=np.uint16)
    hb = rng.integers(0, 1 << 16, b_bytes // 2 + 64, dtype=np.uint16)
    da = torch.from_numpy(ha.view(np.int16)).cuda()
    db = torch.from_numpy(hb.view(np.int16)).cuda()
    sums = probe.stream_read(da, db, a_bytes, b_bytes, num_blocks=blocks)
    torch.cuda.synchronize()
    got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    want = (word_sum(ha[:a_bytes // 2]) + word_sum(hb[:b_bytes // 2])) % (1 << 32)
    assert got == want


PAGE_CASES = [
    # (seed, dtype, batch, hkv, head_dim, page_size, lengths, split_keys)
    (61, "bf16", 5, 4, 128, 16, [0, 1, 17, 1000, 513], 0),
    (62, "fp16", 3, 2, 64, 32, [16400, 31, 64], 0),  # > 64 tiles per wave: two page loads
    (63, "bf16", 2, 3, 256, 16, [300, 15], 0),
    (64, "fp16", 4, 1, 32, 48, [95, 96, 97, 1], 0),
    (65, "bf16", 4, 2, 128, 16, [1000, 0, 257, 16], 256),  # splits, some empty
    (66, "fp16", 2, 3, 64, 32, [5000, 4000], 2048),
    (67, "fp16", 4, 8, 64, 16, [700, 33, 1200, 5], 0),  # XCD order of 128-byte slices
]


@pytest.mark.gpu
@pytest.mark.parametrize("spec", PAGE_CASES, ids=lambda s: "seed%d_d%d" % (s[0], s[4]))
def test_page_read_checksum(plib, spec):
    import torch
    from split_kv_paged_amd import probe
    seed, dt, B, hkv, d, P, lens, split_keys = spec
    case("page_read seed=%d %s B=%d Hkv=%d d=%d page=%d L=%s split_keys=%d"
         % (seed, dt, B, hkv, d, P, lens, split_keys))
    wl = W.make_paged(seed, dt, B, 1, hkv, hkv, d, P, lens, spare_pages=2)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dt]
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()
    sums = probe.page_read(dev(wl.k_cache), dev(wl.v_cache),
                           torch.from_numpy(wl.block_table).cuda(),
                           torch.from_numpy(wl.cache_seqlens.astype(np.int32)).cuda(),
                           max_seqlen_k=wl.max_seqlen_k, split_keys=split_keys)
    torch.cuda.synchronize()
    per_split = sums.cpu().numpy().view(np.uint32).astype(np.uint64)
    S = -(-wl.max_seqlen_k // split_keys) if split_keys else 1
    assert per_split.shape == (S, B, hkv)
    got = (per_split.sum(axis=0) % (1 << 32)).astype(np.uint32)
    assert np.array_equal(got, page_sums(wl))
    if split_keys:  # each split read exactly its own keys
        for s in range(S):
            lo, hi = s * split_keys, (s + 1) * split_keys
            want = np.zeros((B, hkv), dtype=np.uint64)
            for b in range(B):
                j = np.arange(lo, min(hi, int(lens[b])))
                if j.size:
                    pg = wl.block_table[b, j // P]
                    for h in range(hkv):
                        want[b, h] = (word_sum(wl.k_cache[pg, j % P, h, :]) +
                                      word_sum(wl.v_cache[pg, j % P, h, :]))
            assert np.array_equal(per_split[s] % (1 << 32), want % (1 << 32)), s
