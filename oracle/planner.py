"""Oracle for the host planning step: the pack_gqa and num_splits rules.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python written
from the prose of the lpnh.cn article "Flash-Attention GQA 性能调优：pack_gqa
与 num_splits 两个开关怎么选":

* section "pack_gqa 怎么选": variable-length queries always pack; otherwise
  a row efficiency (valid rows over rows rounded up to the M tile) is taken
  with and without packing, and packing is chosen when the unpacked
  efficiency falls below 0.9 times the packed one.  The page's snippet takes
  the efficiencies as single-precision quotients and multiplies by the
  double literal 0.9; the same precisions are used here.
* section "num_splits 怎么选": (1) when the work units (about batch times KV
  heads) reach 80% of the multiprocessor count, one split; (2) when the KV
  sequence spans at most 4 N tiles, one split; (3) otherwise for every
  candidate split count the last-wave efficiency n_waves / ceil(n_waves) is
  taken and the smallest count within 85% of the best is chosen.  The L2
  rule for single very large KV heads is left out (it never applies to these
  workloads).
* section "常见坑点": a split count above one always runs packed.
* section "pack_gqa 怎么选": a value the caller gives wins over the rule.

Readings (stated where the page is silent): the candidate range of split
counts is 1 .. min(128, n_blocks); the unit count is
batch * heads * ceil(rows / unit_block_m) with heads = KV heads and
rows = seqlen_q * G when packed, query heads and seqlen_q otherwise.  The
page's units are the kernel's thread blocks, each carrying one M tile of
rows; where the kernel's block carries several MFMA tiles of rows,
unit_block_m is the rows one block carries and block_m (the pack rule's
tile) stays the MFMA tile.  unit_block_m defaults to block_m.
"""
import math

import numpy as np

MAX_SPLITS = 128


def _f32(x):
    return np.float32(x)


def round_up(x, m):
    return (x + m - 1) // m * m


def should_pack_gqa(varlen_q, seqlen_q, qhead_per_khead, block_m):
    """Pack decision from row efficiency with and without packing."""
    if varlen_q:
        return True
    nopack = _f32(seqlen_q) / _f32(round_up(seqlen_q, block_m))
    rows = seqlen_q * qhead_per_khead
    pack = _f32(rows) / _f32(round_up(rows, block_m))
    return bool(float(nopack) < 0.9 * float(pack))


def num_splits_heuristic(total_mblocks, num_sms, num_n_blocks, max_splits=MAX_SPLITS):
    """Split count from SM fill and last-wave efficiency."""
    if total_mblocks >= 0.8 * num_sms:
        return 1
    if num_n_blocks <= 4:
        return 1
    max_splits = min(max_splits, num_n_blocks)
    effs = []
    for s in range(1, max_splits + 1):
        n_waves = _f32(total_mblocks * s) / _f32(num_sms)
        effs.append(float(n_waves / _f32(math.ceil(float(n_waves)))))
    best = max(effs)
    for s in range(1, max_splits + 1):
        if effs[s - 1] >= 0.85 * best:
            return s
    return 1


def plan(batch, seqlen_q, num_heads_q, num_heads_kv, max_seqlen_k, num_sms, block_m, block_n,
         num_splits=0, pack_gqa=-1, varlen_q=False, unit_block_m=None):
    """(num_splits, pack) for one call.

    num_splits: 0 = rule, else the caller's value.  pack_gqa: -1 = rule,
    0/1 = caller's value (still forced on when num_splits > 1).
    unit_block_m: rows one thread block carries (default block_m), for the
    unit count of the split rule.
    """
    unit_m = block_m if unit_block_m is None else unit_block_m
    G = num_heads_q // num_heads_kv
    if pack_gqa < 0:
        pack = should_pack_gqa(varlen_q, seqlen_q, G, block_m)
    else:
        pack = bool(pack_gqa)
    if num_splits <= 0:
        heads = num_heads_kv if pack else num_heads_q
        rows = seqlen_q * G if pack else seqlen_q
        total = batch * heads * ((rows + unit_m - 1) // unit_m)
        n_blocks = (max_seqlen_k + block_n - 1) // block_n
        splits = num_splits_heuristic(total, num_sms, n_blocks)
    else:
        splits = num_splits
    if splits > 1:
        pack = True
    return splits, pack
