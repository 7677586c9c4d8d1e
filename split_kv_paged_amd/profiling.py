"""Text summaries of rocprofv3 results for the decode kernels.

rocprofv3 writes one SQLite database per run (``<dir>/**/<name>_results.db``).
This module reads the views it defines (``top_kernels``, ``kernels`` and
``counters_collection``) and turns them into short Markdown summaries:

  python -m split_kv_paged_amd.profiling trace  <dir> --out <file.md> ...
  python -m split_kv_paged_amd.profiling pmc    <dir> [<dir> ...] --out <file.md> ...
  python -m split_kv_paged_amd.profiling traffic --fetch <dir> --write <dir> ...

``traffic`` converts the FETCH_SIZE and WRITE_SIZE counters of one kernel
into HBM bytes per launch.  Each counter is scaled by the ratio of known
bytes to what the same counter reads for a plain device-to-device copy of
known size in the same run (on gfx950 FETCH_SIZE counts a 128-byte read
request as 64 bytes, so the raw figure is about half the real traffic).  The
summary ends with ``key: value`` lines that bench.py reads back, including a
digest of the kernel sources' code (comments and layout ignored): once the
code changes, the figure no longer describes the built kernel and bench.py
reports no traffic.
"""
import argparse
import collections
import glob
import hashlib
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|(?://[^\n]*|/\*.*?\*/|\s)+', re.S)


def code_text(text):
    """C++ source with comments removed and whitespace runs collapsed to
    one space (string literals kept as written), so that a digest of it
    changes with the code and not with its comments or layout."""
    def keep(m):
        t = m.group(0)
        if t.startswith('"'):
            return t
        return " "
    return _TOKENS.sub(keep, text).strip()


def source_digest():
    """sha256 over the code (comments and layout ignored) of the library's
    kernel and host sources (csrc/)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if path.endswith((".hip", ".cpp", ".h")):
            h.update(os.path.basename(path).encode())
            with open(path, encoding="utf-8") as f:
                h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def _db(path):
    if path.endswith(".db"):
        return path
    dbs = sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))
    if not dbs:
        raise SystemExit("no rocprofv3 *_results.db under %s" % path)
    return dbs[-1]


def trace_rows(path):
    """(name, calls, total_us, avg_us, percent) per kernel, longest first."""
    con = sqlite3.connect(_db(path))
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels order by total_duration desc").fetchall()
    con.close()
    return rows


def kernel_resources(path):
    """name -> (grid_x, workgroup_x, lds bytes) of the first dispatch.

    The register counts in the same table are left out: on gfx950 they follow
    an allocation granule that differs from the code object's own
    next-free-VGPR count, which is what limits occupancy."""
    con = sqlite3.connect(_db(path))
    out = {}
    for r in con.execute("select name, grid_x, workgroup_x, lds_size from kernels order by id"):
        out.setdefault(r[0], r[1:])
    con.close()
    return out


def counter_means(path):
    """{(kernel, counter): (dispatches, mean per dispatch)}; instances of one
    dispatch are summed first."""
    con = sqlite3.connect(_db(path))
    per = {}
    for k, c, dsp, v in con.execute("select kernel_name, counter_name, dispatch_id, value "
                                    "from counters_collection"):
        key = (k, c, dsp)
        if c.startswith("GRBM_"):  # one clock seen by every instance: take the max
            per[key] = max(per.get(key, 0.0), v)
        else:
            per[key] = per.get(key, 0.0) + v
    con.close()
    acc = collections.defaultdict(list)
    for (k, c, _), v in per.items():
        acc[(k, c)].append(v)
    return {key: (len(vs), sum(vs) / len(vs)) for key, vs in acc.items()}


def _pick(names, sub):
    hits = [n for n in names if sub in n]
    if not hits:
        raise SystemExit("no kernel matching %r among %s" % (sub, sorted(set(names))))
    return hits[0]


def _short(name, width=90):
    return name if len(name) <= width else name[:width - 3] + "..."


def cmd_trace(a):
    rows = trace_rows(a.dir)
    res = kernel_resources(a.dir)
    lines = ["# %s" % a.title, "", "Command (from the repository root, one MI355X):", "",
             "    %s" % a.command, "",
             "From the `top_kernels` view of the rocprofv3 database (microseconds):", "",
             "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for n, calls, tot, avg, pct in rows:
        lines.append("| %s | %d | %.3f | %.3f | %.2f |" % (_short(n), calls, tot, avg, pct))
    if a.kernel:
        k = _pick([r[0] for r in rows], a.kernel)
        avg = next(r[3] for r in rows if r[0] == k)
        g, wg, lds = res.get(k, (0,) * 3)
        lines += ["", "Kernel `%s`: grid %d threads, workgroup %d, LDS %d bytes."
                  % (_short(k, 120), g, wg, lds)]
        if a.bytes:
            gbs = a.bytes / (avg * 1e-6) / 1e9
            lines += ["Algorithmic bytes per launch: %d. At the average duration: %.1f GB/s "
                      "(%.1f%% of 8 TB/s)." % (a.bytes, gbs, gbs / 80.0)]
    lines += [""] + ["%s" % x for x in (a.note or [])]
    _write(a.out, lines)


def cmd_pmc(a):
    lines = ["# %s" % a.title, "", "Commands (from the repository root, one MI355X):", ""]
    lines += ["    %s" % c for c in a.command] + [""]
    table = {}
    for d in a.dirs:
        table.update(counter_means(d))
    kernels = sorted({k for k, _ in table})
    if a.kernel:
        kernels = [k for k in kernels if any(s in k for s in a.kernel)]
    counters = sorted({c for _, c in table})
    lines += ["Mean per dispatch (instances summed):", "",
              "| kernel | " + " | ".join(counters) + " |",
              "|---|" + "---|" * len(counters)]
    for k in kernels:
        cells = []
        for c in counters:
            v = table.get((k, c))
            cells.append("" if v is None else "%.6g" % v[1])
        lines.append("| %s | %s |" % (_short(k), " | ".join(cells)))
    derived = []
    for k in kernels:
        v = {c: table[(k, c)][1] for c in counters if (k, c) in table}
        # rocprofv3 stores GRBM_GUI_ACTIVE summed over the XCDs; the derived
        # expressions take one XCD's clock (reduce(..., max))
        gui = v.get("GRBM_GUI_ACTIVE", 0.0) / a.xcds
        parts = []
        if gui and "SQ_WAVE_CYCLES" in v:  # waves resident per cycle, of 32 per CU
            parts.append("occupancy %.1f%%" % (400.0 * v["SQ_WAVE_CYCLES"] / gui / a.cus / 32))
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            parts.append("MFMA busy %.2f%%" % (100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                (gui * a.cus * 4)))
        if gui and "SQ_ACTIVE_INST_VALU" in v:
            parts.append("VALU busy %.1f%%" % (100.0 * v["SQ_ACTIVE_INST_VALU"] / a.cus / gui))
        if "SQ_LDS_BANK_CONFLICT" in v and v.get("SQ_LDS_IDX_ACTIVE"):
            c = v["SQ_LDS_BANK_CONFLICT"]
            parts.append("LDS bank conflicts %.4f per access" % (c / max(v["SQ_LDS_IDX_ACTIVE"]
                                                                       - c, 1.0)))
        if parts:
            derived.append("- `%s`: %s." % (_short(k, 60), ", ".join(parts)))
    if derived:
        lines += ["", "Derived with the rocprofv3 expressions (OccupancyPercent, MfmaUtil, "
                  "VALUBusy, LdsBankConflict) over %d CUs, with one XCD's GRBM_GUI_ACTIVE "
                  "(the stored value / %d):" % (a.cus, a.xcds), ""] + derived
    lines += [""] + list(a.note or [])
    _write(a.out, lines)


def cmd_traffic(a):
    f = counter_means(a.fetch)
    w = counter_means(a.write)
    kf = _pick([k for k, c in f if c == "FETCH_SIZE"], a.kernel)
    kw = _pick([k for k, c in w if c == "WRITE_SIZE"], a.kernel)
    cf = _pick([k for k, c in f if c == "FETCH_SIZE"], a.copy_kernel)
    cw = _pick([k for k, c in w if c == "WRITE_SIZE"], a.copy_kernel)
    # the calibration copy is the largest dispatch of the copy kernel
    copy_fetch = _max_dispatch(a.fetch, cf, "FETCH_SIZE")
    copy_write = _max_dispatch(a.write, cw, "WRITE_SIZE")
    sf = a.copy_bytes / (copy_fetch * 1024.0)
    sw = a.copy_bytes / (copy_write * 1024.0)
    n_f, fetch_kib = f[(kf, "FETCH_SIZE")]
    n_w, write_kib = w[(kw, "WRITE_SIZE")]
    fetch_b = fetch_kib * 1024.0 * sf
    write_b = write_kib * 1024.0 * sw
    traffic = fetch_b + write_b
    lines = ["# %s" % a.title, "",
             "Commands (from the repository root, one MI355X), one counter per run:", ""]
    lines += ["    %s" % c for c in a.command] + ["",
              "| | FETCH_SIZE KiB per dispatch | WRITE_SIZE KiB per dispatch | dispatches |",
              "|---|---|---|---|",
              "| `%s` | %.1f | %.1f | %d / %d |" % (_short(kf), fetch_kib, write_kib, n_f, n_w),
              "| calibration copy of %d bytes (`%s`) | %.1f | %.1f | 1 / 1 |"
              % (a.copy_bytes, _short(cf, 40), copy_fetch, copy_write), "",
              "Scale factors (known bytes / counter bytes of the copy): fetch %.4f, write %.4f."
              % (sf, sw),
              "HBM bytes per launch of the kernel: fetch %.0f + write %.0f = %.0f." % (
                  fetch_b, write_b, traffic)]
    if a.algorithmic_bytes:
        lines.append("Algorithmic bytes per launch: %d; traffic / algorithmic = %.4f." % (
            a.algorithmic_bytes, traffic / a.algorithmic_bytes))
    lines += [""] + list(a.note or []) + ["", "Values read by bench.py:", "", "```",
              "workload: %s" % a.workload, "num_splits: %d" % a.num_splits,
              "source_digest: %s" % source_digest(),
              "fetch_bytes_per_launch: %.0f" % fetch_b,
              "write_bytes_per_launch: %.0f" % write_b,
              "traffic_bytes_per_launch: %.0f" % traffic, "```"]
    _write(a.out, lines)


def _max_dispatch(path, kernel, counter):
    con = sqlite3.connect(_db(path))
    per = collections.defaultdict(float)
    for dsp, v in con.execute("select dispatch_id, value from counters_collection where "
                              "kernel_name = ? and counter_name = ?", (kernel, counter)):
        per[dsp] += v
    con.close()
    return max(per.values())


def read_traffic(path):
    """key -> value of the ``key: value`` block of a traffic summary."""
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", " ")):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    return vals


def _write(out, lines):
    text = "\n".join(lines).rstrip() + "\n"
    if out == "-":
        sys.stdout.write(text)
    else:
        with open(out, "w") as f:
            f.write(text)


def main(argv=None):
    ap = argparse.ArgumentParser(description="rocprofv3 summaries")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--kernel", help="substring naming the kernel to describe")
    t.add_argument("--bytes", type=int, help="algorithmic bytes per launch of that kernel")
    t.add_argument("--note", action="append")
    t.add_argument("--out", default="-")
    p = sub.add_parser("pmc")
    p.add_argument("dirs", nargs="+")
    p.add_argument("--title", required=True)
    p.add_argument("--command", action="append", required=True)
    p.add_argument("--kernel", action="append", help="substrings of kernels to keep")
    p.add_argument("--cus", type=int, default=256)
    p.add_argument("--xcds", type=int, default=8)
    p.add_argument("--note", action="append")
    p.add_argument("--out", default="-")
    r = sub.add_parser("traffic")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--copy-kernel", default="copyBuffer")
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--algorithmic-bytes", type=int)
    r.add_argument("--workload", required=True)
    r.add_argument("--num-splits", type=int, required=True)
    r.add_argument("--title", required=True)
    r.add_argument("--command", action="append", required=True)
    r.add_argument("--note", action="append")
    r.add_argument("--out", default="-")
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "pmc": cmd_pmc, "traffic": cmd_traffic}[a.cmd](a)


if __name__ == "__main__":
    main()
