"""Summarise rocprofv3 hardware-counter runs of a bench step: per-kernel averages and ratios.

Input: rocprofv3 SQLite result databases of the same command, each from one
``--pmc`` pass (a pass holds only as many counters as the hardware collects at
once).  GRBM_GUI_ACTIVE, included in every pass, identifies the dispatch's duration in
GPU-busy cycles (summed over the XCDs); the per-SIMD counters are normalised by the CUs' busy
cycles (SQ_BUSY_CU_CYCLES, summed over compute units), which needs no such assumption.

Output: a Markdown table per kernel (stdout, or ``--md``) with the per-dispatch
average of every counter and these ratios:

  MFMA busy     SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs * SQ_BUSY_CU_CYCLES)
                (the share of the busy compute units' SIMD-cycles in which the matrix core ran;
                one v_mfma_f32_32x32x16 counts 32 cycles)
  co-exec       SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES
                (the share of matrix-core busy cycles in which the SIMD's vector ALU also ran)
  VALU / MFMA   SQ_INSTS_VALU / SQ_INSTS_MFMA
  wait          SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave cycles spent waiting on any dependency)
  LDS wait      SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES
  LDS conflicts SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS
  L2 hit        TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)

    python -m dynamic_sparse_attention_dsv_amd.profile_counters P1.db P2.db ... \\
        --kernels attn_fwd_bf16_kernel attn_bwd_dkdv_bf16_kernel --command "..." --md out.md

With ``--clocks``, the one database given must come from a run that took the kernel trace and
the counters GRBM_GUI_ACTIVE and SQ_BUSY_CU_CYCLES together; the table then gives each kernel's
effective clock over its dispatch: GRBM_GUI_ACTIVE / XCDs / duration (the GPU-busy cycles are
summed over the XCDs) and SQ_BUSY_CU_CYCLES / CUs / duration (the compute units' busy cycles).
"""
from __future__ import annotations

import argparse
import collections
import sqlite3

from .profile_summary import short


def per_kernel(db: str) -> dict:
    """{kernel: {counter: average value per dispatch}} of one counter database."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    con = sqlite3.connect(db)
    for name, counter, val in con.execute("select kernel_name, counter_name, value from counters_collection"):
        vals[short(name)][counter].append(val)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}


def merge(dbs) -> dict:
    out = collections.defaultdict(dict)
    for db in dbs:
        for k, cs in per_kernel(db).items():
            for c, v in cs.items():
                out[k].setdefault(c, v)  # GRBM_GUI_ACTIVE is in every pass: keep the first
    return out


def ratios(c: dict, cus: int) -> dict:
    def div(a, b, scale=1.0):
        return None if a not in c or b not in c or not c[b] else c[a] / (c[b] * scale)
    r = {"MFMA busy": div("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", 4),
         "co-exec": div("SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES"),
         "VALU / MFMA": div("SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
         "wait": div("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
         "LDS wait": div("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
         "LDS conflicts": div("SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS")}
    h, m = c.get("TCC_HIT_sum"), c.get("TCC_MISS_sum")
    r["L2 hit"] = None if h is None or m is None or h + m == 0 else h / (h + m)
    return r


def to_markdown(data: dict, kernels, cus: int, command: str, title: str) -> str:
    out = [f"# {title}", "", "Commands (repository root, one MI355X, `export TMPDIR=/tmp`):", ""]
    out += ["    " + ln for ln in command.split("\n")] + [""]
    out += ["Per-dispatch averages over the profiled step; ratios as defined in "
            "`dynamic_sparse_attention_dsv_amd/profile_counters.py`.", ""]
    names = [k for k in data if any(k.startswith(p) for p in kernels)]
    ratio_keys = ["MFMA busy", "co-exec", "VALU / MFMA", "wait", "LDS wait", "LDS conflicts", "L2 hit"]
    out += ["| kernel | " + " | ".join(ratio_keys) + " |", "|---" * (len(ratio_keys) + 1) + "|"]
    for k in names:
        r = ratios(data[k], cus)
        cells = []
        for key in ratio_keys:
            v = r[key]
            cells.append("-" if v is None else (f"{v:.2f}" if key == "VALU / MFMA" else f"{100 * v:.1f} %"))
        out.append(f"| {k} | " + " | ".join(cells) + " |")
    counters = sorted({c for k in names for c in data[k]})
    out += ["", "Raw counters (per dispatch):", "", "| counter | " + " | ".join(names) + " |",
            "|---" * (len(names) + 1) + "|"]
    for c in counters:
        out.append(f"| {c} | " + " | ".join(f"{data[k].get(c, float('nan')):.4g}" for k in names) + " |")
    return "\n".join(out) + "\n"


def clocks(db: str, kernels, xcds: int, cus: int):
    """[(kernel, avg ms, GHz from GRBM_GUI_ACTIVE, GHz from SQ_BUSY_CU_CYCLES)] of one database."""
    con = sqlite3.connect(db)
    dur = {short(n): avg_us for n, avg_us in con.execute("select name, average from top_kernels")}
    cnt = per_kernel(db)
    rows = []
    for k, avg_us in dur.items():
        if not any(k.startswith(p) for p in kernels) or k not in cnt:
            continue
        t = avg_us * 1e-6
        g, b = cnt[k].get("GRBM_GUI_ACTIVE"), cnt[k].get("SQ_BUSY_CU_CYCLES")
        rows.append((k, avg_us / 1e3, None if g is None else g / xcds / t / 1e9,
                     None if b is None else b / cus / t / 1e9))
    return rows


def clocks_markdown(rows, command: str, title: str) -> str:
    out = [f"# {title}", "", "Command (repository root, one MI355X, `export TMPDIR=/tmp`):", ""]
    out += ["    " + ln for ln in command.split("\n")] + [""]
    out += ["Effective clock over each kernel's dispatch, from the kernel trace and two counters of the "
            "same run (`profile_counters.py --clocks`).", "",
            "| kernel | avg ms | GHz (GRBM_GUI_ACTIVE / 8 XCDs) | GHz (SQ_BUSY_CU_CYCLES / 256 CUs) |",
            "|---|---|---|---|"]
    for k, ms, g1, g2 in rows:
        f = lambda v: "-" if v is None else f"{v:.3f}"
        out.append(f"| {k} | {ms:.3f} | {f(g1)} | {f(g2)} |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("dbs", nargs="+")
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--kernels", nargs="+", required=True, help="device kernel name prefixes to report")
    ap.add_argument("--command", required=True)
    ap.add_argument("--title", default="Hardware counters")
    ap.add_argument("--md")
    ap.add_argument("--clocks", action="store_true", help="effective clocks from one trace+counter database")
    ap.add_argument("--xcds", type=int, default=8)
    a = ap.parse_args()
    if a.clocks:
        md = clocks_markdown(clocks(a.dbs[0], a.kernels, a.xcds, a.cus), a.command, a.title)
    else:
        md = to_markdown(merge(a.dbs), a.kernels, a.cus, a.command, a.title)
    if a.md:
        with open(a.md, "w") as fh:
            fh.write(md)
    else:
        print(md)


if __name__ == "__main__":
    main()
