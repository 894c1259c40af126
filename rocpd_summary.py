"""Summaries of rocprofv3 databases (rocpd SQLite) for this library's kernels.

    python rocpd_summary.py kernels RUN_results.db
        per-kernel calls and durations of a --kernel-trace run (markdown table)

    python rocpd_summary.py traffic FETCH.db WRITE.db CALIB_MIB
        per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of two --pmc runs,
        each scaled by what the same counter read for the largest plain copy
        (__amd_rocclr_copyBuffer) of CALIB_MIB MiB in the same run; prints a
        markdown table and a JSON object of bytes per dispatch

    python rocpd_summary.py traffic-json FETCH.db WRITE.db CALIB_MIB WORKLOAD OUT.json SOURCE [COMMIT] [--groups G,...]
        the same figures summed per library call (forward scan, backward scan,
        projection forward, projection backward, the delta rule's token form,
        chunk form and backward) and merged into OUT.json under
        "WORKLOAD:fwd", ":bwd", ":proj_fwd", ":proj_bwd", ":delta_token",
        ":delta_chunk", ":delta_bwd" (the file bench.py reads); SOURCE names
        the summary the figures come from and COMMIT the source revision of
        the kernels that were counted; --groups keeps only the named calls

    python rocpd_summary.py counters TRACE.db PMC.db [PMC.db ...]
        per-kernel averages of every counter in the --pmc runs, with the
        kernel's average duration from the --kernel-trace run and derived
        ratios (VALU busy, wave time waiting, LDS bank conflicts)

Only the standard library is used; nothing here runs on the GPU.
"""
from __future__ import annotations

import json
import sqlite3
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _short(name: str) -> str:
    s = name.replace("rglru::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return s if len(s) <= 90 else s[:90] + "..."


def kernels(db: str) -> str:
    con = sqlite3.connect(db)
    rows = con.execute("""select name, count(*), sum(duration), avg(duration), min(duration), max(duration)
                          from kernels group by name order by sum(duration) desc""").fetchall()
    out = ["| kernel | calls | total us | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for n, c, tot, avg, mn, mx in rows:
        out.append(f"| `{_short(n)}` | {c} | {tot / 1e3:.1f} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    return "\n".join(out)


def _counter(db: str, counter: str):
    con = sqlite3.connect(db)
    rows = con.execute("""select kernel_name, count(*), avg(value) from counters_collection
                          where counter_name = ? group by kernel_name""", (counter,)).fetchall()
    copy_max = con.execute("""select max(value) from counters_collection
                              where counter_name = ? and kernel_name = ?""", (counter, COPY_KERNEL)).fetchone()[0]
    return {n: (c, v) for n, c, v in rows}, copy_max


def traffic(fetch_db: str, write_db: str, calib_mib: float):
    fetch, fcopy = _counter(fetch_db, "FETCH_SIZE")
    write, wcopy = _counter(write_db, "WRITE_SIZE")
    ref_kib = calib_mib * 1024.0
    fscale = ref_kib / fcopy
    wscale = ref_kib / wcopy
    out = [f"calibration: {calib_mib:g} MiB copy read FETCH_SIZE {fcopy:.1f} KiB (scale {fscale:.4f}), "
           f"WRITE_SIZE {wcopy:.1f} KiB (scale {wscale:.4f})", "",
           "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
           "|---|---|---|---|---|---|"]
    per = {}
    for name in sorted(set(fetch) | set(write), key=lambda n: -(fetch.get(n, (0, 0))[1] or 0)):
        if name == COPY_KERNEL or "rglru::" not in name:
            continue
        fc, fv = fetch.get(name, (0, 0.0))
        wc, wv = write.get(name, (0, 0.0))
        rb = fv * fscale * 1024.0
        wb = wv * wscale * 1024.0
        per[_short(name)] = {"read_bytes": round(rb), "write_bytes": round(wb)}
        out.append(f"| `{_short(name)}` | {fc} | {fv:.1f} | {wv:.1f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
    return "\n".join(out), per


# kernels of each library call (matched on the kernel name; the forward's
# last template argument tells the fused instantiation from the plain scan)
GROUPS = {
    "fwd": lambda n: "fwd_kernel<" in n and "delta_fwd_kernel<" not in n and not n.endswith(", true>(FwdArgs)"),
    "bwd": lambda n: ("bwd_kernel<" in n and "delta_bwd_kernel<" not in n) or "bwd_dlam_kernel(" in n,
    "proj_fwd": lambda n: "proj_fwd_kernel(" in n,
    "proj_bwd": lambda n: any(k in n for k in ("proj_dw_kernel(", "proj_dw_reduce_kernel(", "proj_dx_kernel<")),
    "fused_fwd": lambda n: ("fwd_kernel<" in n and n.endswith(", true>(FwdArgs)")) or "w_frag_kernel(" in n,
    "delta_token": lambda n: "delta_fwd_kernel<" in n,
    "delta_chunk": lambda n: any(k in n for k in ("gdn_chunk_prep<", "gdn_chunk_state<", "gdn_chunk_map(")),
    "delta_bwd": lambda n: any(k in n for k in ("delta_bwd_kernel<", "delta_bwd_reduce_qk<", "delta_bwd_reduce_gb(")),
}


def traffic_json(fetch_db: str, write_db: str, calib_mib: float, workload: str, out: str, source: str,
                 commit: str = None, groups=None):
    _, per = traffic(fetch_db, write_db, calib_mib)
    try:
        with open(out) as f:
            doc = json.load(f)
    except FileNotFoundError:
        doc = {}
    for group, match in GROUPS.items():
        names = [n for n in per if match(n)]
        if not names or (groups is not None and group not in groups):
            continue
        rb = sum(per[n]["read_bytes"] for n in names)
        wb = sum(per[n]["write_bytes"] for n in names)
        doc[f"{workload}:{group}"] = {"bytes": rb + wb, "read_bytes": rb, "write_bytes": wb,
                                      "kernels": sorted(names), "source": source}
        if commit:
            doc[f"{workload}:{group}"]["commit"] = commit
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    return doc


N_SIMD = 1024    # 256 CUs x 4 SIMDs
N_XCD = 8


def counters(trace_db: str, pmc_dbs) -> str:
    """Per-kernel counter averages and derived ratios (library kernels only)."""
    con = sqlite3.connect(trace_db)
    dur = {n: d for n, d in con.execute("select name, avg(duration) from kernels group by name")}
    vals = {}
    for db in pmc_dbs:
        c = sqlite3.connect(db)
        for n, cn, v in c.execute("""select kernel_name, counter_name, avg(value) from counters_collection
                                     group by kernel_name, counter_name"""):
            if "rglru::" in n:
                vals.setdefault(n, {})[cn] = v
    names = sorted(vals, key=lambda n: -(dur.get(n) or 0))
    cols = sorted({k for v in vals.values() for k in v})
    out = ["| kernel | us | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
    for n in names:
        d = dur.get(n)
        row = [f"`{_short(n)}`", f"{d / 1e3:.2f}" if d else "-"]
        row += [f"{vals[n].get(k, float('nan')):.4g}" for k in cols]
        out.append("| " + " | ".join(row) + " |")
    out += ["", "| kernel | kernel cycles per XCD | VALU busy per SIMD | VALU instructions per SIMD | "
            "wave time waiting (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) | of it on LDS (SQ_WAIT_INST_LDS) | "
            "LDS bank-conflict cycles per LDS instruction |", "|---|---|---|---|---|---|---|"]

    def ratio(a, b, fmt="{:.3f}"):
        return fmt.format(a / b) if a is not None and b else "-"

    for n in names:
        v = vals[n]
        gui = v.get("GRBM_GUI_ACTIVE")
        xcd = gui / N_XCD if gui else None
        valu = v.get("SQ_ACTIVE_INST_VALU")
        # GRBM_GUI_ACTIVE sums the 8 XCDs; SQ_ACTIVE_INST_VALU counts in
        # 4-cycle units, summed over every wave
        busy = ratio(4 * valu / N_SIMD if valu is not None else None, xcd)
        insts = v.get("SQ_INSTS_VALU")
        cyc = f"{xcd:.0f}" if xcd else "-"
        per_simd = f"{insts / N_SIMD:.0f}" if insts is not None else "-"
        out.append(f"| `{_short(n)}` | {cyc} | {busy} | {per_simd} | "
                   f"{ratio(v.get('SQ_WAIT_INST_ANY'), v.get('SQ_WAVE_CYCLES'))} | "
                   f"{ratio(v.get('SQ_WAIT_INST_LDS'), v.get('SQ_WAVE_CYCLES'))} | "
                   f"{ratio(v.get('SQ_LDS_BANK_CONFLICT'), v.get('SQ_INSTS_LDS'))} |")
    return "\n".join(out)


def main(argv):
    groups = None
    if "--groups" in argv:
        i = argv.index("--groups")
        groups = set(argv[i + 1].split(","))
        argv = argv[:i] + argv[i + 2:]
    if len(argv) >= 2 and argv[0] == "kernels":
        print(kernels(argv[1]))
    elif len(argv) >= 4 and argv[0] == "traffic":
        table, per = traffic(argv[1], argv[2], float(argv[3]))
        print(table)
        print()
        print(json.dumps(per, indent=1))
    elif len(argv) >= 7 and argv[0] == "traffic-json":
        doc = traffic_json(argv[1], argv[2], float(argv[3]), argv[4], argv[5], argv[6],
                           argv[7] if len(argv) >= 8 else None, groups)
        print(json.dumps(doc, indent=1))
    elif len(argv) >= 3 and argv[0] == "counters":
        print(counters(argv[1], argv[2:]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
