#!/usr/bin/env python3
"""Summarises rocprofv3 output of `bench.py --headline-only` runs into the
tables kept under profiles/: kernel durations (from --kernel-trace) and, given
the two counter passes, HBM bytes per dispatch (FETCH_SIZE and WRITE_SIZE,
each scaled by the factor a plain device copy of known size gives).

Dispatches are classified by kernel and position: a bench step launches the
extend attention of every phase in order (phase 0 = the hint prefill of the
top-level prefixes, then the member phases), each followed by its merge
kernel when the plan split tiles, then one decode attention (+ merge) per
decode step.  So the k-th extend dispatch of the run belongs to phase
k mod n_phases, and a merge kernel belongs to the attention dispatch right
before it.

    python3 bench_trace_summary.py trace <run_kernel_trace.csv> --phases N --runs R
    python3 bench_trace_summary.py pmc <FETCH run_counter_collection.csv> <WRITE ...csv> --phases N \\
        --fetch-factor F --write-factor W
    python3 bench_trace_summary.py counters <pass1 csv> <pass2 csv> ... --phases N [--label "extend phase 1"]
    python3 bench_trace_summary.py gaps <run_kernel_trace.csv> --phases N
"""
from __future__ import annotations

import argparse
import collections
import csv

EXTEND = ("attn_bf16_wide_kernel", "attn_bf16_kernel", "attn_f32_kernel")


def _rows(path):
    rows = list(csv.DictReader(open(path)))
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Correlation_Id"
    rows.sort(key=lambda r: int(r[key]))
    return rows


def _short(name: str) -> str:
    for k in ("attn_decode_kernel", "merge_kernel") + EXTEND:
        if k in name:
            i = name.index(k)
            j = name.find("(", i)
            return name[i:j if j > 0 else None]
    return name.split("(")[0][:60]


def classify(names, n_phases: int):
    """-> class label per dispatch (same order)."""
    out, n_ext, last = [], 0, None
    for name in names:
        if any(k in name for k in EXTEND):
            ph = n_ext % n_phases
            n_ext += 1
            role = "hint" if (ph == 0 and n_phases > 1) else "member"
            last = f"extend phase {ph} ({role})"
            out.append(f"{last}: {_short(name)}")
        elif "attn_decode_kernel" in name:
            last = "decode"
            out.append(f"decode: {_short(name)}")
        elif "merge_kernel" in name:
            out.append(f"merge after {last}")
        else:
            out.append(_short(name))
    return out


def trace(path, n_phases, runs):
    """runs: passes of the workload in the traced run (warm-up + timed); the
    last column averages the dispatches of the last pass only, the one whose
    kernels bench.py times with events."""
    rows = _rows(path)
    labels = classify([r["Kernel_Name"] for r in rows], n_phases)
    dur = collections.defaultdict(list)
    for r, lab in zip(rows, labels):
        dur[lab].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    tot = sum(sum(v) for v in dur.values())
    print("| dispatch class | calls | average (us) | total (ms) | share | average, last pass (us) |")
    print("|---|---:|---:|---:|---:|---:|")
    for lab, v in sorted(dur.items(), key=lambda x: -sum(x[1])):
        last = v[-(len(v) // runs):] if runs and len(v) % runs == 0 and len(v) >= runs else None
        tail = f"{sum(last) / len(last):.2f}" if last else "-"
        print(f"| `{lab}` | {len(v)} | {sum(v) / len(v):.2f} | {sum(v) / 1e3:.2f} | {100 * sum(v) / tot:.1f}% | {tail} |")


def pmc(fetch_path, write_path, n_phases, ff, wf):
    res = {}
    for which, path in (("fetch", fetch_path), ("write", write_path)):
        rows = _rows(path)
        labels = classify([r["Kernel_Name"] for r in rows], n_phases)
        acc = collections.defaultdict(list)
        for r, lab in zip(rows, labels):
            acc[lab].append(float(r["Counter_Value"]))
        res[which] = acc
    print("| dispatch class | dispatches | FETCH_SIZE mean KiB | WRITE_SIZE mean KiB | scaled MB/dispatch |")
    print("|---|---:|---:|---:|---:|")
    scaled = {}
    for lab in sorted(res["fetch"], key=lambda k: -sum(res["fetch"][k])):
        f = res["fetch"][lab]
        w = res["write"].get(lab, [0.0])
        fm, wm = sum(f) / len(f), sum(w) / len(w)
        scaled[lab] = (fm * ff + wm * wf) * 1024
        print(f"| `{lab}` | {len(f)} | {fm:,.1f} | {wm:,.1f} | {scaled[lab] / 1e6:,.2f} |")
    # per launch: an attention dispatch plus the merge behind it
    dec = [k for k in scaled if k.startswith("decode: ")]
    if dec:
        b = scaled[dec[0]] + scaled.get("merge after decode", 0.0)
        print(f"\ntraffic_bytes_per_launch[decode]: {b:.0f}")
    mem = sorted({k.split(":")[0] for k in scaled if k.startswith("extend phase") and "(member)" in k})
    if mem:
        per = []
        for ph in mem:
            att = [v for k, v in scaled.items() if k.startswith(ph + ":")][0]
            per.append(att + scaled.get(f"merge after {ph}", 0.0))
        print(f"traffic_bytes_per_launch[extend member]: {sum(per) / len(per):.0f}")


def counters(paths, n_phases, label_prefix):
    """Counter passes (rocprofv3 --pmc, one CSV per pass) over the same run:
    the mean of each counter over the dispatches whose class starts with
    label_prefix, then the derived shares.  GRBM_GUI_ACTIVE is summed over
    the 8 XCDs (active cycles per XCD = GRBM / 8); SQ_*_CYCLES counters are
    summed over the SIMDs (1,024) or CUs (256) as noted."""
    vals = collections.defaultdict(list)
    for path in paths:
        rows = _rows_all(path)
        disp = collections.OrderedDict()
        for r in rows:
            disp.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))[1][r["Counter_Name"]] = float(r["Counter_Value"])
        ids = sorted(disp)
        labels = classify([disp[i][0] for i in ids], n_phases)
        for i, lab in zip(ids, labels):
            if lab.startswith(label_prefix):
                for k, v in disp[i][1].items():
                    vals[k].append(v)
    m = {k: sum(v) / len(v) for k, v in vals.items()}
    print("| counter | mean per dispatch |")
    print("|---|---:|")
    for k in sorted(m):
        print(f"| {k} | {m[k]:,.0f} |")
    grbm = [v for k, v in m.items() if k.startswith("GRBM_GUI_ACTIVE")]
    if grbm:
        act = grbm[0] / 8  # cycles per XCD
        print()
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            print(f"MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1,024 SIMDs)): {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (act * 1024) * 100:.1f}%")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
            print(f"MFMA and VALU co-executing (SQ_VALU_MFMA_COEXEC_CYCLES / (active cycles x 1,024)): {m['SQ_VALU_MFMA_COEXEC_CYCLES'] / (act * 1024) * 100:.1f}%")
        if "SQ_ACTIVE_INST_VALU" in m:
            print(f"VALU busy (SQ_ACTIVE_INST_VALU x 4 / (active cycles x 1,024), rocprof's VALUBusy): "
                  f"{m['SQ_ACTIVE_INST_VALU'] * 4 / (act * 1024) * 100:.1f}%")
        if "SQ_LDS_IDX_ACTIVE" in m:
            print(f"LDS active (SQ_LDS_IDX_ACTIVE / (active cycles x 256 CUs)): {m['SQ_LDS_IDX_ACTIVE'] / (act * 256) * 100:.1f}%")
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_LDS_IDX_ACTIVE" in m:
            print(f"LDS bank-conflict share (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE): {m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE'] * 100:.1f}%")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            print(f"executed bf16 MFMA flops (MOPS x 512): {m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e12:.3f} TFLOP")
    if "SQ_INSTS_MFMA" in m and m["SQ_INSTS_MFMA"] > 0:
        r = 1.0 / m["SQ_INSTS_MFMA"]
        parts = [f"{k[9:]} {m[k] * r:.2f}" for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD") if k in m]
        print("instructions per MFMA instruction (SQ_INSTS_VALU counts the MFMA and transcendental "
              "instructions too): " + ", ".join(parts))


def gaps(path, n_phases, top=12):
    """Idle time of the GPU in the last pass of the workload: from the first
    dispatch after the previous pass's last decode step to the run's last
    dispatch, the span, the time some kernel ran (union of the dispatch
    intervals) and the gaps between consecutive dispatches, summed by the
    classes on either side and listed largest first."""
    rows = _rows(path)
    labels = classify([r["Kernel_Name"] for r in rows], n_phases)
    hint0 = [i for i, l in enumerate(labels) if l.startswith("extend phase 0")]
    if not hint0:
        raise SystemExit("no extend phase 0 dispatch in the trace")
    start = 0
    for i in range(hint0[-1] - 1, -1, -1):
        if labels[i].startswith("decode") or labels[i] == "merge after decode":
            start = i + 1
            break
    win = [(int(rows[i]["Start_Timestamp"]), int(rows[i]["End_Timestamp"]), labels[i]) for i in range(start, len(rows))]
    win.sort()
    span = win[-1][1] - win[0][0]
    busy, cur_s, cur_e = 0, win[0][0], win[0][1]
    gl = []
    for (s0, e0, l0), (s1, e1, l1) in zip(win, win[1:]):
        if s1 > cur_e:
            busy += cur_e - cur_s
            gl.append((s1 - cur_e, l0, l1))
            cur_s, cur_e = s1, e1
        else:
            cur_e = max(cur_e, e1)
    busy += cur_e - cur_s
    print(f"last pass: {len(win)} dispatches, span {span / 1e3:.1f} us, kernels running {busy / 1e3:.1f} us, "
          f"idle {(span - busy) / 1e3:.1f} us in {len(gl)} gaps")
    by = collections.defaultdict(lambda: [0, 0])
    for g, l0, l1 in gl:
        k = (l0.split(": ")[0], l1.split(": ")[0])
        by[k][0] += 1
        by[k][1] += g
    print()
    print("| previous dispatch | next dispatch | gaps | total (us) | mean (us) |")
    print("|---|---|---:|---:|---:|")
    for (a, b), (n, t) in sorted(by.items(), key=lambda x: -x[1][1])[:top]:
        print(f"| `{a}` | `{b}` | {n} | {t / 1e3:.1f} | {t / 1e3 / n:.2f} |")
    print()
    print("largest gaps (us): " + ", ".join(f"{g / 1e3:.1f} ({l0.split(': ')[0]} -> {l1.split(': ')[0]})"
                                            for g, l0, l1 in sorted(gl, reverse=True)[:top]))


def _rows_all(path):
    return list(csv.DictReader(open(path)))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--phases", type=int, required=True)
    t.add_argument("--runs", type=int, default=0, help="workload passes in the run (warm-up + timed)")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("--phases", type=int, required=True)
    p.add_argument("--fetch-factor", type=float, required=True)
    p.add_argument("--write-factor", type=float, required=True)
    c = sub.add_parser("counters")
    c.add_argument("csvs", nargs="+", help="counter_collection.csv of each pass")
    c.add_argument("--phases", type=int, required=True)
    c.add_argument("--label", default="extend phase 1", help="dispatch class prefix to average")
    g = sub.add_parser("gaps")
    g.add_argument("csv")
    g.add_argument("--phases", type=int, required=True)
    a = ap.parse_args()
    if a.cmd == "trace":
        trace(a.csv, a.phases, a.runs)
    elif a.cmd == "gaps":
        gaps(a.csv, a.phases)
    elif a.cmd == "pmc":
        pmc(a.fetch_csv, a.write_csv, a.phases, a.fetch_factor, a.write_factor)
    else:
        counters(a.csvs, a.phases, a.label)


if __name__ == "__main__":
    main()
