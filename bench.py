#!/usr/bin/env python3
"""Benchmark of the prefix-shared paged-KV attention path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
input, with every input already resident in HBM:
  admission (radix-tree match / lock / slot allocation) -> page-table and
  work-list upload -> KV scatter -> extend attention, for every phase (the
  prefix hints first, then the requests that share them) -> decode steps
  (allocation, upload, KV scatter, decode attention) -> finish (insert +
  unlock).  The tree starts empty each step.

Prints ONE JSON line.  `value` = (extend query tokens + decode tokens) per
step / wall time per step.  Kernel-level rates use per-launch durations from
HIP events bound to each attention kernel's dispatch (rdx_timing_*), taken
in the timed region on the launch stream.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
KERNEL_SOURCES = ("prefix_shared_kv_token_amd/csrc/attn_kernels.h", "prefix_shared_kv_token_amd/csrc/plan.h",
                  "prefix_shared_kv_token_amd/csrc/plan.cpp")


def extend_flops(cfg, phase_reqs):
    """Unmasked (query, key) pairs x 4 D Hq: S*P + S(S+1)/2 per request."""
    tot = 0
    for r in phase_reqs:
        S, P = r.own_len, r.prompt_len - r.own_len
        tot += S * P + S * (S + 1) // 2
    return 4 * cfg.head_dim * cfg.n_q_heads * tot


def decode_bytes(wl, t):
    """Algorithmic HBM bytes of decode step t: every distinct KV row read
    once (shared prefixes once, each request's own rows once) for K and V,
    its 4-byte page index, the queries and the outputs."""
    cfg = wl.cfg
    b = 2 if cfg.dtype == "bf16" else 4
    leaves = wl.leaf_requests
    shared = sum(n.length for n in wl.nodes if n.level < cfg.n_levels - 1)
    own = sum(r.own_len + t + 1 for r in leaves)
    rows = shared + own
    kv = rows * 2 * cfg.n_kv_heads * cfg.head_dim * b
    qo = 2 * len(leaves) * cfg.n_q_heads * cfg.head_dim * b
    return kv + qo + 4 * rows


def mixed_launch_work(run, e):
    """(flops, bytes) of one mixed launch, algorithmic: every query token
    attends to positions 0..p of its sequence (4 D Hq per visible key); the
    bytes read every distinct KV row the launch needs once (a group's prefix
    once, each request's own rows once; K and V, plus the 4-byte page
    index), the queries and the outputs."""
    import numpy as np

    cfg = run.cfg
    b = 2 if cfg.dtype == "bf16" else 4
    kind, grp, begin, cnt = e[:, 0], e[:, 1], e[:, 3].astype(np.int64), e[:, 4].astype(np.int64)
    end = begin + cnt
    pairs = int((cnt * begin + cnt * (cnt + 1) // 2).sum())
    flops = 4 * cfg.head_dim * cfg.n_q_heads * pairs
    lp = run.prefix_len[grp].astype(np.int64)
    is_pre = kind == 2
    # prefix rows per group: the whole prefix when a member of the group is in
    # the launch, else as far as the group's prefix chunk reaches
    rows = 0
    for g in np.unique(grp):
        sel = grp == g
        if (~is_pre[sel]).any():
            rows += int(lp[sel][0])
        else:
            rows += int(end[sel].max())
    rows += int((end - lp)[~is_pre].sum())
    n_q = int(cnt.sum())
    nbytes = rows * (2 * cfg.n_kv_heads * cfg.head_dim * b + 4) + 2 * n_q * cfg.n_q_heads * cfg.head_dim * b
    return flops, nbytes


def run_mixed_bench(args, cfg, wl):
    """The token-batched job: one step = the whole job (every prefix, prompt
    and decode token of the workload, in the batcher's iterations)."""
    import numpy as np
    import torch
    from prefix_shared_kv_token_amd import rdx
    from prefix_shared_kv_token_amd.mixed import MixedRun
    from workloads import decode_lengths

    tlen = decode_lengths(wl)
    total = cfg.total_tokens() - (cfg.decode_steps * len(wl.leaf_requests) - int(tlen.sum()))
    m = args.m_threshold or 2 * (total // 5)
    print(f"[bench] mixed {cfg.name}: s_chunk {args.s_chunk}, M {m}: staging", file=sys.stderr, flush=True)
    run = MixedRun(wl, args.s_chunk, m, tlen, items=args.extend_items)
    n_it = len(run.iterations)
    gc.collect()
    gc.freeze()
    go = run.run if args.mixed_python else run.run_native
    for _ in range(args.warmup):
        go()
    # the recording's HIP events are created before the timed region
    rdx.timing_begin(n_it)
    rdx.timing_read(0)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} jobs of {n_it} launches", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i == args.steps - 1:
            rdx.timing_begin(n_it)
        go()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_ms, merge_ms, _ = rdx.timing_read(n_it)
    assert len(attn_ms) == n_it, (len(attn_ms), n_it)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    work = [mixed_launch_work(run, e) for e in run.iterations]
    flops = np.array([w[0] for w in work], np.float64)
    nbytes = np.array([w[1] for w in work], np.float64)
    dur = (attn_ms.astype(np.float64) + merge_ms) / 1e3
    kinds = [set(e[:, 0].tolist()) for e in run.iterations]
    dec_only = np.array([k == {0} for k in kinds])
    has_dec = np.array([0 in k for k in kinds])
    mixed = has_dec & ~dec_only
    peak_tf = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS

    def roof(sel, bound):
        d = dur[sel].sum()
        if bound == "mfma":
            a = flops[sel].sum() / d / 1e12
            return {"bound": "mfma", "achieved": a, "peak": peak_tf, "unit": "TFLOP/s", "frac": a / peak_tf,
                    "traffic": None, "launches": int(sel.sum()), "avg_launch_us": d / max(1, sel.sum()) * 1e6}
        a = nbytes[sel].sum() / d / 1e9
        return {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": a / PEAK_HBM_GBS,
                "traffic": None, "launches": int(sel.sum()), "avg_launch_us": d / max(1, sel.sum()) * 1e6}

    every = np.ones(n_it, bool)
    prefill_heavy = ~dec_only
    roof_all = {"mfma": roof(every, "mfma"), "hbm": roof(every, "hbm")}
    dominant = max(roof_all.values(), key=lambda r: r["frac"])
    line = {
        "metric": "mixed extend+decode tokens/s (token-batched job), 1 MI355X",
        "value": run.n_tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1)*sigma Q/K/V, uniform token ids, output lengths uniform in [1, T])",
        "config": {"workload": f"{cfg.name} token-batched", "levels": [list(l) for l in cfg.levels],
                   "max_decode": cfg.decode_steps, "s_chunk": args.s_chunk, "m_threshold": m,
                   "job_tokens": run.n_tokens, "launches": n_it, "mixed_launches": int(mixed.sum()),
                   "decode_only_launches": int(dec_only.sum()), "parallelism": "none (1 GPU)",
                   "runner": "python" if args.mixed_python else "rdx_job"},
        "roofline": dict(dominant, kernel="extend attention over the mixed batches (all launches)"),
        "roofline_mfma_all": roof_all["mfma"],
        "roofline_hbm_all": roof_all["hbm"],
        "roofline_mfma_with_prefill": roof(prefill_heavy, "mfma") if prefill_heavy.any() else None,
        "roofline_hbm_decode_only": roof(dec_only, "hbm") if dec_only.any() else None,
        "attention_ms_per_job": float(dur.sum() * 1e3),
    }
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline on host cores", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_mixed(run, tlen, args.cpu_seconds)
    print(json.dumps(line, default=float), flush=True)


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed:
    what the compiler sees of it (string and character literals, which these
    sources do not use for comment-like text, are kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """sha256 over the code of the kernel sources and of the planner that
    shapes their launches (comments and layout excluded); a counter summary
    taken from other code does not apply."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch (kind: "decode" or "extend member") from the
    committed rocprofv3 counter summary profiles/traffic_<workload>.md, or
    None when there is none or it was taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch\[" + re.escape(kind) + r"\]:\s*([0-9]+)", text)
    if not m_src or not m_val or m_src.group(1) != kernel_source_digest():
        return None
    return {"bytes_per_launch": int(m_val.group(1)), "source": os.path.relpath(path, ROOT)}


def cpu_host_rows():
    """The oracle's host algorithms timed beside the library's (same inputs
    as the probes): the cache-aware order of the 128-prompt queue, the
    global prefix analysis of 128 BatchLLM-shaped prompts (the oracle's token
    trie; the library's call is timed on all 1,024), and the eviction stream
    served on a 6,000-slot cache with LFU."""
    import numpy as np
    from oracle import TokenTrieCache
    from oracle import schedule as osch
    from oracle.prefix_groups import min_processed
    from workloads import Workload, config_by_name, reuse_stream, waiting_queue

    wl = Workload(config_by_name("batchllm"))
    out = {}
    prompts = [[int(t) for t in p] for p in waiting_queue(wl, 128)]
    t0 = time.perf_counter()
    osch.lpm_order(TokenTrieCache(10 ** 6), prompts)
    out["schedule_ms"] = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    min_processed(prompts)
    out["prefix_groups_128_ms"] = (time.perf_counter() - t0) * 1e3
    stream, _ = reuse_stream()
    c = TokenTrieCache(6000, 1, "lfu")
    t0 = time.perf_counter()
    for p in stream:
        m, slots, node = c.match_prefix(p)
        if node:
            c.lock(node)
        new = c.alloc(len(p) - m)
        k, _ = c.insert(p, list(slots) + new)
        c.free(new[: k - m])
        if node:
            c.unlock(node)
    out["eviction_stream_s"] = time.perf_counter() - t0
    return out


def cpu_baseline_mixed(run, tlen, seconds: float):
    """The oracle on the token-batched job, untuned, on this host's cores:
    its batching of the whole job and its cache model over the whole job,
    plus attention for the first member requests until `seconds` of
    attention work; the attention time is scaled to the job by (query, key)
    pairs."""
    import numpy as np
    from oracle.mixed_run import mixed_groups, run_mixed
    from oracle.run import request_attention
    from oracle.token_batching import batch_iterations

    wl = run.wl
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    groups, _ = mixed_groups(wl, tlen)
    batch_iterations(groups, run.s_chunk, run.m_threshold)
    t_sched = time.perf_counter() - t0
    t0 = time.perf_counter()
    run_mixed(wl, run.s_chunk, run.m_threshold, tlen)
    t_cache = time.perf_counter() - t0
    mem = wl.phases[1].requests
    done, t_attn, pairs_done = 0, 0.0, 0
    while done < len(mem) and t_attn < seconds:
        r = mem[done]
        t1 = time.perf_counter()
        request_attention(wl, r)   # its own tokens and all drawn decode tokens
        t_attn += time.perf_counter() - t1
        first = r.prompt_len - r.own_len
        last = r.prompt_len + r.decode_steps
        pairs_done += (last * (last + 1) - first * (first + 1)) // 2
        done += 1
    _, pos = run.job_sources()
    pairs_all = int((pos + 1).sum())
    est = t_sched + t_cache + t_attn * pairs_all / max(pairs_done, 1)
    return {"value": run.n_tokens / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 NumPy oracle: token batching of the whole job ({t_sched:.2f}s), cache model over "
                      f"the whole job ({t_cache:.2f}s), attention of the first {done} member requests "
                      f"({t_attn:.2f}s, {pairs_done} query-key pairs) scaled to the job's {pairs_all} pairs; "
                      f"BLAS threads = host cores"}


def cpu_baseline(wl, seconds: float):
    """The oracle, untuned, on this host's cores, over a bounded sample: the
    cache model for the whole workload plus attention for the first leaf
    requests until `seconds` of attention work have been done."""
    import numpy as np
    import oracle
    from oracle.run import request_attention

    cores = len(os.sched_getaffinity(0))
    leaves = wl.leaf_requests
    t0 = time.perf_counter()
    oracle.run_workload(wl, attention_for=())
    t_cache = time.perf_counter() - t0
    done, toks, t_attn = 0, 0, 0.0
    while done < len(leaves) and t_attn < seconds:
        r = leaves[done]
        t1 = time.perf_counter()
        request_attention(wl, r)
        t_attn += time.perf_counter() - t1
        toks += r.own_len + r.decode_steps
        done += 1
    # whole-workload tokens / (cache model time + attention time scaled to all leaves)
    frac = done / max(1, len(leaves))
    all_toks = sum(r.own_len + r.decode_steps for r in leaves)
    est = t_cache + t_attn / max(frac, 1e-9)
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": all_toks / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 NumPy oracle: cache model over all {len(wl.all_requests)} requests "
                      f"({t_cache:.2f}s) + attention of the first {done} of {len(leaves)} leaf requests "
                      f"({t_attn:.2f}s, {toks} query tokens), rate scaled to all leaf tokens; "
                      f"BLAS threads = host cores; cpu: {cpu}"}


def _serve_in_order(rdx, tree, prompts, order, priority=None) -> int:
    """Serves the prompts one after another on `tree` (match, lock, allocate
    the rest, insert, free duplicates, unlock) -> cached prompt tokens.
    priority: per prompt, the priority its calls carry."""
    cached = 0
    for i in order:
        p = prompts[i]
        if priority is not None:
            tree.set_priority(int(priority[i]))
        m, slots, node = tree.match_prefix(p)
        if node:
            tree.lock(node)
        new = tree.alloc(len(p) - m)
        k, _ = tree.insert(p, list(slots) + list(new))
        if k > m:
            tree.free(new[: k - m])
        if node:
            tree.unlock(node)
        cached += m
    return cached


def schedule_probe(rdx, window: int = 128, reps: int = 20):
    """Cache-aware ordering (host): one window of `window` waiting requests,
    leaf prompts of the BatchLLM-shaped workload (prefix 2,000 shared by 16,
    suffix 200) in a seeded random arrival order, served one at a time on the
    C++ tree in arrival order and in the rdx_schedule order, with a pool of
    twice the longest prompt (tight) and one holding the whole window
    (roomy).  The hit rate is cached prompt tokens / prompt tokens; `optimum`
    is 1 - (distinct prefixes of the window) / (prompt tokens), what a
    depth-first order reaches once the pool holds the longest prompt."""
    import numpy as np
    from workloads import Workload, config_by_name, waiting_queue

    wl = Workload(config_by_name("batchllm"))
    prompts = waiting_queue(wl, window)
    n = len(prompts)
    total = sum(len(p) for p in prompts)
    longest = max(len(p) for p in prompts)
    everything = rdx.Tree(total)
    _serve_in_order(rdx, everything, prompts, range(n))
    distinct = everything.stats()["cached"]
    out = {"queue": f"{n} leaf prompts of batchllm (2000 shared by 16 + 200), seeded random arrival",
           "prompt_tokens": total, "optimum": 1.0 - distinct / total}
    for name, cap in (("tight", 2 * longest), ("roomy", total)):
        fcfs = _serve_in_order(rdx, rdx.Tree(cap), prompts, range(n))
        tree = rdx.Tree(cap)
        order, _ = tree.schedule(prompts)
        lpm = _serve_in_order(rdx, tree, prompts, [int(i) for i in order])
        out[name] = {"pool_slots": cap, "hit_rate_fcfs": fcfs / total, "hit_rate_lpm": lpm / total}
    # cost of one ordering call against a tree that holds the whole window
    # (every prompt's match walks its full length)
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        everything.schedule(prompts)
        ts.append(time.perf_counter() - t0)
    out["schedule_us"] = float(np.median(ts) * 1e6)
    return out


def prefix_groups_probe(rdx, names=("helpdesk", "batchllm", "longprefix", "multilevel"), reps: int = 5):
    """Global prefix analysis (host): each workload's leaf prompts in a seeded
    random order grouped by rdx_prefix_groups; R_saving = 1 - N_processed /
    N_logical with the groups it finds, beside the saving of the radix tree
    (every shared node computed once, as the attention plans here share
    every level), and the median time of one call."""
    import numpy as np
    from workloads import Workload, config_by_name

    out = {}
    for name in names:
        cfg = config_by_name(name)
        wl = Workload(cfg)
        leaves = wl.leaf_requests
        order = np.random.default_rng(cfg.index).permutation(len(leaves))
        prompts = [wl.prompt_tokens(leaves[i]) for i in order]
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            _, _, ng, proc = rdx.prefix_groups(prompts)
            ts.append(time.perf_counter() - t0)
        n_logical = sum(len(p) for p in prompts)
        distinct = cfg.total_tokens() - cfg.n_leaves * cfg.decode_steps
        out[name] = {"requests": len(prompts), "groups": ng, "r_saving_groups": 1.0 - proc / n_logical,
                     "r_saving_radix": 1.0 - distinct / n_logical, "us": float(np.median(ts) * 1e6)}
    return out


def eviction_probe(rdx, pools=(4000, 6000, 10000)):
    """Eviction orders (host): a stream of 400 requests, half of them
    reusing one of four 1,000-token system prompts (popularity 8:4:2:1) plus
    40 fresh tokens, half one-off 1,500-token prompts, served in arrival
    order on the C++ tree with each policy; the priority policy gives the
    reusing requests priority 1.  Hit rate = cached prompt tokens / prompt
    tokens."""
    from workloads import reuse_stream

    prompts, hot = reuse_stream()
    total = sum(len(p) for p in prompts)
    out = {"stream": "400 requests: 50% one of 4 hot 1000-token prompts (8:4:2:1) + 40, 50% one-off 1500",
           "prompt_tokens": total}
    for cap in pools:
        row = {}
        for pol in ("lru", "lfu", "slru", "priority"):
            row[pol] = _serve_in_order(rdx, rdx.Tree(cap, 1, pol), prompts, range(len(prompts)),
                                       priority=hot.astype(int) if pol == "priority" else None) / total
        out[f"hit_rate_pool_{cap}"] = row
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="batchllm",
                    help="headline workload (default: the largest, BatchLLM micro shape)")
    ap.add_argument("--also", default="helpdesk,longprefix,multilevel",
                    help="other workloads measured after the headline (their fractions as extra keys)")
    ap.add_argument("--also-steps", type=int, default=10)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--shuffle-seed", type=int, default=None,
                    help="scattered pool: twice the slots, a seeded random half left free before each step")
    ap.add_argument("--instrumented-steps", type=int, default=1,
                    help="timed steps (the last ones) whose kernels carry timing events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedule-probe", action="store_true")
    ap.add_argument("--mixed", action="store_true",
                    help="token-batched job: prefill chunks and decode tokens share each launch")
    ap.add_argument("--s-chunk", type=int, default=512)
    ap.add_argument("--mixed-python", action="store_true",
                    help="run the job's iterations from Python (default: rdx_job_* in the library)")
    ap.add_argument("--m-threshold", type=int, default=0,
                    help="KV memory bound in K/V entries (default: a fifth of the job's)")
    ap.add_argument("--extra-slots", type=int, default=0,
                    help="pool slots beyond the workload's tokens (a pool over 2 GiB runs the 64-bit offset kernels)")
    ap.add_argument("--extend-items", type=int, default=0)
    ap.add_argument("--decode-items", type=int, default=0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only; several GPUs are not supported "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}))
        return

    from prefix_shared_kv_token_amd import rdx
    from workloads import Workload, config_by_name

    cfg = config_by_name(args.config)
    wl = Workload(cfg)
    if args.mixed:
        return run_mixed_bench(args, cfg, wl)
    m = measure_workload(args, cfg, wl, args.steps, args.warmup, args.instrumented_steps)
    line = {
        "metric": "extend query-tokens/s + decode tokens/s; % MFMA peak / % HBM GB/s, 1 MI355X",
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "instrumented_steps": m["instrumented_steps"],
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1)*sigma Q/K/V, uniform token ids)",
        "config": m["config"],
        "extend_query_tokens_per_s": m["extend_query_tokens_per_s"],
        "decode_tokens_per_s": m["decode_tokens_per_s"],
        "roofline": m["roofline"],
        "extend_roofline": m["extend_roofline"],
        "extend_roofline_hint_plus_member": m["extend_roofline_hint_plus_member"],
        "hint_extend_roofline": m["hint_extend_roofline"],
        "decode_roofline": m["decode_roofline"],
        "decode_loop_us_per_step": m["decode_loop_us_per_step"],
    }
    if not args.headline_only:
        # the other bf16 workloads, each from an empty tree with its own
        # inputs, fewer steps: their kernel fractions beside the headline's
        others = {}
        for name in args.also.split(","):
            if not name or name == cfg.name:
                continue
            ocfg = config_by_name(name)
            print(f"[bench] also {name}", file=sys.stderr, flush=True)
            om = measure_workload(args, ocfg, Workload(ocfg), args.also_steps, args.warmup, 1)
            others[name] = {k: om[k] for k in ("value", "ms_per_step", "extend_query_tokens_per_s",
                                               "decode_tokens_per_s", "extend_roofline",
                                               "extend_roofline_hint_plus_member", "hint_extend_roofline",
                                               "decode_roofline", "decode_loop_us_per_step")}
            others[name]["config"] = om["config"]
            del om
            import torch
            torch.cuda.empty_cache()
        line["workloads"] = others
    if not args.no_schedule_probe:
        print("[bench] request ordering on the host tree", file=sys.stderr, flush=True)
        line["schedule"] = schedule_probe(rdx)
        line["eviction"] = eviction_probe(rdx)
        line["prefix_groups"] = prefix_groups_probe(rdx)
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline on host cores", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        if not args.no_schedule_probe:
            line["cpu_baseline"]["host_rows"] = cpu_host_rows()
    print(json.dumps(line, default=float), flush=True)


def measure_workload(args, cfg, wl, steps: int, warmup: int, instrumented: int) -> dict:
    """Times `steps` passes of the whole workload (admission, uploads, KV
    scatter, extend of every phase, decode steps, finish; empty tree each
    pass) after `warmup` untimed ones; kernel durations from dispatch-bound
    HIP events on the last `instrumented` passes."""
    import numpy as np
    import torch
    from prefix_shared_kv_token_amd import rdx
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    print(f"[bench] {cfg.name}: building inputs", file=sys.stderr, flush=True)
    shuffled = args.shuffle_seed is not None
    run = WorkloadRun(wl, extend_items=args.extend_items, decode_items=args.decode_items,
                      hole_seed=args.shuffle_seed,
                      extra_slots=(cfg.total_tokens() if shuffled else 0) + args.extra_slots)
    # long-lived objects (inputs, torch, the workload) out of the collector's
    # reach, as a serving process does after start-up: a full collection of
    # them would otherwise land inside some step
    gc.collect()
    gc.freeze()
    for _ in range(warmup):
        run.run(keep_outputs=False)
    torch.cuda.synchronize()
    # kernel durations come from HIP events bound to the dispatches of the
    # last `instrumented` timed steps (an event-bound dispatch costs the host
    # extra time, so instrumenting every step would slow the wall clock the
    # value is computed from)
    n_inst = max(1, min(instrumented, steps))
    per_run = len(wl.phases) + cfg.decode_steps
    n_launch = n_inst * per_run
    print(f"[bench] {cfg.name}: timing {steps} steps ({n_inst} instrumented)", file=sys.stderr, flush=True)
    # the passes without event-bound dispatches also time their whole decode
    # loop (store kernel, attention, merge and the gaps between them) with two
    # events on the stream
    loop_events = []
    # the recording's HIP events are created here, before the timed region
    # (creating them costs the host time that a host-paced decode loop would
    # otherwise absorb inside it)
    rdx.timing_begin(n_launch)
    rdx.timing_read(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i == steps - n_inst:
            rdx.timing_begin(n_launch)
        run.run(keep_outputs=False, loop_events=loop_events if i < steps - n_inst else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    loop_us = [e0.elapsed_time(e1) * 1e3 / n for e0, e1, n in loop_events if n]
    attn_ms, merge_ms, kinds = rdx.timing_read(n_launch)
    assert len(attn_ms) == n_launch, (len(attn_ms), n_launch)
    ms_per_step = (t1 - t0) * 1e3 / steps

    # ---- per-launch kernel durations (ms), reshaped [steps, launches/step] ----
    # an attention launch = its attention kernel + the merge kernel behind it
    # (when the plan split tiles); both durations come from events bound to
    # the dispatches, so their sum excludes the gap between the two
    a_step = attn_ms.reshape(n_inst, -1)
    m_step = merge_ms.reshape(n_inst, -1)
    per_step = a_step + m_step
    n_ph = len(wl.phases)
    # launch order per step: extend of phase 0 .. extend of last phase, decode steps after the last extend
    ext_ms = per_step[:, :n_ph]
    dec_ms = per_step[:, n_ph:]
    member_phases = list(range(1, n_ph)) if n_ph > 1 else [0]
    member_reqs = [r for p in member_phases for r in wl.phases[p].requests]
    member_tokens = sum(r.own_len for r in member_reqs)
    ext_member_s = ext_ms[:, member_phases].sum(axis=1).mean() / 1e3
    ext_flops = extend_flops(cfg, member_reqs)
    dec_total_s = dec_ms.sum(axis=1).mean() / 1e3 if cfg.decode_steps else 0.0
    dec_bytes = sum(decode_bytes(wl, t) for t in range(cfg.decode_steps))
    R = len(wl.leaf_requests)
    tokens_per_step = sum(run.extend_tokens) + run.decode_tokens

    def kernel_us(cols):
        return {"attention_kernel_us": float(a_step[:, cols].mean() * 1e3),
                "merge_kernel_us": float(m_step[:, cols].mean() * 1e3)}

    peak_tf = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS

    def mfma_roof(flops, seconds, launches, tokens, cols):
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": a, "peak": peak_tf, "unit": "TFLOP/s", "frac": a / peak_tf,
                "traffic": None, "avg_launch_us": seconds * 1e6 / launches, **kernel_us(cols),
                "work_per_launch": f"{flops / launches / 1e9:.2f} GFLOP ({tokens / launches:.0f} query tokens)"}

    n_mem = len(member_phases)
    extend_roof = mfma_roof(ext_flops, ext_member_s, n_mem, member_tokens, member_phases)
    # phase A (the hint prefill: causal attention over the top-level
    # prefixes, nothing cached) and A+B over every extend launch
    hint_reqs = wl.phases[0].requests if n_ph > 1 else []
    all_reqs = [r for ph in wl.phases for r in ph.requests]
    all_tokens = sum(r.own_len for r in all_reqs)
    ext_all_s = ext_ms.sum(axis=1).mean() / 1e3
    ab_roof = mfma_roof(extend_flops(cfg, all_reqs), ext_all_s, n_ph, all_tokens, list(range(n_ph)))
    hint_roof = None
    if hint_reqs:
        hint_s = ext_ms[:, 0].mean() / 1e3
        hint_roof = mfma_roof(extend_flops(cfg, hint_reqs), hint_s, 1, sum(r.own_len for r in hint_reqs), [0])
    dec_cols = list(range(n_ph, per_step.shape[1]))
    dec_gbs = dec_bytes / dec_total_s / 1e9 if dec_total_s else 0.0
    decode_roof = {"bound": "hbm", "achieved": dec_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": dec_gbs / PEAK_HBM_GBS, "traffic": None,
                   "avg_launch_us": dec_total_s * 1e6 / max(1, cfg.decode_steps),
                   **(kernel_us(dec_cols) if dec_cols else {}),
                   "work_per_launch": f"{dec_bytes / max(1, cfg.decode_steps) / 1e6:.1f} MB (mean over "
                                      f"{cfg.decode_steps} decode steps)"}
    for kname, roof in (("extend member", extend_roof), ("decode", decode_roof)):
        t = measured_traffic(kname, cfg.name)
        if t is not None:
            roof["traffic"] = t["bytes_per_launch"]
            roof["traffic_source"] = t["source"]
    dominant = decode_roof if dec_total_s >= ext_ms.sum(axis=1).mean() / 1e3 else extend_roof
    dominant = dict(dominant, kernel="decode attention" if dominant is decode_roof else "extend attention")
    return {
        "value": tokens_per_step / (ms_per_step / 1e3),
        "ms_per_step": ms_per_step,
        "instrumented_steps": n_inst,
        "config": {"workload": cfg.name, "levels": [list(l) for l in cfg.levels],
                   "decode_steps": cfg.decode_steps, "q_heads": cfg.n_q_heads, "kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "tokens_per_step": tokens_per_step, "parallelism": "none (1 GPU)",
                   "pool": ((f"scattered: 2x slots, random half free (seed {args.shuffle_seed})" if shuffled
                             else "exact size, ascending free ids")
                            + (f", {args.extra_slots} extra slots" if args.extra_slots else "")),
                   "pool_bytes_per_matrix": run.rt.k_pool.numel() * run.rt.k_pool.element_size()},
        "extend_query_tokens_per_s": member_tokens / ext_member_s,
        "decode_tokens_per_s": cfg.decode_steps * R / dec_total_s if dec_total_s else None,
        "roofline": dominant,
        "extend_roofline": extend_roof,
        "extend_roofline_hint_plus_member": ab_roof,
        "hint_extend_roofline": hint_roof,
        "decode_roofline": decode_roof,
        "decode_loop_us_per_step": float(np.mean(loop_us)) if loop_us else None,
    }


if __name__ == "__main__":
    main()
