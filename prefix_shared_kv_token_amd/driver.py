"""Runs a phase-structured synthetic workload through the Runtime.

Phases (SGLang notes, section 3, frontend hint): the top-level shared
prefixes are prefilled first as hint requests; each later phase admits the
requests one level down, whose shared path is then cached; the deepest
requests decode `decode_steps` tokens each.  Every phase ends with `finish`
(insert + unlock), so the next phase finds its prefixes in the tree.
"""
from __future__ import annotations

import numpy as np

from .runtime import Runtime


class WorkloadRun:
    def __init__(self, wl, device="cuda", extend_items: int = 0, decode_items: int = 0, extra_slots: int = 0,
                 hole_seed: int | None = None, kv_row_pitch: int | None = None):
        import torch

        self.torch = torch
        self.wl = wl
        cfg = wl.cfg
        self.cfg = cfg
        self.num_slots = cfg.total_tokens() + extra_slots
        self.hole_seed = hole_seed
        max_rows = max(len(ph.requests) for ph in wl.phases)
        self.rt = Runtime(cfg.dtype, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, self.num_slots, max_rows,
                          cfg.max_seq_len, device, extend_items, decode_items, kv_row_pitch)
        tdt = self.rt.tdtype
        dev = self.rt.device
        self.inputs = []
        for ph in wl.phases:
            n = sum(r.own_len for r in ph.requests)
            q = torch.empty((n, cfg.n_q_heads, cfg.head_dim), dtype=tdt, device=dev)
            k = torch.empty((n, cfg.n_kv_heads, cfg.head_dim), dtype=tdt, device=dev)
            v = torch.empty_like(k)
            wl.fill_phase(ph, q, k, v)
            self.inputs.append((q, k, v))
        T, R = cfg.decode_steps, len(wl.leaf_requests)
        self.dq = torch.empty((T, R, cfg.n_q_heads, cfg.head_dim), dtype=tdt, device=dev)
        self.dk = torch.empty((T, R, cfg.n_kv_heads, cfg.head_dim), dtype=tdt, device=dev)
        self.dv = torch.empty_like(self.dk)
        if T and R:
            wl.fill_decode(self.dq, self.dk, self.dv)
        self._phase_arrays()
        self.extend_tokens = [sum(r.own_len for r in ph.requests) for ph in wl.phases]
        self.decode_tokens = T * R

    def _phase_arrays(self):
        """Per phase: the prompts concatenated, the matched lengths the
        synthetic queries assume, and the full sequences finish() inserts."""
        wl, cfg = self.wl, self.cfg
        self.prompts = [[wl.prompt_tokens(r) for r in ph.requests] for ph in wl.phases]
        self.generated = wl.decode_token_matrix()
        self.ptok, self.poff, self.expect, self.seq = [], [], [], []
        for pi, ph in enumerate(wl.phases):
            ps = self.prompts[pi]
            self.ptok.append(np.concatenate(ps).astype(np.int32))
            self.poff.append(np.concatenate([[0], np.cumsum([len(p) for p in ps])]).astype(np.int64))
            self.expect.append(np.array([r.prompt_len - r.own_len for r in ph.requests], np.int64))
            if pi == len(wl.phases) - 1 and cfg.decode_steps:
                full = [np.concatenate([p, self.generated[i]]) for i, p in enumerate(ps)]
                self.seq.append((np.concatenate(full).astype(np.int32),
                                 np.concatenate([[0], np.cumsum([len(f) for f in full])]).astype(np.int64)))
            else:
                self.seq.append((self.ptok[-1], self.poff[-1]))

    def fragment(self, tree):
        """Leave only a random subset of the pool free (the rest held as
        private slots), so the workload's pages are scattered."""
        if self.hole_seed is None:
            return
        rng = np.random.default_rng(self.hole_seed)
        allslots = tree.alloc(self.num_slots).copy()
        keep_free = np.sort(rng.choice(allslots, self.cfg.total_tokens(), replace=False))
        tree.free(keep_free)

    def run(self, keep_outputs: bool = True, timers: dict | None = None, record: bool = False,
            loop_events: list | None = None):
        """One pass of every phase.  keep_outputs=False keeps only the last
        decode step's output and no page-table rows.  record=True keeps each
        attention launch (its own plan and buffers) in out["launches"] for
        Runtime.replay.  loop_events: a list that gets (start, end, steps),
        events recorded on the stream around the decode loop."""
        torch = self.torch
        rt = self.rt
        rt.reset()
        rt.record = [] if record else None
        self.fragment(rt.tree)
        cfg = self.cfg
        out = {"extend": [], "decode": None, "matched": [], "rows": [], "plan_info": []}
        n_phases = len(self.wl.phases)
        dec_buf = None
        for pi, ph in enumerate(self.wl.phases):
            reqs = rt.admit_tokens(self.ptok[pi], self.poff[pi])
            if not np.array_equal(reqs.matched, self.expect[pi]):
                j = int(np.flatnonzero(reqs.matched != self.expect[pi])[0])
                raise RuntimeError(f"request {ph.requests[j].rid}: matched {int(reqs.matched[j])}, expected "
                                   f"{int(self.expect[pi][j])} (the synthetic queries cover only the uncached part)")
            q, k, v = self.inputs[pi]
            tm = self._timer(timers, "extend")
            o = rt.extend(reqs, q, k, v, timer=tm)
            out["plan_info"].append(dict(rt.last_info[0]))
            out["extend"].append(o)
            leaf = pi == n_phases - 1
            if leaf and cfg.decode_steps:
                T, R = cfg.decode_steps, len(reqs)
                if keep_outputs:
                    dec_buf = torch.empty((T, R, cfg.n_q_heads, cfg.head_dim), dtype=rt.tdtype, device=rt.device)
                else:
                    dec_buf = torch.empty((1, R, cfg.n_q_heads, cfg.head_dim), dtype=rt.tdtype, device=rt.device)
                tms = [self._timer(timers, "decode") for _ in range(T)] if timers is not None else None
                if loop_events is not None:
                    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    ev[0].record()
                rt.decode_steps(reqs, self.dq, self.dk, self.dv, dec_buf if keep_outputs else dec_buf[0], timers=tms)
                if loop_events is not None:
                    ev[1].record()
                    loop_events.append((ev[0], ev[1], T))
                out["decode"] = dec_buf
            out["matched"].append(reqs.matched.tolist())
            if keep_outputs:
                out["rows"].append([rt.host_pt[r, :k].copy() for r, k in zip(reqs.rows, reqs.kv_len)])
            rt.finish(reqs, seq=self.seq[pi])
        out["launches"] = rt.record
        rt.record = None
        return out

    def _timer(self, timers, key):
        if timers is None:
            return None
        ev = (self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True))
        timers.setdefault(key, []).append(ev)
        return ev
