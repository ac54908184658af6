"""Runs a two-level workload as ONE token-batched job: prefill chunks and
decode tokens of many requests share every attention launch.

BatchLLM explainer: requests sharing a prefix form a group (Throughput-
oriented Token Batching); each iteration's token batch holds every decoding
request's next token, then prefill chunks (distinct prompts of groups whose
prefix is done, then new prefixes) while the KV memory stays under the
threshold (Memory-centric Token Batching) -- the library's rdx_batcher
decides it; one attention launch then covers the whole batch, the shared
prefix of a group attended once for all of that group's tokens in it
(Horizontal Fusion).

At the start of a job the library's global prefix analysis (rdx_prefix_groups,
BatchLLM explainer, Global Prefix Sharing) groups the members' prompts; the
groups it finds are the batcher's groups (for the two-level workloads run
here they are the top-level prefixes, which the staged inputs assume -- a
different grouping is an error).

Per iteration (all computation in the library; this module marshals):
  rdx_batcher_next -> admit the requests that start (one rdx_admit: the
  prefix request of a group, or a member once its group's prefix is in the
  tree) -> one slot per decode token (rdx_alloc) -> plan over the mixed
  batch (chunk: kv_len = chunk end, q_len = chunk; decode: q_len = 1) ->
  upload, KV scatter, attention (the extend kernel; the decode kernel when
  the batch holds decode tokens only) -> finish the requests that completed
  (one rdx_finish: the prefix goes into the tree for the members).

Inputs are staged before the run in the order the tokens are processed
(iteration-major, entry order), as a model's projections would produce them,
so each iteration reads one contiguous slice.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import rdx
from .runtime import Runtime


class _Rows:
    """The per-request arrays Runtime._launch reads."""

    __slots__ = ("nodes", "rows", "rows64", "kv_len", "written")

    def __init__(self, nodes, rows, kv_len, written):
        self.nodes = nodes
        self.rows = rows
        self.rows64 = rows.astype(np.int64)
        self.kv_len = kv_len
        self.written = written


class MixedRun:
    def __init__(self, wl, s_chunk: int, m_threshold: int, decode_len=None, device="cuda", items: int = 0,
                 stage: bool = True, num_slots: int | None = None):
        """decode_len: tokens each member generates (<= the workload's
        decode_steps; all of them by default).  num_slots: KV pool size (the
        workload's distinct tokens by default; a smaller pool makes admissions
        evict finished requests' tokens)."""
        import torch

        self.torch = torch
        cfg = wl.cfg
        if cfg.n_levels != 2:
            raise ValueError("a mixed job needs a two-level sharing tree (prefix, then the members' own tokens)")
        self.wl, self.cfg = wl, cfg
        self.s_chunk, self.m_threshold = s_chunk, m_threshold
        pre = wl.phases[0].requests
        mem = wl.phases[1].requests
        G, M = len(pre), len(mem)
        self.G, self.M = G, M
        gid = {r.node: g for g, r in enumerate(pre)}
        mg = np.array([gid[r.path[0]] for r in mem], np.int64)
        if np.any(np.diff(mg) < 0):
            raise ValueError("members must be listed group by group")
        self.member_group = mg
        self.req_rid = np.array([r.rid for r in pre] + [r.rid for r in mem], np.int64)
        self.member_offsets = np.searchsorted(mg, np.arange(G + 1)).astype(np.int32)
        self.prefix_len = np.array([r.own_len for r in pre], np.int32)
        self.distinct_len = np.array([r.own_len for r in mem], np.int32)
        self.decode_len = np.array([r.decode_steps for r in mem] if decode_len is None else decode_len, np.int32)
        if len(self.decode_len) != M or (M and (self.decode_len.min() < 0
                                                  or self.decode_len.max() > cfg.decode_steps)):
            raise ValueError("decode_len: one length per member, each in [0, decode_steps]")
        # requests: 0..G-1 the groups' prefix requests, G.. the members
        self.req_prompt_len = np.concatenate([self.prefix_len, self.prefix_len[mg] + self.distinct_len]).astype(np.int64)
        self.req_total_len = self.req_prompt_len + np.concatenate([np.zeros(G, np.int64), self.decode_len])
        prompts = [wl.prompt_tokens(r) for r in pre] + [wl.prompt_tokens(r) for r in mem]
        self.member_prompts = prompts[G:]
        # the same prompts as one flat token buffer, as a serving loop holds them
        self._mp_flat = np.concatenate(self.member_prompts).astype(np.int32) if M else np.zeros(0, np.int32)
        self._mp_off = np.concatenate([[0], np.cumsum([len(p) for p in self.member_prompts])]).astype(np.int64)
        gen = [np.zeros(0, np.int32)] * G + [wl.decode_tokens(r)[:t] for r, t in zip(mem, self.decode_len)]
        self.seq_tokens = [np.concatenate([p, g]).astype(np.int32) for p, g in zip(prompts, gen)]
        self.rt = Runtime(cfg.dtype, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, num_slots or cfg.total_tokens(), G + M,
                          cfg.max_seq_len, device, extend_items=items)
        # the job's iterations (the batcher is deterministic: the timed run
        # asks it again and gets the same entries)
        self.iterations = []
        b = self._batcher()
        while True:
            e = b.next()
            if len(e) == 0:
                break
            self.iterations.append(e.copy())
        self.iter_tokens = np.array([int(e[:, 4].sum()) for e in self.iterations], np.int64)
        self.iter_off = np.concatenate([[0], np.cumsum(self.iter_tokens)]).astype(np.int64)
        self.n_tokens = int(self.iter_off[-1])
        if stage:
            self._stage()

    def _analysed_groups(self):
        """The batcher's groups from the global prefix analysis of the
        members' prompts: (prefix per group, member offsets, distinct per
        member)."""
        group, prefix, ng, _ = rdx.prefix_groups_flat(self._mp_flat, self._mp_off)
        mg = self.member_group
        # the analysis numbers groups by first member; members come group by group
        if (ng != self.G or not np.array_equal(group, np.searchsorted(np.unique(mg), mg))
                or not np.array_equal(prefix, self.prefix_len[mg])):
            raise RuntimeError("the prefix analysis grouped the members differently from the workload's "
                               "top-level prefixes (the staged inputs assume those)")
        first = np.searchsorted(group, np.arange(ng))
        return (prefix[first], np.append(first, len(group)).astype(np.int32), np.diff(self._mp_off) - prefix)

    def _batcher(self, analyse: bool = False):
        """The job's batcher; analyse=True derives its groups from the
        members' prompts by the global prefix analysis first."""
        if analyse:
            return rdx.Batcher(*self._analysed_groups(), self.decode_len, self.s_chunk, self.m_threshold)
        return rdx.Batcher(self.prefix_len, self.member_offsets, self.distinct_len, self.decode_len,
                           self.s_chunk, self.m_threshold)

    def run_native(self, keep_rows: bool = False, dry_run: bool = False):
        """The job through rdx_job_* (admissions, decode slots, plans and
        finishes in the library; three calls per iteration)."""
        rt = self.rt
        rt.reset()
        self.matched, self.rows = {}, {}
        prefix, offs, distinct = self._analysed_groups()
        if not hasattr(self, "_seq_flat"):
            # every request's full sequence as one flat buffer (borrowed by the job)
            self._seq_flat = np.concatenate(self.seq_tokens).astype(np.int32)
            self._seq_off = np.concatenate([[0], np.cumsum([len(t) for t in self.seq_tokens])]).astype(np.int64)
        flags = (rdx.JOB_KEEP_ROWS if keep_rows else 0) | (rdx.JOB_DRY_RUN if dry_run else 0)
        job = rdx.Job(rt.tree, prefix, offs, distinct, self.decode_len, self.s_chunk, self.m_threshold,
                      self._seq_flat, self._seq_off, rt.max_rows, rt.ld, flags)
        L = rdx.lib()
        io = rt._io
        io_ref = rt._io_ref
        info = job.info
        plans = rt.plans
        ext, dec = plans[rdx.PLAN_EXTEND], plans[rdx.PLAN_DECODE]
        st = None if dry_run else self.torch.cuda.current_stream().cuda_stream
        q0 = k0 = v0 = o0 = 0
        if not dry_run:
            q0, k0, v0, o0 = self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr()
            qrow = self.q[0].numel() * self.q.element_size()
            krow = self.k[0].numel() * self.k.element_size()
        tok = 0
        it = 0
        while True:
            n, kind = job.prepare(ext, dec)
            if n == 0:
                break
            if not dry_run:
                dp = rt._dev_plan(kind, info.device_bytes)
                ws = rt._workspace(info.workspace_bytes)
                io.dev_plan, io.dev_plan_bytes = dp.data_ptr(), dp.numel()
                io.workspace, io.workspace_bytes = ws.data_ptr(), ws.numel()
                io.q, io.o = q0 + tok * qrow, o0 + tok * qrow
                io.k_new, io.v_new = k0 + tok * krow, v0 + tok * krow
                rdx._check(L.rdx_job_launch(job.handle, rt._desc_ref, io_ref, st, None))
            job.complete()
            tok += n
            it += 1
        if tok != self.n_tokens or it != len(self.iterations):
            raise RuntimeError("the batcher's run differs from the staged one")
        if keep_rows:
            for r in range(self.G + self.M):
                if self.req_total_len[r] == 0:
                    continue
                row, m = job.row(r)
                rid = int(self.req_rid[r])
                self.rows[rid], self.matched[rid] = row, m
        return None if dry_run else self.o

    # ------------------------------------------------------------ inputs
    def job_sources(self):
        """For every token of the job in processing order: (request, position)."""
        req = np.empty(self.n_tokens, np.int64)
        pos = np.empty(self.n_tokens, np.int64)
        o = 0
        G = self.G
        for e in self.iterations:
            for kind, g, m, begin, cnt in e.tolist():
                r = g if kind == rdx.TB_PREFIX else G + m
                req[o:o + cnt] = r
                pos[o:o + cnt] = np.arange(begin, begin + cnt)
                o += cnt
        return req, pos

    def _stage(self):
        """Q/K/V of every job token, in processing order, on the device."""
        torch, wl, cfg, rt = self.torch, self.wl, self.cfg, self.rt
        tdt, dev = rt.tdtype, rt.device
        pre, mem = wl.phases[0].requests, wl.phases[1].requests
        G, M = self.G, self.M
        # sources as the phase-structured run lays them out: prefix tokens
        # request-major, member tokens request-major, decode step-major
        n0 = int(self.prefix_len.sum())
        n1 = int(self.distinct_len.sum())
        T = cfg.decode_steps
        n_src = n0 + n1 + T * M
        sq = torch.empty((n_src, cfg.n_q_heads, cfg.head_dim), dtype=tdt, device=dev)
        sk = torch.empty((n_src, cfg.n_kv_heads, cfg.head_dim), dtype=tdt, device=dev)
        sv = torch.empty_like(sk)
        wl.fill_phase(wl.phases[0], sq[:n0], sk[:n0], sv[:n0])
        wl.fill_phase(wl.phases[1], sq[n0:n0 + n1], sk[n0:n0 + n1], sv[n0:n0 + n1])
        if T and M:
            wl.fill_decode(sq[n0 + n1:].view(T, M, cfg.n_q_heads, cfg.head_dim),
                           sk[n0 + n1:].view(T, M, cfg.n_kv_heads, cfg.head_dim),
                           sv[n0 + n1:].view(T, M, cfg.n_kv_heads, cfg.head_dim))
        off0 = np.concatenate([[0], np.cumsum(self.prefix_len)]).astype(np.int64)
        off1 = n0 + np.concatenate([[0], np.cumsum(self.distinct_len)]).astype(np.int64)
        req, pos = self.job_sources()
        is_pre = req < G
        m = np.where(is_pre, 0, req - G)
        plen = self.prefix_len[self.member_group[m]].astype(np.int64)
        own_end = plen + self.distinct_len[m]
        idx = np.where(is_pre, off0[np.minimum(req, G - 1)] + pos,
                       np.where(pos < own_end, off1[m] + pos - plen, n0 + n1 + (pos - own_end) * M + m))
        it = torch.from_numpy(idx).to(dev)
        self.q = sq.index_select(0, it)
        self.k = sk.index_select(0, it)
        self.v = sv.index_select(0, it)
        del sq, sk, sv
        self.o = torch.empty_like(self.q)

    # ------------------------------------------------------------ run
    def run(self, keep_rows: bool = False):
        """One pass of the whole job; outputs land in self.o (processing
        order).  keep_rows=True records each request's matched length and
        final page-table row (self.matched / self.rows, by request id)."""
        rt = self.rt
        rt.reset()
        self.matched, self.rows = {}, {}
        L = rdx.lib()
        G, M = self.G, self.M
        n_req = G + M
        row = np.full(n_req, -1, np.int32)
        node = np.zeros(n_req, np.int64)
        matched = np.zeros(n_req, np.int64)
        plen_m = self.prefix_len[self.member_group]
        expect = np.concatenate([np.zeros(G, np.int64), plen_m.astype(np.int64)])
        b = self._batcher(analyse=True)
        p32, p64 = rdx._p32, (lambda x: x.ctypes.data_as(rdx.i64p))
        done_n = rdx.i32()
        tok = 0
        it = 0
        while True:
            e = b.next()
            n_e = len(e)
            if n_e == 0:
                break
            kind, grp, mbr, begin, cnt = (e[:, i] for i in range(5))
            req = np.where(kind == rdx.TB_PREFIX, grp, G + mbr).astype(np.int64)
            # admissions: a prefix request at its first chunk, a member at its
            # first distinct chunk (its group's prefix is in the tree by then)
            start = (begin == np.where(kind == rdx.TB_PREFIX, 0, np.where(kind == rdx.TB_DISTINCT,
                                                                            self.prefix_len[grp], -1)))
            if start.any():
                new = req[start]
                toks = [self.seq_tokens[r][: self.req_prompt_len[r]] for r in new]
                offs = np.concatenate([[0], np.cumsum([len(t) for t in toks])]).astype(np.int64)
                nb = rt.admit_tokens(np.concatenate(toks), offs)
                row[new], node[new], matched[new] = nb.rows, nb.nodes, nb.matched
                if keep_rows:
                    for r, mm in zip(new, nb.matched):
                        self.matched[int(self.req_rid[r])] = int(mm)
                if not np.array_equal(nb.matched, expect[new]):
                    raise RuntimeError("a request matched more or less than its group's prefix "
                                       "(the staged queries cover only the uncached tokens)")
            rows = row[req]
            rows64 = rows.astype(np.int64)
            kv_len = (begin + cnt).astype(np.int32)
            dec = kind == rdx.TB_DECODE
            n_dec = int(dec.sum())
            if n_dec:
                if (kv_len[dec] > rt.ld).any():
                    raise RuntimeError("page-table row full")
                slots = rt.tree.alloc(n_dec)
                rt.host_pt[rows64[dec], begin[dec]] = slots
            # new slots in entry order: decode entries come first
            parts = [slots] if n_dec else []
            for i in range(n_dec, n_e):
                parts.append(rt.host_pt[rows[i], begin[i]:begin[i] + cnt[i]])
            new_slots = np.ascontiguousarray(np.concatenate(parts), np.int32)
            rt._rs.kv_len[rows64] = kv_len
            batch = _Rows(node[req], rows, kv_len, rt._rs.written[rows64])
            n = int(cnt.sum())
            sl = slice(tok, tok + n)
            # a batch of decode tokens only runs on the decode kernel (few
            # query rows per key: bandwidth-bound); any prefill chunk makes it
            # an extend launch, its decode tokens sharing the tiles of their
            # group's chunks
            kind_p = rdx.PLAN_DECODE if n_dec == n_e else rdx.PLAN_EXTEND
            rt._launch(kind_p, batch, cnt, new_slots, self.q[sl], self.k[sl], self.v[sl], self.o[sl])
            # requests that completed: insert their sequences, unlock, free rows
            fin = kv_len.astype(np.int64) == self.req_total_len[req]
            if fin.any():
                fr = req[fin]
                toks = [self.seq_tokens[r] for r in fr]
                offs = np.concatenate([[0], np.cumsum([len(t) for t in toks])]).astype(np.int64)
                ft = np.concatenate(toks).astype(np.int32)
                frow = np.ascontiguousarray(row[fr], np.int32)
                fm = np.ascontiguousarray(matched[fr])
                fn = np.ascontiguousarray(node[fr])
                if keep_rows:
                    for r, rw in zip(fr, frow):
                        self.rows[int(self.req_rid[r])] = rt.host_pt[rw, :self.req_total_len[r]].copy()
                rdx._check(L.rdx_finish(rt.tree.handle, len(fr), p32(ft), p64(offs), p32(frow), rt._host_pt_p,
                                        rt.max_rows, rt.ld, p64(fm), p64(fn), ctypes.byref(done_n)))
                rt.free_rows.extend(frow.tolist())
                row[fr] = -1
            tok += n
            it += 1
        if tok != self.n_tokens or it != len(self.iterations):
            raise RuntimeError("the batcher's run differs from the staged one")
        return self.o
