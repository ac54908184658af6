"""Serving loop over the librdx C ABI: admit, extend, decode, finish.

The loop follows the SGLang notes (section 3): a request's prompt is
matched against the radix tree, the matched node is locked, KV slots are
allocated for the rest (evicting LRU leaves when short), and after the
request completes its tokens are inserted so later requests can reuse them.
The frontend hint (a shared prefix sent first on a fork) is just an earlier
batch here.  All computation runs in the library; this module marshals
arguments and keeps a host copy of the page-table rows for `finish`.

Protocol (the oracle models the same call sequence):
  admit:   per request in order: match_prefix, lock, alloc(n - m)
  extend:  one plan upload (page-table rows + work list), kv_store of the new
           tokens, one extend-attention launch
  decode:  per step one alloc(R) (slots to requests in order), one plan
           upload, kv_store of the R new tokens, one decode-attention launch
  finish:  per request: insert(prompt + generated, row), free duplicates,
           unlock
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import rdx


class _RowState:
    """Per page-table row: the KV length of the request holding the row and
    how many of its page-table entries are written on the device."""

    def __init__(self, rows: int):
        self.kv_len = np.zeros(rows, np.int32)
        self.written = np.zeros(rows, np.int32)


class Request:
    """A request admitted by a Runtime.  While it holds its page-table row,
    its KV length and written-entry count live in the runtime's per-row
    arrays (a decode step updates a whole batch at once); finish() freezes
    them into the request."""

    __slots__ = ("prompt", "matched", "node", "row", "new_slots", "_rs", "_frozen")

    def __init__(self, prompt, matched, node, row, new_slots, rs: _RowState, kv_len: int, written: int = 0):
        self.prompt, self.matched, self.node, self.row, self.new_slots = prompt, matched, node, row, new_slots
        self._rs, self._frozen = rs, None
        rs.kv_len[row] = kv_len
        rs.written[row] = written

    @property
    def kv_len(self) -> int:
        return self._frozen[0] if self._frozen else int(self._rs.kv_len[self.row])

    @kv_len.setter
    def kv_len(self, v: int):
        self._rs.kv_len[self.row] = v

    @property
    def written(self) -> int:
        return self._frozen[1] if self._frozen else int(self._rs.written[self.row])

    @written.setter
    def written(self, v: int):
        self._rs.written[self.row] = v

    def _freeze(self):
        self._frozen = (self.kv_len, self.written)


class _DecodeBatch:
    """Node and row arrays of one decode batch, in batch order, and the slot
    buffer its steps allocate into (built once per batch)."""

    def __init__(self, reqs):
        n = len(reqs)
        self.reqs, self.n = reqs, n
        self.node = np.fromiter((r.node for r in reqs), np.int64, n)
        self.row = np.fromiter((r.row for r in reqs), np.int32, n)
        self.row64 = self.row.astype(np.int64)
        self.slots = np.empty(max(1, n), np.int32)
        p32 = rdx._p32
        self.slots_p = p32(self.slots)
        self.node_p = self.node.ctypes.data_as(rdx.i64p)
        self.row_p = p32(self.row)

    def matches(self, reqs) -> bool:
        return (reqs is self.reqs and len(reqs) == self.n
                and (self.n == 0 or (reqs[0].row == self.row[0] and reqs[-1].row == self.row[-1])))


class Runtime:
    def __init__(self, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int, num_slots: int,
                 max_rows: int, ld: int, device="cuda", extend_items: int = 0, decode_items: int = 0):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.desc = rdx.attn_desc(rdx.BF16 if dtype == "bf16" else rdx.F32, num_q_heads, num_kv_heads,
                                  head_dim, num_slots)
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.num_slots, self.ld, self.max_rows = num_slots, ld, max_rows
        self.tree = rdx.Tree(num_slots)
        self.k_pool = torch.zeros((num_slots, num_kv_heads, head_dim), dtype=self.tdtype, device=self.device)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.page_table = torch.zeros((max_rows, ld), dtype=torch.int32, device=self.device)
        self.host_pt = np.zeros((max_rows, ld), np.int32)
        self._rs = _RowState(max_rows)
        self.free_rows = list(range(max_rows - 1, -1, -1))
        self.plans = {rdx.PLAN_EXTEND: rdx.Plan(self.desc, rdx.PLAN_EXTEND, extend_items),
                      rdx.PLAN_DECODE: rdx.Plan(self.desc, rdx.PLAN_DECODE, decode_items)}
        self.dev_plan = {k: torch.empty(0, dtype=torch.uint8, device=self.device) for k in self.plans}
        self.workspace = torch.zeros(0, dtype=torch.uint8, device=self.device)
        self.last_info = {}
        self.record = None   # a list to keep every launch (plan, buffers) for replay
        self._dec = None     # arrays of the current decode batch
        self._info = rdx.PlanInfo()
        self._info_ref = ctypes.byref(self._info)
        self._desc_ref = ctypes.byref(self.desc)
        self._io = rdx.StepIO()
        self._io.page_table = self.page_table.data_ptr()
        self._io.page_table_rows = max_rows
        self._io.k_pool = self.k_pool.data_ptr()
        self._io.v_pool = self.v_pool.data_ptr()
        self._io_ref = ctypes.byref(self._io)
        self._rs_p = (rdx._p32(self._rs.kv_len), rdx._p32(self._rs.written))
        self._host_pt_p = rdx._p32(self.host_pt)

    def reset(self):
        """Empty tree and page-table rows; pools and buffers are kept."""
        self.tree = rdx.Tree(self.num_slots)
        self.free_rows = list(range(self.max_rows - 1, -1, -1))
        self._dec = None

    # ------------------------------------------------------------ buffers
    def _dev_plan(self, kind: int, nbytes: int):
        buf = self.dev_plan[kind]
        if buf.numel() < nbytes:
            buf = self.torch.empty(max(nbytes, 2 * buf.numel()), dtype=self.torch.uint8, device=self.device)
            self.dev_plan[kind] = buf
        return buf

    def _workspace(self, nbytes: int):
        if self.workspace.numel() < nbytes:
            self.workspace = self.torch.empty(max(nbytes, 2 * self.workspace.numel()), dtype=self.torch.uint8,
                                              device=self.device)
        return self.workspace

    # ------------------------------------------------------------ protocol
    def admit(self, prompts) -> list:
        reqs = []
        for p in prompts:
            p = np.ascontiguousarray(p, np.int32)
            m, slots, node = self.tree.match_prefix(p)
            self.tree.lock(node)
            new = self.tree.alloc(len(p) - m).copy()
            if not self.free_rows:
                raise RuntimeError("no free page-table row")
            row = self.free_rows.pop()
            self.host_pt[row, :m] = slots
            self.host_pt[row, m:len(p)] = new
            reqs.append(Request(p, m, node, row, new, self._rs, len(p), 0))
        return reqs

    def _check(self, name, t, rows, heads):
        if (t.device != self.device or t.dtype != self.tdtype or not t.is_contiguous()
                or tuple(t.shape) != (rows, heads, self.d)):
            raise ValueError(f"{name}: expected contiguous {self.tdtype} [{rows}, {heads}, {self.d}] on "
                             f"{self.device}, got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _launch(self, kind: int, reqs, q_len, new_slots, q, k_new, v_new, o, timer=None):
        n_new = int(sum(q_len))
        self._check("q", q, n_new, self.hq)
        self._check("o", o, n_new, self.hq)
        self._check("k_new", k_new, n_new, self.hkv)
        self._check("v_new", v_new, n_new, self.hkv)
        if self.record is not None:
            # a fresh plan + device buffer per launch, kept for replay
            plan = rdx.Plan(self.desc, kind, self.plans[kind].target)
        else:
            plan = self.plans[kind]
        plan.build(self.tree, [r.node for r in reqs], [r.row for r in reqs], [r.kv_len for r in reqs], q_len,
                   [r.written for r in reqs], new_slots, self.ld)
        info = plan.info()
        self.last_info[kind] = info
        if self.record is not None:
            dev = self.torch.empty(max(info["device_bytes"], 64), dtype=self.torch.uint8, device=self.device)
        else:
            dev = self._dev_plan(kind, info["device_bytes"])
        plan.upload(dev, dev.numel(), self.page_table, self.max_rows)
        rdx.kv_store(self.desc, self.k_pool, self.v_pool, k_new, v_new,
                     dev.data_ptr() + info["new_slots_offset"], info["num_new"])
        ws = self._workspace(info["workspace_bytes"])
        fn = rdx.extend_attention if kind == rdx.PLAN_EXTEND else rdx.decode_attention
        if timer is not None:
            timer[0].record()
        fn(self.desc, plan, dev, q, self.k_pool, self.v_pool, self.page_table, o, ws, ws.numel())
        if timer is not None:
            timer[1].record()
        if self.record is not None:
            self.record.append((kind, plan, dev, q, o, info))
        for r in reqs:
            r.written = r.kv_len
        return o

    def replay(self, launches, reps: int = 1):
        """Re-issues recorded attention launches back to back (`reps` times).
        Attention reads the pools and writes O only, so a replay recomputes
        the same outputs; nothing else is launched in between."""
        for _ in range(reps):
            for kind, plan, dev, q, o, info in launches:
                ws = self._workspace(info["workspace_bytes"])
                fn = rdx.extend_attention if kind == rdx.PLAN_EXTEND else rdx.decode_attention
                fn(self.desc, plan, dev, q, self.k_pool, self.v_pool, self.page_table, o, ws, ws.numel())

    def extend(self, reqs, q, k_new, v_new, o=None, timer=None):
        """Queries q [sum new, Hq, D] and new K/V [sum new, Hkv, D] of the requests' uncached
        tokens, request-major.  Returns o [sum new, Hq, D]."""
        q_len = [r.kv_len - r.matched for r in reqs]
        new_slots = np.concatenate([r.new_slots for r in reqs]) if reqs else np.zeros(0, np.int32)
        if o is None:
            o = self.torch.empty_like(q)
        return self._launch(rdx.PLAN_EXTEND, reqs, q_len, new_slots, q, k_new, v_new, o, timer)

    def decode_step(self, reqs, q, k_new, v_new, o=None, timer=None):
        """One new token per request: q [R, Hq, D], k_new/v_new [R, Hkv, D].
        One rdx_decode_step call: slot allocation, page-table rows, plan,
        upload, KV scatter and decode attention (timer, if given, brackets
        the whole step)."""
        if self.record is not None:
            return self._decode_step_recorded(reqs, q, k_new, v_new, o, timer)
        db = self._dec
        if db is None or not db.matches(reqs):
            db = self._dec = _DecodeBatch(reqs)
        n = db.n
        self._check_step(q, k_new, v_new, o, n)
        if o is None:
            o = self.torch.empty_like(q)
        io = self._io
        io.q, io.k_new, io.v_new, io.o = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), o.data_ptr()
        plan = self.plans[rdx.PLAN_DECODE]
        st = self.torch.cuda.current_stream().cuda_stream
        if timer is not None:
            timer[0].record()
        L = rdx.lib()
        for _ in range(2):
            dp, ws = self.dev_plan[rdx.PLAN_DECODE], self.workspace
            io.dev_plan, io.dev_plan_bytes = dp.data_ptr(), dp.numel()
            io.workspace, io.workspace_bytes = ws.data_ptr(), ws.numel()
            rc = L.rdx_decode_step(self.tree.handle, plan.handle, self._desc_ref, n, db.node_p, db.row_p,
                                   self._rs_p[0], self._rs_p[1], self._host_pt_p, self.max_rows, self.ld,
                                   db.slots_p, self._io_ref, st, self._info_ref)
            if rc != rdx.ENOBUFS:
                break
            # buffers too small (nothing changed): grow to the reported sizes and retry
            self._dev_plan(rdx.PLAN_DECODE, self._info.device_bytes)
            self._workspace(self._info.workspace_bytes)
        rdx._check(rc)
        if timer is not None:
            timer[1].record()
        return o

    def _check_step(self, q, k_new, v_new, o, n):
        for name, t, heads in (("q", q, self.hq), ("k_new", k_new, self.hkv), ("v_new", v_new, self.hkv),
                               ("o", o, self.hq)):
            if t is not None:
                self._check(name, t, n, heads)

    def _decode_step_recorded(self, reqs, q, k_new, v_new, o, timer):
        slots = self.tree.alloc(len(reqs)).copy()
        rows = np.fromiter((r.row for r in reqs), np.int64, len(reqs))
        pos = np.fromiter((r.kv_len for r in reqs), np.int64, len(reqs))
        if pos.size and pos.max() >= self.ld:
            raise RuntimeError("page-table row full")
        self.host_pt[rows, pos] = slots
        for r in reqs:
            r.kv_len += 1
        if o is None:
            o = self.torch.empty_like(q)
        return self._launch(rdx.PLAN_DECODE, reqs, [1] * len(reqs), slots, q, k_new, v_new, o, timer)

    def finish(self, reqs, generated=None):
        """Insert each request's prompt + generated tokens, free duplicate slots, unlock."""
        self._dec = None
        for i, r in enumerate(reqs):
            gen = np.zeros(0, np.int32) if generated is None else np.asarray(generated[i], np.int32)
            seq = np.concatenate([r.prompt, gen]).astype(np.int32)
            if len(seq) != r.kv_len:
                raise ValueError("generated tokens do not match the request's length")
            row = self.host_pt[r.row, : r.kv_len]
            k, _ = self.tree.insert(seq, row)
            if k > r.matched:
                self.tree.free(row[r.matched:k])
            self.tree.unlock(r.node)
            r._freeze()
            self.free_rows.append(r.row)
