"""Serving loop over the librdx C ABI: admit, extend, decode, finish.

The loop follows the SGLang notes (section 3): a request's prompt is
matched against the radix tree, the matched node is locked, KV slots are
allocated for the rest (evicting LRU leaves when short), and after the
request completes its tokens are inserted so later requests can reuse them.
The frontend hint (a shared prefix sent first on a fork) is just an earlier
batch here.  All computation runs in the library; this module marshals
arguments and keeps a host copy of the page-table rows for `finish`.

Protocol (the oracle models the same call sequence):
  admit:   one rdx_admit: per request in order match_prefix, lock,
           alloc(n - m), page-table row on the host
  extend:  one plan upload (page-table rows + work list), kv_store of the new
           tokens, one extend-attention launch
  decode:  per step one rdx_decode_step: alloc(R) (slots to requests in
           order), plan, upload, KV scatter, decode attention
  finish:  one rdx_finish: per request insert(prompt + generated, row), free
           duplicates, unlock
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


class Batch:
    """A batch admitted by a Runtime: per-request arrays in batch order (the
    concatenated prompts, their page-table rows, matched lengths, locked
    nodes, and the newly allocated slots, request-major).  While the batch
    holds its rows, the requests' KV lengths and written-entry counts live
    in the runtime's per-row arrays (a decode step updates them in one
    call); finish() freezes them into the batch.  Indexing gives a Request
    view of one request."""

    def __init__(self, rs: _RowState, tokens, offsets, rows, matched, nodes, new_slots):
        self._rs = rs
        self.n = len(rows)
        self.tokens, self.offsets = tokens, offsets
        self.rows = rows                      # int32
        self.rows64 = rows.astype(np.int64)
        self.matched, self.nodes = matched, nodes  # int64
        self.lens = np.diff(offsets)
        self.q_lens = self.lens - matched
        self.new_off = np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int64)
        self.new_slots = new_slots            # int32, request-major
        self._final = None
        # fixed arguments of the per-token decode call
        self.slots = np.empty(max(1, self.n), np.int32)
        self.slots_p = rdx._p32(self.slots)
        self.node_p = self.nodes.ctypes.data_as(rdx.i64p)
        self.row_p = rdx._p32(self.rows)

    def __len__(self):
        return self.n

    def __getitem__(self, i):
        if not -self.n <= i < self.n:
            raise IndexError(i)
        return Request(self, i % self.n)

    def __iter__(self):
        return (Request(self, i) for i in range(self.n))

    @property
    def kv_len(self) -> np.ndarray:
        return self._final[0] if self._final is not None else self._rs.kv_len[self.rows64]

    @property
    def written(self) -> np.ndarray:
        return self._final[1] if self._final is not None else self._rs.written[self.rows64]


class Request:
    """View of request i of a Batch."""

    __slots__ = ("_b", "_i")

    def __init__(self, batch: Batch, i: int):
        self._b, self._i = batch, i

    prompt = property(lambda self: self._b.tokens[self._b.offsets[self._i]:self._b.offsets[self._i + 1]])
    matched = property(lambda self: int(self._b.matched[self._i]))
    node = property(lambda self: int(self._b.nodes[self._i]))
    row = property(lambda self: int(self._b.rows[self._i]))
    new_slots = property(lambda self: self._b.new_slots[self._b.new_off[self._i]:self._b.new_off[self._i + 1]])

    @property
    def kv_len(self) -> int:
        return int(self._b.kv_len[self._i])

    @property
    def written(self) -> int:
        return int(self._b.written[self._i])


class Runtime:
    def __init__(self, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int, num_slots: int,
                 max_rows: int, ld: int, device="cuda", extend_items: int = 0, decode_items: int = 0,
                 kv_row_pitch: int | None = None):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.desc = rdx.attn_desc(rdx.BF16 if dtype == "bf16" else rdx.F32, num_q_heads, num_kv_heads,
                                  head_dim, num_slots)
        # pools with the row pitch the kernels stream fastest (rows padded past
        # the Hkv x head_dim a slot holds), unless the caller gives one
        # (elements; 0 = dense rows)
        if kv_row_pitch is None:
            kv_row_pitch = rdx.kv_row_pitch_recommended(self.desc)
        self.desc.kv_row_pitch = kv_row_pitch
        self.kv_row_pitch = kv_row_pitch or num_kv_heads * head_dim
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.num_slots, self.ld, self.max_rows = num_slots, ld, max_rows
        self.tree = rdx.Tree(num_slots)
        self.k_pool = torch.zeros((num_slots, self.kv_row_pitch), dtype=self.tdtype, device=self.device)
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
    def schedule(self, prompts, fcfs_above: int = 128) -> np.ndarray:
        """Cache-aware order of the waiting prompts (arrival order in): the
        order to admit them in, longest prefix shared with the tree or with a
        request placed ahead first; arrival order above `fcfs_above`."""
        return self.tree.schedule(prompts, fcfs_above)[0]

    def admit(self, prompts) -> Batch:
        """Admit a list of prompts (token id arrays) as one batch."""
        prompts = [np.asarray(p, np.int32) for p in prompts]
        offsets = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int64)
        tokens = np.concatenate(prompts) if prompts else np.zeros(0, np.int32)
        return self.admit_tokens(tokens, offsets)

    def admit_tokens(self, tokens: np.ndarray, offsets: np.ndarray) -> Batch:
        """Admit the prompts tokens[offsets[i]:offsets[i+1]] in one rdx_admit
        call: per request, match, lock the matched node, allocate the rest,
        and fill its page-table row on the host."""
        tokens = np.ascontiguousarray(tokens, np.int32)
        offsets = np.ascontiguousarray(offsets, np.int64)
        n = len(offsets) - 1
        if n > len(self.free_rows):
            raise RuntimeError(f"no free page-table rows for {n} requests ({len(self.free_rows)} free)")
        cut = len(self.free_rows) - n
        rows = np.array(self.free_rows[cut:][::-1], np.int32)
        del self.free_rows[cut:]
        matched = np.zeros(n, np.int64)
        nodes = np.zeros(n, np.int64)
        new_slots = np.empty(max(1, int(offsets[-1] - offsets[0])), np.int32)
        done = rdx.i32()
        p32, p64 = rdx._p32, (lambda x: x.ctypes.data_as(rdx.i64p))
        rc = rdx.lib().rdx_admit(self.tree.handle, n, p32(tokens), p64(offsets), p32(rows), self._host_pt_p,
                                 self.max_rows, self.ld, p64(matched), p64(nodes), p32(new_slots),
                                 ctypes.byref(done))
        if rc != rdx.OK:
            msg = rdx.lib().rdx_last_error().decode()
            k = done.value  # release the requests admitted before the failure
            q = (np.diff(offsets) - matched)[:k]
            off = np.concatenate([[0], np.cumsum(q)]).astype(np.int64)
            for i in range(k):
                self.tree.unlock(int(nodes[i]))
                self.tree.free(new_slots[off[i]:off[i + 1]])
            self.free_rows.extend(rows[::-1].tolist())
            raise rdx.RdxError(rc, msg)
        lens = np.diff(offsets)
        self._rs.kv_len[rows] = lens
        self._rs.written[rows] = 0
        return Batch(self._rs, tokens, offsets, rows, matched, nodes, new_slots)

    def _check(self, name, t, rows, heads):
        if (t.device != self.device or t.dtype != self.tdtype or not t.is_contiguous()
                or tuple(t.shape) != (rows, heads, self.d)):
            raise ValueError(f"{name}: expected contiguous {self.tdtype} [{rows}, {heads}, {self.d}] on "
                             f"{self.device}, got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _launch(self, kind: int, reqs: Batch, q_len, new_slots, q, k_new, v_new, o, timer=None):
        n_new = int(np.sum(q_len))
        self._check("q", q, n_new, self.hq)
        self._check("o", o, n_new, self.hq)
        self._check("k_new", k_new, n_new, self.hkv)
        self._check("v_new", v_new, n_new, self.hkv)
        if self.record is not None:
            # a fresh plan + device buffer per launch, kept for replay
            plan = rdx.Plan(self.desc, kind, self.plans[kind].target)
        else:
            plan = self.plans[kind]
        plan.build(self.tree, reqs.nodes, reqs.rows, reqs.kv_len, q_len, reqs.written, new_slots, self.ld)
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
        self._rs.written[reqs.rows64] = self._rs.kv_len[reqs.rows64]
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

    def extend(self, reqs: Batch, q, k_new, v_new, o=None, timer=None):
        """Queries q [sum new, Hq, D] and new K/V [sum new, Hkv, D] of the requests' uncached
        tokens, request-major.  Returns o [sum new, Hq, D]."""
        q_len = reqs.kv_len - reqs.matched
        new_slots = reqs.new_slots[: int(reqs.new_off[-1])]
        if o is None:
            o = self.torch.empty_like(q)
        return self._launch(rdx.PLAN_EXTEND, reqs, q_len, new_slots, q, k_new, v_new, o, timer)

    def decode_step(self, reqs: Batch, q, k_new, v_new, o=None, timer=None):
        """One new token per request: q [R, Hq, D], k_new/v_new [R, Hkv, D].
        One rdx_decode_step call: slot allocation, page-table rows, plan,
        upload, KV scatter and decode attention (timer, if given, brackets
        the whole step)."""
        if self.record is not None:
            return self._decode_step_recorded(reqs, q, k_new, v_new, o, timer)
        db = reqs
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

    def decode_steps(self, reqs: Batch, q, k_new, v_new, o, timers=None):
        """T decode steps back to back, the same calls as T decode_step calls
        with the tensors checked once: q [T, R, Hq, D], k_new/v_new
        [T, R, Hkv, D]; o [T, R, Hq, D] (step t writes o[t]) or [R, Hq, D]
        (every step writes it: it ends holding the last step's output).
        timers: None, or one event pair per step (then each step goes
        through decode_step)."""
        T = q.shape[0] if q.dim() == 4 else -1
        if T < 0 or k_new.dim() != 4 or v_new.dim() != 4 or k_new.shape[0] != T or v_new.shape[0] != T:
            raise ValueError("decode_steps: q, k_new, v_new must be [T, R, heads, D] with the same T")
        per_step_o = o.dim() == 4
        if per_step_o and o.shape[0] != T:
            raise ValueError("decode_steps: o must be [T, R, Hq, D] or [R, Hq, D]")
        if self.record is not None or timers is not None:
            for t in range(T):
                self.decode_step(reqs, q[t], k_new[t], v_new[t], o=o[t] if per_step_o else o,
                                 timer=timers[t] if timers is not None else None)
            return o
        if T == 0:
            return o
        n = reqs.n
        # every step's slice is checked through the first one: same shape, and
        # contiguous when the first is (slices of a tensor along dim 0)
        self._check_step(q[0], k_new[0], v_new[0], o[0] if per_step_o else o, n)
        q_step, k_step, v_step = (x.stride(0) * x.element_size() for x in (q, k_new, v_new))
        o_step = o.stride(0) * o.element_size() if per_step_o else 0
        q0, k0, v0, o0 = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), o.data_ptr()
        io = self._io
        plan = self.plans[rdx.PLAN_DECODE]
        st = self.torch.cuda.current_stream().cuda_stream
        L = rdx.lib()
        call = L.rdx_decode_step
        args_head = (self.tree.handle, plan.handle, self._desc_ref, n, reqs.node_p, reqs.row_p,
                     self._rs_p[0], self._rs_p[1], self._host_pt_p, self.max_rows, self.ld, reqs.slots_p,
                     self._io_ref, st, self._info_ref)

        def bind_buffers():
            dp, ws = self.dev_plan[rdx.PLAN_DECODE], self.workspace
            io.dev_plan, io.dev_plan_bytes = dp.data_ptr(), dp.numel()
            io.workspace, io.workspace_bytes = ws.data_ptr(), ws.numel()

        bind_buffers()
        for t in range(T):
            io.q, io.k_new, io.v_new, io.o = q0 + t * q_step, k0 + t * k_step, v0 + t * v_step, o0 + t * o_step
            rc = call(*args_head)
            if rc == rdx.ENOBUFS:
                # buffers too small (nothing changed): grow to the reported sizes and retry
                self._dev_plan(rdx.PLAN_DECODE, self._info.device_bytes)
                self._workspace(self._info.workspace_bytes)
                bind_buffers()
                rc = call(*args_head)
            rdx._check(rc)
        return o

    def _check_step(self, q, k_new, v_new, o, n):
        for name, t, heads in (("q", q, self.hq), ("k_new", k_new, self.hkv), ("v_new", v_new, self.hkv),
                               ("o", o, self.hq)):
            if t is not None:
                self._check(name, t, n, heads)

    def _decode_step_recorded(self, reqs: Batch, q, k_new, v_new, o, timer):
        n = reqs.n
        pos = self._rs.kv_len[reqs.rows64].astype(np.int64)
        if n and pos.max() >= self.ld:
            raise RuntimeError("page-table row full")
        slots = self.tree.alloc(n).copy()
        self.host_pt[reqs.rows64, pos] = slots
        self._rs.kv_len[reqs.rows64] += 1
        if o is None:
            o = self.torch.empty_like(q)
        return self._launch(rdx.PLAN_DECODE, reqs, np.ones(n, np.int32), slots, q, k_new, v_new, o, timer)

    def finish(self, reqs: Batch, generated=None, seq=None):
        """One rdx_finish call: per request, insert prompt + generated tokens
        with the row's slots, free the duplicates, unlock.  generated: per
        request the generated token ids (or None); seq: the full sequences
        already concatenated, as (tokens, offsets)."""
        kv = reqs.kv_len.astype(np.int64)
        if seq is not None:
            tokens, offsets = np.ascontiguousarray(seq[0], np.int32), np.ascontiguousarray(seq[1], np.int64)
        elif generated is None:
            tokens, offsets = reqs.tokens, reqs.offsets
        else:
            parts = []
            for i in range(reqs.n):
                parts.append(reqs.tokens[reqs.offsets[i]:reqs.offsets[i + 1]])
                parts.append(np.asarray(generated[i], np.int32))
            tokens = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
            glen = np.array([len(generated[i]) for i in range(reqs.n)], np.int64)
            offsets = np.concatenate([[0], np.cumsum(reqs.lens + glen)]).astype(np.int64)
        if len(offsets) != reqs.n + 1 or not np.array_equal(np.diff(offsets), kv):
            raise ValueError("generated tokens do not match the requests' lengths")
        done = rdx.i32()
        p32, p64 = rdx._p32, (lambda x: x.ctypes.data_as(rdx.i64p))
        rdx._check(rdx.lib().rdx_finish(self.tree.handle, reqs.n, p32(tokens), p64(offsets), p32(reqs.rows),
                                        self._host_pt_p, self.max_rows, self.ld, p64(reqs.matched),
                                        p64(reqs.nodes), ctypes.byref(done)))
        reqs._final = (kv.astype(np.int32), self._rs.written[reqs.rows64].copy())
        self.free_rows.extend(reqs.rows.tolist())
