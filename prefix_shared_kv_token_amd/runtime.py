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

from dataclasses import dataclass

import numpy as np

from . import rdx


@dataclass
class Request:
    prompt: np.ndarray
    matched: int
    node: int
    row: int
    kv_len: int
    written: int = 0
    new_slots: np.ndarray | None = None


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
        self.free_rows = list(range(max_rows - 1, -1, -1))
        self.plans = {rdx.PLAN_EXTEND: rdx.Plan(self.desc, rdx.PLAN_EXTEND, extend_items),
                      rdx.PLAN_DECODE: rdx.Plan(self.desc, rdx.PLAN_DECODE, decode_items)}
        self.dev_plan = {k: torch.empty(0, dtype=torch.uint8, device=self.device) for k in self.plans}
        self.workspace = torch.zeros(0, dtype=torch.uint8, device=self.device)
        self.last_info = {}
        self.record = None   # a list to keep every launch (plan, buffers) for replay

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
            reqs.append(Request(p, m, node, row, len(p), 0, new))
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
        """One new token per request: q [R, Hq, D], k_new/v_new [R, Hkv, D]."""
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
            self.free_rows.append(r.row)
