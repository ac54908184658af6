"""ctypes binding of librdx (argument marshalling only).

Every function here forwards to the C ABI declared in include/rdx.h; the
computation happens in the library (host tree and planner in C++, device
work in HIP kernels).  Device arguments are torch tensors (only their data
pointers cross the boundary) or raw integer addresses; `stream` defaults to
torch's current stream.  If librdx.so is missing this module raises: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RDX_LIB selects another build of the same ABI (the host-only sanitizer
# build, whose device entry points fail with RDX_EUNSUPPORTED)
LIB_PATH = os.environ.get("RDX_LIB") or os.path.join(_HERE, "librdx.so")

OK, EINVAL, ENOSPC, ESTATE, EUNSUPPORTED, EDEVICE, ENOBUFS = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
PLAN_EXTEND, PLAN_DECODE = 0, 1

i32p = ctypes.POINTER(ctypes.c_int32)
i64p = ctypes.POINTER(ctypes.c_int64)
vp = ctypes.c_void_p
i64 = ctypes.c_int64
i32 = ctypes.c_int32


class Stats(ctypes.Structure):
    _fields_ = [(n, i64) for n in ("num_slots", "free", "cached", "evictable", "private",
                                   "nodes", "evictions", "clock")]


class NodeInfo(ctypes.Structure):
    _fields_ = [(n, i64) for n in ("id", "parent", "start", "length", "ref", "last_access", "num_children",
                                   "hits", "priority")]


class AttnDesc(ctypes.Structure):
    _fields_ = [("dtype", i32), ("num_q_heads", i32), ("num_kv_heads", i32), ("head_dim", i32),
                ("sm_scale", ctypes.c_float), ("kv_row_pitch", i32), ("num_slots", i64)]


class Batch(ctypes.Structure):
    _fields_ = [("num_reqs", i32), ("reserved", i32), ("node", i64p), ("row", i32p), ("kv_len", i32p),
                ("q_len", i32p), ("written", i32p), ("new_slots", i32p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, i64) for n in ("device_bytes", "workspace_bytes", "new_slots_offset", "num_new",
                                   "num_items", "num_tiles", "num_jobs", "num_split_tiles",
                                   "num_shared_segments", "key_rows")]


class PlanView(ctypes.Structure):
    _fields_ = [("items", i32p), ("num_items", i64), ("tiles", i32p), ("num_tiles", i64),
                ("jobs", i32p), ("num_jobs", i64), ("tokens", i32p), ("num_tokens", i64),
                ("contribs", i32p), ("num_contribs", i64), ("tile_rows", i32), ("group", i32)]


class StepIO(ctypes.Structure):
    _fields_ = [("dev_plan", vp), ("dev_plan_bytes", i64), ("workspace", vp), ("workspace_bytes", i64),
                ("page_table", vp), ("page_table_rows", i64), ("k_pool", vp), ("v_pool", vp),
                ("q", vp), ("k_new", vp), ("v_new", vp), ("o", vp)]


class TbEntry(ctypes.Structure):
    _fields_ = [("kind", i32), ("group", i32), ("member", i32), ("begin", i32), ("count", i32)]


_SIGS = {
    "rdx_last_error": (ctypes.c_char_p, []),
    "rdx_version": (ctypes.c_char_p, []),
    "rdx_tree_create": (ctypes.c_int, [i64, i32, ctypes.POINTER(vp)]),
    "rdx_tree_destroy": (None, [vp]),
    "rdx_match_prefix": (ctypes.c_int, [vp, i32p, i64, i32p, i64p, i64p]),
    "rdx_lock": (ctypes.c_int, [vp, i64]),
    "rdx_unlock": (ctypes.c_int, [vp, i64]),
    "rdx_alloc": (ctypes.c_int, [vp, i64, i32p]),
    "rdx_free": (ctypes.c_int, [vp, i32p, i64]),
    "rdx_insert": (ctypes.c_int, [vp, i32p, i32p, i64, i64p, i64p]),
    "rdx_evict": (ctypes.c_int, [vp, i64, i64p]),
    "rdx_admit": (ctypes.c_int, [vp, i32, i32p, i64p, i32p, i32p, i64, i64, i64p, i64p, i32p, i32p]),
    "rdx_finish": (ctypes.c_int, [vp, i32, i32p, i64p, i32p, i32p, i64, i64, i64p, i64p, i32p]),
    "rdx_schedule": (ctypes.c_int, [vp, i32, i32p, i64p, i32, i32p, i64p]),
    "rdx_batcher_create": (ctypes.c_int, [i32, i32p, i32p, i32p, i32p, i32, i64, ctypes.POINTER(vp)]),
    "rdx_batcher_destroy": (None, [vp]),
    "rdx_batcher_next": (ctypes.c_int, [vp, vp, i32, i32p]),
    "rdx_tree_set_policy": (ctypes.c_int, [vp, i32]),
    "rdx_tree_set_priority": (ctypes.c_int, [vp, i32]),
    "rdx_prefix_groups": (ctypes.c_int, [i32, i32p, i64p, i32p, i64p, i32p, i64p]),
    "rdx_job_create": (ctypes.c_int, [vp, i32, i32p, i32p, i32p, i32p, i32, i64, i32p, i64p, i32, i64, i32,
                                       ctypes.POINTER(vp)]),
    "rdx_job_destroy": (None, [vp]),
    "rdx_job_prepare": (ctypes.c_int, [vp, vp, vp, i64p, i32p, vp]),
    "rdx_job_launch": (ctypes.c_int, [vp, vp, vp, vp, vp]),
    "rdx_job_complete": (ctypes.c_int, [vp, i32p]),
    "rdx_job_row": (ctypes.c_int, [vp, i32, i32p, i64, i64p, i64p]),
    "rdx_tree_stats": (ctypes.c_int, [vp, ctypes.POINTER(Stats)]),
    "rdx_node_get": (ctypes.c_int, [vp, i64, ctypes.POINTER(NodeInfo), i32p]),
    "rdx_kv_store": (ctypes.c_int, [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, i64, vp]),
    "rdx_kv_row_pitch_recommended": (ctypes.c_int, [ctypes.POINTER(AttnDesc), i32p]),
    "rdx_plan_create": (ctypes.c_int, [ctypes.POINTER(AttnDesc), i32, i32, ctypes.POINTER(vp)]),
    "rdx_plan_destroy": (None, [vp]),
    "rdx_plan_build": (ctypes.c_int, [vp, vp, ctypes.POINTER(Batch), i64]),
    "rdx_plan_get_info": (ctypes.c_int, [vp, ctypes.POINTER(PlanInfo)]),
    "rdx_plan_get_view": (ctypes.c_int, [vp, ctypes.POINTER(PlanView)]),
    "rdx_plan_upload": (ctypes.c_int, [vp, vp, i64, vp, i64, vp]),
    "rdx_extend_attention": (ctypes.c_int, [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
    "rdx_decode_attention": (ctypes.c_int, [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
    "rdx_decode_attention_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp]),
    "rdx_decode_step": (ctypes.c_int, [vp, vp, ctypes.POINTER(AttnDesc), i32, i64p, i32p, i32p, i32p, i32p, i64,
                                       i64, i32p, ctypes.POINTER(StepIO), vp, ctypes.POINTER(PlanInfo)]),
    "rdx_timing_begin": (ctypes.c_int, [i32]),
    "rdx_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), i32p, i32,
                                       i32p]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class RdxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"rdx error {code}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != OK:
        raise RdxError(rc, lib().rdx_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p32(a: np.ndarray):
    return a.ctypes.data_as(i32p)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------- tree
EVICT_POLICIES = {"lru": 0, "lfu": 1, "slru": 2, "priority": 3}


class Tree:
    """rdx_tree: radix tree + slot allocator (host)."""

    def __init__(self, num_slots: int, match_unit: int = 1, policy: str = "lru"):
        h = vp()
        _check(lib().rdx_tree_create(num_slots, match_unit, ctypes.byref(h)))
        self._h = h
        if policy != "lru":
            if policy not in EVICT_POLICIES:
                raise ValueError(f"unknown eviction policy {policy!r}")
            _check(lib().rdx_tree_set_policy(h, EVICT_POLICIES[policy]))
        self.num_slots = num_slots
        self._buf = np.empty(0, np.int32)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.rdx_tree_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def set_priority(self, priority: int):
        _check(lib().rdx_tree_set_priority(self._h, int(priority)))

    def match_prefix(self, tokens):
        t = _i32(tokens)
        out = np.empty(max(1, len(t)), np.int32)
        m, node = i64(), i64()
        _check(lib().rdx_match_prefix(self._h, _p32(t), len(t), _p32(out), ctypes.byref(m), ctypes.byref(node)))
        return m.value, out[: m.value], node.value

    def lock(self, node: int):
        _check(lib().rdx_lock(self._h, node))

    def unlock(self, node: int):
        _check(lib().rdx_unlock(self._h, node))

    def alloc(self, n: int, out: np.ndarray | None = None) -> np.ndarray:
        if out is None:
            out = np.empty(max(1, n), np.int32)
        _check(lib().rdx_alloc(self._h, n, _p32(out)))
        return out[:n]

    def free(self, slots):
        s = _i32(slots)
        _check(lib().rdx_free(self._h, _p32(s), len(s)))

    def insert(self, tokens, slots):
        t, s = _i32(tokens), _i32(slots)
        if len(t) != len(s):
            raise ValueError("tokens and slots differ in length")
        k, node = i64(), i64()
        _check(lib().rdx_insert(self._h, _p32(t), _p32(s), len(t), ctypes.byref(k), ctypes.byref(node)))
        return k.value, node.value

    def evict(self, n_tokens: int) -> int:
        f = i64()
        _check(lib().rdx_evict(self._h, n_tokens, ctypes.byref(f)))
        return f.value

    def schedule(self, prompts, fcfs_above: int = 128):
        """Cache-aware order of the waiting `prompts` (arrival order) ->
        (order, score of each request when placed), both numpy arrays."""
        n = len(prompts)
        offsets = np.zeros(n + 1, np.int64)
        if n:
            np.cumsum([len(p) for p in prompts], out=offsets[1:])
        flat = _i32(np.concatenate([np.asarray(p, np.int32).ravel() for p in prompts]) if n else [])
        if flat.size == 0:
            flat = np.zeros(1, np.int32)
        order = np.empty(max(1, n), np.int32)
        score = np.empty(max(1, n), np.int64)
        _check(lib().rdx_schedule(self._h, n, _p32(flat), offsets.ctypes.data_as(i64p), fcfs_above,
                                  _p32(order), score.ctypes.data_as(i64p)))
        return order[:n], score[:n]

    def stats(self) -> dict:
        s = Stats()
        _check(lib().rdx_tree_stats(self._h, ctypes.byref(s)))
        return {n: getattr(s, n) for n, _ in Stats._fields_}

    def node(self, node_id: int) -> dict:
        info = NodeInfo()
        _check(lib().rdx_node_get(self._h, node_id, ctypes.byref(info), None))
        slots = np.empty(max(1, info.length), np.int32)
        _check(lib().rdx_node_get(self._h, node_id, ctypes.byref(info), _p32(slots)))
        d = {n: getattr(info, n) for n, _ in NodeInfo._fields_}
        d["slots"] = slots[: info.length].copy()
        return d


def prefix_groups(prompts):
    """Global prefix analysis of a batch -> (group id per request, group
    prefix length per request, number of groups, N_processed)."""
    n = len(prompts)
    offsets = np.zeros(n + 1, np.int64)
    if n:
        np.cumsum([len(p) for p in prompts], out=offsets[1:])
    flat = _i32(np.concatenate([np.asarray(p, np.int32).ravel() for p in prompts]) if n else [])
    return prefix_groups_flat(flat, offsets)


def prefix_groups_flat(flat, offsets):
    """prefix_groups of the prompts flat[offsets[i]:offsets[i+1]]."""
    flat = _i32(flat)
    offsets = np.ascontiguousarray(offsets, np.int64)
    n = len(offsets) - 1
    if flat.size == 0:
        flat = np.zeros(1, np.int32)
    group = np.empty(max(1, n), np.int32)
    prefix = np.empty(max(1, n), np.int64)
    ng, proc = i32(), i64()
    _check(lib().rdx_prefix_groups(n, _p32(flat), offsets.ctypes.data_as(i64p), _p32(group),
                                   prefix.ctypes.data_as(i64p), ctypes.byref(ng), ctypes.byref(proc)))
    return group[:n], prefix[:n], ng.value, proc.value


# ------------------------------------------------------------------ batcher
TB_DECODE, TB_DISTINCT, TB_PREFIX = 0, 1, 2


class Batcher:
    """rdx_batcher: throughput-oriented token batching of a job of groups
    (prefix length, members' distinct prompt and decode lengths)."""

    def __init__(self, prefix_len, member_offsets, distinct_len, decode_len, s_chunk: int, m_threshold: int):
        pl, mo, dl, dc = _i32(prefix_len), _i32(member_offsets), _i32(distinct_len), _i32(decode_len)
        self._keep = (pl, mo, dl, dc)
        h = vp()
        _check(lib().rdx_batcher_create(len(pl), _p32(pl), _p32(mo), _p32(dl) if len(dl) else None,
                                        _p32(dc) if len(dc) else None, s_chunk, m_threshold, ctypes.byref(h)))
        self._h = h
        self._cap = len(dl) + len(pl) + 1
        self._buf = np.zeros((self._cap, 5), np.int32)
        self._n = i32()

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.rdx_batcher_destroy(h)
            self._h = None

    def next(self) -> np.ndarray:
        """The next iteration's entries, int32 [n, 5] rows (kind, group,
        member, begin, count); empty once the job is done.  A view of an
        internal buffer, valid until the next call."""
        _check(lib().rdx_batcher_next(self._h, self._buf.ctypes.data, self._cap, ctypes.byref(self._n)))
        return self._buf[: self._n.value]


# ---------------------------------------------------------------------- job
JOB_KEEP_ROWS, JOB_DRY_RUN = 1, 2


class Job:
    """rdx_job: a token-batched job run natively over a tree, one iteration
    per prepare / launch / complete."""

    def __init__(self, tree: "Tree", prefix_len, member_offsets, distinct_len, decode_len, s_chunk: int,
                 m_threshold: int, seq_tokens, seq_offsets, num_rows: int, ld: int, flags: int = 0):
        arrs = [_i32(prefix_len), _i32(member_offsets), _i32(distinct_len), _i32(decode_len)]
        toks = _i32(seq_tokens) if len(seq_tokens) else np.zeros(1, np.int32)
        offs = np.ascontiguousarray(seq_offsets, np.int64)
        h = vp()
        _check(lib().rdx_job_create(tree.handle, len(arrs[0]), *[_p32(a) for a in arrs], s_chunk, m_threshold,
                                    _p32(toks), offs.ctypes.data_as(i64p), num_rows, ld, flags, ctypes.byref(h)))
        self._h = h
        self.tree = tree  # the job borrows the tree and the sequences
        self._keep = (toks, offs)
        self.info = PlanInfo()
        self._n, self._kind, self._fin = i64(), i32(), i32()
        self._refs = (ctypes.byref(self._n), ctypes.byref(self._kind), ctypes.byref(self.info),
                      ctypes.byref(self._fin))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.rdx_job_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def prepare(self, extend_plan: "Plan", decode_plan: "Plan"):
        """-> (query tokens of the next iteration (0: done), plan kind)."""
        _check(lib().rdx_job_prepare(self._h, extend_plan.handle, decode_plan.handle, self._refs[0], self._refs[1],
                                     self._refs[2]))
        return self._n.value, self._kind.value

    def complete(self) -> int:
        _check(lib().rdx_job_complete(self._h, self._refs[3]))
        return self._fin.value

    def row(self, req: int):
        """-> (final page-table row, matched length) of a finished request."""
        n, m = i64(), i64()
        buf = np.empty(1, np.int32)
        rc = lib().rdx_job_row(self._h, req, _p32(buf), 0, ctypes.byref(n), ctypes.byref(m))
        if rc not in (OK, ENOBUFS):
            _check(rc)
        buf = np.empty(max(1, n.value), np.int32)
        _check(lib().rdx_job_row(self._h, req, _p32(buf), len(buf), ctypes.byref(n), ctypes.byref(m)))
        return buf[: n.value], m.value


# --------------------------------------------------------------------- plan
def attn_desc(dtype: int, num_q_heads: int, num_kv_heads: int, head_dim: int, num_slots: int,
              sm_scale: float = 0.0, kv_row_pitch: int = 0) -> AttnDesc:
    return AttnDesc(dtype, num_q_heads, num_kv_heads, head_dim, sm_scale, kv_row_pitch, num_slots)


def kv_row_pitch_recommended(desc: AttnDesc) -> int:
    out = i32(0)
    _check(lib().rdx_kv_row_pitch_recommended(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


class Plan:
    """rdx_plan: work list of one extend or decode launch."""

    def __init__(self, desc: AttnDesc, kind: int, target_items: int = 0):
        h = vp()
        _check(lib().rdx_plan_create(ctypes.byref(desc), kind, target_items, ctypes.byref(h)))
        self._h = h
        self.desc = desc
        self.kind = kind
        self.target = target_items
        self._keep = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.rdx_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def build(self, tree: Tree, node, row, kv_len, q_len, written, new_slots, page_table_ld: int):
        node = np.ascontiguousarray(node, np.int64)
        arrs = [_i32(row), _i32(kv_len), _i32(q_len), _i32(written), _i32(new_slots)]
        b = Batch(len(node), 0, node.ctypes.data_as(i64p), *[_p32(a) for a in arrs])
        self._keep = (node, arrs)
        _check(lib().rdx_plan_build(self._h, tree.handle, ctypes.byref(b), page_table_ld))

    def info(self) -> dict:
        i = PlanInfo()
        _check(lib().rdx_plan_get_info(self._h, ctypes.byref(i)))
        return {n: getattr(i, n) for n, _ in PlanInfo._fields_}

    def view(self) -> dict:
        v = PlanView()
        _check(lib().rdx_plan_get_view(self._h, ctypes.byref(v)))

        def arr(p, n, w):
            if n == 0:
                return np.zeros((0, w), np.int32)
            return np.ctypeslib.as_array(p, shape=(n * w,)).reshape(n, w).copy()

        return dict(items=arr(v.items, v.num_items, 20), tiles=arr(v.tiles, v.num_tiles, 8),
                    jobs=arr(v.jobs, v.num_jobs, 8), tokens=arr(v.tokens, v.num_tokens, 2),
                    contribs=arr(v.contribs, v.num_contribs, 4), tile_rows=v.tile_rows, group=v.group)

    def upload(self, dev_plan, dev_plan_bytes: int, page_table, page_table_rows: int, stream=None):
        _check(lib().rdx_plan_upload(self._h, _ptr(dev_plan), dev_plan_bytes, _ptr(page_table),
                                     page_table_rows, _stream(stream)))


# ------------------------------------------------------------- device ops
def kv_store(desc: AttnDesc, k_pool, v_pool, k_new, v_new, slots, n: int, stream=None):
    _check(lib().rdx_kv_store(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                              _ptr(slots), n, _stream(stream)))


def extend_attention(desc: AttnDesc, plan: Plan, dev_plan, q, k_pool, v_pool, page_table, o,
                     workspace, workspace_bytes: int, stream=None):
    _check(lib().rdx_extend_attention(ctypes.byref(desc), plan.handle, _ptr(dev_plan), _ptr(q), _ptr(k_pool),
                                      _ptr(v_pool), _ptr(page_table), _ptr(o), _ptr(workspace),
                                      workspace_bytes, _stream(stream)))


def decode_attention(desc: AttnDesc, plan: Plan, dev_plan, q, k_pool, v_pool, page_table, o,
                     workspace, workspace_bytes: int, stream=None):
    _check(lib().rdx_decode_attention(ctypes.byref(desc), plan.handle, _ptr(dev_plan), _ptr(q), _ptr(k_pool),
                                      _ptr(v_pool), _ptr(page_table), _ptr(o), _ptr(workspace),
                                      workspace_bytes, _stream(stream)))


def decode_attention_noalloc(desc: AttnDesc, plan: Plan, dev_plan, q, k_pool, v_pool, page_table, o, stream=None):
    _check(lib().rdx_decode_attention_noalloc(ctypes.byref(desc), plan.handle, _ptr(dev_plan), _ptr(q),
                                              _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(o),
                                              _stream(stream)))


def timing_begin(cap: int):
    _check(lib().rdx_timing_begin(cap))


def timing_read(cap: int):
    """-> (attention_ms, merge_ms, kinds) of the launches recorded since
    timing_begin: float32[n] kernel durations (merge 0 where none ran) and
    int32[n] plan kinds, in launch order."""
    ms = np.zeros(max(cap, 1), np.float32)
    mm = np.zeros(max(cap, 1), np.float32)
    kinds = np.zeros(max(cap, 1), np.int32)
    n = i32()
    fp = ctypes.POINTER(ctypes.c_float)
    _check(lib().rdx_timing_read(ms.ctypes.data_as(fp), mm.ctypes.data_as(fp), _p32(kinds), cap, ctypes.byref(n)))
    return ms[: n.value].copy(), mm[: n.value].copy(), kinds[: n.value].copy()
