"""Seeded generation of the synthetic workloads.

Recipe (the same for every consumer):
  * every random stream is `numpy.random.default_rng(SeedSequence([1234,
    config_index, TAG, ids...]))`, so any piece (one node's keys, one
    request's queries) can be regenerated on its own;
  * token ids are uniform integers in [0, vocab); the first token of a
    segment is redrawn until it differs from the first tokens of all its
    sibling segments, so the sharing tree is exactly the intended one;
  * Q, K and V are N(0, 1) * sigma drawn in float32 with torch's CPU
    generator (seeded from the same SeedSequence; its output does not depend
    on the thread count); for bf16 workloads they are then rounded to
    bfloat16 (round to nearest even) and both sides consume the rounded values
    (the GPU as bf16, the oracle upcast to fp64).
K/V belong to a *logical* token (sharing-tree node, offset), so a shared
prefix has one set of keys/values however many requests reuse it.
"""
from __future__ import annotations

import functools
from dataclasses import dataclass, field

import numpy as np
import torch

from .configs import Config

SEED = 1234
TAG_TOK, TAG_K, TAG_V, TAG_Q, TAG_DTOK, TAG_DQ, TAG_DK, TAG_DV = range(1, 9)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Node:
    id: int
    level: int
    parent: int          # -1 for level-0 nodes
    length: int
    children: list = field(default_factory=list)


@dataclass
class Request:
    rid: int             # unique over the workload
    phase: int           # index of the extend phase that admits it
    node: int            # its own (deepest) node
    path: tuple          # node ids from the top level down to `node`
    own_len: int         # tokens of its own node (its new tokens when the rest is cached)
    prompt_len: int
    decode_steps: int    # > 0 only for leaf requests


@dataclass
class Phase:
    index: int
    requests: list


class Workload:
    def __init__(self, cfg: Config):
        self.cfg = cfg
        self.nodes: list[Node] = []
        prev = [None]
        for lvl, (fan, length) in enumerate(cfg.levels):
            cur = []
            for p in prev:
                for _ in range(fan):
                    n = Node(len(self.nodes), lvl, -1 if p is None else p.id, length)
                    self.nodes.append(n)
                    if p is not None:
                        p.children.append(n.id)
                    cur.append(n)
            prev = cur
        self._tokens = self._draw_tokens()
        self.phases: list[Phase] = []
        rid = 0
        for lvl in range(cfg.n_levels):
            reqs = []
            leaf = lvl == cfg.n_levels - 1
            for n in self.nodes:
                if n.level != lvl:
                    continue
                path = self.path(n.id)
                reqs.append(Request(rid, lvl, n.id, path, n.length,
                                    sum(self.nodes[i].length for i in path),
                                    cfg.decode_steps if leaf else 0))
                rid += 1
            self.phases.append(Phase(lvl, reqs))

    # ---------------- structure ----------------
    def path(self, node_id: int) -> tuple:
        p = []
        while node_id >= 0:
            p.append(node_id)
            node_id = self.nodes[node_id].parent
        return tuple(reversed(p))

    @property
    def leaf_requests(self) -> list:
        return self.phases[-1].requests

    @property
    def all_requests(self) -> list:
        return [r for ph in self.phases for r in ph.requests]

    # ---------------- token ids ----------------
    def _rng(self, *ids) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence([SEED, self.cfg.index, *ids]))

    def _draw_tokens(self) -> list:
        toks = [None] * len(self.nodes)
        first_by_parent: dict = {}
        for n in self.nodes:
            rng = self._rng(TAG_TOK, n.id)
            t = rng.integers(0, self.cfg.vocab, size=n.length, dtype=np.int64).astype(np.int32)
            used = first_by_parent.setdefault(n.parent, set())
            if n.length > 0:
                while int(t[0]) in used:
                    t[0] = np.int32(rng.integers(0, self.cfg.vocab))
                used.add(int(t[0]))
            toks[n.id] = t
        return toks

    def node_tokens(self, node_id: int) -> np.ndarray:
        return self._tokens[node_id]

    def prompt_tokens(self, req: Request) -> np.ndarray:
        return np.concatenate([self._tokens[i] for i in req.path]).astype(np.int32)

    def decode_tokens(self, req: Request) -> np.ndarray:
        rng = self._rng(TAG_DTOK, req.rid)
        return rng.integers(0, self.cfg.vocab, size=req.decode_steps, dtype=np.int64).astype(np.int32)

    # ---------------- values ----------------
    def _normal_t(self, shape, *ids) -> torch.Tensor:
        """float32 torch tensor (bf16-representable for bf16 workloads)."""
        seed = int(np.random.SeedSequence([SEED, self.cfg.index, *ids]).generate_state(1, np.uint64)[0]) >> 1
        g = torch.Generator().manual_seed(seed)
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        x *= self.cfg.sigma
        if self.cfg.dtype == "bf16":
            x = x.to(torch.bfloat16).to(torch.float32)
        return x

    def _normal(self, shape, *ids) -> np.ndarray:
        return self._normal_t(shape, *ids).numpy()

    @functools.lru_cache(maxsize=256)
    def node_kv(self, node_id: int):
        """(K, V) of a node's logical tokens, float32 [len, Hkv, D]."""
        c = self.cfg
        shape = (self.nodes[node_id].length, c.n_kv_heads, c.head_dim)
        return self._normal(shape, TAG_K, node_id), self._normal(shape, TAG_V, node_id)

    def request_q(self, req: Request) -> np.ndarray:
        """Queries of the request's own tokens, float32 [own_len, Hq, D]."""
        c = self.cfg
        return self._normal((req.own_len, c.n_q_heads, c.head_dim), TAG_Q, req.rid)

    def decode_q(self, req: Request) -> np.ndarray:
        c = self.cfg
        return self._normal((req.decode_steps, c.n_q_heads, c.head_dim), TAG_DQ, req.rid)

    def decode_kv(self, req: Request):
        c = self.cfg
        shape = (req.decode_steps, c.n_kv_heads, c.head_dim)
        return self._normal(shape, TAG_DK, req.rid), self._normal(shape, TAG_DV, req.rid)

    # ---------------- bulk fill (for device upload) ----------------
    def _fill(self, dst: torch.Tensor, shape, *ids):
        """Draw one piece and copy it into `dst` (any dtype / device), through
        a reused host buffer so large workloads do not churn host memory."""
        n = int(np.prod(shape))
        buf = getattr(self, "_scratch", None)
        if buf is None or buf.numel() < n:
            buf = torch.empty(max(n, 1 << 20), dtype=torch.float32)
            self._scratch = buf
        seed = int(np.random.SeedSequence([SEED, self.cfg.index, *ids]).generate_state(1, np.uint64)[0]) >> 1
        x = buf[:n].view(shape)
        torch.randn(shape, generator=torch.Generator().manual_seed(seed), out=x)
        x *= self.cfg.sigma
        dst.copy_(x)          # to bf16: round to nearest even, as the oracle's copy

    def fill_phase(self, phase: Phase, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        """New-token arrays of an extend phase, request-major, written into
        q [sum own_len, Hq, D] and k, v [sum own_len, Hkv, D]."""
        c = self.cfg
        off = 0
        for r in phase.requests:
            n = r.own_len
            self._fill(q[off:off + n], (n, c.n_q_heads, c.head_dim), TAG_Q, r.rid)
            self._fill(k[off:off + n], (n, c.n_kv_heads, c.head_dim), TAG_K, r.node)
            self._fill(v[off:off + n], (n, c.n_kv_heads, c.head_dim), TAG_V, r.node)
            off += n

    def fill_decode(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        """Decode inputs of the leaf requests, step-major: q [T, R, Hq, D],
        k, v [T, R, Hkv, D]."""
        c = self.cfg
        T = c.decode_steps
        for j, r in enumerate(self.leaf_requests):
            self._fill(q[:, j], (T, c.n_q_heads, c.head_dim), TAG_DQ, r.rid)
            self._fill(k[:, j], (T, c.n_kv_heads, c.head_dim), TAG_DK, r.rid)
            self._fill(v[:, j], (T, c.n_kv_heads, c.head_dim), TAG_DV, r.rid)

    def decode_token_matrix(self) -> np.ndarray:
        """Decode token ids of the leaf requests, [R, T]."""
        return np.stack([self.decode_tokens(r) for r in self.leaf_requests]) if self.leaf_requests else \
            np.zeros((0, self.cfg.decode_steps), np.int32)

    def request_full_kv(self, req: Request, n_decode: int | None = None):
        """Logical K/V of the request's whole sequence: its path nodes, then
        its first `n_decode` decode tokens (all by default)."""
        ks, vs = [], []
        for i in req.path:
            k, v = self.node_kv(i)
            ks.append(k)
            vs.append(v)
        nd = req.decode_steps if n_decode is None else n_decode
        if nd:
            dk, dv = self.decode_kv(req)
            ks.append(dk[:nd])
            vs.append(dv[:nd])
        return np.concatenate(ks), np.concatenate(vs)
