"""Token-level trie model of the radix KV cache (oracle; test infrastructure).

Passages followed:
  * SGLang explainer, RadixAttention section: the cache is a radix tree over
    token ids whose value is the KV pages of those tokens; one page holds one
    token; prefix matching walks from the root and reuses the longest match;
    after a request completes its KV is inserted, splitting a node on partial
    overlap; when memory runs short the least recently accessed leaves with a
    reference count of zero are evicted, recursively.
  * SGLang paper notes, section 3 and Figure 3: reference counts protect
    nodes in use; the KV pool is shared with running requests (no separate
    cache pool); nodes split when a new request shares part of an edge.
  * vLLM-vs-SGLang page, worked example and matching-unit section: the
    reusable length is the match counted from the first token, rounded down
    to the matching unit.
  * vLLM-vs-SGLang page, eviction passage: besides the default LRU, SGLang
    offers LFU, SLRU and priority eviction (named only).

This model keeps ONE TRIE NODE PER TOKEN (deliberately not the edge-
compressed layout of the product's tree).  A radix node ("segment") is a
maximal chain of token nodes carrying the same segment id; its attributes
(id, last access, reference count) live in a side table.

Readings of points the pages leave open (the product's tree follows the same):
  * split on match: a match that ends inside a segment splits it there, so
    the returned node ends exactly at the matched length;
  * the logical clock ticks once per match/insert call; every segment on the
    walked path (a new upper split part included) gets the current tick; the
    lower part of a split keeps its old stamp and its id; the new upper part
    takes the next id and the split segment's reference count;
  * eviction victim: smallest (last access, node id) among segments with
    reference count 0 and no children; whole segments are evicted; evicting
    may free more than asked; parents left childless become candidates;
  * allocation returns the n smallest free slot ids in ascending order and
    evicts only the shortfall; if free + evictable < n nothing changes
    (evictable: tokens of segments with no referenced segment at or below);
  * insert keeps the tree's slots for the part already present and reports
    its length; the caller frees its own duplicates;
  * lock/unlock add/subtract 1 on every segment from the node to the root;
    an underflow is a state error and changes nothing;
  * match unit u > 1 truncates the match to a multiple of u before splitting.
  * eviction policies (the pages name them; these are their textbook forms
    on the same leaves): every match/insert call that stamps a segment also
    counts one access to it and raises its priority to the call's priority
    (set_priority; 0 by default); a new segment starts with one access and
    the call's priority; a split's upper part copies both.  Victim key, the
    smallest first: LRU (last access, id); LFU (accesses, last access, id);
    SLRU (protected = accessed by two or more calls, last access, id) -- the
    probationary segment is evicted before the protected one; priority
    (priority, last access, id).
"""
from __future__ import annotations

import heapq

EINVAL, ENOSPC, ESTATE = -1, -2, -3
POLICIES = ("lru", "lfu", "slru", "priority")
_FREE, _TREE, _PRIVATE = 0, 1, 2


class CacheError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class _Tok:
    __slots__ = ("tok", "slot", "seg", "parent", "children")

    def __init__(self, tok, slot, seg, parent):
        self.tok = tok
        self.slot = slot
        self.seg = seg
        self.parent = parent
        self.children = {}


class _Seg:
    __slots__ = ("id", "last", "ref", "top", "hits", "prio")

    def __init__(self, sid, last, ref, top, hits=1, prio=0):
        self.id = sid
        self.last = last
        self.ref = ref
        self.top = top
        self.hits = hits
        self.prio = prio


class TokenTrieCache:
    def __init__(self, num_slots: int, match_unit: int = 1, policy: str = "lru"):
        if num_slots <= 0 or match_unit < 1 or policy not in POLICIES:
            raise CacheError(EINVAL, "num_slots > 0, match_unit >= 1 and a known policy required")
        self.num_slots = num_slots
        self.unit = match_unit
        self.policy = policy
        self.priority = 0
        self.root = _Tok(None, -1, 0, None)
        self.segs: dict[int, _Seg] = {}
        self.next_id = 1
        self.clock = 0
        self.evictions = 0
        self.free_heap = list(range(num_slots))
        self.state = [_FREE] * num_slots

    # ------------------------------------------------------------ helpers
    def _walk(self, tokens):
        cur, out = self.root, []
        for t in tokens:
            nxt = cur.children.get(int(t))
            if nxt is None:
                break
            out.append(nxt)
            cur = nxt
        return out

    @staticmethod
    def _next_in_seg(tn):
        for c in tn.children.values():
            if c.seg == tn.seg:
                return c
        return None

    def _chain(self, seg: _Seg):
        out, tn = [], seg.top
        while tn is not None:
            out.append(tn)
            tn = self._next_in_seg(tn)
        return out

    def _parent_seg(self, seg: _Seg):
        p = seg.top.parent
        return None if p is self.root else self.segs[p.seg]

    def _is_leaf(self, seg: _Seg) -> bool:
        return not self._chain(seg)[-1].children

    def _split_after(self, tn):
        """Make `tn` the last token of its segment; returns its segment id."""
        x = self.segs[tn.seg]
        below = self._next_in_seg(tn)
        if below is None:
            return x.id
        y = _Seg(self.next_id, x.last, x.ref, x.top, x.hits, x.prio)
        self.next_id += 1
        n = x.top
        while True:
            nxt = self._next_in_seg(n)
            n.seg = y.id
            if n is tn:
                break
            n = nxt
        x.top = below
        self.segs[y.id] = y
        return y.id

    def _stamp(self, tnodes):
        for sid in {tn.seg for tn in tnodes}:
            sg = self.segs[sid]
            sg.last = self.clock
            sg.hits += 1
            sg.prio = max(sg.prio, self.priority)

    def _victim_key(self, s):
        if self.policy == "lfu":
            return (s.hits, s.last, s.id)
        if self.policy == "slru":
            return (1 if s.hits >= 2 else 0, s.last, s.id)
        if self.policy == "priority":
            return (s.prio, s.last, s.id)
        return (s.last, s.id)

    def _path(self, node_id: int):
        if node_id == 0:
            return []
        if node_id not in self.segs:
            raise CacheError(ESTATE, f"node {node_id} is not in the tree")
        out, s = [], self.segs[node_id]
        while s is not None:
            out.append(s)
            s = self._parent_seg(s)
        return out

    def _check_private(self, slots):
        seen = set()
        for s in slots:
            s = int(s)
            if not 0 <= s < self.num_slots:
                raise CacheError(EINVAL, f"slot {s} out of range")
            if self.state[s] != _PRIVATE or s in seen:
                raise CacheError(ESTATE, f"slot {s} is not a private allocated slot")
            seen.add(s)

    def _evict_one(self) -> int:
        leaves = [s for s in self.segs.values() if s.ref == 0 and self._is_leaf(s)]
        if not leaves:
            return 0
        victim = min(leaves, key=self._victim_key)
        chain = self._chain(victim)
        del victim.top.parent.children[victim.top.tok]
        for tn in chain:
            self.state[tn.slot] = _FREE
            heapq.heappush(self.free_heap, tn.slot)
        del self.segs[victim.id]
        self.evictions += 1
        return len(chain)

    # ------------------------------------------------------------ API
    def match_prefix(self, tokens):
        """-> (matched length rounded to the unit, slots of those tokens, node id)."""
        self.clock += 1
        nodes = self._walk(tokens)
        mu = (len(nodes) // self.unit) * self.unit
        if mu == 0:
            return 0, [], 0
        node = self._split_after(nodes[mu - 1])
        self._stamp(nodes[:mu])
        return mu, [tn.slot for tn in nodes[:mu]], node

    def insert(self, tokens, slots):
        """-> (length already present, node id of the end of the sequence)."""
        tokens = [int(t) for t in tokens]
        slots = [int(s) for s in slots]
        if len(tokens) != len(slots):
            raise CacheError(EINVAL, "tokens and slots differ in length")
        nodes = self._walk(tokens)
        k, n = len(nodes), len(tokens)
        self._check_private(slots[k:])
        self.clock += 1
        if k > 0:
            self._split_after(nodes[k - 1])
        if k == n:
            self._stamp(nodes)
            return k, (nodes[-1].seg if n else 0)
        z = _Seg(self.next_id, self.clock, 0, None, 1, self.priority)
        self.next_id += 1
        self.segs[z.id] = z
        cur = nodes[-1] if k else self.root
        for t, s in zip(tokens[k:], slots[k:]):
            tn = _Tok(t, s, z.id, cur)
            cur.children[t] = tn
            if z.top is None:
                z.top = tn
            self.state[s] = _TREE
            cur = tn
        self._stamp(nodes)
        return k, z.id

    def set_priority(self, priority: int):
        """Priority carried by the following match/insert calls."""
        self.priority = int(priority)

    def lock(self, node_id: int):
        for s in self._path(node_id):
            s.ref += 1

    def unlock(self, node_id: int):
        path = self._path(node_id)
        if any(s.ref < 1 for s in path):
            raise CacheError(ESTATE, "reference count underflow")
        for s in path:
            s.ref -= 1

    def evictable_tokens(self) -> int:
        """Tokens of segments with no referenced segment at or below them
        (only those can ever become unreferenced leaves)."""
        pinned = set()
        for s in self.segs.values():
            if s.ref > 0:
                p = s
                while p is not None and p.id not in pinned:
                    pinned.add(p.id)
                    p = self._parent_seg(p)
        return sum(len(self._chain(s)) for s in self.segs.values() if s.id not in pinned)

    def alloc(self, n: int):
        if n < 0:
            raise CacheError(EINVAL, "negative allocation")
        short = n - len(self.free_heap)
        if short > 0 and self.evictable_tokens() < short:
            raise CacheError(ENOSPC, f"need {n}, free {len(self.free_heap)}")
        while len(self.free_heap) < n:
            self._evict_one()
        out = [heapq.heappop(self.free_heap) for _ in range(n)]
        for s in out:
            self.state[s] = _PRIVATE
        return out

    def free(self, slots):
        self._check_private(slots)
        for s in slots:
            s = int(s)
            self.state[s] = _FREE
            heapq.heappush(self.free_heap, s)

    def evict(self, n_tokens: int) -> int:
        freed = 0
        while freed < n_tokens:
            f = self._evict_one()
            if f == 0:
                break
            freed += f
        return freed

    def stats(self) -> dict:
        cached = sum(1 for s in self.state if s == _TREE)
        return dict(
            num_slots=self.num_slots,
            free=len(self.free_heap),
            cached=cached,
            evictable=self.evictable_tokens(),
            private=sum(1 for s in self.state if s == _PRIVATE),
            nodes=len(self.segs),
            evictions=self.evictions,
            clock=self.clock,
        )

    # ------------------------------------------------------------ introspection (tests)
    def resident_sequences(self):
        """Every root-to-leaf token sequence currently in the trie."""
        out, stack = [], [(self.root, [])]
        while stack:
            tn, pre = stack.pop()
            if not tn.children and tn is not self.root:
                out.append(pre)
            for t, c in tn.children.items():
                stack.append((c, pre + [t]))
        return out

    def node_info(self, node_id: int) -> dict:
        s = self.segs[node_id]
        chain = self._chain(s)
        depth, p = 0, s.top.parent
        while p is not self.root:
            depth += 1
            p = p.parent
        return dict(id=s.id, last=s.last, ref=s.ref, start=depth, length=len(chain),
                    slots=[tn.slot for tn in chain], leaf=not chain[-1].children, hits=s.hits, prio=s.prio)

    def evictable_leaves(self):
        return [s.id for s in self.segs.values() if s.ref == 0 and self._is_leaf(s)]

    def slot_partition(self):
        free = {i for i, s in enumerate(self.state) if s == _FREE}
        tree = {i for i, s in enumerate(self.state) if s == _TREE}
        priv = {i for i, s in enumerate(self.state) if s == _PRIVATE}
        return free, tree, priv
