"""Host-side properties of the batch planner (no GPU needed).

For every new token and KV head, the key positions assigned to it over all
work items and jobs must be exactly {0, ..., its position}, each once;
shared segments must be read once per tile instead of once per request;
tiles, contributions and workspace offsets must be consistent."""
import numpy as np
import pytest

from prefix_shared_kv_token_amd import rdx
from workloads import Workload, config_by_name


def _admit_phases(cfg, kind_last="extend"):
    """Runs the admission protocol of every phase on the C++ tree and returns
    the plan inputs of the last extend phase and of one decode step."""
    wl = Workload(cfg)
    tree = rdx.Tree(cfg.total_tokens())
    out = []
    for pi, ph in enumerate(wl.phases):
        reqs = []
        for r in ph.requests:
            p = wl.prompt_tokens(r)
            m, slots, node = tree.match_prefix(p)
            tree.lock(node)
            new = tree.alloc(len(p) - m).copy()
            reqs.append((p, m, node, np.concatenate([slots, new])))
        out.append(reqs)
        if pi < len(wl.phases) - 1:
            for p, m, node, row in reqs:
                k, _ = tree.insert(p, row)
                tree.free(row[m:k])
                tree.unlock(node)
    return wl, tree, out


def _check_coverage(plan, kv_len, q_len, rows, hkv):
    v = plan.view()
    group = v["group"]
    items, tiles, jobs, toks, contribs = v["items"], v["tiles"], v["jobs"], v["tokens"], v["contribs"]
    row_of_req = {r: i for i, r in enumerate(rows)}
    # which request owns a q index, and its position
    q_off = np.concatenate([[0], np.cumsum(q_len)])
    n_tok = int(q_off[-1])
    cover = {}
    seen_tok = np.zeros(n_tok, int)
    for t in tiles:
        assert 0 < t[1] * group <= v["tile_rows"]
        for j in range(t[0], t[0] + t[1]):
            seen_tok[toks[j, 0]] += 1
    assert (seen_tok == 1).all()
    for it, kvh in ((it, h) for it in items for h in range(hkv)):
        tile = tiles[it[0]]
        if tile[2] > 1:
            c = contribs[tile[3] + it[3]]
        for jb in range(it[1], it[2]):
            j = jobs[jb]
            for tl in range(j[3], j[4]):
                qi, pos = toks[tile[0] + tl]
                if tile[2] > 1:
                    assert c[0] <= tl < c[1]
                r = int(np.searchsorted(q_off, qi, side="right") - 1)
                end = min(j[2], pos + 1) if j[5] else j[2]
                for p in range(j[1], end):
                    key = (qi, kvh, p)
                    cover[key] = cover.get(key, 0) + 1
                # the job reads the row of a request that shares these positions
                assert j[0] in row_of_req
    per_row = {}
    for (a, b, p), c in cover.items():
        per_row.setdefault((a, b), []).extend([p] * c)
    for qi in range(n_tok):
        r = int(np.searchsorted(q_off, qi, side="right") - 1)
        pos = kv_len[r] - q_len[r] + (qi - q_off[r])
        for h in range(hkv):
            got = sorted(per_row.get((qi, h), []))
            assert got == list(range(pos + 1)), (qi, h)
    return v


@pytest.mark.parametrize("name,levels,decode", [
    ("batchllm", ((3, 40), (5, 13)), 3),
    ("helpdesk", ((1, 70), (9, 7)), 2),
    ("multilevel", ((1, 20), (3, 9), (2, 5)), 2),
    ("tiny", ((1, 0 + 8), (3, 1)), 1),
])
@pytest.mark.parametrize("target", [0, 1, 4096])
def test_extend_and_decode_plans_cover_each_visible_key_once(name, levels, decode, target):
    cfg = config_by_name(name).replace(levels=levels, decode_steps=decode, n_q_heads=8, n_kv_heads=2)
    wl, tree, phases = _admit_phases(cfg)
    reqs = phases[-1]
    desc = rdx.attn_desc(rdx.BF16, 8, 2, 128, cfg.total_tokens())
    ld = cfg.max_seq_len
    rows = list(range(len(reqs)))
    # extend of the last phase
    plan = rdx.Plan(desc, rdx.PLAN_EXTEND, target)
    kv_len = [len(p) for p, *_ in reqs]
    q_len = [len(p) - m for p, m, *_ in reqs]
    new = np.concatenate([row[m:] for p, m, n, row in reqs])
    plan.build(tree, [n for _, _, n, _ in reqs], rows, kv_len, q_len, [0] * len(reqs), new, ld)
    _check_coverage(plan, kv_len, q_len, rows, 2)
    info = plan.info()
    assert info["num_new"] == sum(q_len)
    # one decode step
    dplan = rdx.Plan(desc, rdx.PLAN_DECODE, target)
    slots = tree.alloc(len(reqs))
    kv1 = [k + 1 for k in kv_len]
    dplan.build(tree, [n for _, _, n, _ in reqs], rows, kv1, [1] * len(reqs), kv_len, slots, ld)
    v = _check_coverage(dplan, kv1, [1] * len(reqs), rows, 2)
    # a shared prefix is attended once per decode tile, not once per request
    n_shared = dplan.info()["num_shared_segments"]
    assert n_shared >= 1
    shared_jobs = [j for j in v["jobs"] if j[5] == 0]
    shared_keys = sum(j[2] - j[1] for j in shared_jobs)
    prefix = sum(length for _, length in levels[:-1])
    assert shared_keys <= prefix * len(v["tiles"]) * (len(levels) - 1)
    if target == 4096 and sum(j[2] - j[1] for j in v["jobs"]) > 64 * len(v["tiles"]):
        assert dplan.info()["num_split_tiles"] > 0 and dplan.info()["workspace_bytes"] > 0


def test_single_request_groups_degrade_to_own_ranges():
    """A prefix node reached by one request of the batch is not shared."""
    cfg = config_by_name("batchllm").replace(levels=((4, 30), (1, 10)), decode_steps=1, n_q_heads=8, n_kv_heads=2)
    wl, tree, phases = _admit_phases(cfg)
    reqs = phases[-1]
    desc = rdx.attn_desc(rdx.BF16, 8, 2, 128, cfg.total_tokens())
    plan = rdx.Plan(desc, rdx.PLAN_EXTEND)
    kv_len = [len(p) for p, *_ in reqs]
    q_len = [len(p) - m for p, m, *_ in reqs]
    new = np.concatenate([row[m:] for p, m, n, row in reqs])
    plan.build(tree, [n for _, _, n, _ in reqs], list(range(len(reqs))), kv_len, q_len, [0] * len(reqs), new, 64)
    assert plan.info()["num_shared_segments"] == 0
    _check_coverage(plan, kv_len, q_len, list(range(len(reqs))), 2)


def test_empty_batch_and_zero_query_requests():
    desc = rdx.attn_desc(rdx.BF16, 4, 4, 64, 16)
    tree = rdx.Tree(16)
    plan = rdx.Plan(desc, rdx.PLAN_DECODE)
    plan.build(tree, [], [], [], [], [], [], 8)
    assert plan.info()["num_items"] == 0
    s = tree.alloc(3)
    plan.build(tree, [0, 0], [0, 1], [3, 0], [3, 0], [0, 0], s, 8)
    assert plan.info()["num_new"] == 3 and plan.info()["num_tiles"] == 1


def test_decode_items_are_sized_in_blocks():
    """Work items are cut in 64-key blocks, not keys: items made of many short
    own-suffix jobs carry no more blocks than items cut from a long shared
    prefix (the longest item sets the launch's end), and cuts fall on block
    boundaries (no block is split between items)."""
    cfg = config_by_name("helpdesk").replace(levels=((1, 1000), (64, 40)), decode_steps=1, n_q_heads=8,
                                             n_kv_heads=2)
    wl, tree, phases = _admit_phases(cfg)
    reqs = phases[-1]
    desc = rdx.attn_desc(rdx.BF16, 8, 2, 128, cfg.total_tokens())
    rows = list(range(len(reqs)))
    kv = [len(p) + 101 for p, *_ in reqs]  # decode step 100: 141 own keys (3 blocks) per request
    target = 32  # 16 records per KV head
    plan = rdx.Plan(desc, rdx.PLAN_DECODE, target)
    plan.build(tree, [n for _, _, n, _ in reqs], rows, kv, [1] * len(reqs), [k - 1 for k in kv],
               tree.alloc(len(reqs)), cfg.max_seq_len + 128)
    v = plan.view()
    job_blocks = [(j[2] - j[1] + 63) // 64 for j in v["jobs"]]
    total = sum(job_blocks)
    # the 1000 shared keys once per decode tile (16 tokens x 4 grouped heads) + 3 blocks per own suffix
    assert len(v["tiles"]) == 4 and total == 4 * 16 + 64 * 3
    per_item = [sum(job_blocks[it[1]:it[2]]) for it in v["items"]]
    assert [int(it[4]) for it in v["items"]] == per_item
    assert max(per_item) <= -(-total // (target // 2))
    assert sum(per_item) == total


def test_split_stays_within_the_item_target():
    """Five small sharing groups and one long one (decode, 2 KV heads, a
    target of 32 items: 16 per head).  Cutting every tile by the same block
    count would round up per tile (5 x 1 + 15 = 20 items per head) and start
    a second round for a few workgroups; the planner hands the 16 items out
    one by one to the tile with the longest pieces, so the count is exact
    and the long tile's pieces are even.  Coverage stays exact."""
    hkv = 2
    prefixes = [np.arange(64, dtype=np.int32) + 1000 * (g + 1) for g in range(5)]
    prefixes.append(np.arange(64 * 200, dtype=np.int32) + 100_000)
    tree = rdx.Tree(64 * 300)
    for p in prefixes:
        m, slots, node = tree.match_prefix(p)
        row = np.concatenate([slots, tree.alloc(len(p) - m)])
        tree.insert(p, row)
    reqs = []
    for g, p in enumerate(prefixes):
        for i in range(2):
            prompt = np.concatenate([p, [7 + i + 10 * g]]).astype(np.int32)
            m, slots, node = tree.match_prefix(prompt)
            tree.lock(node)
            reqs.append((prompt, m, node, np.concatenate([slots, tree.alloc(len(prompt) - m)])))
    desc = rdx.attn_desc(rdx.BF16, hkv, hkv, 128, 64 * 300)
    rows = list(range(len(reqs)))
    kv1 = [len(p) + 1 for p, *_ in reqs]
    plan = rdx.Plan(desc, rdx.PLAN_DECODE, 32)
    plan.build(tree, [n for _, _, n, _ in reqs], rows, kv1, [1] * len(reqs), [len(p) for p, *_ in reqs],
               tree.alloc(len(reqs)), 64 * 201 + 2)
    info = plan.info()
    assert info["num_tiles"] == 6 and info["num_split_tiles"] >= 1
    assert info["num_items"] == 32, info["num_items"]   # 16 per head: 5 small tiles whole + 11 pieces
    v = _check_coverage(plan, kv1, [1] * len(reqs), rows, hkv)
    # the long tile's 11 pieces are of nearly equal length (202 blocks: 18 or 19 each)
    big = [int(it[4]) for it in v["items"] if v["tiles"][it[0]][2] > 1]
    assert len(big) == 11 and sum(big) == 202 and max(big) - min(big) <= 1, big


def test_partial_last_round_is_cut_into_pieces():
    """Extend with 5 tiles per KV head on a target of 4 items per head: one
    full round, then 1 tile that would leave three quarters of the second
    round idle for a whole tile.  That last tile is cut into quarters (4
    pieces fill the round), the others stay whole; coverage stays exact."""
    cfg = config_by_name("helpdesk").replace(levels=((1, 512), (4, 80)), decode_steps=1, n_q_heads=8, n_kv_heads=2)
    wl, tree, phases = _admit_phases(cfg)
    reqs = phases[-1]
    desc = rdx.attn_desc(rdx.BF16, 8, 2, 128, cfg.total_tokens())
    plan = rdx.Plan(desc, rdx.PLAN_EXTEND, 8)
    kv_len = [len(p) for p, *_ in reqs]
    q_len = [len(p) - m for p, m, *_ in reqs]
    rows = list(range(len(reqs)))
    new = np.concatenate([row[m:] for p, m, n, row in reqs])
    plan.build(tree, [n for _, _, n, _ in reqs], rows, kv_len, q_len, [0] * len(reqs), new, cfg.max_seq_len)
    info = plan.info()
    assert sum(q_len) * 4 == 1280 and info["num_tiles"] == 5
    assert info["num_items"] == 2 * (4 + 4)
    assert info["num_split_tiles"] == 1
    v = _check_coverage(plan, kv_len, q_len, rows, 2)
    assert [int(t[2]) for t in v["tiles"]] == [1, 1, 1, 1, 4]
    # halves do not pay: 5 tiles on 3 slots per head (2 left over) stay whole
    plan2 = rdx.Plan(desc, rdx.PLAN_EXTEND, 6)
    plan2.build(tree, [n for _, _, n, _ in reqs], rows, kv_len, q_len, [0] * len(reqs), new, cfg.max_seq_len)
    assert plan2.info()["num_items"] == 2 * 5 and plan2.info()["num_split_tiles"] == 0


@pytest.mark.parametrize("name,items", [("helpdesk", 512), ("longprefix", 256), ("multilevel", 512),
                                        ("batchllm", 512)])
def test_default_decode_launch_size(name, items):
    """Default decode split of the four workloads' first decode step: whole
    workgroups per CU on MI355X's 256 CUs -- two per CU when items are short
    (Helpdesk: 16 items of 9 blocks per head; Multi-level), one per CU when
    each item still gets 32+ blocks (Long-prefix: 32 items of ~41 blocks per
    head); BatchLLM's 64 tiles x 8 heads need no split."""
    cfg = config_by_name(name)
    wl, tree, phases = _admit_phases(cfg)
    reqs = phases[-1]
    desc = rdx.attn_desc(rdx.BF16, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.total_tokens())
    plan = rdx.Plan(desc, rdx.PLAN_DECODE)
    kv1 = [len(p) + 1 for p, *_ in reqs]
    plan.build(tree, [n for _, _, n, _ in reqs], list(range(len(reqs))), kv1, [1] * len(reqs),
               [len(p) for p, *_ in reqs], tree.alloc(len(reqs)), cfg.max_seq_len)
    info = plan.info()
    assert info["num_items"] == items
    if name != "batchllm":
        blocks = [int(it[4]) for it in plan.view()["items"]]
        assert max(blocks) - min(blocks) <= 1 or info["num_tiles"] > 1


def test_multilevel_decode_tiles():
    """Multi-level tree (root 1,024 -> 8 branches of 512 -> 3 forks of 128;
    GQA 32/8), first decode step: 24 leaves x 4 grouped heads = 96 rows in
    64-row decode tiles.  Tiles are cut on branch boundaries: branches 0-4
    (15 leaves, 60 rows), then 5-7 (9 leaves, 36 rows), so every branch is a
    job of exactly one tile and only the root, whose 96 rows cannot share one
    tile, is read by both: 1,024 x 2 + 512 x 8 = 6,144 shared key reads per
    KV head for 5,120 distinct shared keys.  Both tiles' items for a KV head
    run on the same XCD, and the counters show the root's second read is
    served from its L2 (tiles of up to 128 rows, measured, read no fewer HBM
    bytes and ran slower)."""
    cfg = config_by_name("multilevel")
    wl, tree, phases = _admit_phases(cfg)
    reqs = phases[-1]
    desc = rdx.attn_desc(rdx.BF16, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.total_tokens())
    plan = rdx.Plan(desc, rdx.PLAN_DECODE, 8)     # one item per tile and KV head: jobs unsplit
    kv1 = [len(p) + 1 for p, *_ in reqs]
    rows = list(range(len(reqs)))
    plan.build(tree, [n for _, _, n, _ in reqs], rows, kv1, [1] * len(reqs), [len(p) for p, *_ in reqs],
               tree.alloc(len(reqs)), cfg.max_seq_len)
    v = _check_coverage(plan, kv1, [1] * len(reqs), rows, cfg.n_kv_heads)
    assert [int(t[1]) * 4 for t in v["tiles"]] == [60, 36]
    shared = sum(int(j[2] - j[1]) for j in v["jobs"] if j[5] == 0)
    own = sum(int(j[2] - j[1]) for j in v["jobs"] if j[5] == 1)
    assert shared == 1024 * 2 + 512 * 8
    assert own == 24 * (128 + 1)
    # each shared segment's tiles: the root in both, each branch in one
    tiles_of = {}
    for it in v["items"]:
        for jx in range(int(it[1]), int(it[2])):
            j = v["jobs"][jx]
            if j[5] == 0:
                tiles_of.setdefault((int(j[1]), int(j[2]), int(j[0]) if j[1] > 0 else -1), set()).add(int(it[0]))
    root = [t for (k0, k1, _), t in tiles_of.items() if (k0, k1) == (0, 1024)]
    branches = [t for (k0, k1, _), t in tiles_of.items() if (k0, k1) == (1024, 1536)]
    assert root == [{0, 1}]
    assert len(branches) == 8 and all(len(t) == 1 for t in branches)


def test_decode_tiles_cut_on_branch_boundaries():
    """Random two-level groups (a root shared by every request of the group,
    branches shared by runs of them): a branch whose requests fit in one
    decode tile is a job of one tile only, and a tile ends before it is full
    only where the next branch's requests would not fit in it."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        nb = int(rng.integers(2, 9))
        sizes = [int(x) for x in rng.integers(1, 22, nb)]
        root = [int(x) for x in rng.integers(1, 30000, 100)]
        tree = rdx.Tree(200000)
        prompts = []
        for b, n in enumerate(sizes):
            br = [30001 + b] + [int(x) for x in rng.integers(1, 30000, 40)]
            for i in range(n):
                prompts.append(root + br + [31000 + 100 * b + i] + [int(x) for x in rng.integers(1, 30000, 5)])
        nodes = []
        for p in prompts:
            m, slots, node = tree.match_prefix(p)
            new = tree.alloc(len(p) - m)
            node = tree.insert(p, np.concatenate([slots, new]).astype(np.int32))
            nodes.append(node)
        reqs = []
        for p in prompts:
            m, slots, node = tree.match_prefix(p)
            assert m == len(p)
            tree.lock(node)
            reqs.append((p, node))
        hq, hkv = 8, 2   # 4 rows per request: 16 requests per 64-row decode tile
        desc = rdx.attn_desc(rdx.BF16, hq, hkv, 128, 200000)
        plan = rdx.Plan(desc, rdx.PLAN_DECODE, 8)
        kv1 = [len(p) + 1 for p, _ in reqs]
        rows = list(range(len(reqs)))
        plan.build(tree, [n for _, n in reqs], rows, kv1, [1] * len(reqs), [len(p) for p, _ in reqs],
                   tree.alloc(len(reqs)), 256)
        v = _check_coverage(plan, kv1, [1] * len(reqs), rows, hkv)
        tiles_of = {}
        for it in v["items"]:
            for jx in range(int(it[1]), int(it[2])):
                j = v["jobs"][jx]
                if j[5] == 0 and int(j[1]) == 100:   # a branch segment: keys 100 .. 141
                    tiles_of.setdefault(int(j[0]), set()).add(int(it[0]))
        # a branch's job reads the page-table row of its first request
        first_row = {int(sum(sizes[:b])): b for b in range(nb) if sizes[b] >= 2}
        assert set(tiles_of) == set(first_row), (sizes, tiles_of)
        for row, b in first_row.items():
            if sizes[b] <= 16:
                assert len(tiles_of[row]) == 1, (sizes, b, tiles_of[row])
            else:   # larger than a tile: consecutive tiles, no more than needed plus one
                t = sorted(tiles_of[row])
                assert t == list(range(t[0], t[-1] + 1)) and len(t) <= -(-sizes[b] // 16) + 1, (sizes, b, t)
        branch_of = [b for b, n in enumerate(sizes) for _ in range(n)]
        toks = v["tokens"]
        tiles = v["tiles"]
        for t in range(len(tiles) - 1):
            n_tok = int(tiles[t][1])
            if n_tok == 16:
                continue
            nxt = [branch_of[int(toks[int(tiles[t + 1][0]) + i][0])] for i in range(int(tiles[t + 1][1]))]
            first = sum(1 for b in nxt if b == nxt[0])
            assert n_tok + first > 16, (sizes, t, n_tok, first)


@pytest.mark.parametrize("group", [1, 4])
def test_causal_jobs_end_at_the_tiles_last_query(group):
    """A causal prefill (every prompt token new, no cached prefix): a tile's own
    job reads keys only up to its last query position (the coverage check
    fixes that it reads all of them), so a tile iterates no key block that
    is masked for every one of its rows."""
    cfg = config_by_name("batchllm").replace(levels=((3, 700),), decode_steps=1, n_q_heads=8,
                                             n_kv_heads=8 // group)
    wl = Workload(cfg)
    tree = rdx.Tree(cfg.total_tokens())
    reqs = []
    for r in wl.phases[0].requests:
        p = wl.prompt_tokens(r)
        m, slots, node = tree.match_prefix(p)
        assert m == 0
        tree.lock(node)
        reqs.append((p, m, node, tree.alloc(len(p)).copy()))
    hkv = 8 // group
    desc = rdx.attn_desc(rdx.BF16, 8, hkv, 128, cfg.total_tokens())
    plan = rdx.Plan(desc, rdx.PLAN_EXTEND)
    kv_len = [len(p) for p, *_ in reqs]
    new = np.concatenate([row for *_, row in reqs])
    rows = list(range(len(reqs)))
    plan.build(tree, [n for _, _, n, _ in reqs], rows, kv_len, kv_len, [0] * len(reqs), new, cfg.max_seq_len)
    v = _check_coverage(plan, kv_len, kv_len, rows, hkv)
    tiles, jobs, toks = v["tiles"], v["jobs"], v["tokens"]
    n_items_jobs = 0
    for it in v["items"]:
        tile = tiles[it[0]]
        pmax = max(int(toks[tile[0] + t, 1]) for t in range(tile[1]))
        for jb in range(it[1], it[2]):
            j = jobs[jb]
            n_items_jobs += 1
            assert j[5] == 1                   # all keys are the request's own: causal
            assert j[2] <= pmax + 1            # ends at the tile's last query
    assert n_items_jobs > 0
