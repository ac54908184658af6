"""End-to-end serving on the GPU under cache pressure: a seeded waiting
queue (three system prompts of different popularity followed by fresh
suffixes, and one-off prompts) arrives in windows of 4; each window is
ordered by rdx_schedule against the tree as it stands (longest shared prefix
first), then served in batches of 2 through the device path -- admission
(match, lock, allocate, evicting when short), extend, 4 decode steps,
finish (insert, free duplicates, unlock) -- on a pool far smaller than the
queue's tokens, once per eviction policy (LRU, LFU, SLRU, priority), and
once with LRU and prefix matching in 16-token units.

The same calls run on the oracle's cache model with the oracle's ordering
(oracle.schedule.lpm_order) and the same policy: the window orders, every
matched length and every page-table row must be equal bit for bit, and
every extend and decode output must be within 2e-2 of the fp64 oracle's
attention over the request's logical sequence (SGLang paper notes, section
3 cache-aware scheduling and appendix A.2; vLLM-vs-SGLang page, eviction
passage)."""
import numpy as np
import pytest

from oracle import TokenTrieCache, causal_attention
from oracle.schedule import lpm_order
from workloads.gen import bf16_bits_to_f32, bf16_round_bits
from workloads.queue import segment_values, served_queue

pytestmark = pytest.mark.gpu

HQ, HKV, D, T, SIGMA = 8, 2, 128, 4, 0.5
POOL, WINDOW, BATCH = 800, 4, 2
QUEUE = dict(seed=1, popularity=(6, 3, 2), one_offs=8, decode_steps=T)


def _bf16(x):
    return bf16_bits_to_f32(bf16_round_bits(x))


def _request_arrays(segs, gen_seg, n_prompt):
    """Logical K, V [n+T, Hkv, D] and Q [n+T, Hq, D] (bf16-rounded float32)."""
    parts = list(segs) + [(gen_seg, T)]
    k = np.concatenate([_bf16(segment_values(s, n, HKV, D, SIGMA, 0)) for s, n in parts])
    v = np.concatenate([_bf16(segment_values(s, n, HKV, D, SIGMA, 1)) for s, n in parts])
    q = _bf16(segment_values(segs[-1][0], n_prompt + T, HQ, D, SIGMA, 2))
    return q, k, v


def _oracle_batch(cache, prompts, gens, batch, prio):
    cache.set_priority(prio)
    adm = []
    for i in batch:
        m, slots, node = cache.match_prefix(prompts[i])
        cache.lock(node)
        adm.append([i, m, node, list(slots) + cache.alloc(len(prompts[i]) - m)])
    for _ in range(T):
        for a, s in zip(adm, cache.alloc(len(adm))):
            a[3].append(s)
    for i, m, node, row in adm:
        k, _ = cache.insert(np.concatenate([prompts[i], gens[i][1]]), row)
        cache.free(row[m:k])
        cache.unlock(node)
    return {i: (m, np.asarray(row, np.int32)) for i, m, _, row in adm}


@pytest.mark.parametrize("policy,unit", [("lru", 1), ("lfu", 1), ("slru", 1), ("priority", 1), ("lru", 16)],
                         ids=["lru", "lfu", "slru", "priority", "lru-unit16"])
def test_scheduled_serving_under_eviction(policy, unit):
    """unit 16: matching in whole 16-token blocks (vLLM-vs-SGLang page,
    matching-unit passage): a cached prefix is reused up to its last whole
    block, the rest of the prompt is computed again into new slots and
    freed as a duplicate when the request finishes."""
    import torch
    from prefix_shared_kv_token_amd import rdx
    from prefix_shared_kv_token_amd.runtime import Runtime

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    prompts, segs, gens, hot = served_queue(**QUEUE)
    print(f"\n[gpu] serving {len(prompts)} prompts, pool {POOL}, policy {policy}, matching unit {unit}", flush=True)
    ld = max(len(p) for p in prompts) + T
    rt = Runtime("bf16", HQ, HKV, D, POOL, BATCH, ld)
    rt.tree = rdx.Tree(POOL, unit, policy)
    cache = TokenTrieCache(POOL, unit, policy)
    dev, tdt = rt.device, rt.tdtype
    worst, hits, n_out = 0.0, 0, 0
    for w0 in range(0, len(prompts), WINDOW):
        win = list(range(w0, min(w0 + WINDOW, len(prompts))))
        got_order = [win[int(i)] for i in rt.schedule([prompts[i] for i in win])]
        want_order = [win[int(i)] for i in lpm_order(cache, [prompts[i] for i in win])[0]]
        assert got_order == want_order, (w0, got_order, want_order)
        for b0 in range(0, len(got_order), BATCH):
            batch = got_order[b0:b0 + BATCH]
            prio = int(max(hot[i] for i in batch)) if policy == "priority" else 0
            want = _oracle_batch(cache, prompts, gens, batch, prio)
            rt.tree.set_priority(prio)
            reqs = rt.admit([prompts[i] for i in batch])
            arrays = [_request_arrays(segs[i], gens[i][0], len(prompts[i])) for i in batch]
            qs, ks, vs = [], [], []
            for j, i in enumerate(batch):
                m, n = int(reqs.matched[j]), len(prompts[i])
                assert m == want[i][0], (policy, i, m, want[i][0])
                hits += m
                q, k, v = arrays[j]
                qs.append(q[m:n]), ks.append(k[m:n]), vs.append(v[m:n])
            to = lambda xs: torch.as_tensor(np.concatenate(xs)).to(dev, tdt).contiguous()
            o_ext = rt.extend(reqs, to(qs), to(ks), to(vs))
            o_dec = []
            for t in range(T):
                n_of = [len(prompts[i]) for i in batch]
                o_dec.append(rt.decode_step(reqs, to([a[0][n + t:n + t + 1] for a, n in zip(arrays, n_of)]),
                                            to([a[1][n + t:n + t + 1] for a, n in zip(arrays, n_of)]),
                                            to([a[2][n + t:n + t + 1] for a, n in zip(arrays, n_of)])))
            torch.cuda.synchronize()
            rows = [rt.host_pt[r, :k].copy() for r, k in zip(reqs.rows, reqs.kv_len)]
            rt.finish(reqs, generated=[gens[i][1] for i in batch])
            off = 0
            for j, i in enumerate(batch):
                np.testing.assert_array_equal(rows[j], want[i][1])
                m, n = int(reqs.matched[j]), len(prompts[i])
                q, k, v = arrays[j]
                ref = causal_attention(np.concatenate([q[m:n], q[n:n + T]]), k, v, np.r_[m:n, n:n + T])
                got = np.concatenate([o_ext[off:off + n - m].float().cpu().numpy()] +
                                     [o[j:j + 1].float().cpu().numpy() for o in o_dec])
                worst = max(worst, float(np.abs(got - ref).max()))
                n_out += len(got)
                off += n - m
    st, ost = rt.tree.stats(), cache.stats()
    print(f"[gpu] {policy}: cached prompt tokens {hits}, evictions {st['evictions']}, {n_out} outputs, "
          f"max abs err {worst:.3g}", flush=True)
    assert st["evictions"] == ost["evictions"] > 0
    assert worst <= 2e-2
    if unit > 1:
        assert hits > 0 and hits % unit == 0
