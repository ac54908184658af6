"""Degenerate cases of prefix caching on the GPU, through the runtime and
the C ABI, against the oracle's cache model and fp64 attention:

* a prompt that is entirely cached (no extend query token of its own: its
  first new token is a decode token over the cached pages) next to a request
  that extends the same cached prompt and one that shares nothing;
* a batch whose prompts are all cached (an extend launch with no query
  token: no kernel runs);
* empty batches (no request) through admission, extend, the decode step and
  finish;
* a long context: a 40,000-token prompt and a follow-up that reuses it,
  checked on sampled query positions.

Matched lengths and page-table rows are compared bit for bit, outputs
within the bf16 tolerance (SGLang explainer, RadixAttention section: a
cached prefix is reused whole; SGLang paper notes, section 3: reuse leaves
every token's attention unchanged)."""
import numpy as np
import pytest

from oracle import TokenTrieCache, causal_attention
from workloads.gen import bf16_bits_to_f32, bf16_round_bits

pytestmark = pytest.mark.gpu

HQ, HKV, D, SIGMA, T = 8, 2, 128, 0.5, 3
TOL = 2e-2
POOL = 2048


def _bf16(x):
    return bf16_bits_to_f32(bf16_round_bits(np.asarray(x, np.float32)))


def test_fully_cached_prompts_and_empty_batches():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_token_amd.runtime import Runtime

    rng = np.random.default_rng(4242)
    P = rng.integers(0, 32000, 300).astype(np.int32)
    E = rng.integers(0, 32000, 50).astype(np.int32)
    U = rng.integers(0, 32000, 120).astype(np.int32)
    while U[0] == P[0]:
        U[0] = rng.integers(0, 32000)
    # logical K/V per token of each sequence (P's shared by everything that starts with it)
    kv = lambda n: (_bf16(rng.normal(0, SIGMA, (n, HKV, D))), _bf16(rng.normal(0, SIGMA, (n, HKV, D))))
    kP, vP = kv(len(P))
    kE, vE = kv(len(E))
    kU, vU = kv(len(U))
    dev = torch.device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev, torch.bfloat16)
    rt = Runtime("bf16", HQ, HKV, D, POOL, 8, 1024, "cuda")
    cache = TokenTrieCache(POOL)
    print("\n[gpu] edges: fully cached prompt, all-cached batch, empty batches", flush=True)

    # ---- phase 1: P from an empty tree ----
    qP = _bf16(rng.normal(0, SIGMA, (len(P), HQ, D)))
    b1 = rt.admit([P])
    assert b1.matched.tolist() == [0]
    o1 = rt.extend(b1, t(qP), t(kP), t(vP))
    m, _, node = cache.match_prefix(P)
    cache.lock(node)
    row1 = cache.alloc(len(P))
    np.testing.assert_array_equal(rt.host_pt[b1.rows[0], :len(P)], row1)
    ref = causal_attention(qP, kP, vP, np.arange(len(P)))
    assert np.abs(o1.float().cpu().numpy() - ref).max() <= TOL
    rt.finish(b1)
    k_, _ = cache.insert(P, row1)
    cache.free(row1[m:k_])
    cache.unlock(node)

    # ---- empty batch through every step ----
    b0 = rt.admit([])
    z = lambda h: torch.empty((0, h, D), dtype=torch.bfloat16, device=dev)
    assert rt.extend(b0, z(HQ), z(HKV), z(HKV)).shape[0] == 0
    assert rt.decode_step(b0, z(HQ), z(HKV), z(HKV)).shape[0] == 0
    rt.finish(b0, generated=[])
    torch.cuda.synchronize()

    # ---- phase 2: P again (all cached), P + E, U ----
    prompts = [P, np.concatenate([P, E]), U]
    seq_k = [kP, np.concatenate([kP, kE]), kU]
    seq_v = [vP, np.concatenate([vP, vE]), vU]
    b2 = rt.admit(prompts)
    adm = []
    for p in prompts:
        m, slots, node = cache.match_prefix(p)
        cache.lock(node)
        adm.append([m, node, list(slots) + cache.alloc(len(p) - m)])
    assert b2.matched.tolist() == [a[0] for a in adm] == [len(P), len(P), 0]
    q_new = [_bf16(rng.normal(0, SIGMA, (len(p) - a[0], HQ, D))) for p, a in zip(prompts, adm)]
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros((0,))
    o2 = rt.extend(b2, t(cat(q_new)), t(cat([k[a[0]:] for k, a in zip(seq_k, adm)])),
                   t(cat([v[a[0]:] for v, a in zip(seq_v, adm)])))
    got = o2.float().cpu().numpy()
    off = 0
    for i, (p, a) in enumerate(zip(prompts, adm)):
        np.testing.assert_array_equal(rt.host_pt[b2.rows[i], :len(p)], a[2])
        n = len(p) - a[0]
        if n:
            ref = causal_attention(q_new[i], seq_k[i], seq_v[i], np.arange(a[0], len(p)))
            assert np.abs(got[off:off + n] - ref).max() <= TOL, i
        off += n

    # ---- T decode steps for all three ----
    gens = [rng.integers(0, 32000, T).astype(np.int32) for _ in prompts]
    for step in range(T):
        qd = _bf16(rng.normal(0, SIGMA, (len(prompts), HQ, D)))
        kd, vd = kv(len(prompts))
        od = rt.decode_step(b2, t(qd), t(kd), t(vd)).float().cpu().numpy()
        for i, a in enumerate(adm):
            a[2] += cache.alloc(1)
            seq_k[i] = np.concatenate([seq_k[i], kd[i:i + 1]])
            seq_v[i] = np.concatenate([seq_v[i], vd[i:i + 1]])
            L = len(seq_k[i])
            np.testing.assert_array_equal(rt.host_pt[b2.rows[i], :L], a[2])
            ref = causal_attention(qd[i:i + 1], seq_k[i], seq_v[i], np.array([L - 1]))
            assert np.abs(od[i:i + 1] - ref).max() <= TOL, (step, i)
    rt.finish(b2, generated=gens)
    for p, g, (m, node, row) in zip(prompts, gens, adm):
        k_, _ = cache.insert(np.concatenate([p, g]), row)
        cache.free(row[m:k_])
        cache.unlock(node)

    # ---- phase 3: a batch whose prompts are all cached (no extend query token) ----
    b3 = rt.admit([P, U])
    assert b3.matched.tolist() == [len(P), len(U)]
    o3 = rt.extend(b3, z(HQ), z(HKV), z(HKV))
    assert o3.shape[0] == 0
    torch.cuda.synchronize()
    rt.finish(b3)
    st = rt.tree.stats()
    assert st["cached"] == cache.stats()["cached"]


def test_long_context_sampled():
    """One 40,000-token prompt (causal prefill of 625 row tiles per KV head,
    items of up to 625 key blocks), then a 1,000-token follow-up that reuses
    it, then two decode steps; sampled query positions (tile and block
    boundaries, the ends) against the oracle, page-table rows bit for bit."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_token_amd.runtime import Runtime

    rng = np.random.default_rng(777)
    L1, L2 = 40000, 1000
    A = rng.integers(0, 32000, L1).astype(np.int32)
    B = np.concatenate([A, rng.integers(0, 32000, L2).astype(np.int32)])
    kv = lambda n: (_bf16(rng.normal(0, SIGMA, (n, HKV, D))), _bf16(rng.normal(0, SIGMA, (n, HKV, D))))
    kA, vA = kv(L1)
    kB, vB = kv(L2)
    dev = torch.device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev, torch.bfloat16)
    pool = L1 + L2 + 16
    rt = Runtime("bf16", HQ, HKV, D, pool, 4, L1 + L2 + 8, "cuda")
    cache = TokenTrieCache(pool)
    print(f"\n[gpu] long context: {L1} + {L2} tokens, Hq/Hkv {HQ}/{HKV}", flush=True)

    qA = _bf16(rng.normal(0, SIGMA, (L1, HQ, D)))
    b1 = rt.admit([A])
    o1 = rt.extend(b1, t(qA), t(kA), t(vA)).float().cpu().numpy()
    m, _, node = cache.match_prefix(A)
    cache.lock(node)
    row = cache.alloc(L1)
    np.testing.assert_array_equal(rt.host_pt[b1.rows[0], :L1], row)
    pos = np.unique(np.concatenate([[0, 1, 63, 64, 65, 255, 256, L1 // 2, L1 - 65, L1 - 64, L1 - 1],
                                    rng.integers(0, L1, 24)]))
    ref = causal_attention(qA[pos], kA, vA, pos)
    assert np.abs(o1[pos] - ref).max() <= TOL
    rt.finish(b1)
    k_, _ = cache.insert(A, row)
    cache.free(row[m:k_])
    cache.unlock(node)

    qB = _bf16(rng.normal(0, SIGMA, (L2, HQ, D)))
    b2 = rt.admit([B])
    assert b2.matched.tolist() == [L1]
    o2 = rt.extend(b2, t(qB), t(kB), t(vB)).float().cpu().numpy()
    m, slots, node = cache.match_prefix(B)
    assert m == L1
    cache.lock(node)
    row = list(slots) + cache.alloc(L2)
    np.testing.assert_array_equal(rt.host_pt[b2.rows[0], :L1 + L2], row)
    kF, vF = np.concatenate([kA, kB]), np.concatenate([vA, vB])
    sel = np.unique(np.concatenate([[0, 63, 64, L2 - 1], rng.integers(0, L2, 12)]))
    ref = causal_attention(qB[sel], kF, vF, L1 + sel)
    assert np.abs(o2[sel] - ref).max() <= TOL
    for step in range(2):
        qd = _bf16(rng.normal(0, SIGMA, (1, HQ, D)))
        kd, vd = kv(1)
        od = rt.decode_step(b2, t(qd), t(kd), t(vd)).float().cpu().numpy()
        kF, vF = np.concatenate([kF, kd]), np.concatenate([vF, vd])
        ref = causal_attention(qd, kF, vF, np.array([len(kF) - 1]))
        assert np.abs(od - ref).max() <= TOL, step
