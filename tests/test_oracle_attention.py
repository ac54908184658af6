"""Pins of the oracle's attention against facts fixed outside it.

Each test checks the oracle against something other than itself: a brute-
force scalar loop, torch's own attention routine in float64, mathematical
invariants (rows of softmax sum to 1; a shared-prefix split merged by
log-sum-exp equals attention over the unshared sequence), and special cases
with closed forms.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_probs, causal_attention


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _brute(q, k, v, q_pos):
    """Scalar triple loop, no vectorisation: softmax over visible keys."""
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    out = np.zeros((n, hq, d))
    for i in range(n):
        for h in range(hq):
            g = h // (hq // hkv)
            scores = []
            for j in range(int(q_pos[i]) + 1):
                s = 0.0
                for e in range(d):
                    s += q[i, h, e] * k[j, g, e]
                scores.append(s / math.sqrt(d))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for e in range(d):
                acc = 0.0
                for j, wj in enumerate(w):
                    acc += wj * v[j, g, e]
                out[i, h, e] = acc / tot
    return out


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (4, 1)])
def test_matches_brute_force_loop(hq, hkv):
    rng = np.random.default_rng(7)
    L, d = 11, 8
    q_pos = np.array([0, 3, 4, 9, 10])
    q, k, v = _rand(rng, 5, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    np.testing.assert_allclose(causal_attention(q, k, v, q_pos), _brute(q, k, v, q_pos),
                               rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(8)
    L, d, hq, hkv = 37, 16, 8, 2
    q_pos = np.arange(20, 37)
    q, k, v = _rand(rng, 17, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    tq = torch.from_numpy(q).permute(1, 0, 2)                        # [Hq, n, D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    mask = torch.from_numpy(np.arange(L)[None, :] <= q_pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(causal_attention(q, k, v, q_pos),
                               ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_probability_rows_sum_to_one_and_respect_mask():
    rng = np.random.default_rng(9)
    q_pos = np.array([0, 5, 12, 29])
    q, k = _rand(rng, 4, 4, 16), _rand(rng, 30, 2, 16)
    p = attention_probs(q, k, q_pos)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    for i, pos in enumerate(q_pos):
        assert np.all(p[i, :, pos + 1:] == 0.0)
        assert np.all(p[i, :, : pos + 1] > 0.0)


def _lse_merge(parts):
    """Combine partial (o normalised, m, l) states: the log-sum-exp merge."""
    m = np.max([pm for _, pm, _ in parts], axis=0)
    w = [pl * np.exp(pm - m) for _, pm, pl in parts]
    tot = np.sum(w, axis=0)
    return np.sum([wi[..., None] * po for wi, (po, _, _) in zip(w, parts)], axis=0) / tot[..., None]


def _partial(q, k, v, visible):
    d = q.shape[-1]
    s = np.einsum("nhd,lhd->nhl", q, k) / math.sqrt(d)
    s = np.where(visible[:, None, :], s, -np.inf)
    m = s.max(-1)
    e = np.exp(s - m[..., None])
    l = e.sum(-1)
    return np.einsum("nhl,lhd->nhd", e, v) / l[..., None], m, l


def test_shared_prefix_split_equals_unshared_attention():
    """Suffix queries over [prefix | own suffix]: attention over the prefix
    part (no mask) and over the own part (causal), merged by log-sum-exp,
    equals one causal attention over the whole unshared sequence."""
    rng = np.random.default_rng(10)
    P, S, d, h = 23, 9, 16, 3
    k, v = _rand(rng, P + S, h, d), _rand(rng, P + S, h, d)
    q = _rand(rng, S, h, d)
    q_pos = np.arange(P, P + S)
    full = causal_attention(q, k, v, q_pos)
    pre = _partial(q, k[:P], v[:P], np.ones((S, P), bool))
    own = _partial(q, k[P:], v[P:], np.arange(S)[None, :] <= np.arange(S)[:, None])
    np.testing.assert_allclose(full, _lse_merge([pre, own]), rtol=0, atol=1e-12)
    # three-way split of the prefix (split-KV) merges to the same answer
    parts = [_partial(q, k[a:b], v[a:b], np.ones((S, b - a), bool)) for a, b in [(0, 7), (7, 16), (16, P)]]
    np.testing.assert_allclose(full, _lse_merge(parts + [own]), rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(11)
    k, v = _rand(rng, 10, 2, 8), _rand(rng, 10, 2, 8)
    q = np.zeros((3, 2, 8))
    q_pos = np.array([0, 4, 9])
    o = causal_attention(q, k, v, q_pos)
    for i, pos in enumerate(q_pos):
        np.testing.assert_allclose(o[i], v[: pos + 1].mean(axis=0), rtol=0, atol=1e-14)


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(12)
    k, v = _rand(rng, 6, 1, 8), _rand(rng, 6, 1, 8)
    q = _rand(rng, 1, 4, 8) * 50.0
    o = causal_attention(q, k, v, np.array([0]))
    for h in range(4):
        np.testing.assert_array_equal(o[0, h], v[0, 0])


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(13)
    hq, hkv, d, L = 8, 2, 16, 20
    q, k, v = _rand(rng, 5, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    q_pos = np.arange(15, 20)
    rep_k = np.repeat(k, hq // hkv, axis=1)       # head h reads kv head h // (hq/hkv)
    rep_v = np.repeat(v, hq // hkv, axis=1)
    np.testing.assert_allclose(causal_attention(q, k, v, q_pos),
                               causal_attention(q, rep_k, rep_v, q_pos), rtol=0, atol=1e-13)


def test_permuting_prefix_keys_leaves_output_unchanged():
    rng = np.random.default_rng(14)
    P, S = 17, 5
    k, v = _rand(rng, P + S, 2, 8), _rand(rng, P + S, 2, 8)
    q = _rand(rng, S, 2, 8)
    q_pos = np.arange(P, P + S)
    perm = np.concatenate([rng.permutation(P), np.arange(P, P + S)])
    np.testing.assert_allclose(causal_attention(q, k, v, q_pos),
                               causal_attention(q, k[perm], v[perm], q_pos), rtol=0, atol=1e-13)


def test_empty_prefix_is_plain_causal_self_attention():
    rng = np.random.default_rng(15)
    S = 7
    k, v, q = _rand(rng, S, 2, 8), _rand(rng, S, 2, 8), _rand(rng, S, 2, 8)
    np.testing.assert_allclose(causal_attention(q, k, v, np.arange(S)),
                               _brute(q, k, v, np.arange(S)), rtol=0, atol=1e-12)
