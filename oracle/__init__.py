"""ORACLE -- test infrastructure, not part of the product.

A plain, slow, obviously correct CPU implementation (Python + NumPy, float64)
of everything the prefix-shared paged-KV path computes:

  * cache_model.TokenTrieCache -- the radix KV cache as a *token-level* trie
    (one trie node per token), mirroring match / lock / alloc / insert /
    LRU leaf eviction of a page-size-1 radix tree;
  * attention.causal_attention -- softmax attention over each request's full
    logical K/V sequence, with a causal mask, in float64;
  * saving -- saved-token counts, the token-saving ratio, hit rate;
  * run.run_workload -- drives a synthetic workload through the model and
    returns every expected output (match lengths, page tables, counts and
    attention outputs).

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package.  It shares no code with the HIP path and
imports nothing from it; the only common dependency is the seeded input
generator package `workloads`, which holds none of the method's arithmetic.
"""
from .attention import causal_attention, attention_probs
from .cache_model import TokenTrieCache, CacheError, EINVAL, ENOSPC, ESTATE
from .saving import saved_tokens, r_saving, hit_rate, prefill_reduction
from .run import run_workload

__all__ = [
    "causal_attention", "attention_probs", "TokenTrieCache", "CacheError",
    "EINVAL", "ENOSPC", "ESTATE", "saved_tokens", "r_saving", "hit_rate",
    "prefill_reduction", "run_workload",
]
