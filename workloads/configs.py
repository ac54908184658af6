"""The five synthetic workload shapes.

Each shape stands in for a workload the pages describe:
  * tiny        -- a parity-only case (fp32, head_dim 64);
  * helpdesk    -- the internal-helpdesk example on the vLLM-vs-SGLang prefix
                   caching page (worked-example section): a 1,000-token common
                   system prompt followed by 40 distinct question tokens,
                   here scaled to 64 concurrent requests, Llama-7B attention
                   shape (32 query heads = 32 KV heads, head_dim 128);
  * batchllm    -- the BatchLLM explainer's micro-benchmark (token-saving
                   section): prefix 2,000 tokens, sharing degree 16, here 64
                   groups, distinct suffix 200, GQA 32/8;
  * longprefix  -- the same page's extreme case: prefix 16,000, sharing 16;
  * multilevel  -- tree-of-thought / multi-turn sharing from the SGLang paper
                   notes (RadixAttention section, multi-level sharing): root
                   1,024 -> 8 branches of 512 -> 3 forks of 128 each.

`levels` lists (fanout, segment length) from the top of the sharing tree
down: level 0's fanout is the number of independent top-level groups; every
node at level k has `fanout` children at level k+1.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "fp32" or "bf16": storage type of Q/K/V/O
    sigma: float          # Q/K/V ~ N(0, 1) * sigma
    levels: tuple         # ((fanout, length), ...) top-down
    decode_steps: int     # decode tokens generated per leaf request
    vocab: int = 32000
    page_size: int = 1

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    # ---- sizes that follow from the shape (plain counting) ----
    @property
    def n_levels(self) -> int:
        return len(self.levels)

    def nodes_at_level(self, k: int) -> int:
        n = 1
        for fan, _ in self.levels[: k + 1]:
            n *= fan
        return n

    @property
    def n_leaves(self) -> int:
        return self.nodes_at_level(self.n_levels - 1)

    @property
    def leaf_prompt_len(self) -> int:
        return sum(length for _, length in self.levels)

    @property
    def max_seq_len(self) -> int:
        return self.leaf_prompt_len + self.decode_steps

    def total_tokens(self) -> int:
        """Distinct logical tokens that ever hold a KV slot (no eviction)."""
        t = 0
        for k, (_, length) in enumerate(self.levels):
            t += self.nodes_at_level(k) * length
        return t + self.n_leaves * self.decode_steps


CONFIGS = [
    Config("tiny", 0, 4, 4, 64, "fp32", 1.0, ((1, 64), (4, 16)), 8),
    Config("helpdesk", 1, 32, 32, 128, "bf16", 0.5, ((1, 1000), (64, 40)), 128),
    Config("batchllm", 2, 32, 8, 128, "bf16", 0.5, ((64, 2000), (16, 200)), 64),
    Config("longprefix", 3, 32, 8, 128, "bf16", 0.5, ((4, 16000), (16, 256)), 32),
    Config("multilevel", 4, 32, 8, 128, "bf16", 0.5,
           ((1, 1024), (8, 512), (3, 128)), 256),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown config {name!r}; known: {[c.name for c in CONFIGS]}")
