"""Token-saving arithmetic (oracle; test infrastructure only).

* saved_tokens -- the vLLM-vs-SGLang prefix-caching page (worked-example
  section and the matching-unit section): the prefill tokens a request
  skips equal the tokens matched from the start of the prompt, rounded down
  to the engine's matching unit (1 token for SGLang, a 16-token block for
  vLLM).
* r_saving -- the BatchLLM explainer, Equation 2: R = (1 - N_processed /
  N_logical) * 100, N_processed the prefill tokens actually computed,
  N_logical those that would be computed with no prefix sharing.
* hit_rate -- SGLang paper notes, section 3 (cache-aware scheduling):
  cached prompt tokens / prompt tokens.
* prefill_reduction -- SGLang explainer (cache-hit effect section): with
  L_prefix cached and L_new new tokens the prefill work shrinks by
  L_prefix / (L_prefix + L_new); a ratio of token counts.
"""
from __future__ import annotations


def saved_tokens(matched: int, unit: int = 1) -> int:
    if unit < 1 or matched < 0:
        raise ValueError("unit >= 1 and matched >= 0 required")
    return (matched // unit) * unit


def r_saving(n_processed: int, n_logical: int) -> float:
    if n_logical <= 0:
        raise ValueError("N_logical must be positive")
    return (1.0 - n_processed / n_logical) * 100.0


def hit_rate(cached_prompt_tokens: int, prompt_tokens: int) -> float:
    if prompt_tokens <= 0:
        raise ValueError("prompt_tokens must be positive")
    return cached_prompt_tokens / prompt_tokens


def prefill_reduction(l_prefix: int, l_new: int) -> float:
    return l_prefix / (l_prefix + l_new)
