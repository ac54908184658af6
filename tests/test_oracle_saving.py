"""Pins of the token-saving arithmetic and of the oracle's workload driver.

The token-saving ratio R = (1 - N_processed / N_logical) * 100 (BatchLLM
explainer, Equation 2) is checked two ways: the pages' printed percentages
(golden fixture) and closed forms of the five synthetic shapes, each
reproduced by driving the workload through the token-trie cache model.
"""
import json
import os

import pytest

from oracle import prefill_reduction, r_saving, run_workload, saved_tokens
from workloads import CONFIGS, Workload, config_by_name

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _group_closed_form(prefix, sharing, distinct):
    """One hint of `prefix` tokens + `sharing` requests of prefix+distinct."""
    processed = prefix + sharing * distinct
    logical = sharing * (prefix + distinct)
    return r_saving(processed, logical)


def test_printed_r_saving_figures():
    gold = json.load(open(os.path.join(GOLD, "token_saving.json")))
    d = gold["distinct_tokens_for_printed"]
    for row in gold["r_saving_printed"]:
        got = _group_closed_form(row["prefix"], row["sharing"], d)
        assert abs(got - row["percent"]) <= gold["r_saving_printed_precision"], row


def test_prefill_reduction_example():
    gold = json.load(open(os.path.join(GOLD, "token_saving.json")))["reduction_example"]
    got = 100 * prefill_reduction(gold["l_prefix"], gold["l_new"])
    assert abs(got - gold["approx_percent"]) <= gold["tolerance_percent"]


def test_saved_tokens_rounding():
    assert saved_tokens(1000, 1) == 1000
    assert saved_tokens(1000, 16) == 992
    assert saved_tokens(15, 16) == 0
    with pytest.raises(ValueError):
        saved_tokens(5, 0)


# closed forms: N_processed = every extend request's new tokens (hints included),
# N_logical = leaf requests' prompt lengths.
CLOSED = {
    "tiny": (64 + 4 * 16, 4 * 80),
    "helpdesk": (1000 + 64 * 40, 64 * 1040),
    "batchllm": (64 * (2000 + 16 * 200), 1024 * 2200),
    "longprefix": (4 * (16000 + 16 * 256), 64 * 16256),
    "multilevel": (1024 + 8 * 512 + 24 * 128, 24 * (1024 + 512 + 128)),
}


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_workload_token_counts_match_closed_forms(cfg):
    res = run_workload(Workload(cfg), attention_for=())
    proc, logical = CLOSED[cfg.name]
    assert (res.n_processed, res.n_logical) == (proc, logical)
    assert res.r_saving == pytest.approx(r_saving(proc, logical), abs=1e-12)
    # every leaf matched exactly its shared path (no eviction with a full-size pool)
    for r in Workload(cfg).leaf_requests:
        assert res.matched[r.rid] == r.prompt_len - r.own_len
    assert res.stats["evictions"] == 0 and res.stats["free"] == 0


def test_longprefix_at_printed_distinct_length():
    cfg = config_by_name("longprefix").replace(levels=((4, 16000), (16, 200)), decode_steps=0)
    res = run_workload(Workload(cfg), attention_for=())
    assert round(res.r_saving, 1) == 92.6


def test_group_members_share_page_table_prefix():
    cfg = config_by_name("batchllm").replace(levels=((3, 40), (4, 6)), decode_steps=2)
    wl = Workload(cfg)
    res = run_workload(wl, attention_for=())
    for r in wl.leaf_requests:
        hint = wl.phases[0].requests[r.path[0]]
        assert list(res.rows[r.rid][:40]) == list(res.rows[hint.rid])
        assert len(res.rows[r.rid]) == r.prompt_len + cfg.decode_steps
