"""Pins of the oracle's workload driver: the outputs it assembles for a
request equal a scalar brute-force attention written out here over that
request's logical sequence (prefix node, own node, decode tokens)."""
import math

import numpy as np

from oracle import run_workload
from workloads import Workload, config_by_name


def _brute_row(q, ks, vs, pos, g):
    d = q.shape[-1]
    sc = [float(np.dot(q, ks[j, g])) / math.sqrt(d) for j in range(pos + 1)]
    mx = max(sc)
    w = [math.exp(s - mx) for s in sc]
    return sum(wj * vs[j, g].astype(np.float64) for j, wj in enumerate(w)) / sum(w)


def test_tiny_outputs_match_brute_force():
    wl = Workload(config_by_name("tiny"))
    res = run_workload(wl)
    cfg = wl.cfg
    grp = cfg.n_q_heads // cfg.n_kv_heads
    for req in wl.leaf_requests[:2]:
        prefix_k, prefix_v = wl.node_kv(req.path[0])
        own_k, own_v = wl.node_kv(req.node)
        dk, dv = wl.decode_kv(req)
        ks = np.concatenate([prefix_k, own_k, dk]).astype(np.float64)
        vs = np.concatenate([prefix_v, own_v, dv]).astype(np.float64)
        q_ext, q_dec = wl.request_q(req), wl.decode_q(req)
        P = cfg.levels[0][1]
        for i in (0, 7, req.own_len - 1):
            for h in range(cfg.n_q_heads):
                want = _brute_row(q_ext[i, h].astype(np.float64), ks, vs, P + i, h // grp)
                np.testing.assert_allclose(res.extend_out[req.rid][i, h], want, rtol=0, atol=1e-12)
        for t in (0, cfg.decode_steps - 1):
            for h in range(cfg.n_q_heads):
                want = _brute_row(q_dec[t, h].astype(np.float64), ks, vs, req.prompt_len + t, h // grp)
                np.testing.assert_allclose(res.decode_out[req.rid][t, h], want, rtol=0, atol=1e-12)
    # the hint request (no cached prefix) is plain causal self-attention
    hint = wl.phases[0].requests[0]
    k0, v0 = wl.node_kv(hint.node)
    q0 = wl.request_q(hint)
    for i in (0, 31, 63):
        want = _brute_row(q0[i, 1].astype(np.float64), k0.astype(np.float64), v0.astype(np.float64), i, 1)
        np.testing.assert_allclose(res.extend_out[hint.rid][i, 1], want, rtol=0, atol=1e-12)
