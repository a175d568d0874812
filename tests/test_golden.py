"""Regression fixture: stored fp64 oracle outputs on workload 0.

CPU: the oracle still reproduces the stored values (catches an accidental change
to the oracle's arithmetic).  GPU: the HIP path through the C ABI matches them
within the head's tolerances (|dlogp|, |dlse| <= 5e-3, dh relative L2 <= 1e-2).
"""
import json
import os

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import synthetic as syn

HERE = os.path.dirname(os.path.abspath(__file__))
FIX = json.load(open(os.path.join(HERE, "golden", "oracle_workload0.json")))


def _inputs():
    return syn.make_inputs(syn.WORKLOADS[FIX["workload"]], FIX["seed"])


def test_oracle_reproduces_golden():
    inp = _inputs()
    g = np.array(FIX["g"])
    logp, lse, dh = oracle.cce(inp, g=g)
    np.testing.assert_allclose(logp, FIX["logp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, FIX["lse"], rtol=0, atol=1e-12)
    for i, t in enumerate(FIX["dh_tokens"]):
        np.testing.assert_allclose(dh[t], FIX["dh"][i], rtol=1e-12, atol=1e-15)


@pytest.mark.gpu
def test_hip_matches_golden():
    import torch
    from linear_cross_entropy_libcce_amd import cce
    inp = _inputs()
    dev = torch.device("cuda:0")
    head = cce.head_from_numpy(inp, dev)
    h, t, m = cce.tokens_from_numpy(inp, dev)
    logp, lse = cce.cce_forward(h, head, t, m)
    g = torch.tensor(FIX["g"], dtype=torch.float32, device=dev)
    dh = cce.cce_backward(h, head, t, lse, g, m)
    torch.cuda.synchronize()
    assert np.max(np.abs(logp.cpu().numpy() - np.array(FIX["logp"]))) <= 5e-3
    assert np.max(np.abs(lse.cpu().numpy() - np.array(FIX["lse"]))) <= 5e-3
    ref = np.array(FIX["dh"])
    got = dh.cpu().numpy().astype(np.float64)[FIX["dh_tokens"]]
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-2
