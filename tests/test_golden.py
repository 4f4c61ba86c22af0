"""Stored oracle outputs (tests/golden/*.json, written by make_golden.py from
oracle/ alone) as regression pins.

CPU: the seeded inputs still hash to the stored manifest, the oracle still
reproduces the stored O/LSE to 1e-12, and the stored prefix and tree parts
merge to the stored whole (LongSpec, section 2.C: the cache part and the
speculative part combine exactly).
GPU: the HIP path, through the C ABI, against the stored values at the
parity bar.
"""

import json
import os

import numpy as np
import pytest

import oracle
import synth
from util import O_ATOL, LSE_RTOL, assert_parity, device_inputs, run_hip

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(HERE, name + ".json")) as f:
        return json.load(f)


def _tiny():
    g = _load("tiny_tree")
    return g, synth.make_inputs(g["workload"])


def _sparse():
    g = _load("small_bf16_sparse")
    r = dict(g["recipe"])
    seed = r.pop("seed")
    r["ctx"] = tuple(r["ctx"])
    inp = synth.make_inputs(synth.WORKLOADS["sparse64k"].scaled(**r), seed=seed,
                            poison_unselected=True)
    return g, inp


def _arr(g, key):
    return np.array(g[key], dtype=np.float64).reshape(g["o_shape"] if key.startswith("o") else
                                                      g["o_shape"][:-1])


def test_golden_inputs_unchanged():
    for g, inp in (_tiny(), _sparse()):
        assert inp.manifest() == g["manifest"]


def test_golden_tiny_tree_oracle_reproduces():
    g, inp = _tiny()
    o, lse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, inp.parent, bf16=False)
    np.testing.assert_allclose(o, _arr(g, "o"), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _arr(g, "lse"), rtol=0, atol=1e-12)
    anc = np.asarray(oracle.ancestor_mask(inp.parent), dtype=np.uint64).ravel()
    assert [int(x) for x in anc] == g["anc_mask"]


def test_golden_sparse_oracle_reproduces_and_parts_merge():
    g, inp = _sparse()
    assert [int(x) for x in inp.kv_idx.ravel()] == g["kv_idx"]
    for name, parts in (("both", oracle.PART_BOTH), ("prefix", oracle.PART_PREFIX),
                        ("tree", oracle.PART_TREE)):
        o, lse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, inp.parent,
                                    kv_idx=inp.kv_idx, bf16=True, parts=parts)
        np.testing.assert_allclose(o, _arr(g, f"o_{name}"), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, _arr(g, f"lse_{name}"), rtol=0, atol=1e-12)
    # the stored parts merge to the stored whole
    D = g["o_shape"][-1]
    op = np.stack([_arr(g, "o_prefix"), _arr(g, "o_tree")]).reshape(2, -1, D)
    lp = np.stack([_arr(g, "lse_prefix"), _arr(g, "lse_tree")]).reshape(2, -1)
    o_both = _arr(g, "o_both").reshape(-1, D)
    l_both = _arr(g, "lse_both").reshape(-1)
    for row in range(lp.shape[1]):
        om, lm = oracle.lse_merge(lp[:, row], op[:, row])
        np.testing.assert_allclose(om, o_both[row], rtol=0, atol=1e-12)
        assert abs(lm - l_both[row]) <= 1e-12


@pytest.mark.gpu
def test_golden_hip_matches_stored(gpu):
    import long_context_tree_verify_amd as hsv
    for g, inp in (_tiny(), _sparse()):
        dev = device_inputs(inp, gpu)
        o, lse = run_hip(hsv, inp, dev)
        o_ref = _arr(g, "o" if "o" in g else "o_both")
        l_ref = _arr(g, "lse" if "lse" in g else "lse_both")
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "golden",
                      o_atol=O_ATOL, lse_rtol=LSE_RTOL)
