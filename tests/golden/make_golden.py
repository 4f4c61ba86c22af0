"""Write the stored oracle outputs under tests/golden/ (run by hand).

Every value in these files comes from ``oracle/`` alone: the seeded inputs
from ``synth`` are fed to the fp64 oracle and its outputs are written as text.
The pages print no worked example, so these fixtures are regression pins of
the oracle itself (a change to its arithmetic shows up as a diff here, and
the commit that makes it has to name the passage behind it).

Fixtures:

* ``tiny_tree.json`` -- the tiny tree workload (1 sequence, 1 head, D 64,
  fp32, 256 prefix tokens, 8-node tree): verification attention over the
  prefix plus the draft tree under the ancestor mask (LongSpec, section 2.C,
  Hybrid Tree Attention), O and LSE for all 8 rows, and the ancestor masks.
* ``small_bf16_sparse.json`` -- a 2-sequence, 2/1-head, D 64 bf16 case over a
  gathered index set (Dustin, methodology 3: verification over the selected
  subset of a fully indexed cache), with its parts computed separately
  (prefix only, tree only) as the divide-and-aggregate form takes them.

Usage: ``python tests/golden/make_golden.py`` from the repository root.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def _floats(a):
    return [float(x) for x in np.asarray(a, dtype=np.float64).ravel()]


def tiny_tree():
    inp = synth.make_inputs("tiny_tree")
    o, lse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, inp.parent, bf16=False)
    anc = oracle.ancestor_mask(inp.parent)
    return {
        "what": "tiny tree verify: O [B,N,Hq,D] and LSE [B,N,Hq] from the fp64 oracle",
        "passage": "LongSpec, section 2.C (Hybrid Tree Attention)",
        "workload": "tiny_tree",
        "manifest": inp.manifest(),
        "parent": [int(x) for x in inp.parent.ravel()],
        "anc_mask": [int(x) for x in np.asarray(anc, dtype=np.uint64).ravel()],
        "o_shape": list(o.shape),
        "o": _floats(o),
        "lse": _floats(lse),
    }


SMALL = dict(batch=2, n_q_heads=2, n_kv_heads=1, head_dim=64, ctx=(40, 57), n_draft=4,
             n_sel=12, n_recent=4, seed=11)


def small_bf16_sparse():
    wl = synth.WORKLOADS["sparse64k"].scaled(
        **{k: tuple(v) if k == "ctx" else v for k, v in SMALL.items() if k != "seed"})
    inp = synth.make_inputs(wl, seed=SMALL["seed"], poison_unselected=True)
    out = {"what": "sparse bf16 verify: whole, prefix part, tree part (fp64 oracle)",
           "passage": "Dustin, methodology 3 (verification workflow over the selected subset); "
                      "LongSpec, section 2.C (cache part, speculative part, exact merge)",
           "recipe": SMALL, "manifest": inp.manifest(),
           "kv_idx": [int(x) for x in inp.kv_idx.ravel()]}
    for name, parts in (("both", oracle.PART_BOTH), ("prefix", oracle.PART_PREFIX),
                        ("tree", oracle.PART_TREE)):
        o, lse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, inp.parent,
                                    kv_idx=inp.kv_idx, bf16=True, parts=parts)
        out[f"o_{name}"] = _floats(o)
        out[f"lse_{name}"] = _floats(lse)
        out["o_shape"] = list(o.shape)
    return out


def main():
    for name, fn in (("tiny_tree", tiny_tree), ("small_bf16_sparse", small_bf16_sparse)):
        path = os.path.join(HERE, name + ".json")
        with open(path, "w") as f:
            json.dump(fn(), f, indent=0)
            f.write("\n")
        print("wrote", path)


if __name__ == "__main__":
    main()
