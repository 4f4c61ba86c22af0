"""General visibility masks through the explicit anc_mask input, on every
kernel path, against the fp64 oracle.

Block-parallel drafting (FlexDraft page, attention tuning) lets each masked
token see its whole block, later tokens included, and the clean prefix, but
no other block; it is not a tree, so it reaches the kernels as anc_mask.
Also: random masks with bits above the row's own index, rows that see no
draft token at all (prefix only) and rows that see every draft token.
"""

import numpy as np
import pytest

import oracle
import synth
from util import assert_parity, cached_inputs, device_inputs, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


# (workload, overrides): the kernel each one reaches is in the comment
PATHS = [
    ("tree32k", (("ctx", (3000, 3000)),)),                                  # 256 rows, DMA
    ("chain_b16", (("ctx", (700, 1500)), ("batch", 3))),                     # 32 rows, DMA small
    ("tree32k", (("ctx", (2000, 2000)), ("n_draft", 24))),                   # 96 rows, MFMA
    ("tree32k", (("ctx", (1500, 1500)), ("head_dim", 64), ("n_draft", 16))),  # D 64, MFMA
    ("tiny_tree", ()),                                                       # fp32, VALU
    ("sparse64k", (("ctx", (4000, 4000)), ("batch", 2), ("n_sel", 700),
                   ("n_recent", 100))),                                      # sparse, DMA small
]


def _masks(rng, B, N):
    flex = [synth.block_masks(N, blk) for blk in (1, 4, max(1, N // 2), N)]
    masks = []
    for b in range(B):
        m = synth.random_masks(rng, 1, N)[0]
        m[0] = 0                                   # prefix only
        m[-1] = np.uint64((1 << N) - 1)            # every draft token
        masks.append((flex[b % len(flex)], m))
    return masks


@pytest.mark.parametrize("case", range(len(PATHS)))
def test_masks_on_every_path(hsv, gpu, case):
    import torch
    name, over = PATHS[case]
    inp = cached_inputs(name, over)
    dev = device_inputs(inp, gpu)
    B, N = inp.parent.shape
    rng = np.random.Generator(np.random.PCG64(70 + case))
    for kind in range(2):
        anc = np.stack([m[kind] for m in _masks(rng, B, N)])
        o, lse = run_hip(hsv, inp, dev, parent=None,
                         anc=torch.from_numpy(anc.view(np.int64)).to(gpu))
        o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=anc,
                                          kv_idx=inp.kv_idx, bf16=inp.is_bf16)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                      f"{name} {dict(over)} {'flex blocks' if kind == 0 else 'random'}")
