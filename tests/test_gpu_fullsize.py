"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (automatic split plan, bf16 inputs, fp32 output): every output row
against the fp64 oracle, element by element.  The maximum errors over all
rows are logged per workload (they are the error budget's evidence for the
scaled-fp16 split partials)."""

import numpy as np
import pytest

import synth
from util import assert_all_rows, cached_inputs, device_inputs, log, oracle_full, run_hip

pytestmark = pytest.mark.gpu

FULL = ["tiny_tree", "tree32k", "chain_b16", "tree128k", "sparse64k"]


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


@pytest.mark.parametrize("name", FULL)
def test_full_size_all_rows(hsv, gpu, name):
    import torch
    log(f"full-size {name}: generating")
    inp = cached_inputs(name) if name == "tree32k" else synth.make_inputs(name)
    dev = device_inputs(inp, gpu)
    log(f"full-size {name}: running HIP path")
    o, lse = run_hip(hsv, inp, dev)
    o_np, l_np = o.cpu().numpy(), lse.cpu().numpy()
    del dev
    torch.cuda.empty_cache()
    if name == "tree32k":
        o_ref, l_ref = oracle_full(name)
    else:
        o_ref, l_ref = None, None
    o_err, l_err = assert_all_rows(o_np, l_np, inp, f"full-size {name}", o_ref, l_ref)
    log(f"full-size {name}: all {l_np.size} rows max|dO| = {o_err:.3e}, "
        f"max rel dLSE = {l_err:.3e}")


@pytest.mark.parametrize("name", ["tree128k", "sparse64k"])
def test_full_size_f32_partials(hsv, gpu, name):
    """The same full-size calls with the split partials kept in fp32
    (HSV_FLAG_F32_PARTIALS): every row against the oracle, and the error the
    default scaled-fp16 partials add, measured on the same inputs."""
    import torch
    inp = synth.make_inputs(name)
    dev = device_inputs(inp, gpu)
    o16, l16 = run_hip(hsv, inp, dev)
    o32, l32 = run_hip(hsv, inp, dev, flags=hsv.HSV_FLAG_F32_PARTIALS)
    o16, l16, o32, l32 = o16.cpu().numpy(), l16.cpu().numpy(), o32.cpu().numpy(), l32.cpu().numpy()
    del dev
    torch.cuda.empty_cache()
    import oracle
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=inp.kv_idx, bf16=True)
    e32 = assert_all_rows(o32, l32, inp, f"{name} fp32 partials", o_ref, l_ref)
    e16 = assert_all_rows(o16, l16, inp, f"{name} fp16 partials", o_ref, l_ref)
    # the fp16 storage adds at most 2^-11 of a partial row's largest |value|
    vmax = float(np.abs(np.nan_to_num(synth.bf16_bits_to_f32(inp.v))).max())
    assert float(np.abs(o16 - o32).max()) <= 2.0 ** -11 * vmax * 1.05
    log(f"full-size {name}: max|dO| fp32 partials {e32[0]:.3e}, fp16 partials {e16[0]:.3e}")
