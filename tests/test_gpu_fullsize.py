"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (automatic split plan, bf16 inputs, fp32 output): every output row
against the fp64 oracle, element by element.  The maximum errors over all
rows are logged per workload (they are the error budget's evidence for the
scaled-fp16 split partials)."""

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
