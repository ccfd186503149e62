"""Full-output parity of every measured workload with the fp64 oracle.

Each workload runs through `bench.prepare`, i.e. the very calls and launch
configuration the benchmark times, and EVERY output element is compared with
the oracle's full product (elementwise rule: |gpu - ref| <= 1e-4 * sum_k
|a_ik b_jk| plus one bf16 ulp of ref for bf16 output; NaN or Inf fails).  The
violations are counted over the whole output (NVFP4, whose tensor scales
enter as an fp32 alpha, takes the epilogue rule with its two fp32
roundings).  The 8192^3 products cost the
oracle about 20 s each on 16 host threads.  The headline bf16 and MXFP8
products are also run twice and must agree bit for bit.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import bench
import tensor_core_matrix_amd as tcm
from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

R, C = orc.ROW_MAJOR, orc.COL_MAJOR


def _say(msg):
    print(f"[workload] {msg}", file=sys.stderr, flush=True)


def _run(name, calls=1):
    _say(f"{name}: GPU call")
    pr = bench.prepare(name, torch, inp, tcm)
    for _ in range(max(calls, pr.sets)):
        pr.fn()
    torch.cuda.synchronize()
    return pr


def _oracle(w, x):
    """The oracle's full product (ref, abssum) for workload w's host inputs."""
    if w.dtype == "nvfp4":
        ga, gb = w.globals
        return orc.gemm_nvfp4(inp.raw(x["A"]), inp.raw(x["B"]), inp.raw(x["SA"]),
                              inp.raw(x["SB"]), ga, gb)
    if w.dtype == "e4m3" and (w.a_order == "col" or w.b_order == "row"):
        lda = w.M if w.a_order == "col" else w.K
        ldb = w.N if w.b_order == "row" else w.K
        return orc.gemm_mx_ld(inp.raw(x["A"]), C if w.a_order == "col" else R, lda,
                              inp.raw(x["B"]), R if w.b_order == "row" else C, ldb,
                              inp.raw(x["SA"]), inp.raw(x["SB"]), w.M, w.N, w.K)
    if w.dtype in ("e4m3", "e2m1", "e2m3", "e3m2"):
        return orc.gemm_mx(inp.raw(x["A"]), inp.raw(x["B"]), inp.raw(x["SA"]), inp.raw(x["SB"]),
                           dtype=orc.DTYPE_NAMES[w.dtype])
    dt = orc.DTYPE_NAMES[w.dtype]
    if w.b_order == "row":
        return orc.gemm_ld(dt, inp.raw(x["A"]), R, w.K, inp.raw(x["B"]), R, w.N, w.M, w.N, w.K)
    return orc.gemm_tn(dt, inp.raw(x["A"]), inp.raw(x["B"]))


def _full_parity(name, pr, out):
    w = pr.w
    _say(f"{name}: oracle, {w.batch} x {w.M} x {w.N} x {w.K}")
    ref, s = _oracle(w, pr.host)
    got = out.cpu().double().numpy()
    if w.dtype == "nvfp4":
        # the tensor scales' product gA gB is formed in fp32 and multiplied
        # into the fp32 sum: the epilogue rule's two fp32 roundings (alpha 1,
        # the scales inside the oracle's sums)
        ok, worst, nbad = orc.check_epi(got, ref, 1.0, s, np.zeros(1), w.out_dtype)
    else:
        ok, worst, nbad = orc.check(got, ref, s, w.out_dtype == "bf16")
    _say(f"{name}: {got.size} outputs, {nbad} violations, worst err/bound {worst:.3g}")
    assert ok, f"{name}: {nbad} of {got.size} outputs outside tolerance (worst {worst:.3g})"
    del ref, s, got
    gc.collect()


@pytest.mark.parametrize("name", ["tile_f16", "bf16_4096", "bf16_8192", "mxfp8_8192",
                                  "mxfp4_8192", "mxfp6_8192", "nvfp4_8192", "bf16_8192_nn",
                                  "mxfp8_8192_mn"])
def test_workload_full_output(name):
    pr = _run(name)
    _full_parity(name, pr, pr.outs[0])
    if name == "tile_f16":
        # the page's own check on its single-tile example
        ref, _ = orc.gemm_tn(orc.F16, inp.raw(pr.host["A"]), inp.raw(pr.host["B"]))
        torch.testing.assert_close(pr.outs[0].cpu(), torch.from_numpy(ref).float(),
                                   rtol=2e-4, atol=2e-4)


def test_workload_batched_full_output_every_set():
    """All 1024 problems of every rotated input/output set: set 0 against the
    oracle in full, the other sets (the same inputs in other buffers) equal to
    it bit for bit."""
    pr = _run("batched")
    assert pr.sets >= 2
    _full_parity("batched", pr, pr.outs[0])
    for k in range(1, pr.sets):
        assert torch.equal(pr.outs[k], pr.outs[0]), f"set {k} differs from set 0"


@pytest.mark.parametrize("name", ["bf16_8192", "mxfp8_8192"])
def test_workload_repeat_runs_bitwise_identical(name):
    """Two calls of the timed launch on the same inputs: the same bits (the
    persistent schedule and the summation order do not depend on timing)."""
    pr = _run(name)
    first = pr.outs[0].clone()
    pr.i = 0
    pr.outs[0].fill_(float("nan"))
    pr.fn()
    torch.cuda.synchronize()
    assert torch.equal(pr.outs[0].view(torch.int16), first.view(torch.int16))
