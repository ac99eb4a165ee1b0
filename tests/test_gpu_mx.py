"""GPU parity of the MxA8W4 mode (FP8 activations, FP4 weights given (e,n,k),
E8M0 block scales) against the float64 oracle, through the C ABI.

The matrix core accumulates in fp32 in an order of its own, so each output
element is checked against the oracle's error bound for any fp32 evaluation
order (oracle/mx.py); the ordered combine must also be run-to-run identical.
"""
import numpy as np
import pytest

from oracle import mx as MX
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = {
    "ragged_shared": dict(seed=1, m=300, k=256, n=288, e=3, output_bs=200, bsdp=40, shared_offset=7),
    "counts_uncovered": dict(seed=2, m=700, k=384, n=544, e=5, group_list_type=1, uncovered=13, output_bs=333),
    "no_logit_identity": dict(seed=3, m=257, k=128, n=64, e=2, with_logit=False, with_row_index=False,
                              output_bs=257),
    "many_empty": dict(seed=4, m=900, k=256, n=256, e=40, empty_frac=0.7, output_bs=300),
    "single_row": dict(seed=5, m=1, k=128, n=32, e=1, output_bs=1),
    "long_k": dict(seed=6, m=400, k=2048, n=320, e=2, output_bs=150, bsdp=20, shared_offset=100),
    # k a multiple of 512: block scales copied 8 k-slices at a time
    "k_512_one_scale_group": dict(seed=7, m=1000, k=512, n=512, e=4, output_bs=500),
    "k_1536_many_tiles": dict(seed=8, m=2000, k=1536, n=768, e=3, output_bs=700, bsdp=30, shared_offset=5),
    "k_512_many_empty": dict(seed=10, m=900, k=512, n=256, e=40, empty_frac=0.7, output_bs=300),
    # one group past 512 plus 128: the dword-per-pair path
    "k_640_dword_path": dict(seed=9, m=600, k=640, n=288, e=3, output_bs=300),
}


def _check(p, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} elements outside the bound; worst excess "
                           f"{float((err - bound).max())} at {np.argwhere(bad)[0].tolist()}")
    # the bound is a worst case; typical errors sit far inside it (a wrong
    # block scale or k pairing would not)
    assert float(np.median(err / np.maximum(bound, 1e-300))) < 0.02


@pytest.mark.parametrize("name", list(CASES), ids=list(CASES))
def test_mx_random_case_all_elements(name):
    p = W.mx_problem(**CASES[name])
    ref, bound, _ = MX.run(p)
    d = G.to_device(p)
    for det, combine in ((True, "auto"), (False, "atomic"), (False, "auto")):
        out, _ = G.run_gpu(p, d, deterministic=det, combine=combine)
        _check(p, out.cpu().numpy(), ref, bound)


def test_mx_ordered_is_run_to_run_identical():
    p = W.mx_problem(**CASES["ragged_shared"])
    d = G.to_device(p)
    a, _ = G.run_gpu(p, d, deterministic=True)
    b, _ = G.run_gpu(p, d, deterministic=True)
    G.assert_bitexact(b.cpu().numpy(), a.cpu().numpy())


def test_mx_workload_sampled_rows():
    p = W.make_mx_config("mxa8w4", 0)
    rng = np.random.default_rng(100)
    dsel = np.array(sorted(set(rng.choice(p.output_bs, size=24, replace=False).tolist())
                           | {0, p.output_bs - 1, 4095, 4096, 12287, 12288}), dtype=np.int64)
    ref, bound = MX.out_rows(p, dsel)
    d = G.to_device(p)
    out, _ = G.run_gpu(p, d, deterministic=True)
    _check(p, out.cpu().numpy()[dsel], ref, bound)
    out2, _ = G.run_gpu(p, d, deterministic=False, combine="atomic")
    _check(p, out2.cpu().numpy()[dsel], ref, bound)


# ---------------------------------------------------------------- FP8 mode

FP8_CASES = {
    "ragged_bf16_shared": dict(seed=11, m=300, k=256, n=272, e=3, scale_bf16=True, output_bs=200, bsdp=40,
                               shared_offset=7),
    "counts_uncovered": dict(seed=12, m=700, k=192, n=528, e=5, group_list_type=1, uncovered=13, output_bs=333),
    "no_factors_identity": dict(seed=13, m=257, k=64, n=16, e=2, with_scale=False, with_pts=False,
                                with_logit=False, with_row_index=False, output_bs=257),
    "many_empty": dict(seed=14, m=900, k=128, n=256, e=40, empty_frac=0.7, output_bs=300),
    "long_k": dict(seed=15, m=400, k=2048, n=320, e=2, output_bs=150, bsdp=20, shared_offset=100),
}


@pytest.mark.parametrize("name", list(FP8_CASES), ids=list(FP8_CASES))
def test_fp8_random_case_all_elements(name):
    p = W.fp8_problem(**FP8_CASES[name])
    ref, bound, _ = MX.run(p)
    d = G.to_device(p)
    for det, combine in ((True, "auto"), (False, "atomic")):
        out, _ = G.run_gpu(p, d, deterministic=det, combine=combine)
        _check(p, out.cpu().numpy(), ref, bound)



@pytest.mark.parametrize("name", list(FP8_CASES), ids=list(FP8_CASES))
def test_fp8_untransposed_weights(name):
    """FP8 weights given (e,k,n) (full-quant notes: x2 transposed or not)."""
    p = W.with_untransposed_fp8_weights(W.fp8_problem(**FP8_CASES[name]))
    ref, bound, _ = MX.run(p)
    d = G.to_device(p)
    for det, combine in ((True, "auto"), (False, "atomic")):
        out, _ = G.run_gpu(p, d, deterministic=det, combine=combine)
        _check(p, out.cpu().numpy(), ref, bound)


def test_fp8_untransposed_ordered_is_run_to_run_identical():
    """The ordered combine is run-to-run identical with (e,k,n) weights."""
    p = W.with_untransposed_fp8_weights(W.fp8_problem(**FP8_CASES["long_k"]))
    d = G.to_device(p)
    a, _ = G.run_gpu(p, d, deterministic=True)
    b, _ = G.run_gpu(p, d, deterministic=True)
    G.assert_bitexact(b.cpu().numpy(), a.cpu().numpy())


def test_fp8_transposed_workload_sampled_rows():
    """The FP8 workload (weights (e,k,n)) with its weights given transposed, (e,n,k)."""
    p = W.with_transposed_weights(W.make_fp8_config("fp8", 0))
    assert p.x2_transposed and p.x2.shape == (p.e, p.n, p.k)
    rng = np.random.default_rng(102)
    dsel = np.array(sorted(set(rng.choice(p.output_bs, size=24, replace=False).tolist())
                           | {0, p.output_bs - 1, 4095, 4096, 12287, 12288}), dtype=np.int64)
    ref, bound = MX.out_rows(p, dsel)
    d = G.to_device(p)
    out, _ = G.run_gpu(p, d, deterministic=True)
    _check(p, out.cpu().numpy()[dsel], ref, bound)


@pytest.mark.parametrize("name", ["ragged_bf16_shared", "many_empty"])
def test_fp8_per_tensor_scale(name):
    """pertokenScale of shape (1): one static per-tensor activation scale."""
    p = W.with_per_tensor_scale(W.fp8_problem(**FP8_CASES[name]))
    ref, bound, _ = MX.run(p)
    d = G.to_device(p)
    for det, combine in ((True, "auto"), (False, "atomic")):
        out, _ = G.run_gpu(p, d, deterministic=det, combine=combine)
        _check(p, out.cpu().numpy(), ref, bound)

def test_fp8_workload_sampled_rows():
    p = W.make_fp8_config("fp8", 0)
    rng = np.random.default_rng(101)
    dsel = np.array(sorted(set(rng.choice(p.output_bs, size=24, replace=False).tolist())
                           | {0, p.output_bs - 1, 4095, 4096, 12287, 12288}), dtype=np.int64)
    ref, bound = MX.out_rows(p, dsel)
    d = G.to_device(p)
    out, _ = G.run_gpu(p, d, deterministic=True)
    _check(p, out.cpu().numpy()[dsel], ref, bound)
