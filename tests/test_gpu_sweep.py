"""GPU parity over a seeded sweep of random shapes and options, through the C ABI.

Each int8 case draws m, k, n, e, the weight type (int8, int8 given (e,n,k),
int4), the groupList type, the rowIndex type, a sharedInput block, rows past
the groups, a tile hint, a grid cap and the ordered combine's row lookup; the
ordered combine must equal the oracle bit for bit (with the int32
accumulators), the unordered one within max|err| <= 1e-5 * max|ref|.  Each
FP8 / MxA8W4 case draws its shape and options likewise and must stay within
the MX oracle's bound, the ordered combine bit-identical under both tiles
and a capped grid.  The draws are fixed by the seed, so a failing case is
named by its index.
"""
import numpy as np
import pytest

import oracle
from oracle import mx as MX
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

N_CASES = 160
N_FP_CASES = 48


def _case(i):
    rng = np.random.default_rng(9000 + i)
    kind = ("int8", "int8", "int8_nk", "int4")[int(rng.integers(0, 4))]
    int4 = kind == "int4"
    m = int(rng.choice([1, 7, 63, 300, 1000, 2500, 6000]))
    k = 64 * int(rng.integers(1, 17))
    n = (32 if int4 else 16) * int(rng.integers(1, 50))
    e = int(rng.choice([1, 2, 5, 17, 64, 300]))
    obs = int(rng.integers(1, max(2, m // 2) + 2))
    bsdp = int(rng.integers(0, obs + 1)) if rng.random() < 0.5 else 0
    kw = dict(int4=int4, group_list_type=int(rng.integers(0, 2)),
              row_index_dtype=np.int32 if rng.random() < 0.4 else np.int64,
              scale_bf16=bool(rng.random() < 0.3), output_bs=obs, bsdp=bsdp,
              shared_offset=int(rng.integers(0, obs - bsdp + 1)) if bsdp else 0,
              empty_frac=float(rng.choice([0.0, 0.3, 0.8])), uncovered=int(rng.integers(0, m // 10 + 1)))
    p = W.random_problem(9000 + i, m, k, n, e, **kw)
    if kind == "int8_nk":
        p = W.with_transposed_weights(p)
    tile = int(rng.choice([0, 0, 32, 64, 128, 256]))
    cap = int(rng.choice([0, 0, 3, 8, 40]))
    lookup = int(rng.integers(0, 3))
    return p, [0, tile, cap, lookup]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_sweep(i):
    p, tc = _case(i)
    ref, ref_acc = oracle.run(p)
    cov = G.covered_mask(p)
    d = G.to_device(p)
    out, acc = G.run_gpu(p, d, deterministic=True, want_acc=True, tuning_config=tc)
    acc = acc.cpu().numpy()
    assert (acc[cov] == ref_acc[cov]).all(), f"case {i}: int32 accumulators differ (tuning {tc})"
    assert (acc[~cov] == -0x55555556).all(), f"case {i}: rows outside every group were written"
    G.assert_bitexact(out.cpu().numpy(), ref)
    out, _ = G.run_gpu(p, d, deterministic=True, tuning_config=tc)  # the guard-free epilogue
    G.assert_bitexact(out.cpu().numpy(), ref)
    out, _ = G.run_gpu(p, d, deterministic=False, combine="atomic", tuning_config=tc)
    G.assert_close_atomic(out.cpu().numpy(), ref)


def _fp_case(i):
    rng = np.random.default_rng(19000 + i)
    mx = bool(rng.random() < 0.5)
    m = int(rng.choice([1, 40, 300, 1000, 2500]))
    e = int(rng.choice([1, 3, 17, 64]))
    obs = int(rng.integers(1, max(2, m // 2) + 2))
    common = dict(group_list_type=int(rng.integers(0, 2)), output_bs=obs,
                  empty_frac=float(rng.choice([0.0, 0.3, 0.8])), uncovered=int(rng.integers(0, m // 10 + 1)))
    if mx:
        k, n = 32 * int(rng.integers(1, 33)), 32 * int(rng.integers(1, 25))
        p = W.mx_problem(19000 + i, m, k, n, e, **common)
    else:
        k, n = 64 * int(rng.integers(1, 17)), 16 * int(rng.integers(1, 49))
        p = W.fp8_problem(19000 + i, m, k, n, e, scale_bf16=bool(rng.random() < 0.3), **common)
        if rng.random() < 0.5:
            p = W.with_untransposed_fp8_weights(p)
    cap = int(rng.choice([0, 3, 8]))
    return p, cap


def _within(p, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), f"{int(bad.sum())} elements outside the bound, worst excess {float((err - bound).max())}"
    if err.size >= 1024:  # typical errors sit far inside the worst-case bound
        assert float(np.median(err / np.maximum(bound, 1e-300))) < 0.02


@pytest.mark.parametrize("i", range(N_FP_CASES))
def test_random_sweep_fp8_mx(i):
    p, cap = _fp_case(i)
    ref, bound, _ = MX.run(p)
    d = G.to_device(p)
    base, _ = G.run_gpu(p, d, deterministic=True)
    base = base.cpu().numpy()
    _within(p, base, ref, bound)
    for tile in (0, 256):
        out, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[0, tile, cap])
        G.assert_bitexact(out.cpu().numpy(), base)
        out, _ = G.run_gpu(p, d, deterministic=False, combine="atomic", tuning_config=[0, tile, cap])
        _within(p, out.cpu().numpy(), ref, bound)
