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
    # k a multiple of 32 or 64 but not of 128 (Atlas 350 MxA8W4 notes: k % 32
    # == 0): block scales padded to whole dwords in the workspace; k % 64 ==
    # 32 leaves the last k-step half filled (an odd count of k-steps also
    # shifts the scale ring's pairing between tiles)
    "k_96_half_step": dict(seed=20, m=300, k=96, n=288, e=3, output_bs=120, bsdp=20, shared_offset=50),
    "k_160_half_step": dict(seed=21, m=500, k=160, n=544, e=4, output_bs=200, group_list_type=1),
    "k_224_half_step_continuous": dict(seed=22, m=700, k=224, n=512, e=3, output_bs=300, uncovered=7),
    "k_192_odd_steps": dict(seed=23, m=600, k=192, n=256, e=4, output_bs=250, empty_frac=0.3),
    "k_320_odd_steps_continuous": dict(seed=24, m=900, k=320, n=288, e=3, output_bs=400, bsdp=30, shared_offset=3),
    "k_32_single_half_step": dict(seed=25, m=200, k=32, n=64, e=2, output_bs=80),
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


@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_fp8_maximum_expert_count(layout):
    """e = 1024 with FP8 weights: the group table's scans full, most experts
    empty or a few rows, both tiles, a capped grid."""
    p = W.fp8_problem(24, 3000, 256, 256, 1024, empty_frac=0.6, output_bs=700)
    if layout == "kn":
        p = W.with_untransposed_fp8_weights(p)
    _check_capped(p)


def test_mx_fp8_maximum_k():
    """k = 65536 (1024 k-steps per tile) for MxA8W4 and FP8, both tiles."""
    _check_capped(W.mx_problem(28, 96, 65536, 256, 2, empty_frac=0.0, output_bs=60))
    _check_capped(W.fp8_problem(27, 96, 65536, 256, 2, empty_frac=0.0, output_bs=60))


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


# ---------------------------------------------------------------- many tiles per workgroup

GRID_CAPPED = ["ragged_shared", "counts_uncovered", "long_k", "k_512_one_scale_group", "k_1536_many_tiles",
               "k_640_dword_path", "many_empty", "k_224_half_step_continuous", "k_320_odd_steps_continuous",
               "k_160_half_step"]


@pytest.mark.parametrize("name", GRID_CAPPED, ids=GRID_CAPPED)
def test_mx_grid_capped(name):
    """The persistent GEMM with its grid capped (tuningConfig[2]), so that
    each workgroup runs many tiles through the continuous pipeline's
    handoff, with either tile (128 x 256, or 256 x 256 with eight waves):
    within the bound, and the ordered combine bit-identical to the uncapped
    launch (each element's k-loop is the same whatever tile runs where)."""
    _check_capped(W.mx_problem(**CASES[name]))


def _check_capped(p):
    ref, bound, _ = MX.run(p)
    d = G.to_device(p)
    base, _ = G.run_gpu(p, d, deterministic=True)
    base = base.cpu().numpy()
    for tile in (0, 256):
        for cap in ((0, 3, 8, 16) if tile else (3, 8, 16)):
            out, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[0, tile, cap])
            G.assert_bitexact(out.cpu().numpy(), base)
            _check(p, out.cpu().numpy(), ref, bound)
            out, _ = G.run_gpu(p, d, deterministic=False, combine="atomic", tuning_config=[0, tile, cap])
            _check(p, out.cpu().numpy(), ref, bound)


@pytest.mark.parametrize("name", list(FP8_CASES), ids=list(FP8_CASES))
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_fp8_grid_capped(name, layout):
    p = W.fp8_problem(**FP8_CASES[name])
    if layout == "kn":
        p = W.with_untransposed_fp8_weights(p)
    _check_capped(p)


# ---------------------------------------------------------------- the matrix core's block arithmetic

# E4M3 codes (sign, exponent bias 7, 3 mantissa bits) and E2M1 codes used below
E4M3 = {256.0: 0x78, -256.0: 0xF8, 2.0 ** -4: 0x18, 2.0 ** -5: 0x10, 2.0 ** -6: 0x08, 1.0: 0x38, 3.0: 0x44,
        7.0: 0x4E}
E2M1_ONE = 0x2


def test_constructed_codes_decode_as_intended():
    for v, c in E4M3.items():
        assert MX.fp8_e4m3_value(c) == v
    assert MX.fp4_e2m1_value(E2M1_ONE) == 1.0


def _mx_block_problem(rows, col1_rows, row_scale_block0):
    """m = 8 rows, k = 128, n = 32, one expert, unit scales except the row
    block-0 scales given.  Weight column 0 is 1.0 on k 0..31 (scale block
    0); column 1 is 1.0 at k = 0 (block 0, first instruction) and k = 64
    (block 2, second instruction); other weights 0.  rows: {row: {k: value}}."""
    m, k, n = 8, 128, 32
    x1 = np.zeros((m, k), dtype=np.uint8)
    for i, vals in {**rows, **col1_rows}.items():
        for kk, v in vals.items():
            x1[i, kk] = E4M3[v]
    x2 = np.zeros((1, n, k // 2), dtype=np.uint8)
    x2[0, 0, :16] = E2M1_ONE | (E2M1_ONE << 4)   # k 0..31 of column 0
    x2[0, 1, 0] = E2M1_ONE                        # k = 0 (low nibble)
    x2[0, 1, 32] = E2M1_ONE                       # k = 64
    pts = np.full((m, k // 64, 2), 127, dtype=np.uint8)
    for i, code in row_scale_block0.items():
        pts[i, 0, 0] = code
    scale = np.full((1, n, k // 64, 2), 127, dtype=np.uint8)
    return W.Problem("mx-blocks", m, k, n, 1, x1, x2, False, scale, False, pts, None,
                     np.array([m], dtype=np.int64), 0, None, None, 0, m, 0, np.array([m]), True, mx=True)


def test_mx_block_arithmetic_matches_the_tolerance_model():
    """The basis of the MxA8W4/FP8 tolerance (oracle/mx.py), measured through
    the library: y = acc exactly here (no logit, unit scales, one row per
    destination), so out is the matrix core's fp32 accumulator.
      * inside one 32-k block, products are aligned to the largest: one 2^-12
        or 2^-13 below it is kept exactly, one 2^-14 below it is dropped;
      * any block's error stays within 2^-7 * max|x1 block| * max|w block|
        (the oracle's per-block term), also for 15 dropped terms and for two
        largest terms that cancel;
      * block sums of successive instructions are added into the fp32
        accumulator with round-to-nearest-even (2^24 + 3 -> 2^24 + 4,
        2^24 + 1 -> 2^24, 2^24 + 7 -> 2^24 + 8; truncation would give
        2^24 + 2, 2^24, 2^24 + 6)."""
    rows = {
        0: {0: 256.0, 1: 2.0 ** -4},                               # 2^-12 below: kept
        1: {0: 256.0, 1: 2.0 ** -5},                               # 2^-13 below: kept
        2: {0: 256.0, 1: 2.0 ** -6},                               # 2^-14 below: dropped
        3: {0: 256.0, **{kk: 2.0 ** -6 for kk in range(1, 16)}},   # fifteen 2^-14 below
        4: {0: 256.0, 1: -256.0, 2: 2.0 ** -6},                    # the largest two cancel
    }
    col1 = {5: {0: 256.0, 64: 3.0}, 6: {0: 256.0, 64: 1.0}, 7: {0: 256.0, 64: 7.0}}
    p = _mx_block_problem(rows, col1, {5: 143, 6: 143, 7: 143})  # 2^16 on block 0 of rows 5-7
    d = G.to_device(p)
    out, _ = G.run_gpu(p, d, deterministic=True)
    out = out.cpu().numpy().astype(np.float64)
    exact = [sum(v for kk, v in rows[i].items() if kk < 32) for i in range(5)]
    got = out[:5, 0]
    assert got[0] == 256.0 + 2.0 ** -4
    assert got[1] == 256.0 + 2.0 ** -5
    assert got[2] == 256.0
    for i in range(5):
        assert abs(got[i] - exact[i]) <= 2.0 ** -7 * 256.0, (i, got[i], exact[i])
    assert got[3] <= exact[3]
    assert out[5, 1] == 2.0 ** 24 + 4
    assert out[6, 1] == 2.0 ** 24
    assert out[7, 1] == 2.0 ** 24 + 8


def test_fp8_block_arithmetic_matches_the_tolerance_model():
    """The FP8 mode runs the same instruction with unit block scales: the
    same kept/dropped threshold inside a 32-k block, and round-to-nearest-even
    when instruction sums are added into the accumulator (four instructions of
    64 products 2^16 make 2^24 exactly; a fifth adds 3 or 7)."""
    m, k, n = 4, 320, 16
    x1 = np.zeros((m, k), dtype=np.uint8)
    x2 = np.zeros((1, n, k), dtype=np.uint8)   # (e,n,k)
    x2[0, 0, :32] = E4M3[1.0]                   # column 0: 1.0 on k 0..31
    x2[0, 1, :] = E4M3[256.0]                   # column 1: 256 on k 0..255 ...
    x2[0, 1, 256:] = E4M3[1.0]                  # ... and 1.0 on the fifth instruction's k
    x1[0, 0], x1[0, 1] = E4M3[256.0], E4M3[2.0 ** -5]
    x1[1, 0], x1[1, 1] = E4M3[256.0], E4M3[2.0 ** -6]
    x1[2, :256], x1[2, 256] = E4M3[256.0], E4M3[3.0]
    x1[3, :256], x1[3, 256] = E4M3[256.0], E4M3[7.0]
    p = W.Problem("fp8-blocks", m, k, n, 1, x1, x2, False, None, False, None, None,
                  np.array([m], dtype=np.int64), 0, None, None, 0, m, 0, np.array([m]), True, fp8=True)
    d = G.to_device(p)
    out, _ = G.run_gpu(p, d, deterministic=True)
    out = out.cpu().numpy().astype(np.float64)
    assert out[0, 0] == 256.0 + 2.0 ** -5
    assert out[1, 0] == 256.0
    assert out[2, 1] == 2.0 ** 24 + 4
    assert out[3, 1] == 2.0 ** 24 + 8
