"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bars: int32 accumulators bit-exact; the ordered (deterministic) combine
bit-exact; the unordered combine within max|err| <= 1e-5 * max|ref|.
Small cases compare every element and span several tiles with ragged tails;
the five named workloads run at full size and are checked on sampled rows
that the oracle evaluates one by one.
"""
import copy
import json
import os

import numpy as np
import pytest

import oracle
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_full(p, *, hints=(None,), modes=("ordered", "atomic")):
    ref, ref_acc = oracle.run(p)
    cov = G.covered_mask(p)
    d = G.to_device(p)
    for hint in hints:
        tc = None if hint is None else list(hint) if isinstance(hint, tuple) else [hint]
        for mode in modes:
            det = mode == "ordered"
            out, acc = G.run_gpu(p, d, deterministic=det, combine="auto" if det else "atomic", want_acc=True,
                                 tuning_config=tc)
            acc = acc.cpu().numpy()
            assert (acc[cov] == ref_acc[cov]).all(), f"acc mismatch (hint={hint}, mode={mode})"
            assert (acc[~cov] == -0x55555556).all(), "rows outside every group were written"
            if det:
                G.assert_bitexact(out.cpu().numpy(), ref)
            else:
                G.assert_close_atomic(out.cpu().numpy(), ref)


# ---------------------------------------------------------------- the pages' worked example

@pytest.mark.parametrize("glt", [0, 1])
def test_worked_example_padded(glt):
    """The per-token quant matmul example, zero-padded to k = 64, n = 16
    (zeros change no product); the 2x3 corner must equal the printed output."""
    g = json.load(open(os.path.join(GOLDEN, "pertoken_matmul_worked_example.json")))
    x1 = np.zeros((2, 64), dtype=np.int8)
    x1[:, :2] = g["x"]
    x2 = np.zeros((1, 64, 16), dtype=np.int8)
    x2[0, :2, :3] = g["weight"]
    s = np.ones((1, 1, 16), dtype=np.float32)
    s[0, 0, :3] = g["deqScale"]
    p = W.Problem("worked", 2, 64, 16, 1, x1, x2, False, s, False, np.array(g["perTokenScale"], dtype=np.float32),
                  None, np.array([2], dtype=np.int64), glt, np.array([0, 1], dtype=np.int64), None, 0, 2, 0,
                  np.array([2]))
    for det in (True, False):
        out, acc = G.run_gpu(p, deterministic=det, combine="auto" if det else "atomic", want_acc=True)
        assert out.cpu().numpy()[:, :3].tolist() == g["output"]
        assert acc.cpu().numpy()[:, :3].tolist() == g["integer_products_from_the_page_derivation"]


# ---------------------------------------------------------------- random cases, every element

CASES = {
    "ragged_n_shared": dict(seed=1, m=300, k=128, n=272, e=3, output_bs=200, bsdp=40, shared_offset=7),
    "counts_i32_bf16_uncovered": dict(seed=2, m=700, k=256, n=528, e=5, group_list_type=1,
                                      row_index_dtype=np.int32, scale_bf16=True, uncovered=13, output_bs=333),
    "int4": dict(seed=3, m=520, k=192, n=544, e=4, int4=True, output_bs=260, bsdp=100, shared_offset=160),
    "no_factors_identity": dict(seed=4, m=257, k=64, n=16, e=2, with_scale=False, with_pts=False,
                                with_logit=False, with_row_index=False, output_bs=257),
    "many_empty_experts": dict(seed=5, m=1000, k=128, n=256, e=64, empty_frac=0.8, output_bs=300),
    "single_row": dict(seed=6, m=1, k=64, n=32, e=1, output_bs=1),
    "int4_counts_many_tiles": dict(seed=7, m=1100, k=320, n=800 - 800 % 32, e=3, int4=True, group_list_type=1,
                                   output_bs=500),
    "full_int8_range": dict(seed=8, m=333, k=448, n=400, e=3, lo=-128, hi=127, output_bs=100),
    # k >= 192: the continuous copy pipeline (tiles of 64 or more rows)
    "long_k_no_factors": dict(seed=15, m=600, k=320, n=272, e=3, with_scale=False, with_pts=False,
                              with_logit=False, with_row_index=False, output_bs=600),
    "long_k_i32_index_bf16_shared": dict(seed=16, m=900, k=256, n=528, e=4, row_index_dtype=np.int32,
                                         scale_bf16=True, output_bs=450, bsdp=100, shared_offset=350),
    "long_k_many_empty": dict(seed=17, m=1500, k=192, n=256, e=40, empty_frac=0.7, output_bs=400, uncovered=20),
}


@pytest.mark.parametrize("name", list(CASES), ids=list(CASES))
def test_random_case_all_elements(name):
    p = W.random_problem(**CASES[name])
    _check_full(p, hints=(None, 8, 100, 300, (0, 256)))  # every tile variant


# int8 weights given transposed, (e,n,k) (parameter notes: transposed x2)
TB_CASES = ["ragged_n_shared", "counts_i32_bf16_uncovered", "many_empty_experts", "single_row", "full_int8_range",
            "long_k_no_factors", "long_k_i32_index_bf16_shared", "long_k_many_empty"]


@pytest.mark.parametrize("name", TB_CASES, ids=TB_CASES)
def test_random_case_transposed_weights(name):
    p = W.with_transposed_weights(W.random_problem(**CASES[name]))
    _check_full(p, hints=(None, 8, 100, 300, (0, 256)))



# one static per-tensor activation scale (function description: static
# pertensor-perchannel): pertokenScale of shape (1)
PT_CASES = ["ragged_n_shared", "int4", "many_empty_experts", "single_row", "long_k_i32_index_bf16_shared"]


@pytest.mark.parametrize("name", PT_CASES, ids=PT_CASES)
def test_random_case_per_tensor_scale(name):
    p = W.with_per_tensor_scale(W.random_problem(**CASES[name]))
    _check_full(p, hints=(None, 8, 300, (0, 256)))


def test_per_tensor_scale_transposed_weights():
    p = W.with_per_tensor_scale(W.with_transposed_weights(W.random_problem(**CASES["long_k_no_factors"])), 0.75)
    _check_full(p, hints=(None, 8, (0, 256)))

def test_zero_rows_gives_seed():
    p = W.random_problem(9, 0, 64, 64, 2, output_bs=20, bsdp=6, shared_offset=3)
    ref, _ = oracle.run(p)
    for det in (True, False):
        out, _ = G.run_gpu(p, deterministic=det, combine="auto" if det else "atomic")
        G.assert_bitexact(out.cpu().numpy(), ref)


def test_long_segment_path():
    """More than 1024 rows into one destination takes the reducer's scanning path."""
    p = W.random_problem(10, 1500, 64, 64, 3, output_bs=3, bsdp=3, shared_offset=0)
    p.row_index[:] = 0
    p.row_index[::7] = 2
    _check_full(p, hints=(None,))


def test_many_destinations_scan_in_chunks():
    """output_bs above the index scan's LDS chunk (32768 destinations): the
    offsets are built over several chunks with a carry."""
    p = W.random_problem(14, 3000, 64, 16, 3, output_bs=70001, bsdp=5000, shared_offset=60000)
    _check_full(p, hints=(None,))


def test_extreme_accumulators_round_like_the_oracle():
    """x1 = x2 = -128, k = 2048: acc = 2^25 (above 2^24); plus mixed
    magnitudes whose int32 -> fp32 conversion must round to nearest even."""
    m, k, n = 64, 2048, 64
    x1 = np.full((m, k), -128, dtype=np.int8)
    x1[1::2, ::3] = 127
    x2 = np.full((1, k, n), -128, dtype=np.int8)
    x2[0, ::5, 1::2] = 101
    p = W.Problem("extreme", m, k, n, 1, x1, x2, False, np.full((1, 1, n), 1.25, dtype=np.float32), False,
                  np.linspace(0.5, 2, m).astype(np.float32), np.linspace(0.1, 1, m).astype(np.float32),
                  np.array([m], dtype=np.int64), 0, (np.arange(m) // 2).astype(np.int64), None, 0, m // 2, 0,
                  np.array([m]))
    _check_full(p)


# ---------------------------------------------------------------- invariants on the device

def test_gpu_rowindex_permutation_permutes_output():
    p = W.random_problem(11, 600, 128, 256, 4, output_bs=150)
    perm = np.random.default_rng(0).permutation(p.output_bs)
    q = copy.deepcopy(p)
    q.row_index = perm[p.row_index].astype(p.row_index.dtype)
    o, _ = G.run_gpu(p, deterministic=True)
    qo, _ = G.run_gpu(q, deterministic=True)
    G.assert_bitexact(qo.cpu().numpy()[perm], o.cpu().numpy())


def test_gpu_int4_equals_int8():
    p = W.random_problem(12, 400, 256, 512, 3, lo=-8, hi=7, output_bs=123)
    q = copy.deepcopy(p)
    q.x2 = W.pack_int4(p.x2)
    q.x2_int4 = True
    for det in (True,):
        o, a = G.run_gpu(p, deterministic=det, want_acc=True)
        qo, qa = G.run_gpu(q, deterministic=det, want_acc=True)
        assert (a.cpu().numpy() == qa.cpu().numpy()).all()
        G.assert_bitexact(qo.cpu().numpy(), o.cpu().numpy())


def test_gpu_empty_experts_with_nan_scale():
    p = W.random_problem(13, 300, 64, 128, 5, empty_frac=0.0, output_bs=90)
    counts = np.diff(np.concatenate([[0], p.group_list]))
    q = copy.deepcopy(p)
    q.e = p.e + 2
    q.group_list = np.cumsum(np.insert(counts, [0, 3], 0)).astype(np.int64)
    q.x2 = np.insert(p.x2, [0, 3], 77, axis=0)
    q.scale = np.insert(p.scale, [0, 3], np.nan, axis=0).astype(np.float32)
    o, _ = G.run_gpu(p, deterministic=True)
    qo, _ = G.run_gpu(q, deterministic=True)
    G.assert_bitexact(qo.cpu().numpy(), o.cpu().numpy())


# ---------------------------------------------------------------- named workloads at full size

def _sample_rows(p, rng, count=48):
    d = set(rng.choice(p.output_bs, size=min(count, p.output_bs), replace=False).tolist())
    d |= {0, p.output_bs - 1}
    if p.shared_input is not None:
        o, b = p.shared_input_offset, p.bsdp
        d |= {x for x in (o - 1, o, o + b - 1, o + b) if 0 <= x < p.output_bs}
    return np.array(sorted(d), dtype=np.int64)


def _sample_src(p, rng, count=48):
    s, e = oracle.group_ranges(p)
    rows = set(rng.choice(max(int(e[-1]), 1), size=min(count, max(int(e[-1]), 1)), replace=False).tolist())
    for a, b in list(zip(s, e))[:8]:
        if b > a:
            rows |= {int(a), int(b) - 1}
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed", "int4", "prefill"])
def test_named_workload(name):
    _check_named(W.make_config(name, 0), name)


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_named_workload_transposed_weights(name):
    _check_named(W.with_transposed_weights(W.make_config(name, 0)), name)


def _check_named(p, name):
    import torch
    rng = np.random.default_rng(100)
    d = G.to_device(p)
    if name == "tiny":
        ref, ref_acc = oracle.run(p)
        dsel = np.arange(p.output_bs)
        isel = np.arange(p.m)
    else:
        dsel = _sample_rows(p, rng)
        isel = _sample_src(p, rng)
        ref = oracle.out_rows(p, dsel)
        ref_acc = oracle.acc_rows(p, isel)
        ref_full = None
    # int32 accumulators (the dump is written by the same launch as the output)
    out, acc = G.run_gpu(p, d, deterministic=True, want_acc=True)
    got_acc = acc[torch.from_numpy(isel).cuda()].cpu().numpy()
    del acc
    assert (got_acc == (ref_acc if name != "tiny" else ref_acc[isel])).all()
    G.assert_bitexact(out.cpu().numpy()[dsel], ref if name != "tiny" else ref[dsel])
    out2, _ = G.run_gpu(p, d, deterministic=False, combine="atomic")
    G.assert_close_atomic(out2.cpu().numpy()[dsel], ref if name != "tiny" else ref[dsel])
    out3, _ = G.run_gpu(p, d, deterministic=False, combine="auto")
    G.assert_close_atomic(out3.cpu().numpy()[dsel], ref if name != "tiny" else ref[dsel])


def test_ordered_mode_is_run_to_run_identical():
    p = W.make_config("decode", 1)
    d = G.to_device(p)
    a, _ = G.run_gpu(p, d, deterministic=True)
    b, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[0, 256])
    c, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[8])
    a = a.cpu().numpy()
    G.assert_bitexact(b.cpu().numpy(), a)
    G.assert_bitexact(c.cpu().numpy(), a)
