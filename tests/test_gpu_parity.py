"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bars: int32 accumulators bit-exact; the ordered (deterministic) combine
bit-exact; the unordered combine within max|err| <= 1e-5 * max|ref|.
Small cases compare every element and span several tiles with ragged tails,
also with the GEMM's grid capped so that each workgroup runs many tiles; the
five named workloads run at full size and are compared on every output
element (the int32 accumulators on sampled rows).
"""
import copy
import json
import os

import numpy as np
import pytest

import oracle
from quantized_moe_grouped_amd import binding as B
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
    # int4 weights with k % 128 == 0: the 128-row tile's 128-k stages
    "int4_k512": dict(seed=21, m=1300, k=512, n=544, e=4, int4=True, empty_frac=0.0, output_bs=450, bsdp=30,
                      shared_offset=100),
    # k % 128 == 0 with more k-steps than stages: the 256-row tile's 128-k stages past its prologue
    "k512_256_row_tiles": dict(seed=19, m=1400, k=512, n=528, e=4, empty_frac=0.0, output_bs=500, bsdp=80,
                               shared_offset=60),
}


# tile hints covering every tile variant, and the ordered combine's two row
# lookups (tuningConfig[3]: 1 bucket index, 2 scan of rowIndex)
HINTS = (None, 8, 100, 300, (0, 256), (0, 0, 0, 1), (0, 0, 0, 2), (0, 64, 0, 1), (8, 0, 0, 1))


@pytest.mark.parametrize("name", list(CASES), ids=list(CASES))
def test_random_case_all_elements(name):
    p = W.random_problem(**CASES[name])
    _check_full(p, hints=HINTS)


# int8 weights given transposed, (e,n,k) (parameter notes: transposed x2)
TB_CASES = ["ragged_n_shared", "counts_i32_bf16_uncovered", "many_empty_experts", "single_row", "full_int8_range",
            "long_k_no_factors", "long_k_i32_index_bf16_shared", "long_k_many_empty", "k512_256_row_tiles"]


@pytest.mark.parametrize("name", TB_CASES, ids=TB_CASES)
def test_random_case_transposed_weights(name):
    p = W.with_transposed_weights(W.random_problem(**CASES[name]))
    _check_full(p, hints=HINTS)



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

# ---------------------------------------------------------------- many tiles per workgroup

def _check_grid_capped(p, caps=(3, 8, 16), tiles=(0, 32, 64, 128, 256)):
    """The persistent GEMM with its grid capped (tuningConfig[2]): every
    workgroup runs many tiles in a row, through the continuous pipeline's
    tile-to-tile handoff (next tile's k-slices and row factors copied under
    this tile's last k-steps, epilogue stores still in flight at the next
    tile's first wait) or the dynamic queues.  Outputs are compared without
    the accumulator dump, so the guard-free epilogue is the one checked:
    ordered bit-exact, atomic within the tolerance; the int32 accumulators
    in a separate run with the dump."""
    ref, ref_acc = oracle.run(p)
    cov = G.covered_mask(p)
    d = G.to_device(p)
    for cap in caps:
        for tile in tiles:
            tc = [0, tile, cap, 1 + (caps.index(cap) + tiles.index(tile)) % 2]  # both row lookups
            out, _ = G.run_gpu(p, d, deterministic=True, tuning_config=tc)
            G.assert_bitexact(out.cpu().numpy(), ref)
            out, _ = G.run_gpu(p, d, deterministic=False, combine="atomic", tuning_config=tc)
            G.assert_close_atomic(out.cpu().numpy(), ref)
            out, acc = G.run_gpu(p, d, deterministic=True, want_acc=True, tuning_config=tc)
            acc = acc.cpu().numpy()
            assert (acc[cov] == ref_acc[cov]).all(), f"acc mismatch (tile {tile}, grid cap {cap})"
            assert (acc[~cov] == -0x55555556).all()
            G.assert_bitexact(out.cpu().numpy(), ref)


@pytest.mark.parametrize("name", list(CASES), ids=list(CASES))
def test_grid_capped_all_elements(name):
    _check_grid_capped(W.random_problem(**CASES[name]))


@pytest.mark.parametrize("name", TB_CASES, ids=TB_CASES)
def test_grid_capped_transposed_weights(name):
    _check_grid_capped(W.with_transposed_weights(W.random_problem(**CASES[name])))


# ---------------------------------------------------------------- hybrid combine

HYB_CASES = ["counts_i32_bf16_uncovered", "int4_counts_many_tiles", "full_int8_range", "long_k_no_factors",
             "long_k_i32_index_bf16_shared", "long_k_many_empty", "int4_k512", "k512_256_row_tiles"]


def _check_hybrid(p, splits=(1, 3, 7), tiles=None, caps=(0, 8)):
    """The hybrid combine (tuningConfig[4] atomic column tiles in every 8):
    the plan takes it, every output element is written, the atomic tiles'
    columns are within the unordered tolerance and the ordered tiles'
    columns bit-exact (the ordered combine's fold), with the grid capped or
    not and under both row lookups."""
    if tiles is None:  # the 256-row tile takes the hybrid combine with int8 weights and k % 128 == 0
        tiles = (128, 256) if not p.x2_int4 and p.k % 128 == 0 else (128,)
    ref, _ = oracle.run(p)
    d = G.to_device(p)
    for a in splits:
        for tile in tiles:
            for cap in caps:
                tc = [0, tile, cap, 1 + (a + tiles.index(tile)) % 2, a]
                plan = G.plan_of(p, d, tuning_config=tc)
                assert plan["combine"] == "hybrid" and plan["hybrid_atomic"] == a, plan
                out, _ = G.run_gpu(p, d, tuning_config=tc)
                G.assert_hybrid(out.cpu().numpy(), ref, a)


@pytest.mark.parametrize("name", HYB_CASES, ids=HYB_CASES)
def test_hybrid_combine(name):
    p = W.random_problem(**CASES[name])
    _check_hybrid(p)


def test_hybrid_combine_many_column_tiles():
    """More than 8 column tiles and a ragged n tail: the second period of
    atomic tiles and a partial last tile in either class; also with
    transposed weights."""
    p = W.random_problem(31, 700, 256, 2320, 3, output_bs=300, bsdp=60, shared_offset=200, uncovered=9)
    _check_hybrid(p, splits=(1, 2, 5, 7))
    _check_hybrid(W.with_transposed_weights(p), splits=(3,), caps=(0,))


def test_hybrid_request_ignored_where_unavailable():
    """tuningConfig[4] is honoured only where AUTO may take the hybrid
    combine: deterministic calls, a forced combine and short k keep their
    own plans and results."""
    p = W.random_problem(**CASES["long_k_no_factors"])
    ref, _ = oracle.run(p)
    d = G.to_device(p)
    assert G.plan_of(p, d, deterministic=True, tuning_config=[0, 0, 0, 0, 3])["combine"] == "ordered"
    assert G.plan_of(p, d, combine="atomic", tuning_config=[0, 0, 0, 0, 3])["combine"] == "atomic"
    out, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[0, 0, 0, 0, 3])
    G.assert_bitexact(out.cpu().numpy(), ref)
    q = W.random_problem(**CASES["ragged_n_shared"])  # k = 128: the tile-by-tile loop
    dq = G.to_device(q)
    assert G.plan_of(q, dq, tuning_config=[0, 128, 0, 0, 3])["combine"] != "hybrid"


def test_grid_capped_single_workgroup():
    """One workgroup runs every tile of a case with a ragged n tail, an empty
    expert and two group tails, in both loop structures."""
    p = W.random_problem(18, 700, 256, 528, 5, output_bs=300, bsdp=50, shared_offset=100, empty_frac=0.3)
    _check_grid_capped(p, caps=(1,), tiles=(0, 32, 64, 128))
    q = W.random_problem(19, 600, 256, 544, 4, int4=True, output_bs=200)
    _check_grid_capped(q, caps=(1,), tiles=(0, 64, 128))


@pytest.mark.parametrize("glt", [0, 1])
def test_maximum_expert_count(glt):
    """e = 1024, the largest groupList the library takes ("aclnnGroupedMatmul
    FinalizeRoutingWeightNzV2", parameter notes: e <= 1024 on the A2/A3
    parts): the group table's scans fill every entry (four per thread with
    256 threads, two with 512), most experts empty or a few rows, under every
    tile height and a capped grid, with k long enough for the continuous
    pipeline and for the 256-row tile's 128-k stages."""
    p = W.random_problem(20 + glt, 4000, 256, 272, 1024, group_list_type=glt, empty_frac=0.6, output_bs=900,
                         bsdp=64, shared_offset=30)
    _check_full(p, hints=(None, (0, 256), (0, 128), (0, 64), (0, 32), (0, 256, 16), (0, 64, 8)))


@pytest.mark.parametrize("int4", [False, True], ids=["int8", "int4"])
def test_maximum_k(int4):
    """k = 65536, the largest the library takes: 512 k-steps of the
    256-row tile (1024 of the others) per tile, and some rows all -128 against
    weights all -128, whose accumulators reach 2^30 (int8)."""
    p = W.random_problem(25 + int4, 96, 65536, 288 if int4 else 272, 2, int4=int4, empty_frac=0.0, output_bs=60)
    if not int4:
        x1 = np.array(p.x1)
        x1[:8] = -128
        x2 = np.array(p.x2)
        x2[:, :, :40] = -128
        p.x1, p.x2 = x1, x2
    _check_full(p, hints=(None, (0, 256), (0, 32), (0, 256, 3)))


def test_zero_rows_gives_seed():
    p = W.random_problem(9, 0, 64, 64, 2, output_bs=20, bsdp=6, shared_offset=3)
    ref, _ = oracle.run(p)
    for det in (True, False):
        out, _ = G.run_gpu(p, deterministic=det, combine="auto" if det else "atomic")
        G.assert_bitexact(out.cpu().numpy(), ref)


def test_long_segment_path():
    """More than 1024 rows into one destination take the reducer's long-segment
    path, with either row lookup."""
    p = W.random_problem(10, 1500, 64, 64, 3, output_bs=3, bsdp=3, shared_offset=0)
    p.row_index[:] = 0
    p.row_index[::7] = 2
    _check_full(p, hints=(None, (0, 0, 0, 1), (0, 0, 0, 2)))


def test_long_segments_split_columns():
    """Destinations averaging more than 1024 rows: each destination's fold
    runs over chunks of the covered rows with the running sum kept in out, and
    its columns are split over several workgroups; one destination receives
    no row (seed only), rows past the groups stay out."""
    p = W.random_problem(67, 5000, 64, 2048, 3, output_bs=3, bsdp=2, shared_offset=1, uncovered=300)
    rng = np.random.default_rng(68)
    p.row_index[:] = rng.integers(0, 2, size=p.m)
    _check_full(p, hints=(None, (0, 0, 0, 1), (0, 0, 0, 2), (0, 256, 4, 2)))


def test_many_destinations_scan_in_chunks():
    """output_bs above the index scan's LDS chunk (32768 destinations): the
    offsets are built over several chunks with a carry."""
    p = W.random_problem(14, 3000, 64, 16, 3, output_bs=70001, bsdp=5000, shared_offset=60000)
    _check_full(p, hints=(None, (0, 0, 0, 2)))


@pytest.mark.parametrize("ri", ["int64", "int32", "identity", "long"])
def test_scan_lookup_over_several_chunks(ri):
    """The ordered combine's rowIndex scan (4096 rows per pass) over several
    passes, with a covered count that is not a multiple of 16 (the scalar
    tail) and every rowIndex form, and a destination receiving 3000 rows (the
    long-segment fold); the bucket index on the same inputs."""
    kw = dict(row_index_dtype=np.int32) if ri == "int32" else {}
    if ri == "identity":
        kw = dict(with_row_index=False)
    p = W.random_problem(66, 9000, 64, 64, 3, output_bs=9000 if ri == "identity" else 700, uncovered=37,
                         bsdp=50, shared_offset=10, **kw)
    if ri == "long":
        p.row_index[::3] = 5
    _check_full(p, hints=((0, 0, 0, 2), (0, 0, 0, 1)))


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

def _sample_src(p, rng, count=48):
    s, e = oracle.group_ranges(p)
    rows = set(rng.choice(max(int(e[-1]), 1), size=min(count, max(int(e[-1]), 1)), replace=False).tolist())
    for a, b in list(zip(s, e))[:8]:
        if b > a:
            rows |= {int(a), int(b) - 1}
    return np.array(sorted(rows), dtype=np.int64)


_NAMED_REF = {}


def _named_ref(name, p):
    """The oracle's whole output of a named workload (computed once per
    session; the transposed-weights form of a workload has the same)."""
    if name not in _NAMED_REF:
        _NAMED_REF[name] = oracle.run(p, want_acc=False)[0]
    return _NAMED_REF[name]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "decode", "skewed", "int4", "prefill"])
def test_named_workload(name):
    _check_named(W.make_config(name, 0), name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_named_workload_transposed_weights(name):
    _check_named(W.with_transposed_weights(W.make_config(name, 0)), name)


def _check_named(p, name):
    """A named workload at full size, every output element against the
    oracle: the ordered combine (deterministic = 1) and the library's own
    choice without the accumulator dump -- the launch the benchmark times --
    bit-exact when that choice is the ordered combine, and the atomic
    combine within the tolerance; the int32 accumulators of sampled rows from
    a run with the dump (whose output must be bit-exact too)."""
    import torch
    ref = _named_ref(name, p)
    d = G.to_device(p)
    args, keep = B.make_args(d["x1"], d["x2"], d["group_list"], torch.empty((p.output_bs, p.n), device="cuda"),
                             scale=d["scale"], pertoken_scale=d["pertoken_scale"], logit=d["logit"],
                             row_index=d["row_index"], shared_input=d["shared_input"],
                             shared_input_offset=p.shared_input_offset if p.shared_input is not None else 0,
                             group_list_type=p.group_list_type, transpose_x2=p.x2_transposed)
    auto_plan = B.plan(args)
    del keep
    out, _ = G.run_gpu(p, d, deterministic=True)
    G.assert_bitexact(out.cpu().numpy(), ref)
    del out
    out, _ = G.run_gpu(p, d, deterministic=False, combine="auto")
    if auto_plan["combine"] == "ordered":
        G.assert_bitexact(out.cpu().numpy(), ref)
    else:
        G.assert_close_atomic(out.cpu().numpy(), ref)
    del out
    out, _ = G.run_gpu(p, d, deterministic=False, combine="atomic")
    G.assert_close_atomic(out.cpu().numpy(), ref)
    del out
    isel = np.arange(p.m) if name == "tiny" else _sample_src(p, np.random.default_rng(100))
    out, acc = G.run_gpu(p, d, deterministic=True, want_acc=True)
    got_acc = acc[torch.from_numpy(isel).cuda()].cpu().numpy()
    del acc
    assert (got_acc == oracle.acc_rows(p, isel)).all()
    G.assert_bitexact(out.cpu().numpy(), ref)


def test_ordered_mode_is_run_to_run_identical():
    p = W.make_config("decode", 1)
    d = G.to_device(p)
    a, _ = G.run_gpu(p, d, deterministic=True)
    b, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[0, 256])
    c, _ = G.run_gpu(p, d, deterministic=True, tuning_config=[8])
    a = a.cpu().numpy()
    G.assert_bitexact(b.cpu().numpy(), a)
    G.assert_bitexact(c.cpu().numpy(), a)
