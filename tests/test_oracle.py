"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: values the pages
print, closed forms, invariants of the definition, an exact rational error
bound, the float64-BLAS identity for the integer GEMM, and a separately
written pure-Python brute force on tiny inputs.
"""
import copy
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from quantized_moe_grouped_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _worked_problem(group_list_type, row_index, output_bs, logit=None):
    g = _load("pertoken_matmul_worked_example.json")
    x = np.array(g["x"], dtype=np.int8)
    w = np.array(g["weight"], dtype=np.int8)[None]
    s = np.array(g["deqScale"], dtype=np.float32).reshape(1, 1, 3)
    pts = np.array(g["perTokenScale"], dtype=np.float32)
    gl = np.array([2], dtype=np.int64)  # one expert holding both rows: same list for both types
    return W.Problem("worked", 2, 2, 3, 1, x, w, False, s, False, pts,
                     None if logit is None else np.array(logit, dtype=np.float32),
                     gl, group_list_type, np.array(row_index, dtype=np.int64), None, 0,
                     output_bs, 0, np.array([2]))


# ---------------------------------------------------------------- values printed on the pages

@pytest.mark.parametrize("glt", [0, 1])
def test_worked_example_pertoken_matmul(glt):
    g = _load("pertoken_matmul_worked_example.json")
    p = _worked_problem(glt, [0, 1], 2)
    out, acc = oracle.run(p)
    assert acc.tolist() == g["integer_products_from_the_page_derivation"]
    assert out.tolist() == g["output"]
    bout, bacc = brute.brute(p)
    assert bacc.tolist() == g["integer_products_from_the_page_derivation"]
    assert bout.tolist() == g["output"]


def test_combine_from_worked_example():
    g = _load("combine_from_worked_example.json")
    p = _worked_problem(0, g["rowIndex"], g["outputBS"], logit=g["logit"])
    out, _ = oracle.run(p)
    assert out.tolist() == g["output"]
    assert brute.brute(p)[0].tolist() == g["output"]


def test_int4_nibble_decoding():
    g = _load("int4_nibbles.json")
    words = np.array([int(h, 16) for h in g["words_hex"]], dtype=np.uint32).view(np.int32)
    kk = len(words)
    x1 = np.eye(kk, dtype=np.int8)                       # row i of acc = row i of W
    x2 = words.reshape(1, kk, 1)
    p = W.Problem("nibbles", kk, kk, 8, 1, x1, x2, True, None, False, None, None,
                  np.array([kk], dtype=np.int64), 0, None, None, 0, kk, 0, np.array([kk]))
    out, acc = oracle.run(p)
    assert acc.tolist() == g["values"]
    assert out.tolist() == [[float(v) for v in r] for r in g["values"]]
    assert brute.brute(p)[1].tolist() == g["values"]
    # the generator's packer agrees with the hand-decoded fixture
    assert (W.pack_int4(np.array(g["values"], dtype=np.int8)).reshape(-1) == words).all()


# ---------------------------------------------------------------- brute force on tiny inputs

def _tiny_cases():
    cases = []
    rng = np.random.default_rng(1234)
    for seed in range(60):
        m = int(rng.integers(1, 20))
        k = int(rng.integers(1, 12))
        n = int(rng.choice([8, 16]))
        e = int(rng.integers(1, 5))
        kw = dict(
            int4=bool(seed % 5 == 0),
            scale_bf16=bool(seed % 3 == 0),
            group_list_type=seed % 2,
            row_index_dtype=np.int32 if seed % 4 == 1 else np.int64,
            with_scale=seed % 7 != 3,
            with_pts=seed % 6 != 2,
            with_logit=seed % 8 != 5,
            with_row_index=seed % 9 != 4,
            uncovered=int(rng.integers(0, 3)) if m > 3 else 0,
        )
        obs = int(rng.integers(1, 10)) if kw["with_row_index"] else m
        kw["output_bs"] = obs
        if seed % 4 == 0 and obs > 1:
            kw["bsdp"] = int(rng.integers(1, obs))
            kw["shared_offset"] = int(rng.integers(0, obs - kw["bsdp"] + 1))
        cases.append((seed, m, k, n, e, kw))
    return cases


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: f"s{c[0]}")
def test_brute_force_matches_oracle(case):
    seed, m, k, n, e, kw = case
    p = W.random_problem(seed, m, k, n, e, **kw)
    out, acc = oracle.run(p)
    bout, bacc = brute.brute(p)
    assert (acc.astype(np.int64) == bacc).all()
    # bit-exact, comparing -0.0 and +0.0 as equal
    assert np.array_equal(out, bout)


# ---------------------------------------------------------------- exact integer GEMM

def test_acc_equals_float64_blas():
    """Every partial sum is an integer below 2**53, so float64 BLAS is exact
    in any summation order."""
    p = W.random_problem(7, 384, 2048, 256, 3, empty_frac=0.0)
    _, acc = oracle.run(p)
    start, end = oracle.group_ranges(p)
    for g in range(p.e):
        a = p.x1[start[g]:end[g]].astype(np.float64)
        ref = a @ p.x2[g].astype(np.float64)
        assert (acc[start[g]:end[g]].astype(np.float64) == ref).all()


def test_acc_closed_form_extremes():
    """x1[i][:] = a_i and x2[g][:, j] = b_gj give acc = k * a_i * b_gj,
    including the extreme -128 * -128 products."""
    k, n, e = 2048, 32, 2
    a = np.array([-128, 127, -1, 0, 5, -128], dtype=np.int8)
    m = a.shape[0]
    b = np.stack([np.linspace(-128, 127, n).astype(np.int8), np.full(n, -128, dtype=np.int8)])
    x1 = np.repeat(a[:, None], k, axis=1)
    x2 = np.repeat(b[:, None, :], k, axis=1)
    p = W.Problem("closed", m, k, n, e, x1, x2, False, None, False, None, None,
                  np.array([3, 6], dtype=np.int64), 0, None, None, 0, m, 0, np.array([3, 3]))
    _, acc = oracle.run(p)
    for i in range(m):
        g = 0 if i < 3 else 1
        assert (acc[i] == k * int(a[i]) * b[g].astype(np.int64)).all()


# ---------------------------------------------------------------- invariants

def _base(seed=3, **kw):
    args = dict(empty_frac=0.3, output_bs=40, bsdp=12, shared_offset=5)
    args.update(kw)
    return W.random_problem(seed, 96, 64, 48, 6, **args)


def test_group_list_types_agree():
    p0 = _base(group_list_type=0)
    p1 = copy.deepcopy(p0)
    p1.group_list = np.diff(np.concatenate([[0], p0.group_list])).astype(np.int64)
    p1.group_list_type = 1
    o0, a0 = oracle.run(p0)
    o1, a1 = oracle.run(p1)
    assert (a0 == a1).all() and np.array_equal(o0, o1)


def test_empty_groups_contribute_nothing():
    p = _base(empty_frac=0.0, seed=5)
    o, a = oracle.run(p)
    # insert two empty experts with garbage weights and NaN scales
    counts = np.diff(np.concatenate([[0], p.group_list]))
    q = copy.deepcopy(p)
    ins = [0, 3]
    rng = np.random.default_rng(0)
    new_counts = np.insert(counts, ins, 0)
    q.e = p.e + len(ins)
    q.group_list = np.cumsum(new_counts).astype(np.int64)
    q.x2 = np.insert(p.x2, ins, rng.integers(-128, 128, size=(p.k, p.n), dtype=np.int8), axis=0)
    q.scale = np.insert(p.scale, ins, np.nan, axis=0).astype(np.float32)
    qo, qa = oracle.run(q)
    assert (qa == a).all() and np.array_equal(qo, o)


def test_uncovered_rows_have_no_effect():
    p = _base(uncovered=10)
    o, _ = oracle.run(p)
    q = copy.deepcopy(p)
    rng = np.random.default_rng(9)
    q.x1[-10:] = rng.integers(-128, 128, size=(10, p.k), dtype=np.int8)
    q.pertoken_scale[-10:] = np.inf
    q.logit[-10:] = np.nan
    q.row_index[-10:] = -7          # outside the output: never read for uncovered rows
    qo, _ = oracle.run(q)
    assert np.array_equal(qo, o)


def test_row_index_permutation_permutes_output():
    p = _base(bsdp=0, shared_offset=0)
    p.shared_input = None
    o, _ = oracle.run(p)
    perm = np.random.default_rng(4).permutation(p.output_bs)
    q = copy.deepcopy(p)
    q.row_index = perm[p.row_index].astype(p.row_index.dtype)
    qo, _ = oracle.run(q)
    assert np.array_equal(qo[perm], o)


def test_zero_activations_give_the_seed():
    p = _base()
    p.x1[:] = 0
    o, a = oracle.run(p)
    assert (a == 0).all()
    seed = np.zeros((p.output_bs, p.n), dtype=np.float32)
    seed[p.shared_input_offset:p.shared_input_offset + p.bsdp] = W.bf16_bits_to_f32(p.shared_input)
    assert np.array_equal(o, seed)


@pytest.mark.parametrize("s", [-3, 1, 5])
def test_logit_power_of_two_scales_output(s):
    p = _base(bsdp=0)
    p.shared_input = None
    o, _ = oracle.run(p)
    q = copy.deepcopy(p)
    q.logit = (p.logit * np.float32(2.0 ** s)).astype(np.float32)
    qo, _ = oracle.run(q)
    assert np.array_equal(qo, (o * np.float32(2.0 ** s)).astype(np.float32))


def test_int4_equals_int8_with_small_values():
    p = W.random_problem(11, 80, 96, 64, 4, lo=-8, hi=7, bsdp=10, output_bs=30)
    q = copy.deepcopy(p)
    q.x2 = W.pack_int4(p.x2)
    q.x2_int4 = True
    o, a = oracle.run(p)
    qo, qa = oracle.run(q)
    assert (a == qa).all() and np.array_equal(o, qo)


def test_transposed_weights_equal_untransposed():
    """Weights given as (e,n,k) (parameter notes: transposed x2) compute the
    same result as the (e,k,n) form; the brute force indexes the transposed
    array directly, the C oracle receives it transposed back."""
    p = W.random_problem(12, 70, 96, 48, 3, bsdp=8, output_bs=30)
    q = W.with_transposed_weights(p)
    assert q.x2.shape == (p.e, p.n, p.k) and q.x2_transposed
    o, a = oracle.run(p)
    qo, qa = oracle.run(q)
    assert (a == qa).all() and np.array_equal(o, qo)
    small = W.random_problem(13, 9, 32, 8, 2, bsdp=2, output_bs=6)
    ts = W.with_transposed_weights(small)
    bo, ba = brute.brute(ts)
    so, sa = oracle.run(small)
    assert (sa.astype(np.int64) == ba).all() and np.array_equal(so, bo)
    # reading the (e,n,k) bytes as (e,k,n), i.e. dropping the transpose, changes the result
    wrong = copy.deepcopy(q)
    wrong.x2_transposed = False
    wo, _ = oracle.run(wrong)
    assert not np.array_equal(wo, o)


def test_missing_factors_equal_unit_factors():
    p = _base()
    q = copy.deepcopy(p)
    q.scale, q.pertoken_scale, q.logit = None, None, None
    r = copy.deepcopy(p)
    r.scale = np.ones_like(p.scale)
    r.pertoken_scale = np.ones_like(p.pertoken_scale)
    r.logit = np.ones_like(p.logit)
    assert np.array_equal(oracle.run(q)[0], oracle.run(r)[0])



def test_per_tensor_scale_is_every_rows_scale():
    """A pertokenScale of shape (1) ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2",
    function description: static pertensor-perchannel) scales every row: the
    same as a per-token array holding that value in every entry; with no seed,
    a power of two 2**s gives 2**s times the unscaled output exactly; the
    brute force agrees on a tiny case."""
    p = _base()
    v = float(p.pertoken_scale[3])
    q = W.with_per_tensor_scale(p, v)
    assert q.pertoken_scale.shape == (1,)
    r = copy.deepcopy(p)
    r.pertoken_scale = np.full(p.m, v, dtype=np.float32)
    assert np.array_equal(oracle.run(q)[0], oracle.run(r)[0])
    base = _base(bsdp=0)
    base.shared_input = None
    none = copy.deepcopy(base)
    none.pertoken_scale = None
    for s in (-3, 5):
        two = W.with_per_tensor_scale(base, 2.0 ** s)
        assert np.array_equal(oracle.run(two)[0], oracle.run(none)[0] * np.float32(2.0 ** s))
    small = W.with_per_tensor_scale(W.random_problem(21, 11, 32, 8, 2, bsdp=2, output_bs=7), 0.37)
    bo, ba = brute.brute(small)
    so, sa = oracle.run(small)
    assert (sa.astype(np.int64) == ba).all() and np.array_equal(so, bo)
    bad = copy.deepcopy(p)
    bad.pertoken_scale = np.ones(2, dtype=np.float32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.run(bad)
    assert e.value.status == "SHAPE"

def test_absent_row_index_is_identity():
    p = _base(with_row_index=False, output_bs=96, bsdp=0)
    q = copy.deepcopy(p)
    q.row_index = np.arange(p.m, dtype=np.int64)
    assert np.array_equal(oracle.run(p)[0], oracle.run(q)[0])


def test_sampled_rows_match_whole_output():
    p = _base()
    o, a = oracle.run(p)
    d = np.array([0, 7, 13, 39, 5])
    assert np.array_equal(oracle.out_rows(p, d), o[d])
    i = np.array([0, 1, 50, 95, 94])
    assert (oracle.acc_rows(p, i) == a[i]).all()


# ---------------------------------------------------------------- exact rational error bound

def test_rounding_error_within_bound():
    """Against the exact real value of the definition (fractions), the fp32
    result errs by at most (t + 4) u sum|terms| per element, u = 2**-24, t the
    number of rows added into that element (4 roundings per term, one per add)."""
    p = W.random_problem(21, 40, 32, 16, 3, output_bs=6, bsdp=3, shared_offset=2,
                         scale_bf16=True)
    out, acc = oracle.run(p)
    ranges = brute.ranges(p)
    u = Fraction(1, 2 ** 24)
    seedv = np.zeros((p.output_bs, p.n), dtype=np.float32)
    seedv[2:5] = W.bf16_bits_to_f32(p.shared_input)
    exact = [[Fraction(float(seedv[d, j])) for j in range(p.n)] for d in range(p.output_bs)]
    absum = [[abs(exact[d][j]) for j in range(p.n)] for d in range(p.output_bs)]
    terms = [[0] * p.n for _ in range(p.output_bs)]
    sc = W.bf16_bits_to_f32(p.scale)
    for g, (s, e) in enumerate(ranges):
        for i in range(s, e):
            d = int(p.row_index[i])
            for j in range(p.n):
                t = (Fraction(int(acc[i, j])) * Fraction(float(sc[g, 0, j]))
                     * Fraction(float(p.pertoken_scale[i])) * Fraction(float(p.logit[i])))
                exact[d][j] += t
                absum[d][j] += abs(t)
                terms[d][j] += 1
    worst = 0.0
    for d in range(p.output_bs):
        for j in range(p.n):
            err = abs(Fraction(float(out[d, j])) - exact[d][j])
            bound = (terms[d][j] + 4) * u * absum[d][j] * Fraction(101, 100)
            assert err <= bound, (d, j, float(err), float(bound))
            if absum[d][j]:
                worst = max(worst, float(err / absum[d][j]))
    assert worst < 1e-6


# ---------------------------------------------------------------- strict validation

def _expect(code, p):
    with pytest.raises(oracle.OracleError) as ei:
        oracle.run(p)
    assert ei.value.status == code


def test_validation_errors():
    p = _base(group_list_type=0)
    q = copy.deepcopy(p); q.group_list = q.group_list.copy(); q.group_list[2] = q.group_list[1] - 1
    if q.group_list[2] >= 0:
        _expect("GROUPLIST", q)
    q = copy.deepcopy(p); q.group_list = q.group_list.copy(); q.group_list[-1] = p.m + 1
    _expect("GROUPLIST", q)
    q = copy.deepcopy(p); q.group_list = q.group_list.copy(); q.group_list[0] = -1
    _expect("GROUPLIST", q)
    q = copy.deepcopy(p); q.group_list_type = 2
    _expect("GROUPLIST", q)
    q = copy.deepcopy(p); q.row_index = q.row_index.copy(); q.row_index[0] = p.output_bs
    _expect("ROWINDEX", q)
    q = copy.deepcopy(p); q.shared_input_offset = p.output_bs - p.bsdp + 1
    _expect("SHARED", q)
    q = copy.deepcopy(p); q.group_list_type = 1
    q.group_list = np.full(p.e, p.m // p.e + 1, dtype=np.int64)
    _expect("GROUPLIST", q)


# ---------------------------------------------------------------- generators

def test_bf16_encoding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (W.f32_to_bf16_bits(x) == ref).all()


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed"])
def test_named_configs_shapes(name):
    p = W.make_config(name, 0)
    assert p.x1.shape == (p.m, p.k)
    assert p.covered_rows == p.m
    start, end = oracle.group_ranges(p)
    assert end[-1] == p.m and (np.diff(start) >= 0).all()
    assert p.row_index.min() >= 0 and p.row_index.max() < p.output_bs
    # every token gets the same number of rows
    cnt = np.bincount(p.row_index.astype(np.int64), minlength=p.output_bs)
    assert (cnt == p.m // p.output_bs).all()


# ---------------------------------------------------------------- the clamped reading of broken device data

@pytest.mark.parametrize("gl,glt,m,want", [
    ([3, 2, 7], 0, 5, [3, 3, 5]),          # decreasing entry kept at the running maximum; past m clamped
    ([-4, 2, 1, 9], 0, 6, [0, 2, 2, 6]),   # negative entry read as 0
    ([3, 4, 2], 1, 5, [3, 5, 5]),          # counts past m: the running sum stops at m
    ([-2, 2, 1], 1, 10, [0, 2, 3]),        # negative count read as 0
    ([2, 5, 5, 9], 0, 9, [2, 5, 5, 9]),    # a list that keeps the rule is read plainly
    ([2, 3, 0, 4], 1, 9, [2, 5, 5, 9]),
])
def test_clamped_group_ends_hand_derived(gl, glt, m, want):
    """Ends under the library's reading of a broken groupList (entries clamped
    to [0, m]; running maximum for type 0, running sum capped at m for type
    1), against values worked out by hand."""
    assert oracle.clamped_ends(np.array(gl, dtype=np.int64), glt, m).tolist() == want


def test_clamped_problem_of_a_valid_problem_is_the_problem():
    p = W.random_problem(31, 120, 64, 48, 4, output_bs=40, bsdp=10, shared_offset=5, group_list_type=1)
    q, rows = oracle.clamped_problem(p)
    ref, _ = oracle.run(p)
    got, _ = oracle.run(q)
    assert rows == p.output_bs
    assert np.array_equal(got[:rows], ref)
    assert not got[rows:].any()


def test_clamped_problem_drops_rows_sent_outside_the_output():
    """Rows whose rowIndex lies outside [0, outputBS) contribute nothing: the
    clamped problem equals the same problem with those rows sent to row 0
    with a zero routing weight (their products are then +-0)."""
    p = W.random_problem(32, 150, 64, 32, 3, output_bs=30)
    bad = np.array([3, 77, 149])
    p.row_index[bad[:2]] = -1
    p.row_index[bad[2]] = p.output_bs
    q, rows = oracle.clamped_problem(p)
    got, _ = oracle.run(q)
    z = copy.deepcopy(p)
    z.row_index[bad] = 0
    z.logit[bad] = 0.0
    ref, _ = oracle.run(z)
    assert np.array_equal(got[:rows], ref)


def test_clamped_problem_reads_a_broken_group_list():
    """A type-0 list with a decreasing entry and an end past m equals the
    list of its clamped ends; rows past the last end contribute nothing."""
    p = W.random_problem(33, 100, 64, 32, 4, output_bs=25)
    p.group_list = np.array([40, 30, 70, 500], dtype=np.int64)
    q, rows = oracle.clamped_problem(p)
    assert q.group_list.tolist() == [40, 40, 70, 100]
    r = copy.deepcopy(p)
    r.group_list = np.array([40, 40, 70, 100], dtype=np.int64)
    ref, _ = oracle.run(r)
    got, _ = oracle.run(q)
    assert np.array_equal(got[:rows], ref)
    with pytest.raises(oracle.OracleError):
        oracle.run(p)  # the oracle itself keeps the rule strictly
