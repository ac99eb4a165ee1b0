"""Pins of the activation-quantisation and routing-permute oracle (CPU):
exactly representable rows, round-half-to-even ties, zero rows, the rounding
bound, power-of-two scaling, a pure-Python permute, groupList types, and the
composition with the grouped matmul oracle against a float64 MoE layer."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import quant as Q
from quantized_moe_grouped_amd import workloads as W


def _rp(hidden_f32, ids, e, K, weights=None, offset=0, glt=1):
    hidden_f32 = np.asarray(hidden_f32, dtype=np.float32)
    T, k = hidden_f32.shape
    return W.RouteProblem("t", T, k, K, e, W.f32_to_bf16_bits(hidden_f32), np.asarray(ids, dtype=np.int64).reshape(T, K),
                          weights, offset, glt)


def test_exactly_representable_rows_round_trip():
    """x = s * q with s a power of two and max|q| = 127: amax = 127 s, so
    scale = s and inv = 1/s exactly, x * inv = q exactly, and the codes come
    back unchanged (|q| <= 127 fits bf16's 8-bit significand)."""
    rng = np.random.default_rng(1)
    T, k = 6, 96
    q = rng.integers(-127, 128, size=(T, k))
    q[np.arange(T), rng.integers(0, k, size=T)] = np.where(rng.integers(0, 2, size=T) == 1, 127, -127)
    s = np.exp2(rng.integers(-12, 6, size=(T, 1))).astype(np.float32)
    x = (q * s).astype(np.float32)
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)), x)
    got_q, got_s = Q.quantize(W.f32_to_bf16_bits(x))
    assert (got_q == q).all()
    assert np.array_equal(got_s, s[:, 0])


def test_ties_round_to_even():
    """Values exactly halfway between codes, (c + 1/2) * s with amax = 127 s,
    round to the even code (the reading: round to nearest even)."""
    s = np.float32(2.0 ** -5)
    halves = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 100.5, 125.5, -126.5], dtype=np.float32)
    x = np.concatenate([[127.0], halves, np.zeros(5)]).astype(np.float32)[None, :] * s
    q, scale = Q.quantize(W.f32_to_bf16_bits(x))
    assert scale[0] == s
    assert q[0, 1:11].tolist() == [0, 2, 2, 4, 0, -2, -2, 100, 126, -126]


def test_zero_row_has_zero_scale_and_codes():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 3] = -0.75
    q, scale = Q.quantize(W.f32_to_bf16_bits(x))
    assert scale[0] == 0.0 and (q[0] == 0).all()
    assert q[1, 3] == -127 and np.count_nonzero(q[1]) == 1


def test_rounding_error_bound_and_extremes():
    """Round to nearest: |x - q*scale| <= scale/2 up to the roundings of scale
    and of x*inv; an entry of largest magnitude maps to +-127."""
    rp = W.route_problem(3, 64, 256, 2, 4)
    q, scale = Q.quantize(rp.hidden)
    x = W.bf16_bits_to_f32(rp.hidden).astype(np.float64)
    err = np.abs(x - q.astype(np.float64) * scale[:, None].astype(np.float64))
    assert (err <= scale[:, None] * (0.5 + 2.0 ** -16)).all()
    amax_at = np.abs(x).argmax(axis=1)
    assert (np.abs(q[np.arange(64), amax_at]) == 127).all()
    assert (np.abs(q.astype(np.int64)) <= 127).all()


@pytest.mark.parametrize("p", [-7, 3])
def test_power_of_two_scaling(p):
    """Multiplying a token's values by 2^p (exact in bf16) multiplies its scale
    by 2^p and leaves its codes unchanged."""
    rp = W.route_problem(4, 16, 128, 2, 4)
    x = W.bf16_bits_to_f32(rp.hidden)
    q0, s0 = Q.quantize(rp.hidden)
    q1, s1 = Q.quantize(W.f32_to_bf16_bits(x * np.float32(2.0 ** p)))
    assert (q0 == q1).all() and np.array_equal(s1, s0 * np.float32(2.0 ** p))


def _brute_permute(ids, e, offset):
    """Pure Python: local entries sorted by (expert, entry index)."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    keys = sorted((g - offset, f) for f, g in enumerate(flat) if 0 <= g - offset < e)
    return [f for _, f in keys], [sum(1 for g, _ in keys if g == x) for x in range(e)]


@pytest.mark.parametrize("seed,T,K,e,offset,repeat", [
    (5, 40, 4, 6, 0, False), (6, 33, 2, 3, 2, False), (7, 17, 1, 1, 0, False),
    (8, 25, 3, 5, 0, True), (9, 50, 8, 16, 4, False), (10, 1, 2, 4, 0, False)])
def test_permute_matches_brute_force(seed, T, K, e, offset, repeat):
    rp = W.route_problem(seed, T, 64, K, e, expert_offset=offset, repeat_slots=repeat)
    order, counts = Q.permute(rp.expert_ids, e, offset)
    b_order, b_counts = _brute_permute(rp.expert_ids, e, offset)
    assert order.tolist() == b_order and counts.tolist() == b_counts
    r = Q.run(rp)
    rows = r["rows"]
    assert rows == sum(b_counts)
    t = [f // K for f in b_order]
    assert r["row_index"][:rows].tolist() == t
    assert r["logit"][:rows].tolist() == [float(rp.topk_weights.reshape(-1)[f]) for f in b_order]
    q, s = Q.quantize(rp.hidden)
    assert (r["x1"][:rows] == q[t]).all() and np.array_equal(r["pertoken_scale"][:rows], s[t])


def test_group_list_types_and_dropped_entries():
    ids = [[0, 3], [5, 1], [1, 1], [7, 2]]  # e = 4, offset 0: ids 5 and 7 belong to other ranks
    rp1 = _rp(np.ones((4, 32)), ids, 4, 2, glt=1)
    rp0 = _rp(np.ones((4, 32)), ids, 4, 2, glt=0)
    r1, r0 = Q.run(rp1), Q.run(rp0)
    assert r1["group_list"].tolist() == [1, 3, 1, 1]
    assert r0["group_list"].tolist() == [1, 4, 5, 6]
    assert r1["rows"] == 6
    assert r1["row_index"][:6].tolist() == [0, 1, 2, 2, 3, 0]  # expert 0: t0; expert 1: t1, t2, t2; 2: t3; 3: t0


def test_composition_with_the_grouped_matmul_is_the_moe_layer():
    """Quantise and permute, then the grouped matmul oracle with the combine by
    rowIndex: each token's output must be the float64 MoE layer
    sum_j w_tj * (q_t * scale_t) @ (W_g * S_g) up to fp32 roundings -- which
    holds only if x1, pertokenScale, logit and rowIndex stay aligned."""
    T, k, n, K, e = 24, 64, 32, 3, 5
    rp = W.route_problem(11, T, k, K, e)
    r = Q.run(rp)
    rng = np.random.default_rng(12)
    x2 = rng.integers(-127, 128, size=(e, k, n), dtype=np.int8)
    S = rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32)
    p = W.Problem("moe", T * K, k, n, e, r["x1"], x2, False, S, False, r["pertoken_scale"], r["logit"],
                  r["group_list"], 1, r["row_index"], None, 0, T, 0, r["group_list"])
    out, _ = oracle.run(p)
    q, s = Q.quantize(rp.hidden)
    ref = np.zeros((T, n))
    for t in range(T):
        for j in range(K):
            g = int(rp.expert_ids[t, j])
            ref[t] += float(rp.topk_weights[t, j]) * ((q[t].astype(np.float64) * float(s[t])) @ x2[g].astype(np.float64)) * S[g, 0].astype(np.float64)
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())
    # a misaligned rowIndex (rows shifted by one) breaks it
    bad = W.Problem("bad", T * K, k, n, e, r["x1"], x2, False, S, False, r["pertoken_scale"], r["logit"],
                    r["group_list"], 1, np.roll(r["row_index"], 1), None, 0, T, 0, r["group_list"])
    assert not np.allclose(oracle.run(bad)[0], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_dispatch_config_shapes():
    rp = W.make_route_config("dispatch", 0)
    assert (rp.T, rp.k, rp.K, rp.e) == (16384, 2048, 8, 32)
    _, counts = Q.permute(rp.expert_ids, rp.e)
    assert counts.sum() == 131072 and counts.min() > 3500 and counts.max() < 4700


# ---------------------------------------------------------------- FP8 outputs (per token; MX per 32 k)

def test_e4m3_encoder_matches_torch_and_rounds_ties_to_even():
    """The encoder against torch's float8_e4m3fn conversion (a library
    routine) on fp32 values over the whole range, and on values exactly
    half-way between codes (ties go to the even code)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    v = np.concatenate([np.linspace(-448, 448, 20001),
                        rng.uniform(-1, 1, 20000) * np.exp2(rng.integers(-12, 9, 20000))]).astype(np.float32)
    v = np.clip(v, -448, 448)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (Q.e4m3_encode(v) == want).all()
    # 84 lies half-way between 80 (mantissa 010) and 88 (011): the even one;
    # 2^-9 * 1.5 half-way between the subnormals 1 and 2 (x 2^-9): code 2
    assert Q.e4m3_encode(np.array([84.0, 92.0, -84.0, 1.5 * 2.0 ** -9], np.float32)).tolist() == \
        [0x6A, 0x6C, 0xEA, 0x02]


def _decode(codes):
    from oracle.mx import FP8_TABLE
    return FP8_TABLE[np.asarray(codes)]


def test_fp8_per_token_exact_rows_and_bound():
    """x = s * v with v on the E4M3 grid and max|v| = 448: amax = 448 s, so
    scale = s, inv = 1/s (s a power of two) and the codes decode to v exactly;
    random rows decode within half an E4M3 step (relative 2^-4) of x/scale."""
    rng = np.random.default_rng(42)
    from oracle.mx import FP8_TABLE
    grid = FP8_TABLE[np.arange(0, 0x7F)]
    v = rng.choice(grid, size=(5, 64)) * rng.choice([-1.0, 1.0], size=(5, 64))
    v[:, 7] = 448.0
    s = np.exp2(rng.integers(-10, 4, size=(5, 1)))
    x = (v * s).astype(np.float32)
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)), x)
    codes, scale = Q.quantize_fp8(W.f32_to_bf16_bits(x))
    assert np.array_equal(scale, s[:, 0].astype(np.float32))
    assert np.array_equal(_decode(codes), v)
    rp = W.route_problem(43, 40, 256, 2, 3)
    codes, scale = Q.quantize_fp8(rp.hidden)
    xr = W.bf16_bits_to_f32(rp.hidden).astype(np.float64)
    dq = _decode(codes) * scale[:, None]
    assert (np.abs(dq - xr) <= np.abs(xr) * 2.0 ** -4 + scale[:, None] * 2.0 ** -9 * 1.01).all()


def test_mx_block_scales_follow_the_block_maximum():
    """Each 32-value block gets E8M0 code floor(log2(amax)) - 8 + 127: a block
    whose largest magnitude is 2^e * 1.x gets code e + 119; values scaled by
    2^p shift the code by p; an all-zero block gets code 0 and zero elements;
    values in [448, 512) after scaling saturate to 448; blocks are independent."""
    x = np.zeros((2, 96), np.float32)
    x[0, :32] = np.linspace(-3.0, 3.0, 32)        # amax 3 = 1.5 * 2^1 -> code 120
    x[0, 32:64] = 0.0                              # zero block -> code 0
    x[0, 64:96] = 2.0 ** -20                       # amax 2^-20 -> code 99
    x[1, :32] = 1.96875 * 2.0 ** 5                 # amax 63 -> 63 / 2^-3 = 504 -> saturates to 448
    x[1, 32:64] = np.linspace(0.0, 1.0, 32) * 2.0 ** 7
    x[1, 64:96] = -(2.0 ** 100)
    codes, sc = Q.quantize_mx(W.f32_to_bf16_bits(x))
    assert sc.tolist() == [[120, 0, 99], [124, 126, 219]]
    assert (codes[0, 32:64] == 0).all()
    assert (_decode(codes[1, :32]) == 448.0).all()
    assert (codes[1, 64:96] == Q.e4m3_encode(np.float32(-256.0))).all()
    two = Q.quantize_mx(W.f32_to_bf16_bits(x * np.float32(2.0 ** 3)))
    assert (two[0] == codes).all() and (two[1][sc > 0] == sc[sc > 0] + 3).all()


def test_fp8_modes_permute_like_int8():
    """The FP8 and MX modes route rows exactly as the int8 mode; only x1 and
    pertokenScale change, to the per-token codes and scales."""
    rp = W.route_problem(44, 50, 128, 4, 5, expert_offset=1, n_gate=7)
    r8 = Q.run(rp)
    for mode, qf in (("fp8", Q.quantize_fp8), ("mx", Q.quantize_mx)):
        rp.mode = mode
        r = Q.run(rp)
        rows = r["rows"]
        assert rows == r8["rows"] and (r["row_index"] == r8["row_index"]).all()
        assert (r["group_list"] == r8["group_list"]).all() and np.array_equal(r["logit"], r8["logit"])
        q, s = qf(rp.hidden)
        t = r["row_index"][:rows]
        assert (r["x1"][:rows] == q[t]).all() and np.array_equal(r["pertoken_scale"][:rows], s[t])
    rp.mode = "int8"


def test_mx_composition_with_the_mx_matmul_oracle():
    """MX producer -> MxA8W4 grouped-matmul oracle (FP4 weights) equals the
    float64 layer built from the decoded codes and block scales."""
    from oracle import mx as MX
    T, k, n, K, e = 20, 128, 32, 2, 3
    rp = W.route_problem(45, T, k, K, e, group_list_type=0)
    rp.mode = "mx"
    r = Q.run(rp)
    m = T * K
    base = W.mx_problem(46, m, k, n, e, output_bs=T)
    p = dataclasses.replace(base, x1=r["x1"], pertoken_scale=r["pertoken_scale"].reshape(m, k // 64, 2),
                            logit=r["logit"], group_list=r["group_list"], group_list_type=0,
                            row_index=r["row_index"], shared_input=None, counts=np.diff(np.r_[0, r["group_list"]]))
    out, bound, _ = MX.run(p)
    a = _decode(r["x1"]).reshape(m, k // 32, 32) * MX.E8M0_TABLE[r["pertoken_scale"]][:, :, None]
    ref = np.zeros((T, n))
    ends = r["group_list"]
    for g in range(e):
        s0 = 0 if g == 0 else ends[g - 1]
        wg = MX._scaled_weights(p, g)  # (n, k) with its block scales
        for i in range(s0, ends[g]):
            ref[r["row_index"][i]] += r["logit"][i] * (a[i].reshape(k) @ wg.T)
    assert (np.abs(out - ref) <= bound + 1e-12).all()
