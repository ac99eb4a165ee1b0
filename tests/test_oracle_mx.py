"""MxA8W4 oracle pins (CPU): element decoding against the format definitions
and torch's own conversions, closed forms, block-scale locality, an
independent pure-Python evaluation, agreement with the int8 oracle on
integer-valued inputs, and the error bound against fp32 evaluations."""
import copy

import numpy as np
import pytest

import oracle
from oracle import mx as MX
from quantized_moe_grouped_amd import workloads as W


def test_fp8_e4m3_table_matches_torch():
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(MX.FP8_TABLE)
    assert (both_nan | (ref == MX.FP8_TABLE)).all()
    assert np.isnan(MX.FP8_TABLE).sum() == 2  # 0x7F and 0xFF
    assert MX.FP8_TABLE[0x7E] == 448.0 and MX.FP8_TABLE[0x01] == 2.0 ** -9


def test_fp4_e2m1_table_is_the_format_table():
    # OCP MX v1.0, FP4 E2M1 values
    assert MX.FP4_TABLE.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                                     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e8m0_table_matches_torch():
    import torch
    ref = torch.arange(255, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert (ref == MX.E8M0_TABLE[:255]).all()
    assert np.isnan(MX.E8M0_TABLE[255])


def test_fp4_unpack_low_nibble_first():
    codes = MX.unpack_fp4(np.array([[0x21, 0xF7]], dtype=np.uint8))
    assert codes.tolist() == [[1, 2, 7, 15]]


def test_closed_form_constant_inputs():
    p = W.mx_problem(1, 40, 128, 64, 2, bsdp=0, output_bs=40, with_row_index=False, with_logit=False)
    p.x1[:] = 0x3C      # 1.5
    p.x2[:] = 0x55      # 3.0 in both nibbles
    p.pertoken_scale[:] = 129
    p.scale[:] = 125
    out, _, acc = MX.run(p)
    s, e = MX.group_ranges(p)
    want = 128 * 1.5 * 3.0 * 2.0 ** (129 - 127) * 2.0 ** (125 - 127)
    assert (acc[: e[-1]] == want).all()
    assert (out[: e[-1]] == want).all()


def test_block_scale_acts_on_its_32_k_only():
    p = W.mx_problem(2, 24, 256, 40, 1, empty_frac=0.0, output_bs=24, with_row_index=False, with_logit=False)
    _, _, acc = MX.run(p)
    i, blk = 5, 3
    q = copy.deepcopy(p)
    q.pertoken_scale[i, blk // 2, blk % 2] += 1
    _, _, acc2 = MX.run(q)
    # the block's own partial sum, from the definitions, element by element
    part = np.zeros(p.n)
    for j in range(p.n):
        for kk in range(32 * blk, 32 * blk + 32):
            byte = int(p.x2[0, j, kk // 2])
            wc = byte & 0xF if kk % 2 == 0 else byte >> 4
            part[j] += (MX.fp8_e4m3_value(int(p.x1[i, kk])) * MX.e8m0_value(int(p.pertoken_scale[i, blk // 2, blk % 2]))
                        * MX.fp4_e2m1_value(wc) * MX.e8m0_value(int(p.scale[0, j, blk // 2, blk % 2])))
    assert np.allclose(acc2[i] - acc[i], part, rtol=1e-12, atol=1e-12)
    others = np.arange(p.m) != i
    assert (acc2[others] == acc[others]).all()


@pytest.mark.parametrize("seed", [3, 4])
def test_brute_force_matches_oracle(seed):
    p = W.mx_problem(seed, 9, 64, 6, 3, empty_frac=0.2, output_bs=5, bsdp=2, shared_offset=1)
    _, _, acc = MX.run(p)
    b = MX.brute(p)
    assert np.allclose(acc, b, rtol=1e-12, atol=0.0)


def _int_codes():
    fp8 = {v: c for c in range(256) if not np.isnan(MX.FP8_TABLE[c]) and (v := MX.FP8_TABLE[c]) == int(v)
           and abs(v) <= 16}
    fp4 = {v: c for c in range(16) if (v := MX.FP4_TABLE[c]) == int(v)}
    return fp8, fp4


def test_integer_inputs_agree_with_the_int8_oracle():
    """FP8/FP4 holding small integers with unit scales compute the integer
    GEMM: acc equals the int8 oracle's int32 accumulator exactly."""
    rng = np.random.default_rng(7)
    fp8, fp4 = _int_codes()
    v8 = np.array(sorted(fp8)), np.array([fp8[v] for v in sorted(fp8)], dtype=np.uint8)
    v4 = np.array(sorted(fp4)), np.array([fp4[v] for v in sorted(fp4)], dtype=np.uint8)
    p = W.mx_problem(8, 50, 128, 48, 3, output_bs=30)
    a_idx = rng.integers(0, len(v8[0]), size=(p.m, p.k))
    w_idx = rng.integers(0, len(v4[0]), size=(p.e, p.n, p.k))
    p.x1 = v8[1][a_idx]
    wcodes = v4[1][w_idx]
    p.x2 = (wcodes[..., 0::2] | (wcodes[..., 1::2] << 4)).astype(np.uint8)
    p.pertoken_scale[:] = 127
    p.scale[:] = 127
    _, _, acc = MX.run(p)
    q = W.Problem("int", p.m, p.k, p.n, p.e, v8[0][a_idx].astype(np.int8),
                  np.ascontiguousarray(np.transpose(v4[0][w_idx], (0, 2, 1))).astype(np.int8), False, None, False,
                  None, None, p.group_list, p.group_list_type, p.row_index, None, 0, p.output_bs, 0, p.counts)
    _, iacc = oracle.run(q)
    s, e = MX.group_ranges(p)
    cov = np.zeros(p.m, dtype=bool)
    for a, b in zip(s, e):
        cov[a:b] = True
    assert (acc[cov] == iacc[cov].astype(np.float64)).all()


def test_bound_covers_fp32_evaluations():
    """fp32 accumulation in two orders (forward, and pairwise by blocks of 16),
    the rounded logit product and the fp32 ordered combine all stay within
    the bound."""
    p = W.mx_problem(9, 60, 256, 32, 2, output_bs=20, bsdp=6, shared_offset=3)
    out, bound, _ = MX.run(p)
    s, e = MX.group_ranges(p)
    ri = np.asarray(p.row_index)
    for order in ("forward", "blocks"):
        y = np.zeros((p.m, p.n), dtype=np.float32)
        for g in range(p.e):
            rows = np.arange(s[g], e[g])
            if rows.size == 0:
                continue
            a = MX._scaled_rows(p, rows).astype(np.float32)   # exact in fp32
            w = MX._scaled_weights(p, g).astype(np.float32)
            prod = a[:, None, :] * w[None, :, :]              # exact products
            if order == "forward":
                acc = np.zeros(prod.shape[:2], dtype=np.float32)
                for kk in range(p.k):
                    acc = (acc + prod[:, :, kk]).astype(np.float32)
            else:
                parts = prod.reshape(prod.shape[0], prod.shape[1], -1, 16).sum(axis=3, dtype=np.float32)
                acc = parts.sum(axis=2, dtype=np.float32)
            y[rows] = (acc * np.asarray(p.logit)[rows, None]).astype(np.float32)
        got = np.zeros((p.output_bs, p.n), dtype=np.float32)
        for d in range(p.output_bs):
            got[d] = MX._seed_row(p, d).astype(np.float32)
        for i in range(int(e[-1])):
            got[ri[i]] = (got[ri[i]] + y[i]).astype(np.float32)
        assert (np.abs(got.astype(np.float64) - out) <= bound).all(), order
    # not vacuous: well below the output's scale
    assert bound.max() <= 0.05 * np.abs(out).max()


def test_sampled_rows_match_whole_output():
    p = W.mx_problem(10, 80, 128, 32, 3, output_bs=25, bsdp=5, shared_offset=20)
    out, bound, _ = MX.run(p)
    d = np.array([0, 3, 21, 24])
    o, b = MX.out_rows(p, d)
    assert np.allclose(o, out[d], rtol=1e-13, atol=1e-13) and np.allclose(b, bound[d], rtol=1e-9)


def test_mx_config_shapes():
    p = W.make_mx_config("mxa8w4", 0)
    assert p.x1.shape == (131072, 2048) and p.x2.shape == (32, 7168, 1024)
    assert p.pertoken_scale.shape == (131072, 32, 2) and p.scale.shape == (32, 7168, 32, 2)
    assert int(p.counts.sum()) == 131072 and p.mx and p.x2_transposed


def _block_truncated_acc(p, rows, g, keep_bits):
    """The matrix core's in-block arithmetic as modelled by the bound: in each
    32-k block every product is truncated toward zero on the grid 2^(e - keep_bits),
    e the exponent of the block's largest |product|; block sums added in fp32."""
    a = MX._scaled_rows(p, rows)
    w = MX._scaled_weights(p, g)
    prod = a[:, None, :] * w[None, :, :]
    blk = prod.reshape(prod.shape[0], prod.shape[1], -1, 32)
    big = np.abs(blk).max(axis=3, keepdims=True)
    e = np.floor(np.log2(np.where(big > 0, big, 1.0)))
    grid = np.exp2(e - keep_bits)
    sums = (np.trunc(blk / grid) * grid).sum(axis=3)
    acc = np.zeros(sums.shape[:2], dtype=np.float32)
    for b in range(sums.shape[2]):
        acc = (acc + sums[:, :, b].astype(np.float32)).astype(np.float32)
    return acc


def test_bound_covers_the_block_alignment_model():
    """Products truncated 13 bits below their block's largest (what the matrix
    core was measured to do) and 12 bits (the bound's margin) stay inside it."""
    p = W.mx_problem(11, 70, 512, 40, 2, output_bs=70, with_row_index=False)
    out, bound, acc = MX.run(p)
    s, e = MX.group_ranges(p)
    L = np.asarray(p.logit, dtype=np.float64)
    for keep in (13, 12):
        for g in range(p.e):
            rows = np.arange(s[g], e[g])
            if rows.size == 0:
                continue
            y = (_block_truncated_acc(p, rows, g, keep) * L[rows, None].astype(np.float32)).astype(np.float64)
            assert (np.abs(y - out[rows]) <= bound[rows]).all(), keep


# ---------------------------------------------------------------- FP8 mode (x1 and x2 FP8 E4M3)

@pytest.mark.parametrize("seed", [21, 22])
def test_fp8_brute_force_matches_oracle(seed):
    p = W.fp8_problem(seed, 9, 64, 6, 3, empty_frac=0.2, output_bs=5, bsdp=2, shared_offset=1)
    _, _, acc = MX.run(p)
    assert np.allclose(acc, MX.brute(p), rtol=1e-12, atol=0.0)


def test_fp8_integer_inputs_agree_with_the_int8_oracle():
    """Integer-valued FP8 activations and weights compute the integer GEMM:
    acc equals the int8 oracle's int32 accumulator, and y (= the output with
    identity routing) agrees with the int8 oracle's fp32 epilogue to within
    its three roundings."""
    rng = np.random.default_rng(23)
    fp8, _ = _int_codes()
    vals = np.array(sorted(fp8))
    codes = np.array([fp8[v] for v in sorted(fp8)], dtype=np.uint8)
    p = W.fp8_problem(24, 60, 128, 40, 3, output_bs=60, with_row_index=False, scale_bf16=True)
    a_idx = rng.integers(0, len(vals), size=(p.m, p.k))
    w_idx = rng.integers(0, len(vals), size=(p.e, p.n, p.k))
    p.x1, p.x2 = codes[a_idx], codes[w_idx]
    out, _, acc = MX.run(p)
    q = W.Problem("int", p.m, p.k, p.n, p.e, vals[a_idx].astype(np.int8),
                  np.ascontiguousarray(np.transpose(vals[w_idx], (0, 2, 1))).astype(np.int8), False, p.scale, True,
                  p.pertoken_scale, p.logit, p.group_list, p.group_list_type, None, None, 0, p.output_bs, 0, p.counts)
    iout, iacc = oracle.run(q)
    s, e = MX.group_ranges(p)
    cov = np.zeros(p.m, dtype=bool)
    for a, b in zip(s, e):
        cov[a:b] = True
    assert (acc[cov] == iacc[cov].astype(np.float64)).all()
    rel = np.abs(iout[cov].astype(np.float64) - out[cov]) / np.maximum(np.abs(out[cov]), 1e-30)
    assert rel.max() <= 4 * 2.0 ** -24


def test_fp8_bound_covers_fp32_evaluation():
    p = W.fp8_problem(25, 50, 256, 24, 2, output_bs=18, bsdp=4, shared_offset=2)
    out, bound, _ = MX.run(p)
    s, e = MX.group_ranges(p)
    ri = np.asarray(p.row_index)
    y = np.zeros((p.m, p.n), dtype=np.float32)
    for g in range(p.e):
        rows = np.arange(s[g], e[g])
        if rows.size == 0:
            continue
        acc = _block_truncated_acc(p, rows, g, 13)
        S = np.asarray(p.scale, dtype=np.float32)[g, 0]
        v = (acc * S[None, :]).astype(np.float32)
        v = (v * np.asarray(p.pertoken_scale, dtype=np.float32)[rows, None]).astype(np.float32)
        y[rows] = (v * np.asarray(p.logit, dtype=np.float32)[rows, None]).astype(np.float32)
    got = np.stack([MX._seed_row(p, d) for d in range(p.output_bs)]).astype(np.float32)
    for i in range(int(e[-1])):
        got[ri[i]] = (got[ri[i]] + y[i]).astype(np.float32)
    assert (np.abs(got.astype(np.float64) - out) <= bound).all()
    assert bound.max() <= 0.05 * np.abs(out).max()


def test_fp8_per_tensor_scale_is_every_rows_scale():
    """A pertokenScale of shape (1) (static pertensor-perchannel) is the same as
    a per-token array holding that value in every entry, and a power of two
    2**s scales every row's output by 2**s exactly (no seed)."""
    p = W.fp8_problem(26, 40, 64, 16, 2, output_bs=25, bsdp=0)
    v = float(p.pertoken_scale[5])
    q = W.with_per_tensor_scale(p, v)
    r = copy.deepcopy(p)
    r.pertoken_scale = np.full(p.m, v, dtype=np.float32)
    oq, bq, _ = MX.run(q)
    orr, br, _ = MX.run(r)
    assert np.array_equal(oq, orr) and np.array_equal(bq, br)
    none = copy.deepcopy(p)
    none.pertoken_scale = None
    on, _, _ = MX.run(none)
    o8, _, _ = MX.run(W.with_per_tensor_scale(p, 8.0))
    assert np.array_equal(o8, on * 8.0)


def test_fp8_untransposed_weights_equal_transposed():
    """FP8 weights given (e,k,n) instead of (e,n,k) ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2",
    full-quant notes: x2 transposed or not) compute the same result; the brute
    force indexes the (e,k,n) array directly; reading the bytes with the other
    layout changes the result."""
    p = W.fp8_problem(27, 30, 64, 32, 3, output_bs=20, bsdp=3, shared_offset=2)
    q = W.with_untransposed_fp8_weights(p)
    assert q.x2.shape == (p.e, p.k, p.n) and not q.x2_transposed
    op, bp, ap = MX.run(p)
    oq, bq, aq = MX.run(q)
    assert np.array_equal(op, oq) and np.array_equal(bp, bq) and np.array_equal(ap, aq)
    small = W.with_untransposed_fp8_weights(W.fp8_problem(28, 7, 64, 6, 2, output_bs=4))
    _, _, acc = MX.run(small)
    assert np.allclose(acc, MX.brute(small), rtol=1e-12, atol=0.0)
    wrong = copy.deepcopy(q)
    wrong.x2_transposed = True
    wrong.x2 = np.ascontiguousarray(q.x2.reshape(p.e, p.n, p.k))  # (e,k,n) bytes read as (e,n,k)
    assert not np.array_equal(MX.run(wrong)[0], op)


# ---------------------------------------------------------------- k % 64 == 32 ("aclnnGroupedMatmulFinalize
# RoutingWeightNzV2", Atlas 350 MxA8W4 notes: k % 32 == 0, scales of shape (.., ceil(k/64), 2))

@pytest.mark.parametrize("k", [32, 96, 160])
def test_half_pair_k_brute_force_matches_oracle(k):
    """k a multiple of 32 but not of 64: the pure-Python brute force (which
    indexes scale byte b of block b directly) agrees with the oracle."""
    p = W.mx_problem(40 + k, 7, k, 32, 2, output_bs=5)
    assert p.pertoken_scale.shape == (7, (k + 63) // 64, 2)
    out, bound, acc = MX.run(p)
    cov = np.zeros(p.m, dtype=bool)
    s, e = MX.group_ranges(p)
    for a, b in zip(s, e):
        cov[a:b] = True
    assert np.allclose(acc[cov], MX.brute(p)[cov], rtol=1e-12, atol=0.0)


def test_half_pair_scale_byte_is_not_read():
    """With k % 64 == 32 the second byte of each row's (and column's) last
    scale pair stands for no block: changing it (to 0, or 255, the NaN code)
    leaves every output as it was."""
    p = W.mx_problem(50, 40, 96, 64, 3, output_bs=20, bsdp=5, shared_offset=3)
    ref, _, _ = MX.run(p)
    for v in (0, 255, 131):
        q = copy.deepcopy(p)
        q.pertoken_scale[:, -1, 1] = v
        q.scale[:, :, -1, 1] = v
        got, _, _ = MX.run(q)
        assert np.array_equal(got, ref)


def test_half_pair_equals_zero_padded_k():
    """A k = 96 problem equals the k = 128 problem whose k 96..127 hold zero
    activations and weights (any scales there): the closed form of the
    shortened sum."""
    p = W.mx_problem(51, 30, 96, 64, 2, output_bs=12)
    q = copy.deepcopy(p)
    q.k = 128
    q.x1 = np.zeros((p.m, 128), dtype=np.uint8)
    q.x1[:, :96] = p.x1
    q.x2 = np.zeros((p.e, p.n, 64), dtype=np.uint8)
    q.x2[:, :, :48] = p.x2
    pts = np.full((p.m, 4), 140, dtype=np.uint8)          # blocks 0..3; block 3 covers k 96..127
    pts[:, :3] = p.pertoken_scale.reshape(p.m, 4)[:, :3]
    q.pertoken_scale = pts.reshape(p.m, 2, 2)
    sc = np.full((p.e, p.n, 4), 121, dtype=np.uint8)
    sc[:, :, :3] = p.scale.reshape(p.e, p.n, 4)[:, :, :3]
    q.scale = sc.reshape(p.e, p.n, 2, 2)
    a, _, _ = MX.run(p)
    b, _, _ = MX.run(q)
    assert np.array_equal(a, b)
