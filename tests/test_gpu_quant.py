"""GPU parity of the producer step (dynamic per-token int8 quantisation and
routing permute) against its CPU oracle, through the C ABI: every output
bit-exact (codes, scales, logits and row indices are decided in the same
fp32 operations on both sides; rows past the covered count are undefined and
not compared).  Also the composition: the producer's outputs fed to the
grouped matmul on the device equal the two oracles chained."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant as Q
from quantized_moe_grouped_amd import binding as B
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = {
    "small": dict(seed=1, T=100, k=64, K=4, e=6),
    "ep_offset_i32": dict(seed=2, T=300, k=256, K=8, e=16, n_gate=64, expert_offset=16, ids_dtype=np.int32,
                          group_list_type=0),
    "zero_tokens_repeats": dict(seed=3, T=257, k=128, K=3, e=5, zero_tokens=4, repeat_slots=True),
    "single": dict(seed=4, T=1, k=16, K=1, e=1),
    "many_chunks": dict(seed=5, T=3000, k=2048, K=8, e=64),
    "ragged_k": dict(seed=6, T=77, k=1040, K=2, e=3, n_gate=7, expert_offset=2),
    "no_tokens": dict(seed=7, T=0, k=32, K=2, e=4),
    "k_4096": dict(seed=11, T=90, k=4096, K=2, e=4),         # rows held in registers, 4 steps
    "k_8208_reread": dict(seed=12, T=40, k=8208, K=3, e=5),  # rows longer than 4096: read twice
    "e_1024": dict(seed=13, T=200, k=32, K=8, e=1024),       # one thread per expert in the base kernel
}


def _host(v):
    if v is None:
        return None
    if v.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu):
        v = v.view(torch.uint8)
    return v.cpu().numpy()


def _run_gpu(rp, ri_dtype=torch.int64):
    dev = torch.device("cuda:0")
    hidden = torch.from_numpy(rp.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(np.ascontiguousarray(rp.expert_ids)).to(dev)
    w = None if rp.topk_weights is None else torch.from_numpy(rp.topk_weights).to(dev)
    out = B.quant_permute(hidden, ids, rp.e, topk_weights=w, expert_offset=rp.expert_offset,
                          group_list_type=rp.group_list_type, row_index_dtype=ri_dtype, mode=rp.mode)
    torch.cuda.synchronize()
    return {k: _host(v) for k, v in out.items() if k != "workspace"}


def _compare(rp, got, ref):
    rows = ref["rows"]
    assert (got["group_list"] == ref["group_list"]).all()
    assert (got["x1"][:rows] == ref["x1"][:rows]).all()
    if rp.mode == "mx":
        assert (got["pertoken_scale"].reshape(len(got["pertoken_scale"]), -1)[:rows] == ref["pertoken_scale"][:rows]).all()
    else:
        assert np.array_equal(got["pertoken_scale"][:rows].view(np.uint32),
                              ref["pertoken_scale"][:rows].view(np.uint32))
    assert (got["row_index"][:rows].astype(np.int64) == ref["row_index"][:rows]).all()
    if ref["logit"] is not None:
        assert np.array_equal(got["logit"][:rows].view(np.uint32), ref["logit"][:rows].view(np.uint32))


@pytest.mark.parametrize("name", list(CASES), ids=list(CASES))
def test_quant_permute_bitexact(name):
    rp = W.route_problem(**CASES[name])
    ref = Q.run(rp)
    _compare(rp, _run_gpu(rp), ref)
    if name in ("small", "ep_offset_i32"):
        _compare(rp, _run_gpu(rp, torch.int32), ref)


def test_quant_permute_without_weights():
    rp = W.route_problem(8, 50, 96, 2, 3)
    rp.topk_weights = None
    ref = Q.run(rp)
    got = _run_gpu(rp)
    assert got["logit"] is None
    _compare(rp, got, ref)


def test_dispatch_workload_bitexact():
    """The prefill workload's producer step at full size: 16384 tokens,
    k = 2048, top-8 of 32 experts; every output compared."""
    rp = W.make_route_config("dispatch", 0)
    ref = Q.run(rp)
    assert ref["rows"] == 131072
    _compare(rp, _run_gpu(rp), ref)


def test_composition_with_the_grouped_matmul():
    """Producer outputs fed to the grouped matmul on the device, ordered
    combine: bit-equal to the producer oracle chained into the matmul oracle."""
    T, k, n, K, e = 640, 256, 272, 4, 6
    rp = W.route_problem(9, T, k, K, e)
    ref = Q.run(rp)
    rng = np.random.default_rng(10)
    x2 = rng.integers(-127, 128, size=(e, k, n), dtype=np.int8)
    S = rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32)
    p = W.Problem("moe", T * K, k, n, e, ref["x1"], x2, False, S, False, ref["pertoken_scale"], ref["logit"],
                  ref["group_list"], 1, ref["row_index"], None, 0, T, 0, ref["group_list"])
    want, _ = oracle.run(p)
    dev = torch.device("cuda:0")
    hidden = torch.from_numpy(rp.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    qp = B.quant_permute(hidden, torch.from_numpy(rp.expert_ids).to(dev), e,
                         topk_weights=torch.from_numpy(rp.topk_weights).to(dev))
    out = torch.empty((T, n), dtype=torch.float32, device=dev)
    B.gmm_finalize_routing(qp["x1"], torch.from_numpy(x2).to(dev), qp["group_list"], out,
                           scale=torch.from_numpy(S).to(dev), pertoken_scale=qp["pertoken_scale"],
                           logit=qp["logit"], row_index=qp["row_index"], group_list_type=1, deterministic=True)
    torch.cuda.synchronize()
    G.assert_bitexact(out.cpu().numpy(), want)


# ---------------------------------------------------------------- FP8 outputs

FP8_CASES = ["small", "ep_offset_i32", "zero_tokens_repeats", "single", "many_chunks", "k_4096", "k_8208_reread"]


@pytest.mark.parametrize("mode", ["fp8", "mx"])
@pytest.mark.parametrize("name", FP8_CASES, ids=FP8_CASES)
def test_quant_permute_fp8_bitexact(name, mode):
    kw = dict(CASES[name])
    if mode == "mx" and kw["k"] % 64:
        kw["k"] = kw["k"] // 64 * 64 + 64
    rp = W.route_problem(**kw)
    rp.mode = mode
    _compare(rp, _run_gpu(rp), Q.run(rp))


@pytest.mark.parametrize("mode", ["fp8", "mx"])
def test_dispatch_workload_fp8_bitexact(mode):
    rp = W.make_route_config("dispatch", 0)
    rp.mode = mode
    _compare(rp, _run_gpu(rp), Q.run(rp))


def test_mx_producer_feeds_the_mx_matmul():
    """MX producer on the device feeding the MxA8W4 grouped matmul on the
    device: within the MxA8W4 oracle's bound of the oracles chained."""
    import dataclasses
    from oracle import mx as MX
    T, k, n, K, e = 200, 256, 288, 4, 5
    rp = W.route_problem(34, T, k, K, e, group_list_type=0)
    rp.mode = "mx"
    r = Q.run(rp)
    m = T * K
    base = W.mx_problem(35, m, k, n, e, output_bs=T)
    p = dataclasses.replace(base, x1=r["x1"], pertoken_scale=r["pertoken_scale"].reshape(m, k // 64, 2),
                            logit=r["logit"], group_list=r["group_list"], group_list_type=0,
                            row_index=r["row_index"], shared_input=None,
                            counts=np.diff(np.r_[0, r["group_list"]]))
    ref, bound, _ = MX.run(p)
    dev = torch.device("cuda:0")
    hidden = torch.from_numpy(rp.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    qp = B.quant_permute(hidden, torch.from_numpy(rp.expert_ids).to(dev), e,
                         topk_weights=torch.from_numpy(rp.topk_weights).to(dev), group_list_type=0, mode="mx")
    d = G.to_device(p)
    out = torch.empty((T, n), dtype=torch.float32, device=dev)
    B.gmm_finalize_routing(qp["x1"], d["x2"], qp["group_list"], out, scale=d["scale"],
                           pertoken_scale=qp["pertoken_scale"], logit=qp["logit"], row_index=qp["row_index"],
                           group_list_type=0, deterministic=True, transpose_x2=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= bound).all()


# ---------------------------------------------------------------- seeded sweep

N_SWEEP = 60


def _sweep_case(i):
    rng = np.random.default_rng(29000 + i)
    mode = ("int8", "int8", "fp8", "mx")[int(rng.integers(0, 4))]
    T = int(rng.choice([0, 1, 33, 500, 2000]))
    K = int(rng.integers(1, 9))
    e = int(rng.choice([1, 4, 32, 300, 1024]))
    off = int(rng.choice([0, 0, 8]))
    n_gate = e + off + int(rng.choice([0, 0, 5]))
    K = min(K, n_gate)
    k = (64 * int(rng.integers(1, 65))) if mode == "mx" else (16 * int(rng.integers(1, 260)))
    rp = W.route_problem(29000 + i, T, k, K, e, n_gate=n_gate, expert_offset=off,
                         ids_dtype=np.int32 if rng.random() < 0.4 else np.int64,
                         with_weights=bool(rng.random() < 0.8), group_list_type=int(rng.integers(0, 2)),
                         zero_tokens=int(rng.integers(0, 3)) if T else 0, repeat_slots=bool(rng.random() < 0.2))
    rp.mode = mode
    return rp, (torch.int32 if rng.random() < 0.3 else torch.int64)


@pytest.mark.parametrize("i", range(N_SWEEP))
def test_quant_permute_sweep(i):
    """Seeded draws of tokens, hidden size, top-K, expert count and offset
    (ids of other ranks), id and rowIndex types, weights or none, groupList
    type, zero tokens, repeated experts and the output encoding (int8, FP8,
    MX): every output bit-exact."""
    rp, ri_dtype = _sweep_case(i)
    got = _run_gpu(rp, ri_dtype)
    ref = Q.run(rp)
    if rp.topk_weights is None:
        assert got["logit"] is None
    _compare(rp, got, ref)
