"""GPU tests of the library's contract beyond the arithmetic, through the C ABI.

* Device data that break the operator's rules ("aclnnGroupedMatmulFinalizeRouting
  WeightNzV2", common constraints: the groupList rule; rowIndex a destination
  row) are documented by the header as memory-safe, with the clamped reading:
  the kernels must touch nothing outside the buffers they are given, and the
  rows inside the contract must equal the oracle's evaluation of that reading.
  Every buffer is cut from a larger allocation whose guard rows on both sides
  hold a sentinel; the guards must come back unchanged.
* A call on a side stream with no workspace given: the binding's workspace
  must not be handed to other work while the kernels still run.
"""
import copy

import numpy as np
import pytest

import oracle
from quantized_moe_grouped_amd import binding as B
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

GUARD = 64          # guard rows on each side of x1, out and acc_out
GUARD_BYTES = 4096  # guard bytes on each side of the workspace


def _broken(p, kind):
    """Break the device-data contract of a valid problem."""
    q = copy.deepcopy(p)
    m = p.m
    if kind == "type0":
        # a decreasing entry, and ends past m
        q.group_list = np.array([m // 4, m // 8, m // 2, m + 1000] + [m + 7] * (p.e - 4), dtype=np.int64)
        q.group_list_type = 0
    else:
        # counts whose sum passes m, one negative count
        q.group_list = np.array([m // 2, -3, m // 2, m // 2] + [5] * (p.e - 4), dtype=np.int64)
        q.group_list_type = 1
    rng = np.random.default_rng(7)
    rows = rng.choice(m, size=12, replace=False)
    big = np.iinfo(q.row_index.dtype).max
    bad = [-1, p.output_bs, -5, p.output_bs + 3, big, -big] * 2
    q.row_index[rows] = np.array(bad, dtype=np.int64).astype(q.row_index.dtype)
    return q


def _run_guarded(p, d, *, deterministic, combine, tuning_config=None, want_acc=False):
    import torch
    x1_big = torch.full((p.m + 2 * GUARD, p.k), 127, dtype=torch.int8, device="cuda")
    x1_big[GUARD:GUARD + p.m] = d["x1"]
    x1 = x1_big[GUARD:GUARD + p.m]
    out_big = torch.full((p.output_bs + 2 * GUARD, p.n), -7.25, dtype=torch.float32, device="cuda")
    out = out_big[GUARD:GUARD + p.output_bs]
    acc_big = acc = None
    if want_acc:
        acc_big = torch.full((p.m + 2 * GUARD, p.n), -0x55555556, dtype=torch.int32, device="cuda")
        acc = acc_big[GUARD:GUARD + p.m]
    dd = dict(d)
    dd["x1"] = x1
    args, keep = B.make_args(x1, dd["x2"], dd["group_list"], out, scale=dd["scale"],
                             pertoken_scale=dd["pertoken_scale"], logit=dd["logit"], row_index=dd["row_index"],
                             shared_input=dd["shared_input"],
                             shared_input_offset=p.shared_input_offset if p.shared_input is not None else 0,
                             group_list_type=p.group_list_type, deterministic=deterministic, combine=combine,
                             acc_out=acc, tuning_config=tuning_config)
    need = B.workspace_size(args)
    ws_big = torch.full((need + 2 * GUARD_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = ws_big[GUARD_BYTES:GUARD_BYTES + need]
    B.run(args, ws)
    torch.cuda.synchronize()
    del keep
    # guards unchanged
    assert (x1_big[:GUARD] == 127).all() and (x1_big[GUARD + p.m:] == 127).all()
    og = torch.cat([out_big[:GUARD], out_big[GUARD + p.output_bs:]])
    assert (og == -7.25).all(), "a write landed outside out"
    wg = torch.cat([ws_big[:GUARD_BYTES], ws_big[GUARD_BYTES + need:]])
    assert (wg == 0xA5).all(), "a write landed outside the workspace"
    if want_acc:
        ag = torch.cat([acc_big[:GUARD], acc_big[GUARD + p.m:]])
        assert (ag == -0x55555556).all(), "a write landed outside acc_out"
    return out.cpu().numpy(), None if acc is None else acc.cpu().numpy()


CONTRACT_CASES = {
    "int8_cont": dict(seed=41, m=900, k=256, n=528, e=6, output_bs=300, bsdp=40, shared_offset=20),
    "int8_short_k": dict(seed=42, m=700, k=128, n=272, e=6, output_bs=200, row_index_dtype=np.int32),
    "int4_cont": dict(seed=43, m=800, k=320, n=544, e=5, int4=True, output_bs=250),
    "many_experts": dict(seed=44, m=1200, k=192, n=256, e=40, empty_frac=0.5, output_bs=400),
}


@pytest.mark.parametrize("kind", ["type0", "type1"])
@pytest.mark.parametrize("name", list(CONTRACT_CASES), ids=list(CONTRACT_CASES))
def test_broken_device_data_stay_in_bounds(name, kind):
    p = _broken(W.random_problem(**CONTRACT_CASES[name]), kind)
    q, rows = oracle.clamped_problem(p)
    ref, ref_acc = oracle.run(q)
    ref = ref[:rows]
    cov = G.covered_mask(q)
    d = G.to_device(p)
    for tc in (None, [0, 0, 8], [0, 64, 16]):
        out, acc = _run_guarded(p, d, deterministic=True, combine="auto", tuning_config=tc, want_acc=True)
        assert (acc[cov] == ref_acc[cov]).all(), f"acc differs (tuning {tc})"
        assert (acc[~cov] == -0x55555556).all(), "rows outside the clamped groups were written"
        G.assert_bitexact(out, ref)
        out, _ = _run_guarded(p, d, deterministic=True, combine="auto", tuning_config=tc)
        G.assert_bitexact(out, ref)
        out, _ = _run_guarded(p, d, deterministic=False, combine="atomic", tuning_config=tc)
        G.assert_close_atomic(out, ref)


def test_side_stream_call_keeps_its_workspace():
    """gmm_finalize_routing on a side stream allocates its workspace (the
    ordered combine's 64 MiB of per-row contributions) from that stream's
    pool: memory allocated and overwritten on the default stream right after
    the call, while the kernels still run, must not be that workspace."""
    import torch
    p = W.random_problem(45, 8192, 2048, 2048, 8, output_bs=1024)
    ref, _ = oracle.run(p, want_acc=False)
    d = G.to_device(p)
    side = torch.cuda.Stream()
    out = torch.full((p.output_bs, p.n), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        B.gmm_finalize_routing(d["x1"], d["x2"], d["group_list"], out, scale=d["scale"],
                               pertoken_scale=d["pertoken_scale"], logit=d["logit"], row_index=d["row_index"],
                               group_list_type=p.group_list_type, deterministic=True, stream=side)
        junk = torch.empty(p.m * p.n * 4 + (1 << 20), dtype=torch.uint8, device="cuda")
        junk.fill_(0xFF)
        torch.cuda.synchronize()
        G.assert_bitexact(out.cpu().numpy(), ref)
        del junk
