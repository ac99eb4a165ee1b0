"""The allocation-free entry point (gmm_finalize_routing_noalloc) against the
existing one (gmm_finalize_routing with a caller-allocated workspace), through
the C ABI: the ordered combine bit-identical, the unordered combine within
max|err| <= 1e-5 * max|ref|, on calls in a row of decreasing size that share
the library's scratch array.  Collected last: run alone in a fresh process or
after the other tests."""
import ctypes

import numpy as np
import pytest

from quantized_moe_grouped_amd import binding as B
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _args(p, d, out, combine, deterministic=False):
    return B.make_args(d["x1"], d["x2"], d["group_list"], out, scale=d["scale"],
                       pertoken_scale=d["pertoken_scale"], logit=d["logit"], row_index=d["row_index"],
                       shared_input=d["shared_input"],
                       shared_input_offset=p.shared_input_offset if p.shared_input is not None else 0,
                       group_list_type=p.group_list_type, combine=combine, deterministic=deterministic,
                       transpose_x2=getattr(p, "x2_transposed", False))


def _both(p, combine, deterministic=False):
    """Outputs of the existing entry point and of the allocation-free one."""
    import torch
    d = G.to_device(p)
    ref = torch.full((p.output_bs, p.n), float("nan"), dtype=torch.float32, device="cuda")
    args, keep = _args(p, d, ref, combine, deterministic)
    ws = torch.empty(max(B.workspace_size(args), 1), dtype=torch.uint8, device="cuda")
    assert B.workspace_size(args) <= B.NOALLOC_SCRATCH_BYTES
    B.run(args, ws)
    torch.cuda.synchronize()
    got = torch.full((p.output_bs, p.n), float("nan"), dtype=torch.float32, device="cuda")
    args2, keep2 = _args(p, d, got, combine, deterministic)
    before = torch.cuda.memory_allocated()
    stream = torch.cuda.current_stream().cuda_stream
    st = B.lib().gmm_finalize_routing_noalloc(ctypes.byref(args2), ctypes.c_void_p(stream))
    assert st == B.OK, B.STATUS_NAMES.get(st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() <= before  # nothing allocated (other tensors may be freed meanwhile)
    del keep, keep2, ws
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_the_allocating_entry_point_on_shrinking_calls():
    # 1: the decode workload, ordered combine (about 117 MB of scratch)
    p1 = W.make_config("decode", 0)
    ref, got = _both(p1, "ordered")
    G.assert_bitexact(got, ref)
    # 2: a smaller problem right after, ordered, with a shared block and bf16
    #    scales: stale contributions and buckets of call 1 must not leak in
    p2 = W.random_problem(61, 700, 256, 528, 5, output_bs=300, bsdp=40, shared_offset=20, scale_bf16=True)
    ref, got = _both(p2, "auto", deterministic=True)
    G.assert_bitexact(got, ref)
    # 3: smaller still, unordered (atomic) combine with int4 weights
    p3 = W.random_problem(62, 300, 192, 256, 3, int4=True, output_bs=100)
    ref, got = _both(p3, "atomic")
    G.assert_close_atomic(got, ref)
    # 4: the second problem again, after the atomic call
    ref, got = _both(p2, "ordered")
    G.assert_bitexact(got, ref)


def test_noalloc_rejects_an_ordered_plan_larger_than_its_scratch():
    import torch
    p = W.random_problem(63, 5000, 64, 7168, 2, output_bs=100)  # 5000 * 7168 * 4 > 128 MiB
    d = G.to_device(p)
    out = torch.zeros((p.output_bs, p.n), dtype=torch.float32, device="cuda")
    args, keep = _args(p, d, out, "ordered")
    with pytest.raises(B.GmmfrError) as ei:
        B.run_noalloc(args)
    assert ei.value.code == B.ERR_WORKSPACE
    # the same problem with the atomic combine fits (1 KiB of queue counters)
    args, keep = _args(p, d, out, "atomic")
    B.run_noalloc(args)
    torch.cuda.synchronize()
    del keep


def test_noalloc_replays_under_graph_capture():
    """The allocation-free entry point inside a captured HIP graph (the
    callers it exists for): each replay, with other work and a smaller eager
    call on the shared scratch between replays, equals the eager result of the
    allocating entry point -- bit-exact in the ordered combine.  The scratch
    array's address is looked up by an eager call before the capture."""
    import torch
    p = W.random_problem(64, 900, 256, 528, 4, output_bs=300, bsdp=40, shared_offset=30)
    q = W.random_problem(65, 200, 128, 272, 3, output_bs=90)
    ref, got = _both(p, "ordered")
    G.assert_bitexact(got, ref)
    d = G.to_device(p)
    out = torch.full((p.output_bs, p.n), float("nan"), dtype=torch.float32, device="cuda")
    args, keep = _args(p, d, out, "ordered")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.run_noalloc(args)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.run_noalloc(args)
    for it in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        G.assert_bitexact(out.cpu().numpy(), ref)
        qref, qgot = _both(q, "ordered")  # an eager call in between rewrites the scratch
        G.assert_bitexact(qgot, qref)
    del keep, graph
