"""The library under HIP graph capture: a call captured once (through
torch.cuda.graph, on the capture stream) and replayed several times, with
eager work and synchronisations between replays, gives the eager result on
every replay -- bit-exact in the ordered combine, within the unordered
tolerance with atomics.  No hipMemsetAsync is recorded (the buffers that
must start at zero are cleared by the library's own kernels)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant as Q
from quantized_moe_grouped_amd import binding as B
from quantized_moe_grouped_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["ordered", "atomic"])
def test_captured_call_replays_match_eager(mode):
    p = W.random_problem(31, 900, 256, 528, 4, row_index_dtype=np.int32, scale_bf16=True, output_bs=450,
                         bsdp=100, shared_offset=350)
    ref, _ = oracle.run(p)
    d = G.to_device(p)
    det = mode == "ordered"
    out = torch.full((p.output_bs, p.n), float("nan"), dtype=torch.float32, device="cuda")
    args, keep = B.make_args(d["x1"], d["x2"], d["group_list"], out, scale=d["scale"],
                             pertoken_scale=d["pertoken_scale"], logit=d["logit"], row_index=d["row_index"],
                             shared_input=d["shared_input"], shared_input_offset=p.shared_input_offset,
                             group_list_type=p.group_list_type, deterministic=det,
                             combine="auto" if det else "atomic")
    ws = torch.empty(max(B.workspace_size(args), 1), dtype=torch.uint8, device="cuda")
    B.run(args, ws)  # eager first (also loads the kernels)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.run(args, ws)
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0x5A)  # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        if det:
            G.assert_bitexact(got, eager)
            G.assert_bitexact(got, ref)
        else:
            G.assert_close_atomic(got, ref)
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work between replays
    del keep


def test_captured_producer_and_matmul_replay():
    """The producer step and the grouped matmul captured together."""
    T, k, n, K, e = 300, 256, 272, 4, 6
    rp = W.route_problem(32, T, k, K, e)
    ref = Q.run(rp)
    rng = np.random.default_rng(33)
    x2 = rng.integers(-127, 128, size=(e, k, n), dtype=np.int8)
    S = rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32)
    p = W.Problem("moe", T * K, k, n, e, ref["x1"], x2, False, S, False, ref["pertoken_scale"], ref["logit"],
                  ref["group_list"], 1, ref["row_index"], None, 0, T, 0, ref["group_list"])
    want, _ = oracle.run(p)
    dev = torch.device("cuda:0")
    hidden = torch.from_numpy(rp.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(rp.expert_ids).to(dev)
    w = torch.from_numpy(rp.topk_weights).to(dev)
    m = T * K
    x1 = torch.empty((m, k), dtype=torch.int8, device=dev)
    pts = torch.empty(m, dtype=torch.float32, device=dev)
    lg = torch.empty(m, dtype=torch.float32, device=dev)
    ri = torch.empty(m, dtype=torch.int64, device=dev)
    gl = torch.empty(e, dtype=torch.int64, device=dev)
    qa, qk = B.make_qp_args(hidden, ids, x1, pts, ri, gl, topk_weights=w, logit=lg)
    qws = torch.empty(max(B.qp_workspace_size(qa), 1), dtype=torch.uint8, device=dev)
    out = torch.empty((T, n), dtype=torch.float32, device=dev)
    ga, gk = B.make_args(x1, torch.from_numpy(x2).to(dev), gl, out, scale=torch.from_numpy(S).to(dev),
                         pertoken_scale=pts, logit=lg, row_index=ri, group_list_type=1, deterministic=True)
    gws = torch.empty(max(B.workspace_size(ga), 1), dtype=torch.uint8, device=dev)
    import ctypes

    def step():
        st = B.lib().gmm_quant_permute(ctypes.byref(qa), ctypes.c_void_p(qws.data_ptr()),
                                       ctypes.c_size_t(qws.numel()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        B.run(ga, gws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        out.fill_(float("nan"))
        x1.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        G.assert_bitexact(out.cpu().numpy(), want)
    del qk, gk
