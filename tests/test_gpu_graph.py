"""The entry points in a captured graph (torch.cuda.CUDAGraph on the HIP
stream): forward, split-K forward + reduce, both backward settings and the
joint backward call are captured once and replayed several times, with eager
work and synchronisations in between; every replay must equal the eager
results bitwise (all of these kernels are deterministic, and the calls clear
nothing with memset and allocate nothing themselves)."""
import numpy as np
import pytest
import torch

from attention_kl_divergence_skl_amd import synth
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    w = synth.Workload("graph", 1, 2, 300, 420, 128, 128, "bf16", True, 1 / np.sqrt(128), 1 / np.sqrt(128),
                       synth.Recipe("corr", noise=0.4), "random", 77)
    say("[graph] capture forward, split-K, both backward settings, joint backward")
    _, t = to_device(w)
    q1, k1, q2, k2, g = t["q1"], t["k1"], t["q2"], t["k2"], t["g"]
    splits = 3
    ws_bytes = gpu_lib.skl_forward_splitk_workspace_size(q1, k1, q2, k2, splits)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    none = torch.empty(0, dtype=torch.float32, device="cuda")

    def run():
        kl, l1, l2 = gpu_lib.skl_forward(q1, k1, q2, k2, w.scale1, w.scale2, True)
        gpu_lib.skl_forward_splitk(q1, k1, q2, k2, w.scale1, w.scale2, True, splits, ws=ws)
        skl_kl, s1, s2 = gpu_lib.skl_reduce(ws, splits, w.B, w.H, w.NQ)
        dq2, dk2 = gpu_lib.skl_backward_student(q1, k1, q2, k2, l1, l2, g, w.scale1, w.scale2, True)
        dq1, dk1 = gpu_lib.skl_backward_teacher(q1, k1, q2, k2, l1, l2, kl, g, w.scale1, w.scale2, True)
        joint = gpu_lib.skl_backward_joint(q1, k1, q2, k2, l1, l2, kl, g, w.scale1, w.scale2, True, ws=none)
        return [kl, l1, l2, skl_kl, s1, s2, dq2, dk2, dq1, dk1, *joint]

    eager = [x.clone() for x in run()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    for rep in range(4):
        # unrelated eager work between replays, then the replay
        junk = torch.randn(1 << 20, device="cuda").mul_(3.0).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"
        del junk
