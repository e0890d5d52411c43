"""The library's calls captured in a HIP graph: every replay equals the eager
result bit for bit. The kernels are deterministic and the library zeroes and
copies memory with kernels of its own (no memset or copy nodes), so a captured
forward, gated forward or run of decode steps must reproduce the eager run
exactly on every replay, with the program's own eager work between replays."""
import numpy as np
import pytest

from kernelized_linear_attention_phi_amd import inputs as gen
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kata():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_phi_amd as k
    k.lib()
    return k


def _ws(torch, nbytes):
    return torch.full((max(nbytes, 4) // 4,), float("nan"), device="cuda")


@pytest.mark.parametrize("dk,C", [(16, 64), (32, 128)])
def test_graph_replays_equal_eager(kata, dk, C):
    import torch
    B, H, T, dv = 2, 2, 1000, 64
    q, k, v = gen.gaussian_qkv(B, H, T, dk, dv, seed=2100 + dk, dtype="bf16")
    g = gen.log_decays(B, H, T, seed=2101, gmin=-0.1)
    qd, kd, vd, gd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g)
    D = kata.feature_dim(dk, "psd")
    N, steps = 64, 6
    q1, k1, v1 = gen.gaussian_qkv(1, steps, N, dk, dv, seed=2102, dtype="bf16")
    g1 = gen.log_decays(1, steps, N, seed=2103, gmin=-0.3)
    q1d, k1d, v1d, g1d = dev(q1[0], "bf16"), dev(k1[0], "bf16"), dev(v1[0], "bf16"), dev(g1[0])
    S1_0 = torch.rand((N, D, dv), device="cuda") * 0.01
    z1_0 = torch.rand((N, D), device="cuda") + 1.0

    ws_scan = _ws(torch, kata.chunked_fwd_workspace(B, H, T, dk, dv, C, 1, True, "psd", "scan"))
    ws_seq = _ws(torch, kata.chunked_fwd_workspace(B, H, T, dk, dv, C, 1, True, "psd", "sequential"))
    ws_dec = _ws(torch, kata.chunked_fwd_decay_workspace(B, H, T, dk, dv, C, 1, "scan"))

    def buffers():
        nan = float("nan")
        return {"o": torch.full_like(vd, nan), "o_seq": torch.full_like(vd, nan),
                "o_dec": torch.full_like(vd, nan),
                "S": torch.full((B, H, D, dv), nan, device="cuda"),
                "z": torch.full((B, H, D), nan, device="cuda"),
                "S_dec": torch.full((B, H, D, dv), nan, device="cuda"),
                "z_dec": torch.full((B, H, D), nan, device="cuda"),
                "o1": torch.full((steps, N, dv), nan, device="cuda").to(torch.bfloat16),
                "S1": S1_0.clone(), "z1": z1_0.clone()}

    def work(b):
        kata.chunked_fwd_into(qd, kd, vd, b["o"], C, True, ws_scan, S_out=b["S"], z_out=b["z"])
        kata.chunked_fwd_into(qd, kd, vd, b["o_seq"], C, True, ws_seq, prefix="sequential")
        kata.chunked_fwd_decay_into(qd, kd, vd, gd, b["o_dec"], C, ws_dec, S_out=b["S_dec"],
                                    z_out=b["z_dec"])
        for t in range(steps):
            kata.decode_step_decay(q1d[t], k1d[t], v1d[t], g1d[t], b["S1"], b["z1"], out=b["o1"][t])

    say(f"graph eager dk={dk} C={C}")
    eager = buffers()
    work(eager)
    torch.cuda.synchronize()
    for name, t in eager.items():
        assert torch.isfinite(t.float()).all(), f"eager {name} not finite"

    cap = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(cap)                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph replay {rep} dk={dk} C={C}")
        for name, t in cap.items():                # eager work between replays
            t.fill_(float("nan"))
        cap["S1"].copy_(S1_0)
        cap["z1"].copy_(z1_0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in eager:
            assert torch.equal(cap[name], eager[name]), f"replay {rep}: {name} differs from eager"
