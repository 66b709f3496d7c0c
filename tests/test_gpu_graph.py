"""The entry points queue only kernel launches on the caller's stream (no allocation, no
synchronisation, no memset), so a HIP graph can capture them.  Each test captures one
call with torch.cuda.graph, replays it several times with eager work and host
synchronisations in between, and checks every replay against the eager call's bits."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import PATH_CHUNKED, PATH_FUSED, t

pytestmark = pytest.mark.gpu

D = 128
REPLAYS = 4


def _replay_and_check(graph, reset, outputs, expected):
    for r in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        # unrelated eager work between the replays
        junk = torch.randn(1 << 20, device=outputs[0].device)
        junk.mul_(2.0).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, expected):
            assert torch.equal(got, want), r


def test_decode_step_in_a_graph(device):
    case = ki.decode_case(340, 4, 6, 1, "graph-decode")
    H = case.H
    print(f"[graph] decode B={case.B} H={H}", flush=True)
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    x = case.step(0)
    xs = [t(getattr(x, n), device) for n in "qkvzbg"]
    s0, c0 = t(case.state, device), t(case.conv_state, device)
    state, conv = s0.clone(), c0.clone()
    out = torch.empty((case.B, H * D), dtype=torch.float32, device=device)
    kda.kda_decode_step(cfg, *xs, *prm, state, conv, out=out)
    torch.cuda.synchronize()
    expected = [out.clone(), state.clone(), conv.clone()]

    def reset():
        state.copy_(s0)
        conv.copy_(c0)
        out.fill_(float("nan"))

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            kda.kda_decode_step(cfg, *xs, *prm, state, conv, out=out, stream=s)
    _replay_and_check(g, reset, [out, state, conv], expected)


def test_decode_multi_in_a_graph(device):
    case = ki.decode_case(341, 3, 4, 4, "graph-multi")
    H, T = case.H, 4
    print(f"[graph] decode-multi B={case.B} H={H} T={T}", flush=True)
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    steps = [case.step(i) for i in range(T)]
    xs = [t(np.ascontiguousarray(np.stack([getattr(s_, n) for s_ in steps], axis=1)), device) for n in "qkvzbg"]
    s0, c0 = t(case.state, device), t(case.conv_state, device)
    so, co = torch.empty_like(s0), torch.empty_like(c0)
    nt = torch.tensor([4, 1, 3], dtype=torch.int32, device=device)
    # rows of tokens past a sequence's count are left as they were: a finite marker, so
    # that torch.equal can compare them
    out = torch.full((case.B, T, H * D), -7.0, dtype=torch.float32, device=device)
    kda.kda_decode_multi(cfg, *xs, *prm, s0, c0, state_out=so, conv_state_out=co, n_tokens=nt, out=out)
    torch.cuda.synchronize()
    expected = [out.clone(), so.clone(), co.clone()]
    assert (expected[0][1, 1:] == -7.0).all()

    def reset():
        out.fill_(-7.0)
        so.zero_()
        co.zero_()

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            kda.kda_decode_multi(cfg, *xs, *prm, s0, c0, state_out=so, conv_state_out=co, n_tokens=nt, out=out,
                                 stream=s)
    _replay_and_check(g, reset, [out, so, co], expected)


@pytest.mark.parametrize("path", [PATH_FUSED, PATH_CHUNKED], ids=["fused", "chunked"])
def test_prefill_in_a_graph(device, path):
    case = ki.prefill_case(342, 4, [70, 1, 200, 0, 129], True, "graph-prefill")
    H = case.H
    print(f"[graph] prefill path={path} H={H} lens={np.diff(case.cu_seqlens).tolist()}", flush=True)
    cfg = kda.KdaConfig(num_heads=H, prefill_path=path)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    xs = [t(getattr(case.x, n), device) for n in "qkvzbg"]
    cu = t(case.cu_seqlens, device)
    s0, c0 = t(case.initial_state, device), t(case.initial_conv_state, device)
    out = torch.empty((case.N, H * D), dtype=torch.float32, device=device)
    fs, fcs = torch.empty_like(s0), torch.empty_like(c0)
    wsb = kda.kda_prefill_workspace_bytes(cfg, case.B, case.N)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device) if wsb else None
    kda.kda_prefill(cfg, cu, *xs, *prm, s0, c0, out=out, final_state=fs, final_conv_state=fcs, workspace=ws)
    torch.cuda.synchronize()
    expected = [out.clone(), fs.clone(), fcs.clone()]

    def reset():
        out.fill_(float("nan"))
        fs.zero_()
        fcs.zero_()
        if ws is not None:
            ws.fill_(0xA5)  # the workspace's contents on entry are ignored

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            kda.kda_prefill(cfg, cu, *xs, *prm, s0, c0, out=out, final_state=fs, final_conv_state=fcs, workspace=ws,
                            stream=s)
    _replay_and_check(g, reset, [out, fs, fcs], expected)
