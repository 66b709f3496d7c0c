"""q, k and v as row-strided views of one fused [tokens, 3*H*D] projection output (the
qkv_row_stride argument of every entry point): decode, multi-token decode, pooled decode
and prefill (both layouts) give exactly the bits of the same call on dense copies, and
write nothing outside their outputs."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import PATH_CHUNKED, PATH_FUSED, t

pytestmark = pytest.mark.gpu

D = 128


def _fused(q, k, v, pad):
    """[rows, 3*H*D + pad] buffer holding q | k | v side by side (pad columns of junk), and
    the three strided views into it."""
    HD = q.shape[-1]
    lead = q.shape[:-1]
    buf = torch.full((*lead, 3 * HD + pad), 7.0, dtype=q.dtype, device=q.device)
    buf[..., :HD] = q
    buf[..., HD:2 * HD] = k
    buf[..., 2 * HD:3 * HD] = v
    return buf, buf[..., :HD], buf[..., HD:2 * HD], buf[..., 2 * HD:3 * HD]


@pytest.mark.parametrize("pad", [0, 8])
def test_decode_step_on_strided_views(device, pad):
    case = ki.decode_case(610, 5, 6, 2, "strided-decode")
    print(f"[strided] decode B={case.B} H={case.H} pad={pad}", flush=True)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    cfg = kda.KdaConfig(num_heads=case.H)
    res = []
    for strided in (False, True):
        st, cs = t(case.state, device), t(case.conv_state, device)
        outs = []
        for i in range(2):
            xs = [t(getattr(case.step(i), n), device) for n in "qkvzbg"]
            if strided:
                buf, xs[0], xs[1], xs[2] = _fused(xs[0], xs[1], xs[2], pad)
                before = buf.clone()
            outs.append(kda.kda_decode_step(cfg, *xs, *prm, st, cs))
            if strided:
                torch.cuda.synchronize()
                assert torch.equal(buf, before)  # read only
        torch.cuda.synchronize()
        res.append((outs, st, cs))
    (o0, s0, c0), (o1, s1, c1) = res
    for a, b in zip(o0, o1):
        assert torch.equal(a, b)
    assert torch.equal(s0, s1) and torch.equal(c0, c1)


def test_decode_multi_and_slots_on_strided_views(device):
    case = ki.decode_case(611, 4, 3, 5, "strided-multi")
    B, H, T = case.B, case.H, 5
    print(f"[strided] decode_multi B={B} H={H} T={T}", flush=True)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    cfg = kda.KdaConfig(num_heads=H)
    steps = [case.step(i) for i in range(T)]
    xs = [t(np.ascontiguousarray(np.stack([getattr(s, n) for s in steps], axis=1)), device) for n in "qkvzbg"]
    _, sq, sk, sv = _fused(xs[0], xs[1], xs[2], 16)
    nt = torch.tensor([5, 2, 0, 4], dtype=torch.int32, device=device)
    outs = []
    for qkv in (xs[:3], [sq, sk, sv]):
        st, cs = t(case.state, device), t(case.conv_state, device)
        o = kda.kda_decode_multi(cfg, *qkv, *xs[3:], *prm, st, cs, n_tokens=nt,
                                 out=torch.zeros((B, T, H * D), device=device))
        torch.cuda.synchronize()
        outs.append((o, st, cs))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    # pooled one-token decode: rows scattered over a pool of 7 entries
    slots = torch.tensor([6, 0, 3, 1], dtype=torch.int32, device=device)
    x0 = [t(getattr(case.step(0), n), device) for n in "qkvzbg"]
    _, q0, k0, v0 = _fused(x0[0], x0[1], x0[2], 0)
    pool = torch.randn((7, H, D, D), device=device)
    cpool = torch.randn((7, 3 * H * D, 3), device=device)
    res = []
    for qkv in (x0[:3], [q0, k0, v0]):
        sp, cp = pool.clone(), cpool.clone()
        o = kda.kda_decode_step_slots(cfg, slots, *qkv, *x0[3:], *prm, sp, cp)
        torch.cuda.synchronize()
        res.append((o, sp, cp))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("path", [pytest.param(PATH_FUSED, id="fused"), pytest.param(PATH_CHUNKED, id="chunked")])
def test_prefill_on_strided_views(device, path):
    case = ki.prefill_case(612, 3, [70, 0, 2, 200], True, "strided-prefill")
    print(f"[strided] prefill path={path} B={case.B} N={case.N} H={case.H}", flush=True)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    cfg = kda.KdaConfig(num_heads=case.H, prefill_path=path)
    cu = t(case.cu_seqlens.astype(np.int32), device)
    xs = [t(getattr(case.x, n), device) for n in "qkvzbg"]
    buf, sq, sk, sv = _fused(xs[0], xs[1], xs[2], 24)
    before = buf.clone()
    res = []
    for qkv in (xs[:3], [sq, sk, sv]):
        st, cs = t(case.initial_state, device), t(case.initial_conv_state, device)
        res.append(kda.kda_prefill(cfg, cu, *qkv, *xs[3:], *prm, st, cs))
        torch.cuda.synchronize()
    assert torch.equal(buf, before)
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
