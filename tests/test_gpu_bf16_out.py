"""GPU tests of the bf16 output option (kda_config.out_dtype = KDA_OUT_BF16): every output
is the fp32 path's output rounded to the nearest bf16 (ties to even), bit for bit, and the
states and conv windows are the fp32 path's bits, for one-token decode, multi-token decode
and prefill on both layouts (the fp32 path itself is checked against the oracle
elsewhere)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import PATH_CHUNKED, PATH_FUSED, t

pytestmark = pytest.mark.gpu

D = 128


def _cfgs(H, **kw):
    return kda.KdaConfig(num_heads=H, **kw), kda.KdaConfig(num_heads=H, out_dtype=torch.bfloat16, **kw)


def _params(case, dev):
    p = case.params
    return [t(p.conv_w, dev), t(p.A_log, dev), t(p.dt_bias, dev), t(p.norm_w, dev)]


def test_decode_step(device):
    case = ki.decode_case(350, 5, 6, 2, "bf16-decode")
    print(f"[bf16-out] decode B={case.B} H={case.H}", flush=True)
    c32, c16 = _cfgs(case.H)
    prm = _params(case, device)
    s32, cv32 = t(case.state, device), t(case.conv_state, device)
    s16, cv16 = s32.clone(), cv32.clone()
    for i in range(2):
        xs = [t(getattr(case.step(i), n), device) for n in "qkvzbg"]
        o32 = kda.kda_decode_step(c32, *xs, *prm, s32, cv32)
        o16 = kda.kda_decode_step(c16, *xs, *prm, s16, cv16)
        torch.cuda.synchronize()
        assert o16.dtype == torch.bfloat16
        assert torch.equal(o16, o32.to(torch.bfloat16)), i
        assert torch.equal(s16, s32) and torch.equal(cv16, cv32), i


def test_decode_multi(device):
    case = ki.decode_case(351, 3, 4, 4, "bf16-multi")
    T = 4
    print(f"[bf16-out] decode-multi B={case.B} H={case.H} T={T}", flush=True)
    c32, c16 = _cfgs(case.H)
    prm = _params(case, device)
    steps = [case.step(i) for i in range(T)]
    xs = [t(np.ascontiguousarray(np.stack([getattr(s_, n) for s_ in steps], axis=1)), device) for n in "qkvzbg"]
    nt = torch.tensor([4, 0, 2], dtype=torch.int32, device=device)
    s0, c0 = t(case.state, device), t(case.conv_state, device)
    so32, co32, so16, co16 = (torch.empty_like(x) for x in (s0, c0, s0, c0))
    o32 = torch.full((case.B, T, case.H * D), 5.0, dtype=torch.float32, device=device)
    o16 = torch.full((case.B, T, case.H * D), 5.0, dtype=torch.bfloat16, device=device)
    kda.kda_decode_multi(c32, *xs, *prm, s0, c0, state_out=so32, conv_state_out=co32, n_tokens=nt, out=o32)
    kda.kda_decode_multi(c16, *xs, *prm, s0, c0, state_out=so16, conv_state_out=co16, n_tokens=nt, out=o16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert (o16[1] == 5.0).all() and (o16[2, 2:] == 5.0).all()  # rows not applied: untouched
    assert torch.equal(so16, so32) and torch.equal(co16, co32)


@pytest.mark.parametrize("path", [PATH_FUSED, PATH_CHUNKED], ids=["fused", "chunked"])
def test_prefill(device, path):
    case = ki.prefill_case(352, 4, [130, 1, 64, 0, 77], True, "bf16-prefill")
    print(f"[bf16-out] prefill path={path} lens={np.diff(case.cu_seqlens).tolist()}", flush=True)
    c32, c16 = _cfgs(case.H, prefill_path=path)
    prm = _params(case, device)
    xs = [t(getattr(case.x, n), device) for n in "qkvzbg"]
    cu = t(case.cu_seqlens, device)
    s0, c0 = t(case.initial_state, device), t(case.initial_conv_state, device)
    o32, fs32, fc32 = kda.kda_prefill(c32, cu, *xs, *prm, s0, c0)
    o16, fs16, fc16 = kda.kda_prefill(c16, cu, *xs, *prm, s0, c0)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(fs16, fs32) and torch.equal(fc16, fc32)
