"""GPU parity of kda_prefill_gate_proj (decay logits z = W_fb f formed inside the library
from f = W_fa x [N, 128] and W_fb [H*D, 128], bf16) against the fp64 oracle given the
same factors: outputs within 2e-2 abs, final states within 5e-3 relative, exact windows,
on both work layouts and in both operand precisions; the layouts agree bit for bit."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import (PATH_CHUNKED, PATH_FUSED, PRECISION_HIGH, PRECISION_STANDARD, PREFILL_OUT_ABS_TOL,
                          PREFILL_STATE_REL_TOL, oracle_cfg, slice_rel, t)

pytestmark = pytest.mark.gpu

D = 128
PATHS = [pytest.param(PATH_FUSED, id="fused"), pytest.param(PATH_CHUNKED, id="chunked")]
PRECS = [pytest.param(PRECISION_STANDARD, id="standard"), pytest.param(PRECISION_HIGH, id="high")]


def _gpu(case, f, w_fb, dev, path, precision):
    cfg = kda.KdaConfig(num_heads=case.H, prefill_path=path, precision=precision)
    p = case.params
    xs = {n: t(getattr(case.x, n), dev) for n in "qkvbg"}
    res = kda.kda_prefill_gate_proj(cfg, t(case.cu_seqlens.astype(np.int32), dev), xs["q"], xs["k"], xs["v"],
                                    t(f, dev), t(w_fb, dev), xs["b"], xs["g"], t(p.conv_w, dev), t(p.A_log, dev),
                                    t(p.dt_bias, dev), t(p.norm_w, dev), t(case.initial_state, dev),
                                    t(case.initial_conv_state, dev))
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res]


def _oracle(case, f, w_fb, pairs):
    import oracle
    x, p = case.x, case.params
    return oracle.forward(oracle_cfg(), case.cu_seqlens, x.q, x.k, x.v, None, x.b, x.g, p.conv_w, p.A_log,
                          p.dt_bias, p.norm_w, case.initial_state, case.initial_conv_state, pairs=pairs,
                          decode=ki.bf16_bits_to_f32, gate_proj=(f, w_fb))


def _check(case, f, w_fb, got, ref, pairs):
    out, fs, fcs = got
    cu, H = case.cu_seqlens, case.H
    wo = ws = 0.0
    for (s, h) in pairs:
        r = ref[(s, h)]
        o = out[cu[s]:cu[s + 1], h * D:(h + 1) * D]
        if o.size:
            wo = max(wo, float(np.max(np.abs(o - r.out))))
        ws = max(ws, slice_rel(fs[s, h], r.state))
        got_c = np.stack([fcs[s, blk * H * D + h * D: blk * H * D + (h + 1) * D] for blk in range(3)])
        np.testing.assert_array_equal(got_c, r.conv_state)
    return wo, ws


@pytest.mark.parametrize("precision", PRECS)
def test_varlen_against_oracle_both_layouts(device, precision):
    case = ki.prefill_case(500, 3, [5, 0, 1, 2, 70, 64, 129, 300], True, "gate-proj-varlen")
    f, w_fb = ki.lowrank_gate(500, case.N, case.H)
    pairs = [(s, h) for s in range(case.B) for h in range(case.H)]
    ref = _oracle(case, f, w_fb, pairs)
    res = {}
    for path in (PATH_FUSED, PATH_CHUNKED):
        print(f"[gate-proj] {case.name} path={path} precision={precision} B={case.B} N={case.N}", flush=True)
        res[path] = _gpu(case, f, w_fb, device, path, precision)
        wo, ws = _check(case, f, w_fb, res[path], ref, pairs)
        print(f"[gate-proj] {case.name} path={path} precision={precision}: out abs err {wo:.3e}, "
              f"state rel err {ws:.3e}", flush=True)
        assert wo <= PREFILL_OUT_ABS_TOL and ws <= PREFILL_STATE_REL_TOL, (wo, ws)
        if precision == PRECISION_HIGH:
            assert wo <= 1e-3 and ws <= 5e-4, (wo, ws)
    for a, b in zip(res[PATH_FUSED], res[PATH_CHUNKED]):
        assert np.array_equal(a, b)


@pytest.mark.timeout(600)
def test_long_sequence_every_head(device):
    """One 8192-token sequence, 96 heads, zero initial state: every head on both layouts."""
    case = ki.prefill_case(2, 96, [8192], False, "gate-proj-1x8192")
    f, w_fb = ki.lowrank_gate(2, case.N, case.H)
    got = {}
    for path in (PATH_FUSED, PATH_CHUNKED):
        print(f"[gate-proj] {case.name} path={path}", flush=True)
        got[path] = _gpu(case, f, w_fb, device, path, PRECISION_STANDARD)
    for a, b in zip(got[PATH_FUSED], got[PATH_CHUNKED]):
        assert np.array_equal(a, b)
    worst = [0.0, 0.0]
    for h0 in range(0, 96, 16):
        pairs = [(0, h) for h in range(h0, h0 + 16)]
        wo, ws = _check(case, f, w_fb, got[PATH_FUSED], _oracle(case, f, w_fb, pairs), pairs)
        worst = [max(worst[0], wo), max(worst[1], ws)]
        print(f"[gate-proj] {case.name}: heads ..{h0 + 15}, out abs err {worst[0]:.3e}, state rel err "
              f"{worst[1]:.3e}", flush=True)
    assert worst[0] <= PREFILL_OUT_ABS_TOL and worst[1] <= PREFILL_STATE_REL_TOL, worst


@pytest.mark.parametrize("path", PATHS)
def test_one_hot_factor_gives_the_z_path(device, path):
    """With a one-hot W_fb (row h*D + i = e_i) the logits are z = f tiled over the heads,
    exactly (one nonzero product per sum, in fp32): the entry point then gives the bits of
    kda_prefill on those logits (which are bf16 values, so nothing is rounded)."""
    H = 2
    case = ki.prefill_case(501, H, [77, 130], True, "gate-proj-one-hot")
    f, _ = ki.lowrank_gate(501, case.N, H)
    w = np.zeros((H * D, D), np.float32)
    for h in range(H):
        w[h * D + np.arange(D), np.arange(D)] = 1.0
    w_fb = ki.to_bf16_bits(w)
    case.x.z[...] = np.tile(f, (1, H))
    got = _gpu(case, f, w_fb, device, path, PRECISION_STANDARD)
    from tests.parity import prefill_gpu
    ref = prefill_gpu(case, device, path=path)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b.cpu().numpy())
