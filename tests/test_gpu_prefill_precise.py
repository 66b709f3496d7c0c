"""GPU parity of kda_prefill with KDA_PRECISION_HIGH (every MFMA operand of the chunk
algebra split into bf16 hi + lo) against the fp64 oracle, at the same bounds as the
standard mode (2e-2 abs on outputs, 5e-3 relative on final states, exact windows):

- the regime the standard mode does not hold: no decay (alpha = 1) and beta = 1 on every
  token, the plain delta rule, at 1,024 and 8,192 tokens, on both work layouts;
- the ordinary cases (single chunk, ragged lengths, varlen with empty and short sequences,
  many sequences, saturated gates, in-place carry) on both layouts;
- the two layouts bit for bit, and bf16 outputs as the fp32 ones rounded;
- the chunked layout's two carry forms (serial after the chunk kernel, and pipelined in its
  launch behind the records' ready words) bit for bit against the fused layout, with bf16
  outputs too, and the pipelined carries' bounded wait."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from tests.parity import (PATH_CHUNKED, PATH_FUSED, PRECISION_HIGH, PREFILL_OUT_ABS_TOL, PREFILL_STATE_REL_TOL,
                          check_prefill, prefill_gpu, t)

pytestmark = pytest.mark.gpu

PATHS = [pytest.param(PATH_FUSED, id="fused"), pytest.param(PATH_CHUNKED, id="chunked")]


def _run_and_check(case, dev, path, in_place=False, bound=None):
    pairs = [(s, h) for s in range(case.B) for h in range(case.H)]
    print(f"[precise] {case.name} path={path} B={case.B} N={case.N} H={case.H}", flush=True)
    out, fs, fcs = prefill_gpu(case, dev, in_place=in_place, path=path, precision=PRECISION_HIGH)
    eo, es = check_prefill(case, out, fs, fcs, pairs)
    print(f"[precise] {case.name} path={path}: out abs err {eo:.3e}, state rel err {es:.3e}", flush=True)
    assert eo <= PREFILL_OUT_ABS_TOL, eo
    assert es <= PREFILL_STATE_REL_TOL, es
    if bound is not None:
        assert eo <= bound[0] and es <= bound[1], (eo, es)
    return out, fs, fcs


def _no_decay_full_beta(T: int, H: int, seed: int):
    """alpha = 1 exactly (z = -300, so exp(A_log) (z + dt_bias) <= -40 and the gate's
    sigmoid is below 5e-18) and beta = 1 (b = 30) on every token, nonzero initial state."""
    case = ki.prefill_case(seed, H, [T], True, f"no-decay-beta1-{T}")
    bf = lambda v: ki.to_bf16_bits(np.float32(v))
    case.x.z[...] = bf(-300.0)
    case.x.b[...] = bf(30.0)
    return case


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1024, 8192])
def test_no_decay_beta_one(device, T, path):
    # the emulated error of this arithmetic is below 1e-4 here; the bound below leaves a
    # 10x margin and still fails the standard mode's 2e-2 by a wide one
    _run_and_check(_no_decay_full_beta(T, 3, 160 + T % 97), device, path, bound=(1e-3, 5e-4))


@pytest.mark.parametrize("path", PATHS)
def test_cfg0_single_chunk(device, path):
    _run_and_check(ki.case0_prefill(), device, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 3, 17, 63, 64, 65, 200])
def test_ragged_lengths_with_initial_state(device, T, path):
    _run_and_check(ki.prefill_case(400 + T, 3, [T], True, f"precise-ragged-{T}"), device, path)


@pytest.mark.parametrize("path", PATHS)
def test_varlen_with_empty_and_short_sequences(device, path):
    _run_and_check(ki.prefill_case(420, 2, [5, 0, 1, 2, 70, 64, 129, 3, 300], True, "precise-varlen"), device, path)


@pytest.mark.parametrize("path", PATHS)
def test_many_sequences(device, path):
    rng = np.random.default_rng(421)
    lengths = rng.choice([0, 1, 7, 64, 65, 100, 130], size=70).tolist()
    _run_and_check(ki.prefill_case(421, 2, lengths, True, "precise-many"), device, path)


@pytest.mark.parametrize("path", PATHS)
def test_saturated_gates_and_in_place(device, path):
    case = ki.prefill_case(422, 3, [150, 150, 200], True, "precise-saturated")
    bf = lambda v: ki.to_bf16_bits(np.float32(v))
    cu = case.cu_seqlens
    rng = np.random.default_rng(423)
    for s in range(case.B):
        for tk in range(cu[s], cu[s + 1]):
            i = tk - cu[s]
            if s == 0:
                z, b = 40.0, 30.0                                   # strongest decay, beta -> 1
            elif s == 1:
                z, b = (40.0 if (i // 16) % 2 == 0 else -40.0), 30.0  # decay on / off per sub-chunk
            else:
                z, b = float(rng.choice([-40.0, 40.0, 0.0])), float(rng.choice([-30.0, 30.0, 0.0]))
            case.x.z[tk] = bf(z)
            case.x.b[tk] = bf(b)
    _run_and_check(case, device, path, in_place=True)


def test_layouts_agree_bitwise(device):
    for lengths, H in (([1, 64, 130, 0, 257], 3), ([2048], 32), ([1024, 2048, 3000, 500, 130], 32)):
        case = ki.prefill_case(424, H, lengths, True, "precise-layouts")
        print(f"[precise] layouts B={case.B} N={case.N} H={H}", flush=True)
        a = prefill_gpu(case, device, path=PATH_FUSED, precision=PRECISION_HIGH)
        b = prefill_gpu(case, device, path=PATH_CHUNKED, precision=PRECISION_HIGH)
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("path", PATHS)
def test_bf16_outputs_are_the_fp32_outputs_rounded(device, path):
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(425, 3, [70, 0, 1, 300], True, "precise-bf16")
    ref = prefill_gpu(case, device, path=path, precision=PRECISION_HIGH)
    p = case.params
    cfg = kda.KdaConfig(num_heads=case.H, prefill_path=path, precision=PRECISION_HIGH, out_dtype=torch.bfloat16)
    xs = [t(getattr(case.x, n), device) for n in "qkvzbg"]
    got = kda.kda_prefill(cfg, t(case.cu_seqlens.astype(np.int32), device), *xs, t(p.conv_w, device),
                          t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device),
                          t(case.initial_state, device), t(case.initial_conv_state, device))
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0].to(torch.bfloat16))
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])


def _precise_modes(case, device, out_dtype=None):
    """The fused layout, then the chunked one with the serial and with the pipelined carry
    (kda_test_pipeline modes 1 and 2)."""
    import gated_delta_rule_31_amd as kda
    runs = [prefill_gpu(case, device, path=PATH_FUSED, precision=PRECISION_HIGH, out_dtype=out_dtype)]
    try:
        for mode in (1, 2):
            kda.kda_test_pipeline(mode)
            runs.append(prefill_gpu(case, device, path=PATH_CHUNKED, precision=PRECISION_HIGH, out_dtype=out_dtype))
    finally:
        kda.kda_test_pipeline(0)
    return runs


@pytest.mark.parametrize("H,lengths", [(32, [8192]), (96, [1000]), (4, [65]), (1, [321]), (16, [700, 0, 1, 2000, 65]),
                                       (32, [1500, 1500, 1500])])
def test_pipelined_carry_agrees_bitwise(device, H, lengths):
    """The high-precision carry pipelined in the chunk workgroups' launch gives the bits of
    its serial form and of the fused kernel (outputs, final states, windows)."""
    case = ki.prefill_case(430 + H, H, lengths, True, "precise-pipe")
    print(f"[precise] pipelined B={case.B} N={case.N} H={H}", flush=True)
    fused, serial, piped = _precise_modes(case, device)
    for x, y, z in zip(fused, serial, piped):
        assert torch.equal(x, y)
        assert torch.equal(x, z)


def test_pipelined_bf16_outputs(device):
    case = ki.prefill_case(436, 8, [900, 77], True, "precise-pipe-bf16")
    fused, serial, piped = _precise_modes(case, device, out_dtype=torch.bfloat16)
    assert fused[0].dtype == torch.bfloat16
    for x, y, z in zip(fused, serial, piped):
        assert torch.equal(x, y)
        assert torch.equal(x, z)


def test_pipelined_wait_times_out(device):
    """The high-precision pipelined carries' wait is bounded too: with the ready words never
    published and a 16-poll bound, the outputs and final states are NaN, the windows exact,
    and the next call is a normal one."""
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(437, 4, [300], True, "precise-pipe-timeout")
    ref = prefill_gpu(case, device, path=PATH_FUSED, precision=PRECISION_HIGH)
    try:
        kda.kda_test_pipeline(2, False, 16)
        got = prefill_gpu(case, device, path=PATH_CHUNKED, precision=PRECISION_HIGH)
        kda.kda_test_pipeline(2)
        again = prefill_gpu(case, device, path=PATH_CHUNKED, precision=PRECISION_HIGH)
    finally:
        kda.kda_test_pipeline(0)
    assert torch.isnan(got[0]).all() and torch.isnan(got[1]).all()
    assert torch.equal(got[2], ref[2])
    for x, y in zip(again, ref):
        assert torch.equal(x, y)
