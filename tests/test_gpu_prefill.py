"""GPU parity of kda_prefill (bf16 inputs, chunk 64, fp32 state) against the fp64 oracle:
max abs error 2e-2 on the gated RMS-normalised outputs, max relative error 5e-3 per
(sequence, head) on final states, exact final conv windows.  Every case runs on both
work layouts (fused; chunk records + carry), which must also agree with each other
bit for bit."""
import functools

import numpy as np
import pytest
import torch

import kda_inputs as ki
from tests.parity import (PATH_CHUNKED, PATH_FUSED, PREFILL_OUT_ABS_TOL, PREFILL_STATE_REL_TOL, DecodeRun,
                          check_prefill, prefill_gpu, slice_rel, t)

pytestmark = pytest.mark.gpu

D = 128

PATHS = [pytest.param(PATH_FUSED, id="fused"), pytest.param(PATH_CHUNKED, id="chunked")]


def _run_and_check(case, dev, path, pairs=None, in_place=False):
    if pairs is None:
        pairs = [(s, h) for s in range(case.B) for h in range(case.H)]
    print(f"[prefill] {case.name} path={path} B={case.B} N={case.N} H={case.H} pairs={len(pairs)}", flush=True)
    out, fs, fcs = prefill_gpu(case, dev, in_place=in_place, path=path)
    eo, es = check_prefill(case, out, fs, fcs, pairs)
    print(f"[prefill] {case.name} path={path}: out abs err {eo:.3e}, state rel err {es:.3e}", flush=True)
    assert eo <= PREFILL_OUT_ABS_TOL, eo
    assert es <= PREFILL_STATE_REL_TOL, es
    return out, fs, fcs


@functools.lru_cache(maxsize=None)
def _case2():
    return ki.case2_prefill()


@functools.lru_cache(maxsize=None)
def _case3():
    return ki.case3_prefill()


@pytest.mark.parametrize("path", PATHS)
def test_cfg0_single_chunk(device, path):
    _run_and_check(ki.case0_prefill(), device, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 3, 17, 63, 64, 65, 200])
def test_ragged_lengths_with_initial_state(device, T, path):
    case = ki.prefill_case(100 + T, 3, [T], True, f"ragged-{T}")
    _run_and_check(case, device, path)


@pytest.mark.parametrize("path", PATHS)
def test_varlen_small_with_empty_and_short_sequences(device, path):
    case = ki.prefill_case(120, 2, [5, 0, 1, 2, 70, 64, 129, 3, 300], True, "varlen-small")
    _run_and_check(case, device, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B", [64, 80])
def test_many_sequences(device, path, B):
    # up to 64 sequences the fused kernel and the carry hand out sequences longest first
    # (ties by index), above that in index order: both sides of the limit, with repeated
    # lengths, empty and 1-token sequences, every (sequence, head) pair checked
    rng = np.random.default_rng(150 + B)
    lengths = rng.choice([0, 1, 7, 64, 65, 100, 130], size=B).tolist()
    case = ki.prefill_case(150 + B, 2, lengths, True, f"many-{B}")
    _run_and_check(case, device, path)


@pytest.mark.parametrize("path", PATHS)
def test_zero_initial_state_multi_chunk(device, path):
    case = ki.prefill_case(121, 4, [333, 190], False, "zero-init")
    _run_and_check(case, device, path)


@pytest.mark.parametrize("path", PATHS)
def test_in_place_state_carry(device, path):
    case = ki.prefill_case(122, 2, [150, 77], True, "in-place")
    _run_and_check(case, device, path, in_place=True)


@pytest.mark.parametrize("path", PATHS)
def test_saturated_gates(device, path):
    """Logits far in the tails, per sequence: the strongest decay (gk -> -5, so G falls by
    about 5 per token and e^{-G} would overflow fp32 within a chunk without the sub-chunk
    references) with beta -> 1; beta -> 0 (no update); strongest and no decay alternating
    every 16 tokens (the sub-chunk boundary) with beta -> 1; a random mix per token.
    (No decay with beta -> 1 on every token has its own test below.)"""
    case = ki.prefill_case(140, 3, [150, 150, 150, 200], True, "saturated")
    bf = lambda v: ki.to_bf16_bits(np.float32(v))
    cu = case.cu_seqlens
    rng = np.random.default_rng(141)
    for s in range(case.B):
        for t in range(cu[s], cu[s + 1]):
            i = t - cu[s]
            if s == 0:
                z, b = 40.0, 30.0
            elif s == 1:
                z, b = 40.0, -30.0
            elif s == 2:
                z, b = (40.0 if (i // 16) % 2 == 0 else -40.0), 30.0
            else:
                z, b = float(rng.choice([-40.0, 40.0, 0.0])), float(rng.choice([-30.0, 30.0, 0.0]))
            case.x.z[t] = bf(z)
            case.x.b[t] = bf(b)
        case.x.g[cu[s]:cu[s + 1], :64] = bf(25.0)  # output gate saturated on one head's channels
    _run_and_check(case, device, path)


def test_layouts_agree_bitwise(device):
    """The chunked layout performs the fused kernel's arithmetic in the same order, so
    the two give identical bits (outputs, final states, final windows)."""
    case = ki.prefill_case(126, 3, [1, 64, 130, 0, 257], True, "layouts")
    a = prefill_gpu(case, device, path=PATH_FUSED)
    b = prefill_gpu(case, device, path=PATH_CHUNKED)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("lengths", [[8192], [1024, 2048, 3000, 500, 130]], ids=["1x8192", "mix5"])
def test_layouts_agree_bitwise_long_segments(device, lengths):
    """With 32 heads the chunked plan gives each chunk-kernel workgroup 16 chunks of the
    8192-token sequence and 8 chunks of the five-sequence batch (the plan's segment length
    follows B, N and H); the records, and so every output bit, stay the fused kernel's."""
    case = ki.prefill_case(127, 32, lengths, True, "long-segments")
    a = prefill_gpu(case, device, path=PATH_FUSED)
    b = prefill_gpu(case, device, path=PATH_CHUNKED)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,H,lengths", [(2, 64, [65, 128]), (3, 43, [129, 1, 70])], ids=["BH128-split", "BH129-one"])
def test_carry_forms_agree_bitwise(device, B, H, lengths):
    """The chunked layout carries B*H <= 128 (sequence, head) pairs with two workgroups per
    pair (each owning 64 value columns, exchanging the RMS sums of every output row) and
    larger batches with one workgroup per pair; either form gives the fused kernel's bits.
    The first case sits at the limit of the split form (2 x 64 pairs, two-chunk sequences:
    the exchange's first chunks and last two epilogues), the second one pair past it."""
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(128 + B, H, lengths, True, f"carry-forms-{B}x{H}")
    assert case.B * case.H == (128 if B == 2 else 129)
    a = prefill_gpu(case, device, path=PATH_FUSED)
    try:
        kda.kda_test_pipeline(1)  # the serial carries (not the pipelined form)
        b = prefill_gpu(case, device, path=PATH_CHUNKED)
    finally:
        kda.kda_test_pipeline(0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_split_carry_wait_times_out(device):
    """The two-workgroup carry's wait for the other half's row sums is bounded: with the
    publishing switched off from the host (kda_test_split_carry) and a 16-poll bound, the
    call returns with NaN outputs and the exact final states and windows, and the next call
    is a normal one again."""
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(130, 4, [200, 70], True, "split-timeout")
    try:
        kda.kda_test_pipeline(1)  # the split carry (not the pipelined form)
        ref = prefill_gpu(case, device, path=PATH_CHUNKED)
        kda.kda_test_split_carry(False, 16)
        got = prefill_gpu(case, device, path=PATH_CHUNKED)
        kda.kda_test_split_carry(True, 0)
        again = prefill_gpu(case, device, path=PATH_CHUNKED)
    finally:
        kda.kda_test_split_carry(True, 0)
        kda.kda_test_pipeline(0)
    assert torch.isnan(got[0]).all()
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])
    for x, y in zip(again, ref):
        assert torch.equal(x, y)


# one sequence: (heads, length) for the pipelined form (carries in the chunk workgroups'
# launch): many chunks, a ragged tail, a single partial chunk, the largest H it takes on
# 256 compute units, one head
PIPE_CASES = [(32, 8192), (96, 1000), (4, 65), (128, 3000), (1, 321)]


@pytest.mark.parametrize("H,T", PIPE_CASES)
def test_pipelined_carry_agrees_bitwise(device, H, T):
    """One sequence with the carries running in the chunk workgroups' launch, each reading
    a record once its ready word is set, gives the bits of the serial carry and of the
    fused kernel: outputs, final states and windows."""
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(140 + H, H, [T], True, f"pipe-{H}x{T}")
    fused = prefill_gpu(case, device, path=PATH_FUSED)
    try:
        kda.kda_test_pipeline(1)
        serial = prefill_gpu(case, device, path=PATH_CHUNKED)
        kda.kda_test_pipeline(2)
        piped = prefill_gpu(case, device, path=PATH_CHUNKED)
    finally:
        kda.kda_test_pipeline(0)
    for x, y, z in zip(fused, serial, piped):
        assert torch.equal(x, y)
        assert torch.equal(x, z)


# several sequences (B*H <= 128): the chunk workgroups take the segments row by row
PIPE_VARLEN = [(16, [700, 0, 1, 2000, 65]), (32, [1500, 1500, 1500]), (64, [3000, 100])]


@pytest.mark.parametrize("H,lengths", PIPE_VARLEN)
def test_pipelined_varlen_agrees_bitwise(device, H, lengths):
    """Several sequences through the pipelined form (empty, 1-token and ragged ones among
    them) give the bits of the serial carry and of the fused kernel."""
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(180 + H, H, lengths, True, f"pipe-varlen-{H}")
    fused = prefill_gpu(case, device, path=PATH_FUSED)
    try:
        kda.kda_test_pipeline(1)
        serial = prefill_gpu(case, device, path=PATH_CHUNKED)
        kda.kda_test_pipeline(2)
        piped = prefill_gpu(case, device, path=PATH_CHUNKED)
    finally:
        kda.kda_test_pipeline(0)
    for x, y, z in zip(fused, serial, piped):
        assert torch.equal(x, y)
        assert torch.equal(x, z)


@pytest.mark.parametrize("seed", [302, 307, 309, 317, 318, 321])
def test_pipelined_random_batches_agree_bitwise(device, seed):
    """Random batches through the pipelined form (1 to 6 sequences of 0 to 3000 tokens,
    B*H <= 128) give the fused kernel's bits."""
    import gated_delta_rule_31_amd as kda
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    H = int(rng.integers(1, 128 // B + 1))
    lengths = [int(x) for x in rng.choice([0, 1, 2, 63, 64, 65, 300, 1000, 3000], size=B)]
    if sum(lengths) == 0:
        lengths[0] = 129
    case = ki.prefill_case(seed, H, lengths, True, f"pipe-random-{seed}")
    fused = prefill_gpu(case, device, path=PATH_FUSED)
    try:
        kda.kda_test_pipeline(2)
        piped = prefill_gpu(case, device, path=PATH_CHUNKED)
    finally:
        kda.kda_test_pipeline(0)
    for x, y in zip(fused, piped):
        assert torch.equal(x, y)


def test_pipelined_reuses_workspace(device):
    """Two different batches through the pipelined form in one workspace, back to back and
    again: each call gives the fused kernel's bits, so no carry reads a record the call
    before left there."""
    import gated_delta_rule_31_amd as kda
    cases = [ki.prefill_case(160 + i, 16, [T], True, f"pipe-ws-{i}") for i, T in enumerate((2000, 1500))]
    refs = [prefill_gpu(c, device, path=PATH_FUSED) for c in cases]
    try:
        kda.kda_test_pipeline(2)
        cfg = kda.KdaConfig(num_heads=16, prefill_path=PATH_CHUNKED)
        ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, 1, 2000), dtype=torch.uint8, device=device)
        for c, ref in [(cases[0], refs[0]), (cases[1], refs[1]), (cases[0], refs[0])]:
            p = c.params
            got = kda.kda_prefill(cfg, t(c.cu_seqlens.astype(np.int32), device), *[t(getattr(c.x, n), device) for n in "qkvzbg"],
                                  t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device),
                                  t(c.initial_state, device), t(c.initial_conv_state, device), workspace=ws)
            torch.cuda.synchronize()
            for x, y in zip(got, ref):
                assert torch.equal(x, y)
    finally:
        kda.kda_test_pipeline(0)


def test_pipelined_wait_times_out(device):
    """The pipelined carries' wait for a record is bounded: with the ready words never
    published (kda_test_pipeline) and a 16-poll bound, the call returns with NaN outputs
    and NaN final states, the windows exact, and the next call is a normal one again."""
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(170, 4, [300], True, "pipe-timeout")
    ref = prefill_gpu(case, device, path=PATH_FUSED)
    try:
        kda.kda_test_pipeline(2, False, 16)
        got = prefill_gpu(case, device, path=PATH_CHUNKED)
        kda.kda_test_pipeline(2)
        again = prefill_gpu(case, device, path=PATH_CHUNKED)
    finally:
        kda.kda_test_pipeline(0)
    assert torch.isnan(got[0]).all() and torch.isnan(got[1]).all()
    assert torch.equal(got[2], ref[2])
    for x, y in zip(again, ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("path", PATHS)
def test_packing_invariance(device, path):
    """Each sequence of a packed batch gives what it gives alone."""
    case = ki.prefill_case(123, 2, [90, 31, 200], True, "packed")
    out, fs, fcs = prefill_gpu(case, device, path=path)
    cu = case.cu_seqlens
    for s in range(case.B):
        alone = ki.PrefillCase(f"alone-{s}", case.seed, case.H, np.array([0, cu[s + 1] - cu[s]], np.int32),
                               case.params,
                               ki.TokenInputs(*(getattr(case.x, n)[cu[s]:cu[s + 1]] for n in "qkvzbg")),
                               case.initial_state[s:s + 1], case.initial_conv_state[s:s + 1])
        o1, f1, c1 = prefill_gpu(alone, device, path=path)
        assert torch.equal(o1, out[cu[s]:cu[s + 1]])
        assert torch.equal(f1[0], fs[s])
        assert torch.equal(c1[0], fcs[s])


@pytest.mark.parametrize("path", PATHS)
def test_prefill_matches_decode_steps(device, path):
    """32 decode steps on the bf16-rounded tokens give the 32-token prefill's result
    (fp32 decode vs chunked bf16-MFMA prefill, within the prefill tolerances)."""
    H, T = 4, 32
    case = ki.prefill_case(124, H, [T], True, "decode-vs-prefill")
    out, fs, fcs = prefill_gpu(case, device, path=path)
    x = case.x.as_f32()
    steps = [ki.TokenInputs(*(getattr(x, n)[i:i + 1] for n in "qkvzbg")) for i in range(T)]
    dcase = ki.DecodeCase("dec", case.seed, 1, H, T, case.params, case.initial_state, case.initial_conv_state,
                          _steps=steps)
    run = DecodeRun(dcase, device)
    outs = [run.step(run.inputs(i)) for i in range(T)]
    torch.cuda.synchronize()
    dec_out = torch.cat(outs).cpu().numpy()
    assert np.max(np.abs(dec_out - out.cpu().numpy())) <= PREFILL_OUT_ABS_TOL
    for h in range(H):
        assert slice_rel(fs[0, h].cpu().numpy(), run.state[0, h].cpu().numpy()) <= PREFILL_STATE_REL_TOL
    assert torch.equal(fcs, run.conv_state)


@pytest.mark.parametrize("path", PATHS)
def test_empty_batch_and_stream(device, path):
    import gated_delta_rule_31_amd as kda
    case = ki.prefill_case(125, 2, [40], True, "stream")
    o1, f1, _ = prefill_gpu(case, device, path=path)
    cfg = kda.KdaConfig(num_heads=2, prefill_path=path)
    p = case.params
    s = torch.cuda.Stream()
    args = [t(getattr(case.x, n), device) for n in "qkvzbg"]
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    cu = t(case.cu_seqlens, device)
    st, cst = t(case.initial_state, device), t(case.initial_conv_state, device)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o2, f2, _ = kda.kda_prefill(cfg, cu, *args, *prm, st, cst, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def _no_decay_full_beta(T: int, H: int, seed: int):
    """Every token with alpha = 1 exactly (z = -300: exp(A_log) (z + dt_bias) <= -40, so
    the sigmoid of the decay gate is below 5e-18 and gk rounds to -0 in fp32) and beta = 1
    (b = 30), from a nonzero initial state: the plain delta rule S = (I - k k^T) S + k v^T,
    the regime that has no decay to wash out rounding errors."""
    case = ki.prefill_case(seed, H, [T], True, f"no-decay-beta1-{T}")
    bf = lambda v: ki.to_bf16_bits(np.float32(v))
    case.x.z[...] = bf(-300.0)
    case.x.b[...] = bf(30.0)
    return case


@pytest.mark.xfail(reason="standard precision: with no decay every bf16 operand rounding persists in the state; "
                          "measured 1.9e-2 to 2.3e-2 output abs error at T = 1024 and 2.7e-2 to 3.2e-2 at 8192 "
                          "(bound 2e-2; the spread is the rounding of different kernel builds). "
                          "KDA_PRECISION_HIGH holds it at 9e-5 (tests/test_gpu_prefill_precise.py)",
                   strict=False)
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1024, 8192])
def test_no_decay_beta_one(device, T, path):
    _run_and_check(_no_decay_full_beta(T, 3, 160 + T % 97), device, path)
