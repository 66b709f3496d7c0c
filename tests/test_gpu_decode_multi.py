"""GPU parity of kda_decode_multi (several known tokens per sequence in one call) against
the fp64 oracle (max relative error 1e-4 per (sequence, head) slice, as for one-token
decode), in both evaluation forms: the default block form (blocks of eight tokens in the
chunk form of the recurrence, the same terms summed in another order) agrees with the
same number of kda_decode_step calls to fp32 rounding (2e-5 relative per slice, windows
exact); the sequential form gives their bits.  Also the verify / roll-back use:
out-of-place candidates, then an in-place commit of the accepted prefix, whose outputs
are the candidates' bits."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import DECODE_REL_TOL, DecodeRun, decode_oracle, slice_rel, t

pytestmark = pytest.mark.gpu

D = 128
BLOCK, SEQUENTIAL = 0, 1  # kda_config.decode_multi_form
FORMS = [pytest.param(BLOCK, id="block"), pytest.param(SEQUENTIAL, id="sequential")]
MULTI_VS_STEPS_REL = 2e-5  # block form against token-by-token fp32, per (sequence, head) slice


def _rel(x: torch.Tensor, r: torch.Tensor) -> float:
    """max over (..., D) slices of max|x - r| / max|r|"""
    x = x.double().reshape(-1, D)
    r = r.double().reshape(-1, D)
    den = r.abs().amax(dim=1).clamp_min(1e-30)
    return float(((x - r).abs().amax(dim=1) / den).max())


class MultiRun:
    """A decode case's first T tokens as [B, T, ...] inputs on the GPU."""

    def __init__(self, case: ki.DecodeCase, T: int, dev, form: int = BLOCK):
        self.case, self.T, self.dev = case, T, dev
        self.cfg = kda.KdaConfig(num_heads=case.H, decode_multi_form=form)
        p = case.params
        self.prm = [t(p.conv_w, dev), t(p.A_log, dev), t(p.dt_bias, dev), t(p.norm_w, dev)]
        steps = [case.step(i) for i in range(T)]
        self.xs = [t(np.ascontiguousarray(np.stack([getattr(s, n) for s in steps], axis=1)), dev) for n in "qkvzbg"]
        self.state0 = t(case.state, dev)
        self.conv0 = t(case.conv_state, dev)

    def call(self, state_in, conv_in, state_out=None, conv_out=None, n_tokens=None):
        B, H = self.case.B, self.case.H
        out = torch.full((B, self.T, H * D), float("nan"), dtype=torch.float32, device=self.dev)
        nt = None if n_tokens is None else torch.tensor(n_tokens, dtype=torch.int32, device=self.dev)
        kda.kda_decode_multi(self.cfg, *self.xs, *self.prm, state_in, conv_in, state_out=state_out,
                             conv_state_out=conv_out, n_tokens=nt, out=out)
        torch.cuda.synchronize()
        return out


def _single_steps(case, n, dev):
    """n kda_decode_step calls on the whole batch: outputs [n][B, H*D], final state, windows."""
    run = DecodeRun(case, dev)
    outs = [run.step(run.inputs(i)).clone() for i in range(n)]
    torch.cuda.synchronize()
    return outs, run.state, run.conv_state


def _window(cst, b, h, H):
    return np.stack([cst[b, blk * H * D + h * D: blk * H * D + (h + 1) * D] for blk in range(3)])


@pytest.mark.parametrize("form", FORMS)
def test_per_sequence_counts_against_oracle(device, form):
    case = ki.decode_case(310, 4, 4, 8, "multi-counts")
    n = [8, 3, 0, 1]
    print(f"[decode-multi] {case.name} B={case.B} H={case.H} T=8 n={n} form={form}", flush=True)
    mr = MultiRun(case, 8, device, form)
    s_out, c_out = torch.empty_like(mr.state0), torch.empty_like(mr.conv0)
    state_in, conv_in = mr.state0.clone(), mr.conv0.clone()
    out = mr.call(state_in, conv_in, s_out, c_out, n_tokens=n).cpu().numpy().reshape(case.B, 8, case.H, D)
    st, cst = s_out.cpu().numpy(), c_out.cpu().numpy()
    # the inputs are left as they were (they are the pre-verify snapshot)
    assert torch.equal(state_in, mr.state0) and torch.equal(conv_in, mr.conv0)
    worst = 0.0
    for b in range(case.B):
        assert np.isnan(out[b, n[b]:]).all()  # rows past the count are not written
        if n[b] == 0:
            np.testing.assert_array_equal(st[b], case.state[b])
            np.testing.assert_array_equal(cst[b], case.conv_state[b])
            continue
        ref = decode_oracle(case, [(b, h) for h in range(case.H)], n[b])
        for h in range(case.H):
            r = ref[(b, h)]
            for i in range(n[b]):
                worst = max(worst, slice_rel(out[b, i, h], r.out[i]))
            worst = max(worst, slice_rel(st[b, h], r.state))
            np.testing.assert_array_equal(_window(cst, b, h, case.H), r.conv_state)
    print(f"[decode-multi] {case.name}: max rel err {worst:.3e}", flush=True)
    assert worst <= DECODE_REL_TOL, worst


@pytest.mark.parametrize("T", [1, 6, 8, 11, 17, 40])
def test_in_place_agrees_with_single_steps(device, T):
    case = ki.decode_case(311, 5, 6, T, f"multi-vs-steps-{T}")
    print(f"[decode-multi] {case.name} B={case.B} H={case.H} T={T}", flush=True)
    mr = MultiRun(case, T, device)
    state, conv = mr.state0.clone(), mr.conv0.clone()
    out = mr.call(state, conv)
    outs, st, cst = _single_steps(case, T, device)
    worst = max(_rel(out[:, i], outs[i]) for i in range(T))
    worst = max(worst, _rel(state, st))
    print(f"[decode-multi] {case.name}: max rel diff against single steps {worst:.3e}", flush=True)
    assert worst <= MULTI_VS_STEPS_REL, worst
    assert torch.equal(conv, cst)


@pytest.mark.parametrize("form", FORMS)
def test_verify_then_commit_accepted_prefix(device, form):
    case = ki.decode_case(312, 3, 4, 6, "multi-verify")
    accepted = [6, 2, 0]
    print(f"[decode-multi] {case.name} B={case.B} H={case.H} T=6 accepted={accepted} form={form}", flush=True)
    mr = MultiRun(case, 6, device, form)
    state, conv = mr.state0.clone(), mr.conv0.clone()
    spec_s, spec_c = torch.empty_like(state), torch.empty_like(conv)
    spec_out = mr.call(state, conv, spec_s, spec_c)  # candidates; `state` is the snapshot
    assert torch.equal(state, mr.state0)
    out = mr.call(state, conv, n_tokens=accepted)    # commit the accepted prefixes in place
    for b, a in enumerate(accepted):
        outs, st, cst = _single_steps(case, a, device) if a else ([], mr.state0, mr.conv0)
        for i in range(a):
            assert torch.equal(out[b, i], spec_out[b, i])  # the commit repeats the candidates' bits
            if form == SEQUENTIAL:
                assert torch.equal(out[b, i], outs[i][b])
            else:
                assert _rel(out[b, i], outs[i][b]) <= MULTI_VS_STEPS_REL
        assert torch.isnan(out[b, a:]).all()
        if a == 0:
            assert torch.equal(state[b], mr.state0[b]) and torch.equal(conv[b], mr.conv0[b])
        elif form == SEQUENTIAL:
            assert torch.equal(state[b], st[b]) and torch.equal(conv[b], cst[b])
        else:
            assert _rel(state[b], st[b]) <= MULTI_VS_STEPS_REL
            assert torch.equal(conv[b], cst[b])
    # a fully accepted sequence ends where the candidates ended
    assert torch.equal(state[0], spec_s[0]) and torch.equal(conv[0], spec_c[0])


@pytest.mark.parametrize("T", [6, 11])
def test_sequential_form_equals_single_steps_bitwise(device, T):
    case = ki.decode_case(311, 5, 6, T, f"multi-seq-vs-steps-{T}")
    print(f"[decode-multi] {case.name} B={case.B} H={case.H} T={T} sequential", flush=True)
    mr = MultiRun(case, T, device, SEQUENTIAL)
    state, conv = mr.state0.clone(), mr.conv0.clone()
    out = mr.call(state, conv)
    outs, st, cst = _single_steps(case, T, device)
    for i in range(T):
        assert torch.equal(out[:, i], outs[i]), i
    assert torch.equal(state, st) and torch.equal(conv, cst)


def test_k3_shape_four_tokens(device):
    case = ki.decode_case(313, 64, 96, 4, "multi-k3")
    print(f"[decode-multi] {case.name} B={case.B} H={case.H} T=4", flush=True)
    mr = MultiRun(case, 4, device)
    state, conv = mr.state0.clone(), mr.conv0.clone()
    out = mr.call(state, conv)
    outs, st, cst = _single_steps(case, 4, device)
    assert _rel(state, st) <= MULTI_VS_STEPS_REL and torch.equal(conv, cst)
    for i in range(4):
        assert _rel(out[:, i], outs[i]) <= MULTI_VS_STEPS_REL
    rng = np.random.default_rng(313)
    pairs = [(0, 0), (63, 95)] + [(int(b), int(h)) for b, h in zip(rng.integers(0, 64, 10), rng.integers(0, 96, 10))]
    ref = decode_oracle(case, pairs, 4)
    o = out.cpu().numpy().reshape(case.B, 4, case.H, D)
    s = state.cpu().numpy()
    worst = 0.0
    for (b, h) in pairs:
        for i in range(4):
            worst = max(worst, slice_rel(o[b, i, h], ref[(b, h)].out[i]))
        worst = max(worst, slice_rel(s[b, h], ref[(b, h)].state))
    assert worst <= DECODE_REL_TOL, worst


def test_pool_verify_and_commit_matches_dense(device):
    """kda_decode_multi_slots over a pool: candidates into a second pool, then the accepted
    prefixes committed in place; every applied output row equals the dense call's bits,
    the committed entries agree with single steps, and a row aimed past the pool leaves
    everything untouched."""
    case = ki.decode_case(314, 3, 4, 5, "multi-slots")
    B, H, T, P = case.B, case.H, 5, 6
    home = [4, 0, 2]
    print(f"[decode-multi] {case.name} B={B} H={H} T={T} P={P} home={home}", flush=True)
    mr = MultiRun(case, T, device)
    pool_s = torch.full((P, H, D, D), 3.0, dtype=torch.float32, device=device)
    pool_c = torch.full((P, 3 * H * D, 3), 3.0, dtype=torch.float32, device=device)
    for bi, e in enumerate(home):
        pool_s[e] = mr.state0[bi]
        pool_c[e] = mr.conv0[bi]
    before_s, before_c = pool_s.clone(), pool_c.clone()
    # rows: the three sequences plus one aimed past the pool (it carries sequence 0's tokens)
    rows = [0, 1, 2, 0]
    slots = torch.tensor(home + [P + 3], dtype=torch.int32, device=device)
    xs = [x[rows].contiguous() for x in mr.xs]
    out = torch.full((4, T, H * D), float("nan"), dtype=torch.float32, device=device)
    cand_s, cand_c = torch.zeros_like(pool_s), torch.zeros_like(pool_c)
    kda.kda_decode_multi_slots(mr.cfg, slots, *xs, *mr.prm, pool_s, pool_c, state_out=cand_s,
                               conv_state_out=cand_c, out=out)
    accepted = torch.tensor([5, 2, 0, 5], dtype=torch.int32, device=device)
    out2 = torch.full_like(out, float("nan"))
    kda.kda_decode_multi_slots(mr.cfg, slots, *xs, *mr.prm, pool_s, pool_c, n_tokens=accepted, out=out2)
    torch.cuda.synchronize()
    dense_out = mr.call(mr.state0.clone(), mr.conv0.clone(), torch.empty_like(mr.state0), torch.empty_like(mr.conv0))
    for bi, e in enumerate(home):
        assert torch.equal(out[bi], dense_out[bi]), bi
        a = int(accepted[bi])
        assert torch.equal(out2[bi, :a], dense_out[bi, :a]) and torch.isnan(out2[bi, a:]).all(), bi
        outs, st, cst = _single_steps(case, a, device) if a else ([], mr.state0, mr.conv0)
        if a == 0:
            assert torch.equal(pool_s[e], st[bi]), bi
        else:
            assert _rel(pool_s[e], st[bi]) <= MULTI_VS_STEPS_REL, bi
        assert torch.equal(pool_c[e], cst[bi]), bi
    assert torch.isnan(out[3]).all() and torch.isnan(out2[3]).all()
    for e in set(range(P)) - set(home):
        assert torch.equal(pool_s[e], before_s[e]) and torch.equal(pool_c[e], before_c[e]), e
        assert (cand_s[e] == 0).all() and (cand_c[e] == 0).all(), e


@pytest.mark.parametrize("regime", ["strongest-decay", "no-decay-beta-one", "mixed"])
def test_extreme_gates_against_oracle(device, regime):
    """The block form at the gates' extremes: the strongest decay (the cumulative log decay
    of a block reaches -40, the bound of its e^{+-G} factors), no decay with beta = 1 (the
    plain delta rule, where the block's triangular solve is least damped), and a mix."""
    import oracle
    from tests.parity import oracle_cfg
    T = 19
    case = ki.decode_case(315, 3, 4, T, f"multi-{regime}")
    mr = MultiRun(case, T, device)
    steps = [case.step(i) for i in range(T)]
    x = {nm: np.ascontiguousarray(np.stack([getattr(s, nm) for s in steps], axis=1)) for nm in "qkvzbg"}
    rng = np.random.default_rng(315)
    if regime == "strongest-decay":
        x["z"][...] = 40.0
        x["b"][...] = 30.0
    elif regime == "no-decay-beta-one":
        x["z"][...] = -300.0
        x["b"][...] = 30.0
    else:
        x["z"][...] = rng.choice([-300.0, 40.0, 0.0], size=x["z"].shape)
        x["b"][...] = rng.choice([-30.0, 30.0, 0.0], size=x["b"].shape)
    mr.xs[3] = t(x["z"].astype(np.float32), device)
    mr.xs[4] = t(x["b"].astype(np.float32), device)
    print(f"[decode-multi] {case.name} B={case.B} H={case.H} T={T}", flush=True)
    state, conv = mr.state0.clone(), mr.conv0.clone()
    out = mr.call(state, conv).cpu().numpy().reshape(case.B, T, case.H, D)
    st = state.cpu().numpy()
    B, H = case.B, case.H
    flat = {nm: x[nm].reshape(B * T, -1) for nm in x}
    p = case.params
    pairs = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle.forward(oracle_cfg(), np.arange(B + 1) * T, flat["q"], flat["k"], flat["v"], flat["z"], flat["b"],
                         flat["g"], p.conv_w, p.A_log, p.dt_bias, p.norm_w, case.state, case.conv_state, pairs=pairs)
    worst = 0.0
    for (b, h) in pairs:
        r = ref[(b, h)]
        for i in range(T):
            worst = max(worst, slice_rel(out[b, i, h], r.out[i]))
        worst = max(worst, slice_rel(st[b, h], r.state))
    print(f"[decode-multi] {case.name}: max rel err {worst:.3e}", flush=True)
    assert worst <= DECODE_REL_TOL, worst
