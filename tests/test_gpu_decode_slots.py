"""GPU parity of kda_decode_step_slots (one token per batch row, states held in a pool
addressed by per-row slot ids) against the fp64 oracle (max relative error 1e-4 per
(sequence, head) slice, as for dense decode), bit-for-bit agreement with
kda_decode_step on the same states gathered into a dense batch, and the skipping of
rows whose slot lies outside the pool."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import DECODE_REL_TOL, DecodeRun, decode_oracle, slice_rel, t

pytestmark = pytest.mark.gpu

D = 128


class Pool:
    """A decode case's sequences parked in a pool of P entries: sequence s at home[s]."""

    def __init__(self, case: ki.DecodeCase, P: int, home, dev):
        self.case, self.P, self.dev = case, P, dev
        self.home = list(home)
        H = case.H
        rng = np.random.default_rng(case.seed + 1000)
        # entries that hold no sequence of the case get unrelated contents (must stay as they are)
        st = rng.standard_normal((P, H, D, D), dtype=np.float32) * np.float32(0.05)
        cs = rng.standard_normal((P, 3 * H * D, 3), dtype=np.float32)
        for s, e in enumerate(self.home):
            st[e] = case.state[s]
            cs[e] = case.conv_state[s]
        self.state = t(st, dev)
        self.conv = t(cs, dev)
        self.cfg = kda.KdaConfig(num_heads=H)
        p = case.params
        self.prm = [t(p.conv_w, dev), t(p.A_log, dev), t(p.dt_bias, dev), t(p.norm_w, dev)]

    def step(self, i: int, rows, out_rows: int | None = None):
        """Decode step i of the case: batch row r carries rows[r] = sequence id, or an int
        slot wrapped as ("raw", slot) for a row aimed at an arbitrary slot (its inputs
        are sequence 0's)."""
        x = self.case.step(i)
        seq = [r[2] if isinstance(r, tuple) else r for r in rows]
        slots = [r[1] if isinstance(r, tuple) else self.home[r] for r in rows]
        xs = [t(np.ascontiguousarray(getattr(x, n)[seq]), self.dev) for n in "qkvzbg"]
        B = len(rows)
        out = torch.full((B, self.case.H * D), float("nan"), dtype=torch.float32, device=self.dev)
        sl = torch.tensor(slots, dtype=torch.int32, device=self.dev)
        kda.kda_decode_step_slots(self.cfg, sl, *xs, *self.prm, self.state, self.conv, out=out)
        torch.cuda.synchronize()
        return out


def test_slots_equal_dense_steps_bitwise_and_skip_outside_rows(device):
    case = ki.decode_case(320, 4, 6, 3, "slots-vs-dense")
    P = 9
    home = [7, 2, 5, 0]
    print(f"[decode-slots] {case.name} B={case.B} H={case.H} P={P} home={home}", flush=True)
    pool = Pool(case, P, home, device)
    before = pool.state.clone(), pool.conv.clone()
    run = DecodeRun(case, device)  # the same sequences as a dense batch
    # rows in a different order every step, plus rows aimed outside the pool
    orders = [[2, 0, ("raw", -1, 0), 3, 1], [1, ("raw", P, 0), 3, 2, 0, ("raw", -7, 0)], [3, 2, 1, 0]]
    for i, rows in enumerate(orders):
        out = pool.step(i, rows)
        ref = run.step(run.inputs(i)).clone()
        torch.cuda.synchronize()
        for r, row in enumerate(rows):
            if isinstance(row, tuple):
                assert torch.isnan(out[r]).all(), (i, r)  # skipped: left as it was
            else:
                assert torch.equal(out[r], ref[row]), (i, r)
    for s, e in enumerate(home):
        assert torch.equal(pool.state[e], run.state[s]) and torch.equal(pool.conv[e], run.conv_state[s]), s
    for e in set(range(P)) - set(home):
        assert torch.equal(pool.state[e], before[0][e]) and torch.equal(pool.conv[e], before[1][e]), e


def test_rotating_rows_against_oracle(device):
    case = ki.decode_case(321, 5, 4, 4, "slots-oracle")
    P = 12
    rng = np.random.default_rng(321)
    home = [int(e) for e in rng.permutation(P)[:case.B]]
    print(f"[decode-slots] {case.name} B={case.B} H={case.H} P={P} home={home}", flush=True)
    pool = Pool(case, P, home, device)
    outs = []
    for i in range(case.n_steps):
        rows = [int(s) for s in rng.permutation(case.B)]
        o = pool.step(i, rows).cpu().numpy().reshape(case.B, case.H, D)
        outs.append({s: o[r] for r, s in enumerate(rows)})
    ref = decode_oracle(case, [(b, h) for b in range(case.B) for h in range(case.H)])
    st, cs = pool.state.cpu().numpy(), pool.conv.cpu().numpy()
    worst = 0.0
    for b in range(case.B):
        for h in range(case.H):
            r = ref[(b, h)]
            for i in range(case.n_steps):
                worst = max(worst, slice_rel(outs[i][b][h], r.out[i]))
            worst = max(worst, slice_rel(st[home[b], h], r.state))
            got_c = np.stack([cs[home[b], blk * case.H * D + h * D: blk * case.H * D + (h + 1) * D]
                              for blk in range(3)])
            np.testing.assert_array_equal(got_c, r.conv_state)
    print(f"[decode-slots] {case.name}: max rel err {worst:.3e}", flush=True)
    assert worst <= DECODE_REL_TOL, worst


def test_k3_shape_half_full_pool(device):
    """64 active rows x 96 heads in a pool of 128 entries, against dense decode."""
    case = ki.decode_case(322, 64, 96, 1, "slots-k3")
    P = 128
    home = [int(e) for e in np.random.default_rng(322).permutation(P)[:case.B]]
    print(f"[decode-slots] {case.name} B={case.B} H={case.H} P={P}", flush=True)
    pool = Pool(case, P, home, device)
    out = pool.step(0, list(range(case.B)))
    run = DecodeRun(case, device)
    ref = run.step(run.inputs(0))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    idx = torch.tensor(home, device=device, dtype=torch.long)
    assert torch.equal(pool.state[idx], run.state) and torch.equal(pool.conv[idx], run.conv_state)
