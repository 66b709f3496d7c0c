"""Full-size GPU parity, every (sequence, head) pair against the fp64 oracle:

- the 1 x 8192-token prefill (96 heads) and the 16-sequence varlen prefill (96 heads,
  nonzero initial states), each on both work layouts and in both operand precisions:
  outputs within 2e-2 abs, final states within 5e-3 relative, final conv windows exact,
  and the two layouts bit-identical in each precision;
- the 512 x 96 decode batch over 32 chained steps: every output of every step and the
  final states within 1e-4 relative, final windows exact.

The oracle runs in batches of pairs (threads over pairs), so host memory stays bounded."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from tests.parity import (DECODE_REL_TOL, PATH_CHUNKED, PATH_FUSED, PRECISION_HIGH, PRECISION_STANDARD,
                          PREFILL_OUT_ABS_TOL, PREFILL_STATE_REL_TOL, DecodeRun, _prefill_oracle, decode_oracle,
                          elem_rel, prefill_gpu, slice_rel)

pytestmark = pytest.mark.gpu

D = 128


def _prefill_all_pairs(case, device, batch_pairs):
    H = case.H
    res = {}
    for prec in (PRECISION_STANDARD, PRECISION_HIGH):
        got = {}
        for path in (PATH_FUSED, PATH_CHUNKED):
            print(f"[full] {case.name} path={path} precision={prec} B={case.B} N={case.N} H={H}", flush=True)
            out, fs, fcs = prefill_gpu(case, device, path=path, precision=prec)
            got[path] = (out.cpu().numpy(), fs.cpu().numpy(), fcs.cpu().numpy())
            del out, fs, fcs
        for x, y in zip(got[PATH_FUSED], got[PATH_CHUNKED]):
            assert np.array_equal(x, y)  # the layouts run the same arithmetic in the same order
        res[prec] = got[PATH_FUSED]
    cu = case.cu_seqlens
    pairs = [(s, h) for s in range(case.B) for h in range(H)]
    worst = {p: [0.0, 0.0, 0.0] for p in res}  # output abs, state rel, state elementwise rel
    for i in range(0, len(pairs), batch_pairs):
        chunk = pairs[i:i + batch_pairs]
        ref = _prefill_oracle(case, chunk)
        for prec, (out, fs, fcs) in res.items():
            w = worst[prec]
            for (s, h) in chunk:
                r = ref[(s, h)]
                o = out[cu[s]:cu[s + 1], h * D:(h + 1) * D]
                if o.size:
                    w[0] = max(w[0], float(np.max(np.abs(o - r.out))))
                w[1] = max(w[1], slice_rel(fs[s, h], r.state))
                w[2] = max(w[2], elem_rel(fs[s, h], r.state))
                got_c = np.stack([fcs[s, blk * H * D + h * D: blk * H * D + (h + 1) * D] for blk in range(3)])
                np.testing.assert_array_equal(got_c, r.conv_state)
        del ref
        print(f"[full] {case.name}: {i + len(chunk)}/{len(pairs)} pairs, out abs err / state rel err "
              "(state elementwise rel err): "
              + ", ".join(f"precision {p}: {w[0]:.3e} / {w[1]:.3e} ({w[2]:.3e})" for p, w in worst.items()),
              flush=True)
    for prec, (wo, ws, _) in worst.items():
        assert wo <= PREFILL_OUT_ABS_TOL, (prec, wo)
        assert ws <= PREFILL_STATE_REL_TOL, (prec, ws)


@pytest.mark.timeout(900)
def test_cfg2_every_head_both_layouts(device):
    _prefill_all_pairs(ki.case2_prefill(), device, 16)


@pytest.mark.timeout(1200)
def test_cfg3_every_pair_both_layouts(device):
    _prefill_all_pairs(ki.case3_prefill(), device, 96)


@pytest.mark.timeout(1200)
def test_cfg4_every_pair_32_chained_steps(device):
    case = ki.case4_decode()
    n = case.n_steps
    print(f"[full] {case.name} B={case.B} H={case.H} steps={n}", flush=True)
    case._steps = [case.step(i) for i in range(n)]  # generated once, shared by both sides
    run = DecodeRun(case, device)
    outs = []
    for i in range(n):
        outs.append(run.step(run.inputs(i)).cpu().numpy().reshape(case.B, case.H, D))
    torch.cuda.synchronize()
    st = run.state.cpu().numpy()
    cst = run.conv_state.cpu().numpy()
    del run
    H = case.H
    worst_o, worst_s, worst_e = 0.0, 0.0, 0.0
    per = 32  # sequences per oracle batch
    for b0 in range(0, case.B, per):
        pairs = [(b, h) for b in range(b0, min(case.B, b0 + per)) for h in range(H)]
        ref = decode_oracle(case, pairs, n)
        for (b, h) in pairs:
            r = ref[(b, h)]
            for i in range(n):
                worst_o = max(worst_o, slice_rel(outs[i][b, h], r.out[i]))
                worst_e = max(worst_e, elem_rel(outs[i][b, h], r.out[i]))
            worst_s = max(worst_s, slice_rel(st[b, h], r.state))
            worst_e = max(worst_e, elem_rel(st[b, h], r.state))
            got_c = np.stack([cst[b, blk * H * D + h * D: blk * H * D + (h + 1) * D] for blk in range(3)])
            np.testing.assert_array_equal(got_c, r.conv_state)
        del ref
        print(f"[full] {case.name}: sequences {b0}..{b0 + per - 1}, out rel err {worst_o:.3e}, "
              f"state rel err {worst_s:.3e} (elementwise rel err {worst_e:.3e})", flush=True)
    assert worst_o <= DECODE_REL_TOL, worst_o
    assert worst_s <= DECODE_REL_TOL, worst_s
