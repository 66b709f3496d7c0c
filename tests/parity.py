"""Shared helpers of the GPU parity tests: upload seeded cases, run the oracle on the
same inputs, and the error metrics the tolerances are stated in.

Metrics (per (sequence, head) slice):
  rel  = max|x - r| / max|r|          -- "max relative error" (decode: 1e-4; prefill states: 5e-3)
  abs  = max|x - r|                   -- "max abs error" (prefill outputs: 2e-2)
  elem = max |x - r| / max(|r|, 1e-3 max|r|)  -- elementwise, reported beside them
"""
from __future__ import annotations

import numpy as np
import torch

import kda_inputs as ki
import oracle

D = 128

DECODE_REL_TOL = 1e-4        # fp32 decode: outputs and states
PREFILL_OUT_ABS_TOL = 2e-2   # bf16-input chunked prefill: gated RMS-normalised outputs
PREFILL_STATE_REL_TOL = 5e-3  # bf16-input chunked prefill: final states


def slice_rel(x: np.ndarray, r: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(x - r)) / den) if den > 0 else float(np.max(np.abs(x)))


def elem_rel(x: np.ndarray, r: np.ndarray) -> float:
    """The elementwise relative error reported beside slice_rel (no bound is stated for it):
    max |x - r| / max(|r|, 1e-3 max|r|) over the slice."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    floor = 1e-3 * np.max(np.abs(r))
    if floor == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), floor)))


def t(a, dev, dtype=None):
    """numpy -> device tensor (uint16 arrays become bf16)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    x = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return x if dtype is None else x.to(dtype)


def oracle_cfg() -> oracle.MixerConfig:
    return oracle.MixerConfig(head_dim=D, conv_size=4, gate_lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-5)


# ------------------------------------------------------------------------------- decode

def decode_oracle(case: ki.DecodeCase, pairs, n_steps: int | None = None):
    """The oracle over ``n_steps`` decode steps for the given (sequence, head) pairs:
    each sequence's steps form a token sequence.  Returns {(b, h): PairResult}."""
    n = case.n_steps if n_steps is None else n_steps
    seqs = sorted({b for b, _ in pairs})
    H = case.H
    # gather, per needed sequence, its n tokens: rows ordered [seq][step]
    rows = {name: [] for name in "qkvzbg"}
    for i in range(n):
        x = case.step(i)
        for name in "qkvzbg":
            rows[name].append(getattr(x, name)[seqs])
    stacked = {name: np.stack(rows[name], axis=1).reshape(len(seqs) * n, -1) for name in rows}
    cu = np.arange(len(seqs) + 1) * n
    idx = {b: j for j, b in enumerate(seqs)}
    sub_pairs = [(idx[b], h) for b, h in pairs]
    p = case.params
    res = oracle.forward(oracle_cfg(), cu, stacked["q"], stacked["k"], stacked["v"], stacked["z"],
                         stacked["b"], stacked["g"], p.conv_w, p.A_log, p.dt_bias, p.norm_w,
                         case.state[seqs], case.conv_state[seqs], pairs=sub_pairs)
    return {(b, h): res[(idx[b], h)] for b, h in pairs}


class DecodeRun:
    """A decode case resident on the GPU."""

    def __init__(self, case: ki.DecodeCase, dev):
        import gated_delta_rule_31_amd as kda
        self.kda = kda
        self.case = case
        self.dev = dev
        self.cfg = kda.KdaConfig(num_heads=case.H)
        p = case.params
        self.conv_w, self.A_log = t(p.conv_w, dev), t(p.A_log, dev)
        self.dt_bias, self.norm_w = t(p.dt_bias, dev), t(p.norm_w, dev)
        self.state = t(case.state, dev)
        self.conv_state = t(case.conv_state, dev)

    def inputs(self, i: int):
        x = self.case.step(i)
        return [t(getattr(x, n), self.dev) for n in "qkvzbg"]

    def step(self, xs, out=None, stream=None):
        return self.kda.kda_decode_step(self.cfg, *xs, self.conv_w, self.A_log, self.dt_bias, self.norm_w,
                                        self.state, self.conv_state, out=out, stream=stream)


# ------------------------------------------------------------------------------- prefill

_ORACLE_CACHE: dict = {}


def prefill_oracle(case: ki.PrefillCase, pairs=None):
    """The oracle on the case's bf16 activations (their exact values) for the pairs
    (memoised per case name, seed and pairs: the tests run each case on both layouts)."""
    key = (case.name, case.seed, case.H, tuple(case.cu_seqlens.tolist()), None if pairs is None else tuple(pairs))
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = _prefill_oracle(case, pairs)
    return _ORACLE_CACHE[key]


def _prefill_oracle(case: ki.PrefillCase, pairs=None):
    x = case.x
    p = case.params
    return oracle.forward(oracle_cfg(), case.cu_seqlens, x.q, x.k, x.v, x.z, x.b, x.g, p.conv_w, p.A_log,
                          p.dt_bias, p.norm_w, case.initial_state, case.initial_conv_state, pairs=pairs,
                          decode=ki.bf16_bits_to_f32)


def check_prefill(case: ki.PrefillCase, out, fs, fcs, pairs):
    """Compare GPU prefill results with the oracle on (sequence, head) pairs.  Returns
    (max output abs error, max state rel error)."""
    ref = prefill_oracle(case, pairs)
    cu = case.cu_seqlens
    H = case.H
    out_np = out.cpu().numpy() if hasattr(out, "cpu") else out
    fs_np = fs.cpu().numpy() if hasattr(fs, "cpu") else fs
    fcs_np = fcs.cpu().numpy() if hasattr(fcs, "cpu") else fcs
    worst_o, worst_s = 0.0, 0.0
    for (s, h) in pairs:
        r = ref[(s, h)]
        o = out_np[cu[s]:cu[s + 1], h * D:(h + 1) * D]
        if o.size:
            worst_o = max(worst_o, float(np.max(np.abs(o - r.out))))
        worst_s = max(worst_s, slice_rel(fs_np[s, h], r.state))
        got_c = np.stack([fcs_np[s, blk * H * D + h * D: blk * H * D + (h + 1) * D] for blk in range(3)])
        np.testing.assert_array_equal(got_c, r.conv_state)  # the window is copied, exact
    return worst_o, worst_s


# kda_config.prefill_path values (kda.PREFILL_*), spelled out so that collecting the
# tests does not need the library
PATH_AUTO, PATH_FUSED, PATH_CHUNKED = 0, 1, 2


PRECISION_STANDARD, PRECISION_HIGH = 0, 1


def prefill_gpu(case: ki.PrefillCase, dev, in_place: bool = False, path: int = PATH_AUTO,
                precision: int = PRECISION_STANDARD, out_dtype=None):
    import gated_delta_rule_31_amd as kda
    cfg = kda.KdaConfig(num_heads=case.H, prefill_path=path, precision=precision,
                        **({} if out_dtype is None else {"out_dtype": out_dtype}))
    p = case.params
    cu = t(case.cu_seqlens.astype(np.int32), dev)
    xs = [t(getattr(case.x, n), dev) for n in "qkvzbg"]
    st = t(case.initial_state, dev)
    cst = t(case.initial_conv_state, dev)
    kw = {}
    if in_place:
        kw = dict(final_state=st, final_conv_state=cst)
    out, fs, fcs = kda.kda_prefill(cfg, cu, *xs, t(p.conv_w, dev), t(p.A_log, dev), t(p.dt_bias, dev),
                                   t(p.norm_w, dev), st, cst, **kw)
    torch.cuda.synchronize()
    return out, fs, fcs
