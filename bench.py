#!/usr/bin/env python3
"""Bench of the KDA mixer hot path on one MI355X.

Headline (``value``): decode state bandwidth, GB/s, of ``kda_decode_step`` on 512
sequences x 96 heads (head dim 128, 3.2 GB of fp32 states), one token per sequence per
step, K chained steps (default 32, each with its own token inputs).  Beside it, in the
same JSON line: the 64 x 96 decode step, multi-token and pooled decode, the prefill of
one 8192-token sequence and of 16 varlen sequences (96 heads, bf16 inputs, chunk 64),
each with its roofline fraction (and the HBM traffic and MFMA / VALU busy fractions that
rocprofv3 counters measured on the same kernel sources, from ``profiles/``), and the
fp64 CPU oracle timed on this host on a bounded sample of the same work.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Every timed workload's generated inputs are hashed and compared with
``tests/golden/input_digests.json``; a mismatch ends the run with exit status 3.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_VALU_PEAK_TFLOPS = 78.6   # 256 CUs x 4 SIMD x 16 lanes x 2 (FMA) x 2.4 GHz, packed fp32 not used
D = 128
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gated_delta_rule_31_amd", "csrc")


def decode_bytes(B: int, H: int) -> int:
    """Algorithmic HBM bytes of one decode step: every byte the step must move once."""
    HD = H * D
    state = 2 * B * H * D * D * 4            # read + write
    conv = 2 * B * 3 * HD * 3 * 4            # read + write
    tok = (3 * B * HD + 2 * B * HD + B * H) * 4  # q, k, v, z, g, b
    out = B * HD * 4
    params = (3 * HD * 4 + HD + H + D) * 4   # conv_w, dt_bias, A_log, norm_w
    return state + conv + tok + out + params


def decode_multi_bytes(B: int, H: int, T: int) -> int:
    """Algorithmic HBM bytes of one T-token decode call: the state and windows move once,
    the token inputs and outputs once per token."""
    HD = H * D
    state = 2 * B * H * D * D * 4
    conv = 2 * B * 3 * HD * 3 * 4
    tok = T * (3 * B * HD + 2 * B * HD + B * H) * 4
    out = T * B * HD * 4
    params = (3 * HD * 4 + HD + H + D) * 4
    return state + conv + tok + out + params


def chunk_flops(L: int, d: int = D) -> int:
    """Algorithmic FLOPs of one chunk of L tokens for one head (multiply-add = 2;
    masked triangles not counted): A, P, the UT inverse, W and U', the three state
    products, and P.U."""
    return (d * L * (L - 1) + d * L * (L + 1) + (L - 1) * L * (L + 1) // 3 + 2 * d * L * (L + 1) +
            6 * L * d * d + d * L * (L + 1))


def prefill_flops(lengths, H: int, chunk: int = 64) -> int:
    tot = 0
    for n in lengths:
        full, rem = divmod(int(n), chunk)
        tot += full * chunk_flops(chunk) + (chunk_flops(rem) if rem else 0)
    return tot * H


def prefill_bytes(N: int, B: int, H: int, initial: bool, out_bytes: int = 4) -> int:
    HD = H * D
    tok = (5 * N * HD + N * H) * 2              # bf16 q, k, v, z, g, b
    out = N * HD * out_bytes                     # fp32 (or bf16) out
    states = B * H * D * D * 4 * (2 if initial else 1)
    conv = B * 3 * HD * 3 * 4 * (2 if initial else 1)
    params = (3 * HD * 4 + HD + H + D) * 4
    return tok + out + states + conv + params


# ---------------------------------------------------------------- profile summaries
# Each summary under profiles/ ends with "- key: value" lines; the bench takes counter
# figures from one only while its kernel_source_sha256 matches the current sources
# (sha256 of the listed files, concatenated in order), so a figure is never reported
# for a kernel that changed after the counters were taken.

# (each list covers the kernel file and every header it includes)
DECODE_SRCS = ["kda_decode.hip", "kda_decode_common.hpp", "kda_device.hpp", "kda_internal.hpp"]
DECODE_MULTI_SRCS = ["kda_decode_multi.hip", "kda_decode_common.hpp", "kda_device.hpp", "kda_internal.hpp"]
PREFILL_SRCS = ["kda_prefill.hip", "kda_carry.hip", "kda_carry.hpp", "kda_device.hpp", "kda_internal.hpp"]


def sources_sha256(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_values(name: str, srcs) -> dict:
    """The "- key: value" lines of profiles/<name>.md, or {} if the file is missing or was
    written for other kernel sources."""
    path = os.path.join(ROOT, "profiles", name + ".md")
    if not os.path.exists(path):
        return {}
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != sources_sha256(srcs):
        return {}
    out = {}
    for k, v in vals.items():
        try:
            out[k] = int(v)
        except ValueError:
            try:
                out[k] = float(v)
            except ValueError:
                out[k] = v
    return out


def recorded_digest(name: str):
    """The digest of case `name`'s generated inputs recorded in tests/golden/input_digests.json
    (None if absent)."""
    try:
        with open(os.path.join(ROOT, "tests", "golden", "input_digests.json")) as f:
            return json.load(f).get(name)
    except OSError:
        return None


class DigestMismatch(RuntimeError):
    pass


def check_digest(case, name: str) -> str:
    import kda_inputs as ki

    d = ki.digest(case)
    want = recorded_digest(name)
    if d != want:
        raise DigestMismatch(f"inputs of {name} hash to {d}, recorded {want}: the generator changed")
    return d


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _tt(dev):
    import torch
    return lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _bf(dev):
    import torch
    return lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


# ---------------------------------------------------------------- decode legs

_CFG4 = []


def cfg4_case():
    """The headline workload's inputs, generated once (the GPU leg and the CPU baseline
    use the same arrays)."""
    import kda_inputs as ki

    if not _CFG4:
        case = ki.case4_decode()
        case._steps = [case.step(i) for i in range(case.n_steps)]
        _CFG4.append(case)
    return _CFG4[0]


def bench_decode_cfg4(args, dev):
    """The headline: 512 sequences x 96 heads, K chained kda_decode_step calls in place
    (token inputs of step i are the workload's step i mod 32), after W warm-up steps.  The
    K steps run as one HIP graph replay (captured and replayed once before the timed
    replay); ms_per_step is the wall clock of the timed replay over K, the kernel average
    the HIP events around it on the replay stream."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = cfg4_case()
    digest = check_digest(case, "cfg4-decode")
    B, H = case.B, case.H
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = _tt(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    state, conv = tt(case.state), tt(case.conv_state)
    xs = [[tt(getattr(case.step(i), n)) for n in "qkvzbg"] for i in range(case.n_steps)]
    out = torch.empty((B, H * D), dtype=torch.float32, device=dev)

    def launch(i, stream=None):
        kda.kda_decode_step(cfg, *xs[i % len(xs)], conv_w, A_log, dt_bias, norm_w, state, conv, out=out,
                            stream=stream)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    # eager launches, one event pair each (includes launch gaps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    kern_eager = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(args.steps):
                launch(i, stream=side)
    g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    g.replay()
    g1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = g0.elapsed_time(g1) / args.steps
    alg = decode_bytes(B, H)
    state_b = 2 * B * H * D * D * 4
    achieved = alg / (kern_ms * 1e-3) / 1e9
    prof = profile_values("decode_kernel_512seq_96head", DECODE_SRCS)
    traffic = prof.get("hbm_bytes_per_launch")
    return dict(
        B=B, H=H, ms_per_step=ms_step, inputs_sha256=digest,
        state_gbs=state_b / (ms_step * 1e-3) / 1e9,
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                  "traffic_over_alg": round(traffic / alg, 4) if traffic else None,
                  "kernel": "decode_kernel", "alg_bytes_per_launch": alg,
                  "kernel_avg_us": round(kern_ms * 1e3, 2), "kernel_avg_us_eager": round(kern_eager * 1e3, 2),
                  "state_only_frac": round(state_b / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    )


def bench_decode_cfg1(args, dev):
    """64 sequences x 96 heads, one step; three state sets (3 x 403 MB) rotate so that the
    256 MB last-level cache cannot serve a step from the previous one."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case1_decode()
    digest = check_digest(case, "cfg1-decode")
    B, H = case.B, case.H
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = _tt(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    n_sets = 3
    states = [tt(case.state) for _ in range(n_sets)]
    convs = [tt(case.conv_state) for _ in range(n_sets)]
    xs = [tt(getattr(case.step(0), n)) for n in "qkvzbg"]
    out = torch.empty((B, H * D), dtype=torch.float32, device=dev)
    steps = max(10, args.steps)

    def launch(i, stream=None):
        kda.kda_decode_step(cfg, *xs, conv_w, A_log, dt_bias, norm_w, states[i % n_sets], convs[i % n_sets],
                            out=out, stream=stream)

    for i in range(args.warmup):
        launch(i)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                launch(i, stream=side)
    g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    g.replay()
    g1.record()
    torch.cuda.synchronize()
    kern_ms = g0.elapsed_time(g1) / steps
    alg = decode_bytes(B, H)
    prof = profile_values("decode_kernel_64seq_96head", DECODE_SRCS)
    return {"workload": "kda-decode-64seq-96head", "inputs_sha256": digest, "kernel_avg_us": round(kern_ms * 1e3, 2),
            "state_gbs": round(2 * B * H * D * D * 4 / (kern_ms * 1e-3) / 1e9, 1), "alg_bytes_per_launch": alg,
            "hbm_frac": round(alg / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": prof.get("hbm_bytes_per_launch")}


def bench_decode_multi(args, dev, T: int, form: int = 0):
    """T known tokens per sequence in one kda_decode_multi call, 64 sequences x 96 heads,
    in place, three state sets rotated as in the one-token leg; form: the call's
    decode_multi_form (0: blocks of eight tokens, the default; 1: token by token)."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case1_decode()
    B, H = case.B, case.H
    cfg = kda.KdaConfig(num_heads=H, decode_multi_form=form)
    p = case.params
    tt = _tt(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    n_sets = 3
    states = [tt(case.state) for _ in range(n_sets)]
    convs = [tt(case.conv_state) for _ in range(n_sets)]
    steps = [ki.token_inputs(case.seed, B, H, step=i) for i in range(T)]
    xs = [tt(np.stack([getattr(x, n) for x in steps], axis=1)) for n in "qkvzbg"]
    out = torch.empty((B, T, H * D), dtype=torch.float32, device=dev)

    def launch(i):
        kda.kda_decode_multi(cfg, *xs, conv_w, A_log, dt_bias, norm_w, states[i % n_sets], convs[i % n_sets],
                             out=out)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    n = max(5, args.steps // 2)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    kern_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    alg = decode_multi_bytes(B, H, T)
    res = {"workload": f"kda-decode-multi-64seq-96head-{T}tok" + ("-sequential" if form else ""), "tokens": T,
           "form": "sequential" if form else "block",
           "kernel_avg_us": round(kern_ms * 1e3, 2), "us_per_token": round(kern_ms * 1e3 / T, 2),
           "tokens_per_s": round(B * T / (kern_ms * 1e-3), 1), "alg_bytes_per_launch": alg,
           "hbm_frac": round(alg / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if T == 8 and not form:
        # HBM bytes and busy fractions from the rocprofv3 summary of this leg, while its
        # kernel sources are the ones measured
        prof = profile_values("decode_multi_kernel_64seq_96head_8tok", DECODE_MULTI_SRCS)
        res["traffic"] = prof.get("hbm_bytes_per_call")
        res["mfma_busy_frac"] = prof.get("mfma_busy_frac")
        res["valu_issue_frac"] = prof.get("valu_issue_frac")
    return res


def bench_decode_slots(args, dev):
    """The 64 x 96 one-token step through kda_decode_step_slots: the 64 rows update
    scattered entries of a 192-entry state pool, a different random set of 64 entries per
    launch (three sets rotated, as the dense leg rotates three state sets)."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case1_decode()
    B, H = case.B, case.H
    P = 3 * B
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = _tt(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    st, cs = tt(case.state), tt(case.conv_state)
    pool = torch.cat([st, st, st])
    conv_pool = torch.cat([cs, cs, cs])
    del st, cs
    perm = np.random.default_rng(7).permutation(P).astype(np.int32)
    slot_sets = [tt(perm[j * B:(j + 1) * B]) for j in range(3)]
    xs = [tt(getattr(case.step(0), n)) for n in "qkvzbg"]
    out = torch.empty((B, H * D), dtype=torch.float32, device=dev)

    def launch(i):
        kda.kda_decode_step_slots(cfg, slot_sets[i % 3], *xs, conv_w, A_log, dt_bias, norm_w, pool, conv_pool,
                                  out=out)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    n = max(5, args.steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    kern_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    alg = decode_bytes(B, H)
    return {"workload": "kda-decode-slots-64rows-192pool-96head", "kernel_avg_us": round(kern_ms * 1e3, 2),
            "hbm_frac": round(alg / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- prefill legs

PREFILL_WORKLOADS = {
    # name: (case factory, digest name, profile summary, workload label)
    "cfg2": ("case2_prefill", "cfg2-prefill", "prefill_1x8192tok_96head", "kda-prefill-1x8192tok-96head"),
    "cfg3": ("case3_prefill", "cfg3-prefill", "prefill_16seq_varlen_96head", "kda-prefill-16seq-varlen-96head"),
}


def prefill_warmup(args) -> int:
    """Untimed calls before each prefill leg's timed ones.  The GPU comes to each leg from
    host-side input generation, and its per-call time keeps falling over the first ten to
    fifteen calls (1.24 -> 1.05 ms on the 8192-token workload), so a leg warms up with at
    least ten calls."""
    return max(10, args.warmup)


def bench_prefill(args, dev, which: str, with_bf16_out: bool = False, with_precise: bool = False):
    """One kda_prefill call on the workload (inputs resident in HBM, outputs, final states
    and the workspace allocated before the timed calls), the layout the library picks
    unless --prefill-path forces one; HIP events around each of n calls."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    factory, dname, pname, label = PREFILL_WORKLOADS[which]
    case = getattr(ki, factory)()
    digest = check_digest(case, dname)
    H, B, N = case.H, case.B, case.N
    path = {"auto": kda.PREFILL_AUTO, "fused": kda.PREFILL_FUSED, "chunked": kda.PREFILL_CHUNKED}[args.prefill_path]
    cfg = kda.KdaConfig(num_heads=H, prefill_path=path)
    p = case.params
    tt, bf = _tt(dev), _bf(dev)
    cu = tt(case.cu_seqlens.astype(np.int32))
    xs = [bf(getattr(case.x, n)) for n in "qkvzbg"]
    prm = [tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)]
    s0 = tt(case.initial_state) if case.initial_state is not None else None
    c0 = tt(case.initial_conv_state) if case.initial_conv_state is not None else None
    lengths = np.diff(case.cu_seqlens)
    initial = case.initial_state is not None
    del case
    out = torch.empty((N, H * D), dtype=torch.float32, device=dev)
    fs = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    fcs = torch.empty((B, 3 * H * D, 3), dtype=torch.float32, device=dev)
    ws_bytes = kda.kda_prefill_workspace_bytes(cfg, B, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def timed(c, o, w=None):
        wsp = ws if w is None else w
        call = lambda: kda.kda_prefill(c, cu, *xs, *prm, s0, c0, out=o, final_state=fs, final_conv_state=fcs,
                                       workspace=wsp)
        for _ in range(prefill_warmup(args)):
            call()
        torch.cuda.synchronize()
        n = args.prefill_steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        t0 = time.perf_counter()
        for i in range(n):
            ev[i][0].record()
            call()
            ev[i][1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per = [s.elapsed_time(e) for s, e in ev]
        log(f"prefill {which}: per-call ms {[round(x, 4) for x in per]}")
        return (t1 - t0) * 1e3 / n, float(np.mean(per))

    ms, kern_ms = timed(cfg, out)
    flops = prefill_flops(lengths, H)
    byts = prefill_bytes(N, B, H, initial=initial)
    tf = flops / (kern_ms * 1e-3) / 1e12
    gbs = byts / (kern_ms * 1e-3) / 1e9
    mf, hf = tf / BF16_PEAK_TFLOPS, gbs / HBM_PEAK_GBS
    layout = args.prefill_path if path else ("chunked" if ws_bytes else "fused")
    prof = profile_values(f"{pname}_{layout}", PREFILL_SRCS)
    traffic = prof.get("hbm_bytes_per_call")
    res = {"workload": label, "sequences": int(B), "tokens": int(N), "inputs_sha256": digest, "layout": layout,
           "workspace_bytes": ws_bytes, "tokens_per_s": round(N / (kern_ms * 1e-3), 1),
           "ms_per_call": round(kern_ms, 4), "ms_per_call_wall": round(ms, 4),
           "mfma_frac": round(mf, 4), "hbm_frac": round(hf, 4), "roofline_frac": round(max(mf, hf), 4),
           "alg_flops": flops, "alg_bytes": byts, "achieved_tflops": round(tf, 2), "achieved_gbs": round(gbs, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(hf, 4), "traffic": traffic,
                        "traffic_over_alg": round(traffic / byts, 4) if traffic else None},
           "counters": {k: prof[k] for k in prof if k.endswith("_frac") or k.endswith("_us")} or None}
    if with_bf16_out:
        cfg16 = kda.KdaConfig(num_heads=H, prefill_path=path, out_dtype=torch.bfloat16)
        out16 = torch.empty((N, H * D), dtype=torch.bfloat16, device=dev)
        _, ms16 = timed(cfg16, out16)
        byts16 = prefill_bytes(N, B, H, initial=initial, out_bytes=2)
        res["bf16_out"] = {"ms_per_call": round(ms16, 4), "tokens_per_s": round(N / (ms16 * 1e-3), 1),
                           "alg_bytes": byts16, "hbm_frac": round(byts16 / (ms16 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if with_precise:
        # the opt-in high-precision mode (every MFMA operand of the chunk algebra split hi + lo),
        # same workload, with its own workspace (larger chunk records)
        cfgp = kda.KdaConfig(num_heads=H, prefill_path=path, precision=kda.PRECISION_HIGH)
        wsp_bytes = kda.kda_prefill_workspace_bytes(cfgp, B, N)
        wsp = torch.empty(wsp_bytes, dtype=torch.uint8, device=dev) if wsp_bytes else None
        _, msp = timed(cfgp, out, wsp)
        res["precision_high"] = {"ms_per_call": round(msp, 4), "tokens_per_s": round(N / (msp * 1e-3), 1),
                                 "workspace_bytes": wsp_bytes, "vs_standard": round(msp / kern_ms, 3),
                                 "hbm_frac": round(byts / (msp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def bench_prefill_gate_proj(args, dev):
    """The one-sequence prefill (8192 tokens, 96 heads) through kda_prefill_gate_proj: the
    decay logits formed inside from f = W_fa x [8192, 128] and W_fb [12288, 128] (bf16)
    instead of read as z [8192, 12288]."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case2_prefill()
    H, B, N = case.H, case.B, case.N
    f, w_fb = ki.lowrank_gate(case.seed, N, H)
    path = {"auto": kda.PREFILL_AUTO, "fused": kda.PREFILL_FUSED, "chunked": kda.PREFILL_CHUNKED}[args.prefill_path]
    cfg = kda.KdaConfig(num_heads=H, prefill_path=path)
    p = case.params
    tt, bf = _tt(dev), _bf(dev)
    cu = tt(case.cu_seqlens.astype(np.int32))
    xs = {n: bf(getattr(case.x, n)) for n in "qkvbg"}
    fd, wd = bf(f), bf(w_fb)
    prm = [tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)]
    del case
    out = torch.empty((N, H * D), dtype=torch.float32, device=dev)
    fs = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    fcs = torch.empty((B, 3 * H * D, 3), dtype=torch.float32, device=dev)
    ws_bytes = kda.kda_prefill_workspace_bytes(cfg, B, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    call = lambda: kda.kda_prefill_gate_proj(cfg, cu, xs["q"], xs["k"], xs["v"], fd, wd, xs["b"], xs["g"], *prm,
                                             None, None, out=out, final_state=fs, final_conv_state=fcs, workspace=ws)
    for _ in range(prefill_warmup(args)):
        call()
    torch.cuda.synchronize()
    n = args.prefill_steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        call()
        ev[i][1].record()
    torch.cuda.synchronize()
    kern_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    # algorithmic bytes: z [N, H*D] replaced by f [N, 128] and W_fb [H*D, 128]
    byts = prefill_bytes(N, B, H, initial=False) - N * H * D * 2 + N * 128 * 2 + H * D * 128 * 2
    flops = prefill_flops([N], H) + 2 * N * H * D * 128  # plus z = W_fb f
    return {"workload": "kda-prefill-gate-proj-1x8192tok-96head", "layout": "chunked" if ws_bytes else "fused",
            "ms_per_call": round(kern_ms, 4), "tokens_per_s": round(N / (kern_ms * 1e-3), 1), "alg_bytes": byts,
            "alg_flops": flops, "hbm_frac": round(byts / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def bench_copy(args, dev):
    """A plain device-to-device copy of 402,653,184 bytes: the calibration of the HBM
    traffic counters and a reference for achievable bandwidth."""
    import torch

    n = 64 * 96 * D * D
    src = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        dst.copy_(src)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return {"bytes_per_copy": 2 * n * 4, "kernel_avg_us": round(ms * 1e3, 2),
            "gbs": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_decode(case, seqs, n_steps, threads):
    """The oracle over n_steps chained decode steps of every head of the given sequences;
    returns the seconds it took."""
    import oracle

    p = case.params
    steps = [case.step(i) for i in range(n_steps)]
    tok = {n: np.stack([getattr(x, n)[seqs] for x in steps], axis=1).reshape(len(seqs) * n_steps, -1)
           for n in "qkvzbg"}
    cu = np.arange(len(seqs) + 1) * n_steps
    t0 = time.perf_counter()
    oracle.forward(oracle.MixerConfig(), cu, tok["q"], tok["k"], tok["v"], tok["z"], tok["b"], tok["g"],
                   p.conv_w, p.A_log, p.dt_bias, p.norm_w, case.state[seqs], case.conv_state[seqs],
                   threads=threads)
    return time.perf_counter() - t0


def cpu_baseline(min_seconds: float = 10.0):
    """The fp64 oracle on this host's cores, on the headline workload: all 96 heads of
    blocks of 16 of the 512 sequences over the workload's 32 chained steps, until
    ``min_seconds`` have run; as state GB/s (the state bytes a GPU step moves per
    (sequence, head) and token).  Beside it, one thread on the 64-step 4-head sequence
    and on the 64 x 96 one-step workload."""
    import kda_inputs as ki

    cores = len(os.sched_getaffinity(0))
    case = cfg4_case()
    per = 16
    done, dt = 0, 0.0
    while dt < min_seconds and done < case.B:
        seqs = list(range(done, min(case.B, done + per)))
        dt += _oracle_decode(case, seqs, case.n_steps, cores)
        done += len(seqs)
    tok_heads = done * case.H * case.n_steps
    res = {"value": round(2 * D * D * 4 * tok_heads / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{done} of 512 sequences x 96 heads x 32 chained decode steps, fp64, {dt:.2f} s on "
                     f"{cores} threads"}
    single = {}
    c0 = ki.case0_decode()
    t0 = _oracle_decode(c0, [0], c0.n_steps, 1)
    single["cfg0"] = {"workload": "1 sequence x 4 heads x 64 decode steps", "seconds": round(t0, 4),
                      "token_heads_per_s": round(4 * 64 / t0, 1)}
    c1 = ki.case1_decode()
    t1 = _oracle_decode(c1, list(range(c1.B)), 1, 1)
    single["cfg1"] = {"workload": "64 sequences x 96 heads x 1 decode step", "seconds": round(t1, 4),
                      "state_gbs": round(2 * D * D * 4 * c1.B * c1.H / t1 / 1e9, 4)}
    res["single_thread"] = single
    return res


def cpu_baseline_prefill(heads_per_batch: int = 4, min_seconds: float = 5.0):
    """The fp64 oracle on this host: batches of heads of the 8192-token prefill until
    ``min_seconds`` of work have run; scaled to 96 heads."""
    import kda_inputs as ki
    import oracle

    case = ki.case2_prefill()
    p = case.params
    cores = len(os.sched_getaffinity(0))
    x = case.x
    done = 0
    t0 = time.perf_counter()
    while done < case.H:
        pairs = [(0, h) for h in range(done, min(case.H, done + heads_per_batch))]
        oracle.forward(oracle.MixerConfig(), case.cu_seqlens, x.q, x.k, x.v, x.z, x.b, x.g, p.conv_w, p.A_log,
                       p.dt_bias, p.norm_w, pairs=pairs, threads=cores, decode=ki.bf16_bits_to_f32)
        done += len(pairs)
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(case.N * done / case.H / dt, 1), "unit": "tokens/s (96 heads)", "cores": cores,
            "kind": "oracle", "sample": f"{done} of 96 heads x {case.N} tokens, fp64, {dt:.2f} s; scaled to 96 heads"}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32, help="timed decode steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-steps", type=int, default=10, help="timed calls of each prefill leg")
    ap.add_argument("--prefill-path", choices=["auto", "fused", "chunked"], default="auto",
                    help="prefill work layout (auto: the library's estimate of the faster one)")
    ap.add_argument("--only", choices=["all", "decode-cfg4", "decode-cfg1", "decode-multi", "decode-multi-8",
                                       "decode-slots", "prefill-cfg2", "prefill-cfg3", "prefill-gate-proj", "copy"],
                    default="all", help="run one part only (counter runs under rocprofv3 use this)")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the KDA decode and prefill paths here run on a single MI355X "
              "and have no multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(0)}")
    try:
        single = {"copy": lambda: bench_copy(args, dev),
                  "decode-cfg4": lambda: bench_decode_cfg4(args, dev),
                  "decode-cfg1": lambda: bench_decode_cfg1(args, dev),
                  "decode-slots": lambda: bench_decode_slots(args, dev),
                  "decode-multi": lambda: [bench_decode_multi(args, dev, T) for T in (4, 8)]
                                          + [bench_decode_multi(args, dev, 8, form=1)],
                  "decode-multi-8": lambda: bench_decode_multi(args, dev, 8),
                  "prefill-cfg2": lambda: bench_prefill(args, dev, "cfg2"),
                  "prefill-cfg3": lambda: bench_prefill(args, dev, "cfg3"),
                  "prefill-gate-proj": lambda: bench_prefill_gate_proj(args, dev)}
        if args.only != "all":
            print(json.dumps({args.only: single[args.only]()}), flush=True)
            return
        log("decode: 512 seq x 96 heads, chained steps (headline)")
        dec = bench_decode_cfg4(args, dev)
        log(f"decode: {dec['ms_per_step'] * 1e3:.1f} us/step, kernel {dec['roofline']['kernel_avg_us']} us, "
            f"{dec['roofline']['frac']:.4f} of HBM peak")
        log("decode: 64 seq x 96 heads")
        dec1 = bench_decode_cfg1(args, dev)
        log(f"decode cfg1: {dec1}")
        log("decode_multi: 64 seq x 96 heads, 4 and 8 tokens per call")
        multi = [bench_decode_multi(args, dev, T) for T in (4, 8)] + [bench_decode_multi(args, dev, 8, form=1)]
        log(f"decode_multi: {multi}")
        log("decode_slots: 64 rows of a 192-entry pool x 96 heads")
        slots = bench_decode_slots(args, dev)
        log(f"decode_slots: {slots}")
        pre2 = pre3 = None
        if not args.skip_prefill:
            log("prefill: 1 x 8192 tokens x 96 heads")
            pre2 = bench_prefill(args, dev, "cfg2", with_bf16_out=True, with_precise=True)
            log(f"prefill cfg2: {pre2}")
            log("prefill: 16 varlen sequences x 96 heads")
            pre3 = bench_prefill(args, dev, "cfg3")
            log(f"prefill cfg3: {pre3}")
            log("prefill with the decay projection inside: 1 x 8192 tokens x 96 heads")
            pre2["gate_proj"] = bench_prefill_gate_proj(args, dev)
            log(f"prefill gate_proj: {pre2['gate_proj']}")
    except DigestMismatch as e:
        print(f"bench.py: {e}", file=sys.stderr, flush=True)
        sys.exit(3)
    cpu = None
    if not args.skip_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu}")
        if pre2 is not None:
            pre2["cpu_baseline"] = cpu_baseline_prefill()
            log(f"cpu baseline prefill: {pre2['cpu_baseline']}")
    line = {
        "metric": "KDA decode state GB/s (% HBM peak) + prefill tokens/s (% MFMA), 96 heads",
        "value": round(dec["state_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kda-decode-512seq-96head-32steps", "batch": dec["B"], "heads": dec["H"],
                   "head_dim": D, "state_dtype": "f32", "inputs_sha256": dec["inputs_sha256"],
                   "inputs_match_recorded": True,
                   "timed_as": "one HIP graph replay of the K chained steps, in place"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_cfg1": dec1,
        "decode_multi": multi,
        "decode_slots": slots,
        "prefill": pre2,
        "prefill_varlen": pre3,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
