#!/usr/bin/env python3
"""Bench of the KDA mixer hot path on one MI355X.

Headline (``value``): decode state bandwidth, GB/s, of ``kda_decode_step`` on 64
sequences x 96 heads (head dim 128, fp32 states), one token per sequence per step.
Beside it, in the same JSON line: the prefill's tokens/s on one 8192-token sequence x 96
heads (bf16 inputs, chunk 64), each with its roofline fraction, and the fp64 CPU oracle
timed on this host on a bounded sample of the same work.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Decode timing rotates three copies of the resident state (3 x 403 MB) so that the
256 MB last-level cache cannot serve a step from the previous one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
D = 128


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


def prefill_bytes(N: int, B: int, H: int, initial: bool) -> int:
    HD = H * D
    tok = (5 * N * HD + N * H) * 2              # bf16 q, k, v, z, g, b
    out = N * HD * 4                             # fp32 out
    states = B * H * D * D * 4 * (2 if initial else 1)
    conv = B * 3 * HD * 3 * 4 * (2 if initial else 1)
    params = (3 * HD * 4 + HD + H + D) * 4
    return tok + out + states + conv + params


ROOT = os.path.dirname(os.path.abspath(__file__))
# the decode kernel's sources: the kernel and the per-token arithmetic it includes
DECODE_SRCS = [os.path.join(ROOT, "gated_delta_rule_31_amd", "csrc", n)
               for n in ("kda_decode.hip", "kda_decode_common.hpp")]
DECODE_PROFILE = os.path.join(ROOT, "profiles", "decode_kernel_64seq_96head.md")


def measured_decode_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None
    if the summary is missing or was taken on a different decode kernel source (the
    sha256 of the kernel's source files, concatenated in DECODE_SRCS order)."""
    import hashlib

    if not os.path.exists(DECODE_PROFILE):
        return None
    vals = {}
    with open(DECODE_PROFILE) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    h = hashlib.sha256()
    for src in DECODE_SRCS:
        with open(src, "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()
    if vals.get("kernel_source_sha256") != sha:
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_digest(name: str):
    """The digest of case `name`'s generated inputs recorded in tests/golden/input_digests.json
    (None if absent)."""
    try:
        with open(os.path.join(ROOT, "tests", "golden", "input_digests.json")) as f:
            return json.load(f).get(name)
    except OSError:
        return None


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bench_decode(args, dev):
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case1_decode()
    B, H = case.B, case.H
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    n_sets = 3
    states = [tt(case.state) for _ in range(n_sets)]
    convs = [tt(case.conv_state) for _ in range(n_sets)]
    x = case.step(0)
    xs = [tt(getattr(x, n)) for n in "qkvzbg"]
    out = torch.empty((B, H * D), dtype=torch.float32, device=dev)

    def launch(i):
        kda.kda_decode_step(cfg, *xs, conv_w, A_log, dt_bias, norm_w, states[i % n_sets], convs[i % n_sets],
                            out=out)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / args.steps
    kern_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    # the same K steps launched as one HIP graph (as a serving loop would replay them):
    # captured and replayed once untimed, then one timed replay
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(args.steps):
                kda.kda_decode_step(cfg, *xs, conv_w, A_log, dt_bias, norm_w, states[i % n_sets],
                                    convs[i % n_sets], out=out, stream=side)
    g.replay()
    torch.cuda.synchronize()
    # the timed replay: wall clock for ms_per_step, and HIP events on the stream the graph
    # is replayed on for the kernels' average duration (the K launches run back to back)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record()
    g.replay()
    g1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kern_graph_ms = g0.elapsed_time(g1) / args.steps
    alg = decode_bytes(B, H)
    state_b = 2 * B * H * D * D * 4
    achieved = alg / (kern_graph_ms * 1e-3) / 1e9
    return dict(
        B=B, H=H, ms_per_step=ms_step, kernel_ms=kern_graph_ms, ms_per_step_eager=ms_eager,
        inputs_sha256=ki.digest(case),
        state_gbs=state_b / (ms_step * 1e-3) / 1e9,
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": "decode_kernel", "alg_bytes_per_launch": alg,
                  "kernel_avg_us": round(kern_graph_ms * 1e3, 2),
                  "kernel_avg_us_eager": round(kern_ms * 1e3, 2),
                  "state_only_frac": round(state_b / (kern_graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    )


def bench_decode_multi(args, dev, T: int):
    """T known tokens per sequence in one kda_decode_multi call, 64 sequences x 96 heads,
    in place, three state sets rotated as in the one-token leg."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case1_decode()
    B, H = case.B, case.H
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
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
    return {"workload": f"kda-decode-multi-64seq-96head-{T}tok", "tokens": T,
            "kernel_avg_us": round(kern_ms * 1e3, 2), "us_per_token": round(kern_ms * 1e3 / T, 2),
            "tokens_per_s": round(B * T / (kern_ms * 1e-3), 1), "alg_bytes_per_launch": alg,
            "hbm_frac": round(alg / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_decode_slots(args, dev):
    """The one-token leg's 64 x 96 workload through kda_decode_step_slots: the 64 rows
    update scattered entries of a 192-entry state pool, a different random set of 64
    entries per launch (three sets rotated, as the dense leg rotates three state sets)."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case1_decode()
    B, H = case.B, case.H
    P = 3 * B
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    st, cs = tt(case.state), tt(case.conv_state)
    pool = torch.cat([st, st, st])
    conv_pool = torch.cat([cs, cs, cs])
    del st, cs
    perm = np.random.default_rng(7).permutation(P).astype(np.int32)
    slot_sets = [tt(perm[j * B:(j + 1) * B]) for j in range(3)]
    x = case.step(0)
    xs = [tt(getattr(x, n)) for n in "qkvzbg"]
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


def bench_decode_cfg4(args, dev):
    """512 sequences x 96 heads (3.2 GB of fp32 states): 32 chained kda_decode_step calls,
    and the same 32 tokens as one kda_decode_multi call."""
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    B, H, T = 512, 96, 32
    case = ki.decode_case(4, B, H, T, "cfg4-decode")
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    conv_w, A_log, dt_bias, norm_w = tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)
    state, conv = tt(case.state), tt(case.conv_state)
    xs = [[tt(getattr(case.step(i), n)) for n in "qkvzbg"] for i in range(T)]
    out = torch.empty((B, H * D), dtype=torch.float32, device=dev)
    # warm-up step, then the 32 chained steps
    kda.kda_decode_step(cfg, *xs[0], conv_w, A_log, dt_bias, norm_w, state, conv, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(T):
        kda.kda_decode_step(cfg, *xs[i], conv_w, A_log, dt_bias, norm_w, state, conv, out=out)
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / T
    alg = decode_bytes(B, H)
    # the same tokens in one call
    mx = [torch.stack([xs[i][j] for i in range(T)], dim=1).contiguous() for j in range(6)]
    del xs
    mout = torch.empty((B, T, H * D), dtype=torch.float32, device=dev)
    kda.kda_decode_multi(cfg, *mx, conv_w, A_log, dt_bias, norm_w, state, conv, out=mout)
    torch.cuda.synchronize()
    e0.record()
    kda.kda_decode_multi(cfg, *mx, conv_w, A_log, dt_bias, norm_w, state, conv, out=mout)
    e1.record()
    torch.cuda.synchronize()
    multi_ms = e0.elapsed_time(e1)
    return {"workload": "kda-decode-512seq-96head-32steps", "step_us": round(step_ms * 1e3, 2),
            "step_hbm_frac": round(alg / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "state_gbs": round(2 * B * H * D * D * 4 / (step_ms * 1e-3) / 1e9, 1),
            "multi_32tok_us": round(multi_ms * 1e3, 2), "multi_us_per_token": round(multi_ms * 1e3 / T, 2)}


def bench_prefill(args, dev):
    import torch

    import kda_inputs as ki
    import gated_delta_rule_31_amd as kda

    case = ki.case2_prefill()
    H = case.H
    path = {"auto": kda.PREFILL_AUTO, "fused": kda.PREFILL_FUSED, "chunked": kda.PREFILL_CHUNKED}[args.prefill_path]
    cfg = kda.KdaConfig(num_heads=H, prefill_path=path)
    p = case.params
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    cu = tt(case.cu_seqlens.astype(np.int32))
    xs = [bf(getattr(case.x, n)) for n in "qkvzbg"]
    prm = [tt(p.conv_w), tt(p.A_log), tt(p.dt_bias), tt(p.norm_w)]
    N = case.N
    out = torch.empty((N, H * D), dtype=torch.float32, device=dev)
    fs = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    fcs = torch.empty((1, 3 * H * D, 3), dtype=torch.float32, device=dev)
    ws_bytes = kda.kda_prefill_workspace_bytes(cfg, 1, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def launch():
        kda.kda_prefill(cfg, cu, *xs, *prm, None, None, out=out, final_state=fs, final_conv_state=fcs,
                        workspace=ws)

    for _ in range(max(1, args.warmup // 2)):
        launch()
    torch.cuda.synchronize()
    n = args.prefill_steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        ev[i][0].record()
        launch()
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / n
    kern_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    flops = prefill_flops([N], H)
    byts = prefill_bytes(N, 1, H, initial=False)
    tf = flops / (kern_ms * 1e-3) / 1e12
    gbs = byts / (kern_ms * 1e-3) / 1e9
    mf, hf = tf / BF16_PEAK_TFLOPS, gbs / HBM_PEAK_GBS
    # the same call with bf16 outputs (kda_config.out_dtype), timed the same way
    cfg16 = kda.KdaConfig(num_heads=H, prefill_path=path, out_dtype=torch.bfloat16)
    out16 = torch.empty((N, H * D), dtype=torch.bfloat16, device=dev)
    launch16 = lambda: kda.kda_prefill(cfg16, cu, *xs, *prm, None, None, out=out16, final_state=fs,
                                       final_conv_state=fcs, workspace=ws)
    launch16()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        launch16()
    e1.record()
    torch.cuda.synchronize()
    ms16 = e0.elapsed_time(e1) / n
    byts16 = byts - N * H * D * 2  # outputs at 2 bytes instead of 4
    return {"workload": "kda-prefill-1x8192tok-96head", "inputs_sha256": ki.digest(case),
            "layout": args.prefill_path if path else
            ("chunked" if ws_bytes else "fused"), "workspace_bytes": ws_bytes,
            "tokens_per_s": round(N / (ms * 1e-3), 1),
            "ms_per_call": round(ms, 4), "kernel_avg_us": round(kern_ms * 1e3, 2),
            "mfma_frac": round(mf, 4), "hbm_frac": round(hf, 4), "roofline_frac": round(max(mf, hf), 4),
            "alg_flops": flops, "alg_bytes": byts, "achieved_tflops": round(tf, 2), "achieved_gbs": round(gbs, 1),
            "bf16_out": {"ms_per_call": round(ms16, 4), "tokens_per_s": round(N / (ms16 * 1e-3), 1),
                         "alg_bytes": byts16, "hbm_frac": round(byts16 / (ms16 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def cpu_baseline(n_steps: int = 16, min_seconds: float = 10.0):
    """The fp64 oracle on this host: ``n_steps`` chained decode steps of all 64 x 96
    (sequence, head) pairs of the decode workload, repeated from the same initial state
    until ``min_seconds`` of work have run."""
    import kda_inputs as ki
    import oracle

    case = ki.case1_decode()
    p = case.params
    cores = len(os.sched_getaffinity(0))
    steps = [case.step(i) if i == 0 else ki.token_inputs(case.seed, case.B, case.H, step=i) for i in range(n_steps)]
    # tokens of sequence b are rows b*n .. b*n+n-1
    tok = {n: np.stack([getattr(x, n) for x in steps], axis=1).reshape(case.B * n_steps, -1) for n in "qkvzbg"}
    cu = np.arange(case.B + 1) * n_steps
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(oracle.MixerConfig(), cu, tok["q"], tok["k"], tok["v"], tok["z"], tok["b"], tok["g"],
                       p.conv_w, p.A_log, p.dt_bias, p.norm_w, case.state, case.conv_state, threads=cores)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    state_b = 2 * case.B * case.H * D * D * 4 * n_steps * reps
    return {"value": round(state_b / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x {n_steps} chained decode steps of all {case.B}x{case.H} (sequence, head) pairs, "
                      f"fp64, {dt:.2f} s"}


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


def bench_copy(args, dev):
    """A plain device-to-device copy of one decode state (402.7 MB read + written): the
    reference for HBM counter readings and achievable bandwidth."""
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--prefill-path", choices=["auto", "fused", "chunked"], default="auto",
                    help="prefill work layout (auto: the library's estimate of the faster one)")
    ap.add_argument("--only", choices=["all", "decode", "decode-multi", "decode-slots", "decode-cfg4", "prefill",
                                       "copy"],
                    default="all",
                    help="run one part only (counter runs under rocprofv3 use this)")
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
    if args.only == "copy":
        print(json.dumps({"copy": bench_copy(args, dev)}), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps({"prefill": bench_prefill(args, dev)}), flush=True)
        return
    if args.only == "decode-cfg4":
        print(json.dumps({"decode_cfg4": bench_decode_cfg4(args, dev)}), flush=True)
        return
    if args.only == "decode-slots":
        print(json.dumps({"decode_slots": bench_decode_slots(args, dev)}), flush=True)
        return
    if args.only == "decode-multi":
        print(json.dumps({"decode_multi": [bench_decode_multi(args, dev, T) for T in (4, 8)]}), flush=True)
        return
    log("decode: 64 seq x 96 heads")
    dec = bench_decode(args, dev)
    log(f"decode: {dec['ms_per_step'] * 1e3:.1f} us/step as a graph, {dec['ms_per_step_eager'] * 1e3:.1f} eager, "
        f"kernel {dec['kernel_ms'] * 1e3:.1f} us")
    dec["roofline"]["traffic"] = measured_decode_traffic()
    multi = slots = None
    if args.only == "all":
        log("decode_multi: 64 seq x 96 heads, 4 and 8 tokens per call")
        multi = [bench_decode_multi(args, dev, T) for T in (4, 8)]
        log(f"decode_multi: {multi}")
        log("decode_slots: 64 rows of a 192-entry pool x 96 heads")
        slots = bench_decode_slots(args, dev)
        log(f"decode_slots: {slots}")
    pre = None
    if args.only == "all" and not args.skip_prefill:
        log("prefill: 1 x 8192 tokens x 96 heads")
        try:
            pre = bench_prefill(args, dev)
            pre["inputs_match_recorded"] = pre["inputs_sha256"] == recorded_digest("cfg2-prefill")
        except Exception as e:  # a prefill failure must not hide the decode line
            pre = {"error": str(e)}
        log(f"prefill: {pre}")
    cpu = None
    if args.only == "all" and not args.skip_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu}")
        if pre is not None and "error" not in pre:
            pre["cpu_baseline"] = cpu_baseline_prefill()
            log(f"cpu baseline prefill: {pre['cpu_baseline']}")
    line = {
        "metric": "KDA decode state GB/s (% HBM peak) + prefill tokens/s (% MFMA), 96 heads",
        "value": round(dec["state_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "ms_per_step_eager": round(dec["ms_per_step_eager"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kda-decode-64seq-96head", "batch": dec["B"], "heads": dec["H"], "head_dim": D,
                   "state_dtype": "f32", "state_sets_rotated": 3, "inputs_sha256": dec["inputs_sha256"],
                   "inputs_match_recorded": dec["inputs_sha256"] == recorded_digest("cfg1-decode"),
                   "timed_as": "one HIP graph replay of the K steps (eager launches: ms_per_step_eager)"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_multi": multi,
        "decode_slots": slots,
        "prefill": pre,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
