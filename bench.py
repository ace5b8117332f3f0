"""Throughput of the CKDA hot path on one MI355X.

A step is one chunked forward, i.e. one ckda_fwd_chunked call: the
chunk-local kernel (gate/sign-fold prep, intra-chunk products, UT/WY
substitution, over every (chunk, head) at once) followed by the
state-passing kernel (state products, output, state update, chunk by
chunk), over the mixer workload of the 1.36B model: B=8, T=4096, H=16,
dk=dv=128, bf16 q/k/v, fp32 gates, state and outputs.  The JSON line's ``value`` is that forward's
tokens/s; the decode workload (256 sequences x 16 heads, 512 recurrent
steps) is reported in the same line as state-streaming GB/s, the backward as
tokens/s, and the same forward with one gate per (token, head), and with
raw q and k that the path L2-normalises itself, as tokens/s; the forward
over few long chains (varlen_64k, long_64k) with and without the segmented
state pass, and the long_64k backward with and without the segmented
reverse pass.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--only fwd|fwd_head_gate|fwd_qk_norm|fwd_long|bwd_long|decode|bwd|options|copy|conv]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix peak
METRIC = "CKDA chunked fwd tokens/s (H16,d128,T4096) + decode GB/s; % of roofline"

# algorithmic bytes per token-head of the forward: q,k,v bf16 (768) + g f32 (512)
# + s int8 (128) + beta f32 (4) + o f32 (512)
FWD_BYTES_PER_TOKEN_HEAD = 768 + 512 + 128 + 4 + 512
# algorithmic flops per token-head of the 64-token chunked method (dense count)
FWD_FLOPS_PER_TOKEN_HEAD = 181.6e3
# decode, per head-step: state read+write (2*64 KiB) + q,k,v bf16 + g + s +
# sign_prod read+write + beta + o
DEC_BYTES_PER_HEAD_STEP = 2 * 128 * 128 * 4 + 3 * 256 + 512 + 128 + 2 * 128 + 4 + 512


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ckda_fwd_traffic__layer_bf16.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_traffic__decode_b256.json")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ckda_bwd_traffic__layer_bwd.json")


def measured_traffic(path=None):
    """HBM bytes per call (forward, the default record; backward) or per step (decode)
    from the committed FETCH_SIZE / WRITE_SIZE runs (calibrated on a plain
    copy), or None when the kernel sources have changed since those counters
    were taken."""
    import hashlib
    path = TRAFFIC_FILE if path is None else path
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        with open(os.path.join(ROOT, "gated_delta_rule_sign_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return float(rec["traffic_bytes_per_call"])


MFMA_FILE = os.path.join(ROOT, "profiles", "ckda_fwd_mfma__layer_bf16.json")


def measured_mfma():
    """Executed bf16 matrix-core flops per forward call and per kernel
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 from the committed counter run), or
    None when the forward kernel sources have changed since then."""
    import hashlib
    try:
        rec = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        with open(os.path.join(ROOT, "gated_delta_rule_sign_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev_tensor(torch, arr):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if arr.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to("cuda:0")


def time_kernel_launches(torch, fn, steps, warmup):
    """Run fn warmup+steps times; time the steps with HIP events on the
    current stream (the stream the library launches on).  Returns (total
    wall ms, per-launch event ms list)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return wall, [a.elapsed_time(b) for a, b in evs]


# head-scalar gate: g f32 and s int8 once per token-head (5 bytes instead of 640)
FWD_HG_BYTES_PER_TOKEN_HEAD = 768 + 4 + 1 + 4 + 512


def bench_fwd(torch, steps, warmup, workload="layer_bf16"):
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    log(f"generating {workload} inputs")
    w = I.make_workload(workload)
    tok = w.tok
    d = {k: dev_tensor(torch, getattr(tok, k)) for k in ("q", "k", "v", "g", "s", "beta")}
    B, T, H, DK = tok.q.shape
    o = torch.empty((B, T, H, 128), dtype=torch.float32, device="cuda:0")
    ht = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(ckda.fwd_workspace_bytes(B, T, H, DK, 128, torch.bfloat16), dtype=torch.uint8,
                     device="cuda:0")
    qk_norm = w.cfg.get("qk") == "raw"   # raw q, k: the path normalises them
    fn = lambda: ckda.fwd(**d, o=o, ht=ht, workspace=ws, qk_norm=qk_norm)
    log("timing forward")
    wall, per = time_kernel_launches(torch, fn, steps, warmup)
    tokens = B * T
    th = B * T * H
    ms = wall / steps
    avg_launch = float(np.mean(per))
    per_th = FWD_HG_BYTES_PER_TOKEN_HEAD if tok.g.ndim == 3 else FWD_BYTES_PER_TOKEN_HEAD
    return dict(w=w, tokens=tokens, ms=ms, launch_ms=avg_launch, launch_all=per,
                bytes=th * per_th, flops=th * FWD_FLOPS_PER_TOKEN_HEAD,
                workspace_bytes=int(ws.numel()))


def bench_fwd_long(torch, steps, warmup, workload):
    """Forward over few long chains (varlen_64k: 16 documents, the longest
    16,637 tokens; long_64k: one 65,536-token sequence), timed with the
    automatic state-pass plan (segments of long chains when the cost model
    takes them) and with whole chains only."""
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    log(f"generating {workload} inputs")
    w = I.make_workload(workload)
    tok = w.tok
    d = {k: dev_tensor(torch, getattr(tok, k)) for k in ("q", "k", "v", "g", "s", "beta")}
    H, DK, DV = w.cfg["H"], w.cfg["DK"], w.cfg["DV"]
    if w.cu_seqlens is not None:
        cu = torch.from_numpy(w.cu_seqlens)
        cu_dev = cu.to("cuda:0")
        h0 = dev_tensor(torch, w.h0)
        Tt = int(w.cu_seqlens[-1])
        N = len(w.cu_seqlens) - 1
        o = torch.empty((Tt, H, DV), dtype=torch.float32, device="cuda:0")
        ht = torch.empty((N, H, DK, DV), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(ckda.fwd_varlen_workspace_bytes(N, Tt, H, DK, DV, torch.bfloat16), dtype=torch.uint8,
                         device="cuda:0")
        fn = lambda: ckda.fwd_varlen(**d, cu_seqlens=cu, cu_seqlens_dev=cu_dev, h0=h0, o=o, ht=ht, workspace=ws)
        tokens, lens = Tt, np.diff(w.cu_seqlens)
    else:
        B, T = w.cfg["B"], w.cfg["T"]
        o = torch.empty((B, T, H, DV), dtype=torch.float32, device="cuda:0")
        ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(ckda.fwd_workspace_bytes(B, T, H, DK, DV, torch.bfloat16), dtype=torch.uint8,
                         device="cuda:0")
        fn = lambda: ckda.fwd(**d, o=o, ht=ht, workspace=ws)
        tokens, lens = B * T, np.full(B, T)
    res = {"workload": workload, "tokens": tokens, "chains": int(len(lens) * H),
           "longest_chain_tokens": int(lens.max())}
    try:
        # the two plans are timed twice, interleaved, and each keeps its faster
        # pass (the first timed pass after input generation runs slow)
        for rep in range(2):
            for mode, G in (("auto", 0), ("whole_chains", -1)):
                ckda.set_segment_chunks(G)
                log(f"timing {workload} forward, state pass {mode} (pass {rep + 1} of 2)")
                wall, per = time_kernel_launches(torch, fn, steps, warmup)
                r = {"ms": wall / steps, "avg_launch_ms": float(np.mean(per)),
                     "tokens_per_s": tokens / (wall / steps * 1e-3)}
                if mode not in res or r["ms"] < res[mode]["ms"]:
                    res[mode] = r
    finally:
        ckda.set_segment_chunks(0)
    res["speedup_auto_vs_whole"] = res["whole_chains"]["ms"] / res["auto"]["ms"]
    return res


def bench_decode(torch, nsteps=512, distinct=64):
    """256 sequences x 16 heads, nsteps sequential steps from a state drawn
    N(0, 0.02).  Step inputs are drawn for `distinct` steps and reused
    cyclically (same shapes and distributions; the state still evolves
    over all nsteps)."""
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    cfg = I.WORKLOADS["decode_b256"]
    N, H, D = cfg["N"], cfg["H"], cfg["DK"]
    seed = I.SEED_BASE + cfg["index"]
    log(f"generating decode inputs ({distinct} distinct steps)")
    rng = np.random.default_rng(seed)
    state0 = I.draw_state(rng, (N, H, D, D), 0.02)
    tok = I.decode_steps(seed, 0, distinct, N, H, D, D, "bf16")
    dq = {k: dev_tensor(torch, getattr(tok, k)) for k in ("q", "k", "v", "g", "s", "beta")}
    state = dev_tensor(torch, state0)
    sp = torch.ones((N, H, D), dtype=torch.int8, device="cuda:0")
    o = torch.empty((N, H, D), dtype=torch.float32, device="cuda:0")
    it = [0]

    def step():
        t = it[0] % distinct
        it[0] += 1
        ckda.decode_step(dq["q"][t], dq["k"][t], dq["v"][t], dq["g"][t], dq["s"][t], dq["beta"][t],
                         state, sp, o=o)

    log("timing decode")
    wall, per = time_kernel_launches(torch, step, nsteps, 8)
    per_step = wall / nsteps
    bytes_step = N * H * DEC_BYTES_PER_HEAD_STEP
    # the same nsteps steps captured in one graph and replayed: the host
    # launches nothing per step, so wall time per step is the kernels' own
    # rate (plus the graph's dispatch gaps)
    log("timing decode as one graph of all steps")
    it[0] = 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the allocator and the library on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    it[0] = 0
    with torch.cuda.graph(graph):
        for _ in range(nsteps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_step = (time.perf_counter() - t0) * 1e3 / (reps * nsteps)
    return dict(ms_per_step=per_step, launch_ms=float(np.mean(per)), bytes_per_step=bytes_step,
                gbs=bytes_step / (float(np.mean(per)) * 1e-3) / 1e9,
                graph_ms_per_step=graph_step, graph_gbs=bytes_step / (graph_step * 1e-3) / 1e9,
                wall_gbs=bytes_step / (per_step * 1e-3) / 1e9,
                seq_steps_per_s=N / (per_step * 1e-3), steps=nsteps)


# backward, per token-head: q,k,v,do bf16 (1024) + g (512) + s (128) + beta (4)
# + chunk-start state checkpoints (128*128*4 per 64 tokens = 1024) + dq,dk,dv,dg
# f32 (2048) + dbeta (4)
BWD_BYTES_PER_TOKEN_HEAD = 1024 + 512 + 128 + 4 + 1024 + 2048 + 4


def bench_bwd(torch, steps, warmup):
    """layer_bwd: the layer_bf16 shapes with a seeded bf16 upstream gradient;
    the forward (with chunk checkpoints) runs once outside the timed region."""
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    log("generating layer_bwd inputs")
    w = I.make_workload("layer_bwd")
    tok = w.tok
    d = {k: dev_tensor(torch, getattr(tok, k)) for k in ("q", "k", "v", "g", "s", "beta")}
    do = dev_tensor(torch, w.do)
    B, T, H, DK = tok.q.shape
    # the forward with checkpoints, its workspace (chunk records) kept for the
    # backward that reads them
    fws = torch.empty(ckda.fwd_workspace_bytes(B, T, H, DK, DK, torch.bfloat16), dtype=torch.uint8, device="cuda:0")
    fwd_ck = lambda: ckda.fwd(**d, want_ckpt=True, workspace=fws)
    _, _, hc = fwd_ck()
    ws = torch.empty(ckda.bwd_workspace_bytes(B, T, H, DK, DK, ckpt_given=True), dtype=torch.uint8, device="cuda:0")
    fn = lambda: ckda.bwd(**d, h_ckpt=hc, do=do, workspace=ws)
    fn_rec = lambda: ckda.bwd(**d, h_ckpt=hc, do=do, workspace=ws, fwd_workspace=fws)
    log("timing backward")
    wall, per = time_kernel_launches(torch, fn, steps, warmup)
    log("timing backward reading the forward's records")
    wall_rec, _ = time_kernel_launches(torch, fn_rec, steps, warmup)
    log("timing the forward with checkpoints")
    wall_fck, _ = time_kernel_launches(torch, fwd_ck, steps, warmup)
    th = B * T * H
    ms = wall / steps
    ms_rec = wall_rec / steps
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), bytes=th * BWD_BYTES_PER_TOKEN_HEAD,
                gbs=th * BWD_BYTES_PER_TOKEN_HEAD / (ms * 1e-3) / 1e9,
                workspace_bytes=int(ws.numel()), ms_with_fwd_records=ms_rec,
                fwd_ckpt_ms=wall_fck / steps, fwd_records_bytes=int(fws.numel()))


def bench_options(torch, steps, warmup):
    """layer_bwd's shapes under the two options that change the per-element
    arithmetic: the gate map (raw pre-activations x ~ 1.5 N(0,1) for the
    gate, y ~ N(0,1) for beta, no s) and q, k normalised in the path (the
    workload's unit rows, which the norm keeps).  Forward with checkpoints
    and backward, each beside the plain call on the same tensors."""
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    log("generating layer_bwd inputs (options)")
    w = I.make_workload("layer_bwd")
    tok = w.tok
    d = {k: dev_tensor(torch, getattr(tok, k)) for k in ("q", "k", "v", "g", "s", "beta")}
    do = dev_tensor(torch, w.do)
    B, T, H, DK = tok.q.shape
    x, y = I.draw_gate_preacts(np.random.default_rng(2024), tuple(tok.g.shape), tuple(tok.beta.shape))
    dm = dict(d, g=dev_tensor(torch, x), s=None, beta=dev_tensor(torch, y))
    ws = torch.empty(ckda.bwd_workspace_bytes(B, T, H, DK, DK, ckpt_given=True), dtype=torch.uint8, device="cuda:0")
    res = {"workload": "layer_bwd shapes (B=8, T=4096, H=16, d=128, bf16) under each option", "unit": "ms"}
    cases = (("plain", d, {}), ("gate_map", dm, {"gate_map": True}), ("qk_norm", d, {"qk_norm": True}))
    for name, dd, kw in cases:   # every variant loaded and run once before any is timed
        _, _, hc = ckda.fwd(**dd, want_ckpt=True, **kw)
        ckda.bwd(**dd, h_ckpt=hc, do=do, workspace=ws, **kw)
    torch.cuda.synchronize()
    for name, dd, kw in cases:
        log(f"timing forward and backward, {name}")
        wall_f, _ = time_kernel_launches(torch, lambda: ckda.fwd(**dd, want_ckpt=True, **kw), steps, warmup)
        _, _, hc = ckda.fwd(**dd, want_ckpt=True, **kw)
        wall_b, _ = time_kernel_launches(torch, lambda: ckda.bwd(**dd, h_ckpt=hc, do=do, workspace=ws, **kw),
                                         steps, warmup)
        res[name] = {"fwd_ckpt_ms": wall_f / steps, "bwd_ms": wall_b / steps}
    return res


def bench_bwd_long(torch, steps=2, warmup=1):
    """Backward of long_64k (one 65,536-token sequence x 16 heads, bf16, a
    seeded bf16 upstream gradient): the reverse (dS) pass with the automatic
    plan (segments of the long chains) and with whole chains, interleaved,
    each keeping its faster pass.  The forward with checkpoints runs once,
    outside the timed region."""
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    log("generating long_64k inputs (backward)")
    w = I.make_workload("long_64k")
    tok = w.tok
    d = {k: dev_tensor(torch, getattr(tok, k)) for k in ("q", "k", "v", "g", "s", "beta")}
    B, T, H, DK = tok.q.shape
    do = torch.randn((B, T, H, DK), generator=torch.Generator().manual_seed(77)).to(torch.bfloat16).to("cuda:0")
    _, _, hc = ckda.fwd(**d, want_ckpt=True)
    ws = torch.empty(ckda.bwd_workspace_bytes(B, T, H, DK, DK, ckpt_given=True), dtype=torch.uint8, device="cuda:0")
    fn = lambda: ckda.bwd(**d, h_ckpt=hc, do=do, workspace=ws)
    res = {"workload": "long_64k backward", "tokens": B * T, "chains": B * H}
    try:
        for rep in range(2):
            for mode, G in (("auto", 0), ("whole_chains", -1)):
                ckda.set_segment_chunks(G)
                log(f"timing long_64k backward, reverse pass {mode} (pass {rep + 1} of 2)")
                wall, per = time_kernel_launches(torch, fn, steps, warmup)
                r = {"ms": wall / steps, "tokens_per_s": B * T / (wall / steps * 1e-3)}
                if mode not in res or r["ms"] < res[mode]["ms"]:
                    res[mode] = r
    finally:
        ckda.set_segment_chunks(0)
    res["speedup_auto_vs_whole"] = res["whole_chains"]["ms"] / res["auto"]["ms"]
    return res


def bench_conv(torch, steps, warmup):
    """The optional short convolution (width 4, SiLU) over one input of the
    layer workload's shapes (B=8, T=4096, 16 x 128 channels, bf16): forward
    and backward, one launch sequence each, HBM-bound."""
    from gated_delta_rule_sign_amd import ckda
    from gated_delta_rule_sign_amd import inputs as I
    B, T, C = 8, 4096, 2048
    log("generating short-conv inputs")
    x, w, _, dy = I.draw_conv(41, (B, T, C), C, B, "bf16", with_state=False)
    xd, wd, dyd = dev_tensor(torch, x), dev_tensor(torch, w), dev_tensor(torch, dy)
    y = torch.empty_like(xd)
    ws = torch.empty(int(ckda.lib().ckda_short_conv_bwd_workspace_bytes(B * T, C)), dtype=torch.uint8,
                     device="cuda:0")
    log("timing short conv")
    _, per_f = time_kernel_launches(torch, lambda: ckda.short_conv(xd, wd, silu=True, y=y), steps, warmup)
    _, per_b = time_kernel_launches(torch, lambda: ckda.short_conv_bwd(xd, wd, dyd, silu=True, workspace=ws),
                                    steps, warmup)
    n = B * T * C
    fb = n * (2 + 2) + C * 16            # x read, y written (bf16), taps
    bb = n * (2 + 4 + 4) + C * 16 * 2    # x and dy read, dx written, taps and dw
    tf, tb = float(np.mean(per_f)), float(np.mean(per_b))
    return {"workload": "q of layer_bf16 (B=8, T=4096, 2048 channels, bf16), width 4, SiLU",
            "fwd_ms": tf, "fwd_gbs": fb / (tf * 1e-3) / 1e9, "fwd_frac_of_hbm_peak": fb / (tf * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bwd_ms": tb, "bwd_gbs": bb / (tb * 1e-3) / 1e9, "bwd_frac_of_hbm_peak": bb / (tb * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_fwd": fb, "algorithmic_bytes_bwd": bb}


def bench_copy(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size (calibration for HBM byte counters)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").uniform_()
    dst = torch.empty_like(src)
    wall, per = time_kernel_launches(torch, lambda: dst.copy_(src), reps, 2)
    copy_ms = float(np.mean(per))
    # a write-only stream of the same size (a fill)
    _, per_w = time_kernel_launches(torch, lambda: dst.fill_(1.0), reps, 2)
    write_ms = float(np.mean(per_w))
    return dict(bytes_read=nbytes, bytes_written=nbytes, launch_ms=copy_ms,
                gbs=2 * nbytes / (copy_ms * 1e-3) / 1e9,
                write_only_gbs=nbytes / (write_ms * 1e-3) / 1e9)


def cpu_baseline(w, min_seconds=10.0, max_passes=8):
    """The float64 CPU oracle on the same workload: all (sequence, head)
    chains of layer_bf16, all tokens and value columns, repeated until about
    `min_seconds` of CPU work (at most `max_passes` passes)."""
    import oracle
    f = w.tok.f64()
    B, T, H, _ = f["q"].shape
    chains = [(b, h) for b in range(B) for h in range(H)]
    threads = oracle.max_threads()
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        oracle.fwd(**f, chains=chains)
        dt += time.perf_counter() - t0
        passes += 1
    # a layer token carries H heads: chain-tokens / H = layer tokens
    return dict(value=passes * len(chains) * T / H / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"the whole forward workload ({len(chains)} (sequence, head) chains x {T} tokens, "
                       f"{f['v'].shape[-1]} value columns), {passes} passes, {dt:.1f} s; float64 token recurrence; "
                       f"value = chain-tokens / {H} heads / seconds",
                seconds=dt, tiny_fp32_one_core=cpu_tiny_one_core())


def cpu_tiny_one_core(min_seconds=1.0):
    """The oracle on tiny_fp32 (B=1, T=256, H=2, d=32) on one thread, repeated
    for about `min_seconds`: the small case's CPU figure beside the layer's."""
    import oracle
    from gated_delta_rule_sign_amd import inputs as I
    f = I.make_workload("tiny_fp32").tok.f64()
    B, T, H, _ = f["q"].shape
    n0 = oracle.max_threads()
    oracle.set_threads(1)
    try:
        passes, dt = 0, 0.0
        while passes == 0 or dt < min_seconds:
            t0 = time.perf_counter()
            oracle.fwd(**f)
            dt += time.perf_counter() - t0
            passes += 1
    finally:
        oracle.set_threads(n0)
    return dict(value=passes * B * T / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"tiny_fp32 (B={B}, T={T}, H={H}, d=32), {passes} passes, {dt:.2f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["fwd", "fwd_head_gate", "fwd_qk_norm", "fwd_long", "bwd_long", "decode", "bwd", "options",
                                       "copy", "conv"], default=None)
    ap.add_argument("--decode-steps", type=int, default=512)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path shards over "
              "(sequence, head) chains with no exchange, so N GPUs is N independent copies.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from gated_delta_rule_sign_amd import ckda
    ckda.lib()

    if args.only == "copy":
        print(json.dumps(bench_copy(torch)))
        return
    if args.only == "decode":
        print(json.dumps(bench_decode(torch, args.decode_steps)))
        return
    if args.only == "conv":
        print(json.dumps(bench_conv(torch, args.steps, args.warmup)))
        return
    if args.only == "bwd":
        print(json.dumps(bench_bwd(torch, args.steps, args.warmup)))
        return
    if args.only == "options":
        print(json.dumps(bench_options(torch, args.steps, args.warmup)))
        return
    if args.only == "bwd_long":
        print(json.dumps(bench_bwd_long(torch)))
        return
    if args.only == "fwd_long":
        print(json.dumps([bench_fwd_long(torch, max(3, args.steps // 4), 3, wl) for wl in ("varlen_64k", "long_64k")]))
        return

    if args.only in ("fwd_head_gate", "fwd_qk_norm"):
        wl = "layer_bf16_head_gate" if args.only == "fwd_head_gate" else "layer_bf16_qk_norm"
        fh = bench_fwd(torch, args.steps, args.warmup, wl)
        print(json.dumps({k: v for k, v in fh.items() if k not in ("w", "launch_all")}))
        return
    fw = bench_fwd(torch, args.steps, args.warmup)
    if args.only == "fwd":
        print(json.dumps({k: v for k, v in fw.items() if k not in ("w", "launch_all")}))
        return
    dec = bench_decode(torch, args.decode_steps)
    bw = bench_bwd(torch, max(3, args.steps // 4), 1)
    fh = bench_fwd(torch, args.steps, args.warmup, "layer_bf16_head_gate")
    fq = bench_fwd(torch, args.steps, args.warmup, "layer_bf16_qk_norm")
    longs = [bench_fwd_long(torch, max(3, args.steps // 4), 3, wl) for wl in ("varlen_64k", "long_64k")]
    bwl = bench_bwd_long(torch)
    cv = bench_conv(torch, args.steps, args.warmup)
    opt = bench_options(torch, max(3, args.steps // 4), 1)
    cpu = None if args.no_cpu else cpu_baseline(fw["w"])
    cp = bench_copy(torch)

    achieved = fw["bytes"] / (fw["launch_ms"] * 1e-3) / 1e9
    traffic = measured_traffic()
    traffic_gbs = None if traffic is None else traffic / (fw["launch_ms"] * 1e-3) / 1e9
    value = fw["tokens"] / (fw["ms"] * 1e-3)
    mf = measured_mfma()
    mfma_exec = None if mf is None else {
        "frac": mf["executed_bf16_flops_per_call"] / (fw["launch_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "executed_tflop_per_call": mf["executed_bf16_flops_per_call"] / 1e12,
        "basis": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per call (committed counter run), over this run's mean "
                 "launch time, against 2.5 PFLOP/s; includes the hi/lo split's three products per pair",
        "busy_frac_per_kernel": {k: v["mfma_busy_frac"] for k, v in mf["kernels"].items()
                                 if v["executed_bf16_flops"] > 0}}
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fw["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layer_bf16: one CKDA mixer of the 1.36B model, forward prefill",
                   "B": 8, "T": 4096, "H": 16, "dk": 128, "dv": 128, "chunk": 64,
                   "inputs": "q,k,v bf16; g,beta f32; s int8", "state_and_outputs": "f32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_gbs": traffic_gbs,
                     "copy_gbs": cp["gbs"],
                     "write_only_gbs": cp["write_only_gbs"],
                     "traffic_frac_of_copy": None if traffic_gbs is None else traffic_gbs / cp["gbs"],
                     "copy_basis": "a 1 GiB device copy (torch copy_) timed in this run, read + write bytes; a 1 GiB "
                                   "fill (write only) beside it; "
                                   "traffic_gbs = the counted HBM bytes of one call over this run's mean launch time",
                     "kernel": "ckda_fwd_chunked call = ckda_chunk_kernel<bf16,128,128> + "
                               "ckda_state_kernel<bf16,128,128,false>",
                     "algorithmic_bytes_per_launch": fw["bytes"],
                     "avg_launch_ms": fw["launch_ms"],
                     "workspace_bytes": fw["workspace_bytes"],
                     "mfma_algorithmic_frac": fw["flops"] / (fw["launch_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "mfma_executed_frac": None if mfma_exec is None else mfma_exec["frac"],
                     "mfma_executed": mfma_exec},
        "decode": {"workload": "decode_b256: 256 seqs x 16 heads, dk=dv=128, 512 steps",
                   "unit": "GB/s", "value": dec["gbs"], "frac_of_hbm_peak": dec["gbs"] / HBM_PEAK_GBS,
                   "basis": "mean HIP-event time of one step's kernel",
                   "graph_gbs": dec["graph_gbs"], "graph_frac_of_hbm_peak": dec["graph_gbs"] / HBM_PEAK_GBS,
                   "graph_ms_per_step": dec["graph_ms_per_step"],
                   "graph_basis": "wall time of the 512 steps captured in one HIP graph and replayed",
                   "wall_gbs": dec["wall_gbs"],
                   "wall_basis": "wall time of 512 host-launched steps (launch gaps included)",
                   "traffic": measured_traffic(DECODE_TRAFFIC_FILE),
                   "ms_per_step": dec["ms_per_step"], "seq_steps_per_s": dec["seq_steps_per_s"],
                   "algorithmic_bytes_per_step": dec["bytes_per_step"]},
        "backward": {"workload": "layer_bwd: layer_bf16 shapes, bf16 upstream gradient, checkpointed states",
                     "unit": "tokens/s", "value": bw["tokens_per_s"], "ms": bw["ms"],
                     "algorithmic_bytes": bw["bytes"], "achieved_gbs": bw["gbs"],
                     "frac_of_hbm_peak": bw["gbs"] / HBM_PEAK_GBS, "workspace_bytes": bw["workspace_bytes"],
                     "traffic": measured_traffic(BWD_TRAFFIC_FILE),
                     "with_forward_records": {
                         "ms": bw["ms_with_fwd_records"],
                         "frac_of_hbm_peak": bw["bytes"] / (bw["ms_with_fwd_records"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "basis": "ckda_bwd_with_records: the backward reads the chunk records the forward with "
                                  "checkpoints left in its workspace (kept between the calls) instead of writing "
                                  "its own",
                         "kept_bytes": bw["fwd_records_bytes"]},
                     "training_step_ms": {"forward_with_checkpoints": bw["fwd_ckpt_ms"],
                                          "plus_backward": bw["fwd_ckpt_ms"] + bw["ms"],
                                          "plus_backward_with_forward_records": bw["fwd_ckpt_ms"] + bw["ms_with_fwd_records"]}},
        "forward_head_gate": {"workload": "layer_bf16_head_gate: layer_bf16 with one signed gate per "
                                          "(token, head) (g f32, s int8 [B,T,H])",
                              "unit": "tokens/s", "value": fh["tokens"] / (fh["ms"] * 1e-3), "ms": fh["ms"],
                              "avg_launch_ms": fh["launch_ms"], "algorithmic_bytes": fh["bytes"],
                              "achieved_gbs": fh["bytes"] / (fh["launch_ms"] * 1e-3) / 1e9,
                              "frac_of_hbm_peak": fh["bytes"] / (fh["launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "forward_qk_norm": {"workload": "layer_bf16_qk_norm: layer_bf16 with raw q, k (row norms spread "
                                        "over two decades) L2-normalised inside the path",
                            "unit": "tokens/s", "value": fq["tokens"] / (fq["ms"] * 1e-3), "ms": fq["ms"],
                            "avg_launch_ms": fq["launch_ms"], "algorithmic_bytes": fq["bytes"],
                            "achieved_gbs": fq["bytes"] / (fq["launch_ms"] * 1e-3) / 1e9,
                            "frac_of_hbm_peak": fq["bytes"] / (fq["launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "forward_long_chains": longs,
        "backward_long_chains": bwl,
        "short_conv": cv,
        "options": opt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
