"""Benchmark of the delta-rule mixer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--decode-reps R] [--graph]
    python bench.py --only prefill2|prefill3|prefill5|decode|conv|chunk_bwd1|chunk_bwd4|prompt_d64 [--steps K]

One step is one prefill call (dn_chunk_fwd) over the DeltaNet layer-prefill workload
(B=4, H=16, T=2048, d_k=d_v=128, bf16 q/k/v, fp32 beta, no decay, zero initial state,
final state returned): 8192 tokens.  K steps run back to back between two device
synchronisations, cycling through several copies of the inputs so the working set
(> 256 MB) does not stay in the Infinity Cache between steps.  The wall clock of the eager
launch loop gives the value (--graph times a HIP-graph replay of the same K steps instead;
both are reported); the average kernel time per call is also taken with HIP events on the
launching stream around the eager loop.  The warmup runs long enough (200 calls, about
12 ms) for the GPU's clocks to settle before the timed region.

The two other full-size prefill workloads (gated GQA B2 T8192 16 -> 32 heads; 8 packed gated
sequences of 32,768 tokens in all) are timed right after it, each warmed for about 20 ms
of back-to-back calls and then timed with events around 10 calls, and each gets its own
roofline block (algorithmic bytes and flops,
rocprofv3 counters) under ``prefill_workloads``.  ``--only`` runs one workload alone (a
prefill workload, the gated decode step, the conv and the fused prologue, or the reverse
pass at B1 or B4) for a rocprofv3 counter pass per workload.  The decode step (256 sequences x 32 heads,
state updated in place) is timed with events around a loop of back-to-back steps and
reported in the same line, and so is the chunkwise reverse pass (dn_chunk_bwd) on the gated
H16 T2048 shape at B1 and B4 (20 calls between events, own roofline block under
``chunk_backward``), and the gated d_k = d_v = 64 prompt of the layer's shape on the same
one-launch kernel at d = 64 (``prompt_d64``).  The fp64 oracle is timed on the host cores on a bounded
sample of the prefill workload.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, TFLOP/s
PREFILL = dict(B=4, T=2048, H=16, D=128, C=64)
PREFILL_WHAT = {
    2: "DeltaNet layer prefill B4 H16 T2048 d128 bf16, no decay, zero initial state, final state",
    3: "gated prefill, GQA 16 q/k heads -> 32 v heads, B2 T8192 d128 bf16, g = -0.1 softplus(z), "
       "final state",
    5: "varlen gated prefill, 8 packed sequences, 32768 tokens, H32 d128 bf16, beta in (0,2), "
       "g = -0.05 softplus(z), initial state per sequence",
}
DECODE = dict(N=256, H=32, D=128)


def prefill_bytes(B, T, Hqk, Hv, D, gated, N, init):
    """Algorithmic HBM bytes of one prefill call: q, k, v read and o written once
    (bf16), beta (and g) read once (fp32), final state written (and initial read)."""
    tok = B * T
    b = tok * (2 * Hqk * D * 2 + Hv * D * 2 + Hv * D * 2) + tok * Hv * 4 * (2 if gated else 1)
    b += N * Hv * D * D * 4 * (2 if init else 1)
    return b


def prefill_flops(tokens, Hqk, Hv, D, C):
    """Algorithmic matrix flops of one prefill call, triangles exploited: per token and
    value head 6 d_k d_v (K M and Q M against the state, K^T Delta into it) plus
    C ((1 + 2/r) d_k + 2 d_v) (the masked Gram products K K^T and Q K^T at half a dense
    tile each, shared by the r = Hv / Hqk value heads of a q/k head, and T R and P Delta
    at half a tile each).  139,264 flop per token-head at r = 1, 131,072 at r = 2."""
    r = Hv // Hqk
    return int(tokens * Hv * (6 * D * D + C * ((1 + 2 / r) * D + 2 * D)))


def prefill_flops_dense(tokens, Hqk, Hv, D, C):
    """The same products with every tile dense (upper triangles and the padded diagonal
    blocks counted): per chunk and value head [K;Q] M (2*2C*D*D), T R (2*C*C*D), P Delta
    (2*C*C*D), K^T Delta (2*C*D*D); per chunk and q/k head K K^T, Q K^T (2*2*C*C*D).
    Reported beside the algorithmic figure as what a dense-tile schedule issues; the
    kernel's own count (its slice workgroups each form A, T and P) comes from the
    rocprofv3 SQ counters."""
    chunks = tokens / C
    per_v = 2 * 2 * C * D * D + 2 * 2 * C * C * D + 2 * C * D * D
    per_qk = 2 * 2 * C * C * D
    return int(chunks * (Hv * per_v + Hqk * per_qk))


def chunk_bwd_bytes(tokens, Hqk, Hv, D, gated, N, init, dfinal):
    """Algorithmic HBM bytes of one chunkwise reverse pass: q, k, v, dL/do read once (bf16),
    beta (and g) read once, dq, dk, dv, dbeta (and dg) written once (fp32), the initial
    state read and its gradient written (when given), dL/d final state read (when given).
    The chunk-start states it recomputes and its workspace traffic are not algorithmic."""
    b = tokens * (2 * Hqk * D * 2 + 2 * Hv * D * 2) + tokens * Hv * 4 * (2 if gated else 1)
    b += tokens * (2 * Hqk * D * 4 + Hv * D * 4) + tokens * Hv * 4 * (2 if gated else 1)
    b += N * Hv * D * D * 4 * ((2 if init else 0) + (1 if dfinal else 0))
    return b


def chunk_bwd_flops(tokens, Hv, D, C):
    """Algorithmic matrix flops of one chunkwise reverse pass, triangles exploited, per token
    and value head (one q/k head per value head): recomputing the chunk-start states, K M
    and K^T Delta (4 d^2) with K K^T and T R (2 C d, half tiles); the gradients, seven
    products against the state or its gradient (K M, K dM', Q^T dO, K^T dX, dO M^T, dX M^T,
    Delta dM'^T: 14 d^2) and eleven half-tile chunk products (K K^T, Q K^T, T R, P^T dO,
    T^T dDelta, dR Delta^T, dO Delta^T, Z K, W K, W^T K, Z^T Q: 11 C d).
    18 d^2 + 13 C d = 401,408 flop per token-head at d = 128, C = 64."""
    return int(tokens * Hv * (18 * D * D + 13 * C * D))


def decode_bytes(N, Hqk, Hv, D):
    return N * Hv * D * D * 4 * 2 + N * (2 * Hqk * D * 2 + 2 * Hv * D * 2 + 2 * Hv * 4)


def code_text(src):
    """A source file's code without its comments and blank lines (a comment edit leaves the
    built kernels, and so their counters, unchanged)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in src.splitlines())
    return "\n".join(line for line in lines if line)


def source_digest():
    """Digest of the code of every kernel source: counters in profiles/traffic.json are used
    only while the code is the one they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "delta_rule_recurrent_chunked_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                h.update(f.encode() + b"\0" + code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(key):
    """Entry ``key`` of profiles/traffic.json (HBM bytes and matrix-core work per call from
    rocprofv3 counters), or None unless the kernel sources are the ones the counters were
    taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    if t.get("source_digest") != source_digest():
        return None
    return t.get(key)


def prefill_roofline(key, kernel, call_us, alg_b, tokens, Hqk, Hv, D, C=64):
    """Roofline block of one prefill workload: algorithmic HBM bytes and matrix flops of
    one call over the call's kernel time (HIP events on the launching stream), against
    MI355X's HBM and dense bf16 peaks; rocprofv3's counted bytes and matrix-core work
    (profiles/traffic.json) while the kernel sources are the ones they were taken on."""
    meas = load_traffic(key) or {}
    achieved = alg_b / (call_us * 1e-6) / 1e9
    alg_f = prefill_flops(tokens, Hqk, Hv, D, C)
    counters = None
    if meas.get("counted_flops_per_call"):
        counters = {"counted_flops_per_call": meas["counted_flops_per_call"],
                    "counted_frac_of_bf16_peak": meas["counted_flops_per_call"] / (call_us * 1e-6)
                    / 1e12 / BF16_PEAK_TFLOPS,
                    "mfma_busy_util": meas.get("mfma_busy_util")}
    return {
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": meas.get("bytes_per_call"),
                     "kernel": kernel, "call_us": call_us, "algorithmic_bytes": alg_b},
        "mfma": {"algorithmic_flops": alg_f, "tflops": alg_f / (call_us * 1e-6) / 1e12,
                 "frac_of_bf16_peak": alg_f / (call_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                 "dense_tile_flops": prefill_flops_dense(tokens, Hqk, Hv, D, C),
                 "counters": counters},
        "tokens_per_s": tokens / (call_us * 1e-6),
    }


def cpu_baseline(x, budget_s=12.0):
    """The fp64 oracle on the host cores, on the same prefill workload, repeated until
    about budget_s seconds of wall time have passed (at least one full call)."""
    import oracle
    f = x.f64()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    toks = reps * x.B * x.T
    return {"value": toks / el, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"full prefill workload (B{x.B} H{x.Hv} T{x.T} d{x.Dk}) x {reps} call(s), "
                      f"{el:.1f} s, fp64 token-by-token recurrence, OpenMP over (sequence, head)"}


def only_part(what, dn, dev, reps, warmup):
    """One workload of the line alone (for a rocprofv3 counter pass): the gated decode step,
    the conv and the fused prologue on the layer shape, the reverse pass at B1 / B4, or the
    gated d = 64 prompt of the layer's shape.
    Returns the average time per call from HIP events on the launching stream."""
    import numpy as np
    import torch
    from synth import make_case

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    calls = []
    if what == "decode":
        y = make_case(B=DECODE["N"], T=1, Hqk=DECODE["H"], Dk=DECODE["D"], dtype="bf16", g_scale=0.1,
                      init_std=0.02, seed=0, decode=True)
        q, k, v = to_dev(y.q)[:, 0], to_dev(y.k)[:, 0], to_dev(y.v)[:, 0]
        b, g = to_dev(y.beta)[:, 0], to_dev(y.g)[:, 0]
        st = [to_dev(y.init) for _ in range(2)]
        out = torch.empty((y.B, y.Hv, y.Dv), dtype=torch.bfloat16, device=dev)
        calls.append(("decode_kernel", lambda i: dn.decode_step(q, k, v, b, g, st[i % 2], out=out)))
    elif what == "conv":
        H, D, B, T = PREFILL["H"], PREFILL["D"], PREFILL["B"], PREFILL["T"]
        rng = np.random.default_rng(3)
        C = 3 * H * D
        x = torch.from_numpy(rng.standard_normal((B, T, C)).astype(np.float32)).to(dev).to(torch.bfloat16)
        w = torch.from_numpy((rng.standard_normal((C, 4)) / 2).astype(np.float32)).to(dev)
        b = torch.zeros(C, dtype=torch.float32, device=dev)
        calls.append(("conv_kernel (plain)", lambda i: dn.causal_conv(x, w, b)))
        calls.append(("conv_kernel (split, head norm)", lambda i: dn.conv_qkv(x, w, b, H, H, D, D)))
    elif what == "prompt_d64":
        T, H = PREFILL["T"], PREFILL["H"]
        B = PREFILL["B"]
        x64 = make_case(B=B, T=T, Hqk=H, Dk=64, dtype="bf16", g_scale=0.1, seed=0)
        q, k, v, b, g = (to_dev(a_) for a_ in (x64.q, x64.k, x64.v, x64.beta, x64.g))
        o = torch.empty((B, T, H, 64), dtype=torch.bfloat16, device=dev)
        s = torch.empty((B, H, 64, 64), dtype=torch.float32, device=dev)
        calls.append(("d64 prompt (one launch)",
                      lambda i: dn.chunk_fwd(q, k, v, b, g, None, out=o, final_state=s)))
    else:
        bb = 1 if what == "chunk_bwd1" else 4
        T, H, D = PREFILL["T"], PREFILL["H"], PREFILL["D"]
        xg = make_case(B=bb, T=T, Hqk=H, Dk=D, dtype="bf16", g_scale=0.1, seed=0)
        gq, gk, gv, gb, gg = (to_dev(a_) for a_ in (xg.q, xg.k, xg.v, xg.beta, xg.g))
        gdo = torch.randn((bb, T, H, D), device=dev).to(torch.bfloat16)
        gws = torch.empty(dn.chunk_bwd_workspace_bytes(bb, T, H, H, D, D, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        calls.append((f"chunk_bwd B{bb}", lambda i: dn.chunk_bwd(gq, gk, gv, gb, gg, None, gdo, workspace=gws)))
    res = {}
    stream = torch.cuda.current_stream(dev)
    for name, fn in calls:
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = {"us_per_call": e0.elapsed_time(e1) * 1e3 / reps, "calls": reps}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-reps", type=int, default=50)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time a HIP-graph replay of the K steps instead of the eager launch loop")
    ap.add_argument("--only", choices=["prefill2", "prefill3", "prefill5", "decode", "conv",
                                       "chunk_bwd1", "chunk_bwd4", "prompt_d64"], default=None,
                    help="run only this prefill workload (a rocprofv3 counter pass per workload) "
                         "and print its timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy five times (calibrates rocprofv3's "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the mixer "
              "runs no collectives; run --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import delta_rule_recurrent_chunked_amd as dn
    from synth import make_case, make_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = 512 << 20
        src = torch.zeros(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)
        return

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def time_prefill_workload(cfg, reps, warmup=3):
        """One prefill workload: `reps` back-to-back calls between HIP events on the launching
        stream (config 2 cycles over four copies of its inputs, so its 139 MB do not stay
        in the 256 MB Infinity Cache; the others exceed it by themselves)."""
        z = make_config(cfg)
        zcu = None if z.cu_seqlens is None else to_dev(z.cu_seqlens.astype(np.int32))
        ncopy = 4 if cfg == 2 else 1
        zsets = []
        for _ in range(ncopy):
            zsets.append(dict(q=to_dev(z.q), k=to_dev(z.k), v=to_dev(z.v), b=to_dev(z.beta),
                              g=to_dev(z.g), i=to_dev(z.init),
                              o=torch.empty((z.B, z.T, z.Hv, z.Dv), dtype=torch.bfloat16, device=dev),
                              s=torch.empty((z.num_seqs, z.Hv, z.Dk, z.Dv), dtype=torch.float32,
                                            device=dev)))

        def zstep(i):
            w = zsets[i % ncopy]
            dn.chunk_fwd(w["q"], w["k"], w["v"], w["b"], w["g"], w["i"], cu_seqlens=zcu, out=w["o"],
                         final_state=w["s"])

        for i in range(warmup):
            zstep(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(reps):
            zstep(i)
        e1.record(st)
        torch.cuda.synchronize()
        z_us = e0.elapsed_time(e1) * 1e3 / reps
        init = z.init is not None
        zb = prefill_bytes(z.B, z.T, z.Hqk, z.Hv, z.Dk, gated=z.g is not None, N=z.num_seqs, init=init)
        kern = "fused_kernel<128, %s, false>" % ("true" if z.g is not None else "false")
        blk = prefill_roofline(f"prefill_config{cfg}", kern, z_us, zb, z.B * z.T, z.Hqk, z.Hv, z.Dk)
        del zsets, zcu
        return dict(workload=PREFILL_WHAT[cfg], **blk)

    if args.only in ("decode", "conv", "chunk_bwd1", "chunk_bwd4", "prompt_d64"):
        print(json.dumps({"only": args.only, **only_part(args.only, dn, dev, args.steps, args.warmup)}),
              flush=True)
        return
    if args.only:
        cfg = int(args.only[-1])
        r = time_prefill_workload(cfg, args.steps, warmup=args.warmup)
        print(json.dumps({"only": args.only, **r}), flush=True)
        return

    # ------------------------------------------------------------------ prefill
    x = make_config(2)
    B, T, Hqk, Hv, D = x.B, x.T, x.Hqk, x.Hv, x.Dk
    base = dict(q=to_dev(x.q), k=to_dev(x.k), v=to_dev(x.v), beta=to_dev(x.beta))
    wsb = dn.workspace_bytes(B, T, Hqk, Hv, D, D, torch.bfloat16)
    sets = []
    for i in range(args.copies):
        s = {k: (t if i == 0 else t.clone()) for k, t in base.items()}
        s["o"] = torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device=dev)
        s["fs"] = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(max(1, wsb), dtype=torch.uint8, device=dev)
        sets.append(s)

    def step(i):
        s = sets[i % len(sets)]
        dn.chunk_fwd(s["q"], s["k"], s["v"], s["beta"], None, None, out=s["o"], final_state=s["fs"],
                     workspace=s["ws"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    # average kernel time per call: HIP events on the launching stream around the eager
    # loop (the launches queue back to back), divided by the call count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    call_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    # the same K steps captured once in a HIP graph and replayed, reported beside the eager
    # loop (on this stack a replayed kernel node starts several microseconds later than an
    # eagerly launched one, so the eager loop is the faster launch path here)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t0
    del graph
    wall = wall_graph if args.graph else wall_eager
    ms_step = wall * 1e3 / args.steps
    tokens = B * T
    alg_b = prefill_bytes(B, T, Hqk, Hv, D, gated=False, N=B, init=False)
    traffic_d = load_traffic("decode_bytes_per_call")
    head_block = prefill_roofline("prefill_config2", "fused_kernel<128, false, false>", call_us, alg_b,
                                  tokens, Hqk, Hv, D)

    # ------------------------------------ the other two full-size prefill workloads, right
    # after the headline and warmed like it (about 20 ms of back-to-back calls each, so the
    # clocks have settled before the timed calls)
    other = {3: time_prefill_workload(3, 10, warmup=80), 5: time_prefill_workload(5, 10, warmup=40)}

    # ------------------------------------------------------------------- decode
    y = make_case(B=DECODE["N"], T=1, Hqk=DECODE["H"], Dk=DECODE["D"], dtype="bf16", g_scale=0.1,
                  init_std=0.02, seed=0, decode=True)
    dq, dk, dv = to_dev(y.q)[:, 0], to_dev(y.k)[:, 0], to_dev(y.v)[:, 0]
    db, dg = to_dev(y.beta)[:, 0], to_dev(y.g)[:, 0]
    dstate = [to_dev(y.init) for _ in range(2)]
    dout = torch.empty((y.B, y.Hv, y.Dv), dtype=torch.bfloat16, device=dev)
    for i in range(3):
        dn.decode_step(dq, dk, dv, db, dg, dstate[i % 2], out=dout)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.decode_reps):
        dn.decode_step(dq, dk, dv, db, dg, dstate[i % 2], out=dout)
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_us = ev0.elapsed_time(ev1) * 1e3 / args.decode_reps
    ev0.record(stream)
    for i in range(args.decode_reps):
        dn.decode_step(dq, dk, dv, db, None, dstate[i % 2], out=dout)
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_plain_us = ev0.elapsed_time(ev1) * 1e3 / args.decode_reps
    state_b = y.B * y.Hv * y.Dk * y.Dv * 4 * 2
    dec_b = decode_bytes(y.B, y.Hqk, y.Hv, y.Dk)
    dec_gbs = state_b / (dec_us * 1e-6) / 1e9

    # ------------- in-rule q/k normalisation: the same two workloads handed raw q and k
    xr = make_case(B=B, T=T, Hqk=Hqk, Dk=D, dtype="bf16", seed=0, qk_raw=True)
    rsets = []
    for i in range(args.copies):
        rsets.append(dict(q=to_dev(xr.q), k=to_dev(xr.k), v=sets[i]["v"], beta=sets[i]["beta"],
                          o=sets[i]["o"], fs=sets[i]["fs"], ws=sets[i]["ws"]))

    def rstep(i):
        s = rsets[i % len(rsets)]
        dn.chunk_fwd(s["q"], s["k"], s["v"], s["beta"], None, None, out=s["o"], final_state=s["fs"],
                     workspace=s["ws"], qk_l2norm=True)

    for i in range(args.warmup):
        rstep(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        rstep(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    norm_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    del rsets
    yr = make_case(B=DECODE["N"], T=1, Hqk=DECODE["H"], Dk=DECODE["D"], dtype="bf16", g_scale=0.1,
                   init_std=0.02, seed=0, decode=True, qk_raw=True)
    rq, rk = to_dev(yr.q)[:, 0], to_dev(yr.k)[:, 0]
    for i in range(3):
        dn.decode_step(rq, rk, dv, db, dg, dstate[i % 2], out=dout, qk_l2norm=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.decode_reps):
        dn.decode_step(rq, rk, dv, db, dg, dstate[i % 2], out=dout, qk_l2norm=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_norm_us = ev0.elapsed_time(ev1) * 1e3 / args.decode_reps
    in_rule_norm = {
        "what": "q and k handed raw (N(0,1) draws) and L2-normalised inside the call "
                "(DN_QK_L2NORM, eps 1e-6); same workloads, same timing as above",
        "prefill": {"kernel": "fused_kernel<128, false, true>", "us_per_call": norm_us,
                    "tokens_per_s": tokens / (norm_us * 1e-6),
                    "hbm_frac": alg_b / (norm_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "traffic": load_traffic("prefill_qk_l2norm_bytes_per_call"),
                    "vs_prenormalised_call": norm_us / call_us},
        "decode": {"kernel": "decode_kernel (normalising)", "us_per_step": dec_norm_us,
                   "hbm_frac": dec_b / (dec_norm_us * 1e-6) / 1e9 / HBM_PEAK_GBS},
    }

    # ------------- gates per key channel (ChannelGates): decode and layer prefill
    yc = make_case(B=DECODE["N"], T=1, Hqk=DECODE["H"], Dk=DECODE["D"], dtype="bf16", g_scale=0.1,
                   init_std=0.02, seed=0, decode=True, g_per_key=True)
    cg = to_dev(yc.g)[:, 0].contiguous()
    for i in range(3):
        dn.decode_step(dq, dk, dv, db, cg, dstate[i % 2], out=dout)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.decode_reps):
        dn.decode_step(dq, dk, dv, db, cg, dstate[i % 2], out=dout)
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_chg_us = ev0.elapsed_time(ev1) * 1e3 / args.decode_reps
    dec_chg_b = dec_b + y.B * y.Hv * y.Dk * 4
    xc = make_case(B=B, T=T, Hqk=Hqk, Dk=D, dtype="bf16", seed=0, g_scale=0.1, g_per_key=True)
    cq, ck, cv, cb, cgp = (to_dev(a) for a in (xc.q, xc.k, xc.v, xc.beta, xc.g))
    co = torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device=dev)
    cs = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
    cws = torch.empty(dn.workspace_bytes(B, T, Hqk, Hv, D, D, torch.bfloat16, g_per_key=True),
                      dtype=torch.uint8, device=dev)
    for _ in range(3):
        dn.chunk_fwd(cq, ck, cv, cb, cgp, None, out=co, final_state=cs, workspace=cws)
    torch.cuda.synchronize()
    creps = 20
    ev0.record(stream)
    for _ in range(creps):
        dn.chunk_fwd(cq, ck, cv, cb, cgp, None, out=co, final_state=cs, workspace=cws)
    ev1.record(stream)
    torch.cuda.synchronize()
    pre_chg_us = ev0.elapsed_time(ev1) * 1e3 / creps
    pre_chg_b = alg_b + B * T * Hv * D * 4
    channel_gates = {
        "what": "log decay per key channel (DN_GATE_PER_KEY, g = -0.1 softplus(N(0,1)) per channel)",
        "decode": {"workload": "256 sequences x 32 heads d128 bf16, state in place",
                   "kernel": "decode_kernel (channel gates)", "us_per_step": dec_chg_us,
                   "hbm_frac": dec_chg_b / (dec_chg_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                   "algorithmic_bytes": dec_chg_b,
                   "traffic": load_traffic("decode_channel_gates_bytes_per_call")},
        "prefill": {"workload": "B4 H16 T2048 d128 bf16, final state returned",
                    "kernel": "chg_prep_kernel + chg_chain_kernel (matrix cores, 64-token chunks)",
                    "us_per_call": pre_chg_us, "tokens_per_s": tokens / (pre_chg_us * 1e-6),
                    "hbm_frac": pre_chg_b / (pre_chg_us * 1e-6) / 1e9 / HBM_PEAK_GBS},
    }
    del cq, ck, cv, cb, cgp, co, cs

    # ---------------- readout epilogue: over the prefill's output, and fused into decode
    from synth import make_epilogue_inputs
    ep_in = make_epilogue_inputs((B, T, Hv, D), "bf16", seed=1)
    ew = to_dev(ep_in["weight"])
    esets = []
    for i in range(args.copies):
        esets.append((sets[i]["o"], to_dev(ep_in["gate"]) if i == 0 else esets[0][1].clone(),
                      torch.empty_like(sets[i]["o"])))
    for i in range(args.warmup):
        eo, eg, ey = esets[i % len(esets)]
        dn.norm_gate(eo, "rms", 1e-6, ew, None, eg, out=ey)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        eo, eg, ey = esets[i % len(esets)]
        dn.norm_gate(eo, "rms", 1e-6, ew, None, eg, out=ey)
    ev1.record(stream)
    torch.cuda.synchronize()
    ng_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    ng_b = B * T * Hv * D * 2 * 3 + D * 4
    del esets
    dep_in = make_epilogue_inputs((y.B, y.Hv, y.Dv), "bf16", seed=2)
    dw, dgt = to_dev(dep_in["weight"]), to_dev(dep_in["gate"])
    for i in range(3):
        dn.decode_step(dq, dk, dv, db, dg, dstate[i % 2], out=dout, norm="rms", norm_weight=dw,
                       out_gate=dgt)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.decode_reps):
        dn.decode_step(dq, dk, dv, db, dg, dstate[i % 2], out=dout, norm="rms", norm_weight=dw,
                       out_gate=dgt)
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_ep_us = ev0.elapsed_time(ev1) * 1e3 / args.decode_reps
    dec_ep_b = dec_b + y.B * y.Hv * y.Dv * 2 + y.Dv * 4
    epilogue = {
        "what": "per-head RMSNorm over d_v with weight, then * silu(gate) (gate shaped like o, bf16)",
        "prefill_output": {"workload": "the B4 H16 T2048 d128 bf16 prefill output",
                           "kernel": "norm_gate_kernel", "us_per_call": ng_us,
                           "roofline": {"bound": "hbm", "achieved": ng_b / (ng_us * 1e-6) / 1e9,
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": ng_b / (ng_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                        "algorithmic_bytes": ng_b,
                                        "traffic": load_traffic("norm_gate_bytes_per_call")}},
        "decode_fused": {"workload": "gated decode step 256 x 32 heads d128 bf16",
                         "kernel": "decode_kernel (fused epilogue)", "us_per_step": dec_ep_us,
                         "hbm_frac": dec_ep_b / (dec_ep_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "vs_plain_step": dec_ep_us / dec_us,
                         "traffic": load_traffic("decode_epilogue_bytes_per_call")},
    }

    # ------------- the token-by-token route on the layer-prefill workload (for context)
    s0 = sets[0]
    dn.recurrent_fwd(s0["q"], s0["k"], s0["v"], s0["beta"], None, None, out=s0["o"],
                     final_state=s0["fs"])
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(3):
        dn.recurrent_fwd(s0["q"], s0["k"], s0["v"], s0["beta"], None, None, out=s0["o"],
                         final_state=s0["fs"])
    ev1.record(stream)
    torch.cuda.synchronize()
    rec_us = ev0.elapsed_time(ev1) * 1e3 / 3
    # the reverse pass on a gated sample of the layer workload (one sequence of 2048 tokens,
    # 16 heads), from the forward's state trace
    xb = make_case(B=1, T=T, Hqk=Hqk, Dk=D, dtype="bf16", g_scale=0.1, seed=0)
    bq, bk, bv, bb_, bg = (to_dev(a_) for a_ in (xb.q, xb.k, xb.v, xb.beta, xb.g))
    _, _, btr = dn.recurrent_fwd(bq, bk, bv, bb_, bg, None, state_trace=True)
    bdo = torch.randn((1, T, Hv, D), device=dev).to(torch.bfloat16)
    dn.recurrent_bwd(bq, bk, bv, bb_, bg, None, btr, bdo)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(3):
        dn.recurrent_bwd(bq, bk, bv, bb_, bg, None, btr, bdo)
    ev1.record(stream)
    torch.cuda.synchronize()
    bwd_us = ev0.elapsed_time(ev1) * 1e3 / 3
    del btr
    recurrent = {"workload": "B4 H16 T2048 d128 bf16, no decay, final state, no trace",
                 "reverse_pass": {"workload": "B1 H16 T2048 d128 bf16 gated, from the state trace",
                                  "kernel": "recurrent_bwd_kernel", "us_per_call": bwd_us,
                                  "tokens_per_s": T / (bwd_us * 1e-6)},
                 "kernel": "recurrent_kernel (token by token, state in registers)",
                 "us_per_call": rec_us, "tokens_per_s": tokens / (rec_us * 1e-6),
                 "vs_chunked_call": rec_us / call_us}

    # ------------- the d = 64 prompt (the one-launch kernel at d_k = d_v = 64)
    x64 = make_case(B=B, T=T, Hqk=Hqk, Dk=64, dtype="bf16", g_scale=0.1, seed=0)
    q64, k64, v64, b64, g64 = (to_dev(a_) for a_ in (x64.q, x64.k, x64.v, x64.beta, x64.g))
    o64 = torch.empty((B, T, Hv, 64), dtype=torch.bfloat16, device=dev)
    s64 = torch.empty((B, Hv, 64, 64), dtype=torch.float32, device=dev)
    for _ in range(3):
        dn.chunk_fwd(q64, k64, v64, b64, g64, None, out=o64, final_state=s64)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(20):
        dn.chunk_fwd(q64, k64, v64, b64, g64, None, out=o64, final_state=s64)
    ev1.record(stream)
    torch.cuda.synchronize()
    d64_us = ev0.elapsed_time(ev1) * 1e3 / 20
    d64_b = prefill_bytes(B, T, Hqk, Hv, 64, True, B, False)
    prompt_d64 = {"workload": f"gated prefill B{B} H{Hv} T{T} d_k=d_v=64 bf16, chunk 64",
                  "path": dn.chunk_fwd_path(B, T, Hqk, Hv, 64, 64, torch.bfloat16),
                  "kernels": "fused_kernel<64, true, false>", "us_per_call": d64_us,
                  "tokens_per_s": tokens / (d64_us * 1e-6),
                  "roofline": {"bound": "hbm", "achieved": d64_b / (d64_us * 1e-6) / 1e9,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": d64_b / (d64_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                               "algorithmic_bytes": d64_b,
                               "traffic": load_traffic("prompt_d64_bytes_per_call")}}

    # ------------- the chunkwise reverse pass (dn_chunk_bwd), gated, H16 T2048, B1 and B4
    chunk_backward = {"what": "dL/dq, dk, dv, dbeta, dg and the initial state's gradient from "
                              "dL/do, through the chunked form (chunk-start states recomputed by "
                              "the prompt kernel), fp32 gradients"}
    for bb in (1, 4):
        xg = make_case(B=bb, T=T, Hqk=Hqk, Dk=D, dtype="bf16", g_scale=0.1, seed=0)
        gq, gk, gv, gb, gg = (to_dev(a_) for a_ in (xg.q, xg.k, xg.v, xg.beta, xg.g))
        gdo = torch.randn((bb, T, Hv, D), device=dev).to(torch.bfloat16)
        gws = torch.empty(dn.chunk_bwd_workspace_bytes(bb, T, Hqk, Hv, D, D, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        for _ in range(5):
            dn.chunk_bwd(gq, gk, gv, gb, gg, None, gdo, workspace=gws)
        torch.cuda.synchronize()
        greps = 20
        ev0.record(stream)
        for _ in range(greps):
            dn.chunk_bwd(gq, gk, gv, gb, gg, None, gdo, workspace=gws)
        ev1.record(stream)
        torch.cuda.synchronize()
        gb_us = ev0.elapsed_time(ev1) * 1e3 / greps
        gbytes = chunk_bwd_bytes(bb * T, Hqk, Hv, D, gated=True, N=bb, init=False, dfinal=False)
        gflops = chunk_bwd_flops(bb * T, Hv, D, 64)
        chunk_backward[f"B{bb}"] = {
            "workload": f"B{bb} H{Hv} T{T} d{D} bf16, g = -0.1 softplus(z), zero initial state",
            "kernels": ("fused_kernel<128, true, false, true> (chunk-start states, second stream) + "
                        "chunk_tp_kernel (T, P) + " if bb == 1 else
                        "fused_kernel<128, true, false, true> (chunk-start states and the T, P records) + ")
                       + "chunk_carry_kernel (dL/dM per chunk) + chunk_grad_kernel<true> (gradients per chunk)",
            "us_per_call": gb_us, "tokens_per_s": bb * T / (gb_us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbytes / (gb_us * 1e-6) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbytes / (gb_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": gbytes,
                         "traffic": load_traffic(f"chunk_bwd_B{bb}_bytes_per_call")},
            "mfma": {"algorithmic_flops": gflops, "tflops": gflops / (gb_us * 1e-6) / 1e12,
                     "frac_of_bf16_peak": gflops / (gb_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                     "counters": load_traffic(f"chunk_bwd_B{bb}_mfma")},
        }
        del gq, gk, gv, gb, gg, gdo, gws

    # ------------ the short causal conv (+ silu) in front of the rule: prompt and decode
    crng = np.random.default_rng(3)
    Cc = 3 * Hv * D
    cx = torch.from_numpy(crng.standard_normal((B, T, Cc)).astype(np.float32)).to(dev).to(torch.bfloat16)
    cw = torch.from_numpy((crng.standard_normal((Cc, 4)) / 2).astype(np.float32)).to(dev)
    cb = torch.zeros(Cc, dtype=torch.float32, device=dev)
    cy = torch.empty_like(cx)
    cst = torch.empty((B, Cc, 3), dtype=torch.bfloat16, device=dev)
    dn.causal_conv(cx, cw, cb, out=cy, final_state=cst)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(20):
        dn.causal_conv(cx, cw, cb, out=cy, final_state=cst)
    ev1.record(stream)
    torch.cuda.synchronize()
    conv_us = ev0.elapsed_time(ev1) * 1e3 / 20
    conv_b = 2 * B * T * Cc * 2 + Cc * 4 * 5 + B * Cc * 3 * 2
    # the fused prologue: the same convolution, split into q, k, v with q and k L2-normalised
    for _ in range(3):
        dn.conv_qkv(cx, cw, cb, Hqk, Hv, D, D)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(20):
        dn.conv_qkv(cx, cw, cb, Hqk, Hv, D, D)
    ev1.record(stream)
    torch.cuda.synchronize()
    qkv_us = ev0.elapsed_time(ev1) * 1e3 / 20
    Cd = 3 * y.Hv * y.Dk
    dx = torch.from_numpy(crng.standard_normal((y.B, Cd)).astype(np.float32)).to(dev).to(torch.bfloat16)
    dwt = torch.from_numpy((crng.standard_normal((Cd, 4)) / 2).astype(np.float32)).to(dev)
    dcs = torch.from_numpy(crng.standard_normal((y.B, Cd, 3)).astype(np.float32)).to(dev).to(torch.bfloat16)
    dyo = torch.empty_like(dx)
    for _ in range(3):
        dn.causal_conv_step(dx, dwt, None, dcs, out=dyo)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.decode_reps):
        dn.causal_conv_step(dx, dwt, None, dcs, out=dyo)
    ev1.record(stream)
    torch.cuda.synchronize()
    cstep_us = ev0.elapsed_time(ev1) * 1e3 / args.decode_reps
    cstep_b = 2 * y.B * Cd * 2 + 2 * y.B * Cd * 3 * 2 + Cd * 4 * 4
    conv = {
        "what": "causal depthwise conv, width 4, + silu, bf16, over the q, k and v channels",
        "prompt": {"workload": f"B{B} T{T}, {Cc} channels (3 x {Hv} heads x {D})",
                   "kernel": "conv_kernel", "us_per_call": conv_us,
                   "roofline": {"bound": "hbm", "achieved": conv_b / (conv_us * 1e-6) / 1e9,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": conv_b / (conv_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                "algorithmic_bytes": conv_b,
                                "traffic": load_traffic("conv_bytes_per_call")}},
        "prologue_conv_qkv": {
            "what": "dn_conv_qkv: the convolution + silu, split into q, k, v tensors, q and k "
                    "L2-normalised per head, in one pass (the rule then runs without in-call norm)",
            "workload": f"B{B} T{T}, {Cc} channels -> q, k [B, T, {Hqk}, {D}], v [B, T, {Hv}, {D}]",
            "kernel": "conv_kernel (split outputs, head norm)", "us_per_call": qkv_us,
            "roofline": {"bound": "hbm", "achieved": conv_b / (qkv_us * 1e-6) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": conv_b / (qkv_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": conv_b,
                         "traffic": load_traffic("conv_qkv_bytes_per_call")}},
        "decode_step": {"workload": f"{y.B} sequences, {Cd} channels, conv state in place",
                        "kernel": "conv_step_kernel", "us_per_step": cstep_us,
                        "hbm_frac": cstep_b / (cstep_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                        "algorithmic_bytes": cstep_b},
    }
    del cx, cy, cst, dx, dcs, dyo

    line = {
        "metric": "prefill tokens/sec + MFMA util; decode-step state GB/s vs HBM peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta sigmoid(N(0,1)))",
        "config": {"workload": "DeltaNet layer prefill B4 H16 T2048 d_k=d_v=128 bf16, no decay, "
                               "zero initial state, chunk 64", "global_batch": B, "seq_len": T,
                   "heads": Hv, "head_dim": D, "parallelism": "single GPU"},
        "roofline": head_block["roofline"],
        "timing": {"loop": "hip_graph_replay" if args.graph else "eager",
                   "ms_per_step_eager": wall_eager * 1e3 / args.steps,
                   "ms_per_step_graph": wall_graph * 1e3 / args.steps},
        "mfma": head_block["mfma"],
        "decode": {"workload": "gated decode step, 256 sequences x 32 heads, d=128, bf16, fp32 state "
                               "in place", "us_per_step": dec_us, "state_GBps": dec_gbs,
                   "roofline": {"bound": "hbm", "achieved": dec_b / (dec_us * 1e-6) / 1e9,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_b / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                "traffic": traffic_d, "kernel": "decode_kernel",
                                "algorithmic_bytes": dec_b},
                   "ungated_us_per_step": dec_plain_us},
        "prefill_workloads": {
            "config2": dict(workload=PREFILL_WHAT[2], **head_block),
            "config3": other[3], "config5": other[5]},
        "in_rule_qk_l2norm": in_rule_norm,
        "channel_gates": channel_gates,
        "readout_epilogue": epilogue,
        "recurrent_route": recurrent,
        "chunk_backward": chunk_backward,
        "prompt_d64": prompt_d64,
        "causal_conv": conv,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
