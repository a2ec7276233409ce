"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * the chunked forward (prefill) over the 32K workload: B=1, T=32768, H=32,
    d_k=d_v=128, C=64, bf16 inputs, fp32 state, per-channel gate
    (kda_chunk_fwd: chunk map, intra-chunk, chunk walk), then
  * one recurrent decode step over 256 sequences x 32 heads, d=128, fp32
    state (kda_recurrent_step).
Inputs are generated once (seeded, synth.CONFIGS / DECODE_CONFIGS) and are
resident in HBM before the timed region.  `value` is prefill tokens/s over
the chunked-forward time of the timed steps.  `roofline` prices the dominant
kernel of the step against HBM with the method's own minimum bytes (bf16 q,
k, v, g, o and beta: 1282 B per head-token); `path_roofline` does the same
for the whole kda_chunk_fwd call, next to its fraction of the bf16 MFMA peak
at the algorithmic FLOP count; `kernels_intermediate` gives each prefill
kernel's rate over the bytes it actually moves (its inputs plus the
intermediates it reads or writes).  Each kernel is timed with HIP events
recorded on the stream it runs on.  `decode` reports 64 decode steps launched
back to back, each timed, in GB/s of the step's algorithmic bytes.  The
oracle (fp64, host cores) is timed on a bounded prefix of the same workload as
`cpu_baseline`.  After the timed steps, the 1M-token prefill (T = 1,048,576,
H = 16) is timed under `long_context`, the chunked backward pass
(kda_chunk_bwd) over the 32K prefill inputs under `backward`, the pre-path
transforms (kda_prepare_inputs on the prefill inputs, the decode step with
them fused in, and the prefill with them fused in, kda_chunk_fwd_raw) under
`prepath`, the d = 64 variant of the prefill at the same model width
(H = 64) under `variant_d64`, and the 32K prefill with 128-token chunks
(kda_chunk_fwd_c128) under `variant_c128` (the 1M prefill with them under
`long_context.c128`).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-backward]
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA chunked fwd tokens/s (H=32,d=128,T=32K) + decode step GB/s; % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published

# Algorithmic figures (per head-token for the chunked path, d = 128, C = 64)
PATH_MIN_BYTES_PER_HT = 1282           # bf16 q, k, v, g, o (5 x 2 x 128) + beta (2)
PATH_FLOP_PER_HT = 139136              # 6 d^2 + (5C - 1) d
INTRA_BYTES_PER_HT = 2154              # reads q,k,v,g,beta (1026); writes W,QG,KdT,U' (4 x 256), P (96: the 6 of
                                       # its 8 fragment blocks on or below the diagonal), Gn (8)
WALK_BYTES_PER_HT = 1384               # reads W,QG,KdT,U' (4 x 256), P (96), Gn (8); writes o (256)
SEG_PASS1_BYTES_PER_HT = 776           # the segmented walk's first pass re-reads W, KdT, U' (3 x 256), Gn (8)
SEG_GROUPS_32K = 8                     # segments per (sequence, head) at 32K x 32 (one workgroup per CU)
DECODE_BYTES_PER_STEP = 1084243968     # state read + write (2 x 536870912) + tokens in (8404992) + o (2097152)


# The files the forward and decode kernels are compiled from (the backward
# pass and the host-side ABI live elsewhere and do not change them).
KERNEL_SOURCES = ("kda_chunk.hip", "kda_chunk128.hip", "kda_chunk_util.h", "kda_decode.hip", "kda_device.h")


def kernel_sources_sha():
    """sha256[:16] over the forward and decode kernel sources, as recorded next
    to counter readings."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        f = os.path.join(ROOT, "gated_delta_rule_48_amd", "csrc", name)
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) recorded in
    profiles/traffic_counters.txt for these exact kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.txt")
    if not os.path.exists(path):
        return None
    sha = kernel_sources_sha()
    with open(path) as f:
        for line in f:
            kv = dict(x.split("=", 1) for x in line.split())
            if kv.get("kernel") == kernel and kv.get("sources_sha") == sha:
                return float(kv["read_bytes"]) + float(kv["write_bytes"])
    return None


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    return lib


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def record(self, i, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i, j):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(self.ev[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)


def _to_dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, prefix_tokens):
    import oracle
    oracle.build(force=False)
    T = prefix_tokens
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    sl = lambda a: np.ascontiguousarray(a[:T])
    t0 = time.perf_counter()
    oracle.recurrence(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), cu_seqlens=[0, T],
                      threads=threads)
    dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"the whole 32K x 32-head prefill workload ({T} tokens, all heads)" if T >= 32768 else
                       f"the first {T} tokens of the 32K x 32-head prefill workload, all heads")
                      + f": fp64 sequential recurrence, {dt:.2f} s on {threads} threads"}


def time_backward(kda, torch, hip, x, d, T, H, dk, dv, stream, steps=5, warmup=2):
    """The chunked backward pass (kda_chunk_bwd) over the same 32K x 32 inputs,
    with seeded cotangents dO ~ N(0,1) (bf16) and dS_T ~ N(0,1); the whole
    call is timed with HIP events on its stream.  Reported beside the
    forward, not part of `value`."""
    import synth
    dO, dST = synth.draw_cotangents(np.random.default_rng(3030), T, 1, H, dk, dv, "bf16")
    dO, dST = _to_dev(dO, torch), torch.from_numpy(dST).cuda()
    ws = torch.empty(kda.chunk_bwd_workspace_size(T, 1, H, dk, dv), dtype=torch.uint8, device="cuda")
    ev = Events(hip, steps + 1)

    def run():
        return kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, dS_T=dST, workspace=ws)

    for _ in range(warmup):
        run()
    ev.record(0, stream)
    for i in range(steps):
        run()
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    ms = [ev.ms(i, i + 1) for i in range(steps)]
    t = float(np.median(ms))
    return {"ms_median": t, "ms_min": float(np.min(ms)), "tokens_per_s": T / (t * 1e-3),
            "workspace_GB": ws.numel() / 1e9,
            "what": "kda_chunk_bwd: dq, dk, dv, dg, dbeta, dS0 of the 32K x 32 prefill for dO, dS_T"}


def time_prepath(kda, torch, hip, x, T, H, dk, stream, S_dec, toks, steps=10):
    """kda_prepare_inputs over the 32K x 32 prefill inputs (q, k, per-channel g
    and beta, read and written once: 2 x (3 d_k + 1) x 2 bytes per head-token),
    and the decode step with the same transforms fused in (kda_recurrent_step_raw)
    on the decode workload, each timed with HIP events on its stream."""
    outs = tuple(torch.empty_like(x[n]) for n in ("q", "k", "g", "beta"))
    ev = Events(hip, steps + 1)
    for _ in range(2):
        kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"], out=outs)
    ev.record(0, stream)
    for i in range(steps):
        kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"], out=outs)
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    t_prep = float(np.median([ev.ms(i, i + 1) for i in range(steps)]))
    prep_bytes = 2 * (3 * dk + 1) * 2 * T * H
    ev2 = Events(hip, steps + 1)
    for i in range(2):
        tk = toks[i % len(toks)]
        kda.recurrent_step_raw(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S_dec)
    ev2.record(0, stream)
    for i in range(steps):
        tk = toks[i % len(toks)]
        kda.recurrent_step_raw(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S_dec)
        ev2.record(i + 1, stream)
    torch.cuda.synchronize()
    t_raw = float(np.median([ev2.ms(i, i + 1) for i in range(steps)]))
    # the prefill with the same transforms fused into its intra-chunk kernel
    # (kda_chunk_fwd_raw), on the prefill inputs taken as raw projections
    dv = x["v"].shape[2]
    o = torch.empty_like(x["v"])
    S_T = torch.empty((1, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.chunk_fwd_workspace_size(T, 1, H, dk, dv), dtype=torch.uint8, device="cuda")
    ev3 = Events(hip, steps + 1)
    for _ in range(2):
        kda.chunk_fwd_raw(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws, check=False)
    ev3.record(0, stream)
    for i in range(steps):
        kda.chunk_fwd_raw(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws, check=False)
        ev3.record(i + 1, stream)
    torch.cuda.synchronize()
    kda.chunk_fwd_check(ws)
    t_fraw = float(np.median([ev3.ms(i, i + 1) for i in range(steps)]))
    return {
        "prefill_raw": {"what": "kda_chunk_fwd_raw: the 32K x 32 prefill from raw projections, pre-path fused "
                                "into the intra-chunk kernel", "ms": t_fraw, "tokens_per_s": T / (t_fraw * 1e-3)},
        "prepare_inputs": {"us": t_prep * 1e3, "bytes": prep_bytes, "GB_per_s": prep_bytes / (t_prep * 1e-3) / 1e9,
                           "frac_hbm_peak": prep_bytes / (t_prep * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "decode_raw_back_to_back": {"us_per_step": t_raw * 1e3,
                                    "GB_per_s": DECODE_BYTES_PER_STEP / (t_raw * 1e-3) / 1e9,
                                    "frac_hbm_peak": DECODE_BYTES_PER_STEP / (t_raw * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }


def time_c128(kda, torch, hip, x, T, H, dk, dv, stream, steps=10):
    """The 32K x 32 prefill with 128-token chunks (kda_chunk_fwd_c128) on the
    same resident inputs, each call's chunk map, intra-chunk kernel and walk
    timed with HIP events on its stream; reported beside the 64-token path,
    not part of `value`."""
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((1, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.chunk_fwd_workspace_size(T, 1, H, dk, dv, chunk=128), dtype=torch.uint8, device="cuda")
    evs = [Events(hip, 4) for _ in range(steps)]
    for _ in range(2):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws, check=False,
                      chunk=128)
    for e in evs:
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws, check=False,
                      chunk=128, events=e.ev)
    torch.cuda.synchronize()
    kda.chunk_fwd_check(ws)
    med = lambda i, j: float(np.median([e.ms(i, j) for e in evs]))
    t = med(0, 3)
    ht = T * H
    return {"what": f"kda_chunk_fwd_c128, T={T}, H={H}, d_k=d_v={dk}, bf16, C=128", "ms": t,
            "tokens_per_s": T / (t * 1e-3),
            "kernels_ms": {"chunk_map": med(0, 1), "intra_chunk": med(1, 2), "chunk_walk": med(2, 3)},
            "method_GB_per_s": PATH_MIN_BYTES_PER_HT * ht / (t * 1e-3) / 1e9,
            "TFLOP_per_s": PATH_FLOP_PER_HT * ht / (t * 1e-3) / 1e12}


def time_long_context(kda, torch, hip, stream, steps=3, with_c128=True):
    """The 1M-token prefill (kda_1m_bf16: B=1, T=1,048,576, H=16, d=128,
    bf16, per-channel gate from N(-1,1)) through kda_chunk_fwd, inputs drawn
    block by block (the recipe of the parity test) and resident in HBM before
    the timed calls; each call timed with HIP events on its stream."""
    import synth
    cfg = synth.CONFIGS["kda_1m_bf16"]
    T, H, dk, dv = cfg.T, cfg.H, cfg.dk, cfg.dv
    shapes = {"q": (T, H, dk), "k": (T, H, dk), "v": (T, H, dv), "g": (T, H, dk), "beta": (T, H)}
    dev = {n: torch.empty(s, dtype=torch.bfloat16, device="cuda") for n, s in shapes.items()}
    for _, start, blk in synth.iter_token_blocks(cfg, workers=8):
        rows = blk["q"].shape[0]
        for n in shapes:
            dev[n][start:start + rows].copy_(torch.from_numpy(blk[n].view(np.int16)).view(torch.bfloat16))
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((1, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.chunk_fwd_workspace_size(T, 1, H, dk, dv), dtype=torch.uint8, device="cuda")
    ev = Events(hip, steps + 1)

    def run():
        kda.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], out=o, S_T=S_T, workspace=ws, check=False)

    run()
    ev.record(0, stream)
    for i in range(steps):
        run()
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    ms = [ev.ms(i, i + 1) for i in range(steps)]
    t = float(np.median(ms))
    ht = T * H
    gbs = PATH_MIN_BYTES_PER_HT * ht / (t * 1e-3) / 1e9
    res = {"what": f"kda_chunk_fwd, kda_1m_bf16: T={T}, H={H}, d_k=d_v={dk}, bf16", "ms_median": t,
           "ms_min": float(np.min(ms)), "tokens_per_s": T / (t * 1e-3), "method_GB_per_s": gbs,
           "frac_hbm_peak": gbs / HBM_PEAK_GBS}
    if with_c128:
        # the same inputs with 128-token chunks (kda_chunk_fwd_c128)
        del ws
        ws = torch.empty(kda.chunk_fwd_workspace_size(T, 1, H, dk, dv, chunk=128), dtype=torch.uint8,
                         device="cuda")
        ev2 = Events(hip, steps + 1)

        def run128():
            kda.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], out=o, S_T=S_T, workspace=ws,
                          check=False, chunk=128)

        run128()
        ev2.record(0, stream)
        for i in range(steps):
            run128()
            ev2.record(i + 1, stream)
        torch.cuda.synchronize()
        kda.chunk_fwd_check(ws)
        t2 = float(np.median([ev2.ms(i, i + 1) for i in range(steps)]))
        res["c128"] = {"what": "kda_chunk_fwd_c128 on the same inputs (C = 128)", "ms_median": t2,
                       "tokens_per_s": T / (t2 * 1e-3)}
    del dev, o, S_T, ws
    torch.cuda.empty_cache()
    return res


def time_d64_variant(kda, torch, hip, stream, T=32768, H=64, steps=5):
    """The d_k = d_v = 64 variant at the same model width (H = 64 heads of 64
    channels, T = 32768, bf16, per-channel gate, seeded inputs of the 32K
    recipe) through kda_chunk_fwd, timed with HIP events; reported beside the
    d = 128 workload, not part of `value`."""
    import synth
    cfg = synth.small_chunk_config(H=H, dk=64, dv=64, dtype="bf16", gate="channel", gate_mu=-1.0, s0_sigma=0.0,
                                   seed=303)
    d = synth.chunk_inputs(cfg, lengths=[T])
    x = {n: _to_dev(d[n], torch) for n in ("q", "k", "v", "g", "beta")}
    o = torch.empty((T, H, 64), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((1, H, 64, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.chunk_fwd_workspace_size(T, 1, H, 64, 64), dtype=torch.uint8, device="cuda")
    ev = Events(hip, steps + 1)
    for _ in range(2):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws, check=False)
    ev.record(0, stream)
    for i in range(steps):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws, check=False)
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    t = float(np.median([ev.ms(i, i + 1) for i in range(steps)]))
    return {"what": f"kda_chunk_fwd, T={T}, H={H}, d_k=d_v=64, bf16", "ms": t, "tokens_per_s": T / (t * 1e-3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-prefix", type=int, default=32768)
    ap.add_argument("--no-backward", action="store_true", help="skip timing the chunked backward pass")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the d = 64 and the 128-token-chunk variants")
    ap.add_argument("--no-long-context", action="store_true", help="skip timing the 1M-token prefill")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one device-to-device copy of exactly 1 GiB before the timed steps, so that a "
                         "counter run (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) has a kernel of known traffic "
                         "to scale by")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the KDA hot path here is not sharded, got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_48_amd as kda
    import synth

    kda.load_library()
    hip = _hip()
    cfg = synth.CONFIGS["kda_32k_bf16"]
    d = synth.chunk_inputs(cfg)
    T, H, dk, dv = int(d["cu_seqlens"][-1]), cfg.H, cfg.dk, cfg.dv
    x = {n: _to_dev(d[n], torch) for n in ("q", "k", "v", "g", "beta")}
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((1, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.chunk_fwd_workspace_size(T, 1, H, dk, dv), dtype=torch.uint8, device="cuda")

    dcfg = synth.DECODE_CONFIGS["decode_256x32"]
    rng = np.random.default_rng(dcfg.seed)
    S_dec = torch.from_numpy(synth.decode_state(dcfg, rng)).cuda()
    n_tok = min(args.steps + args.warmup, 8)
    toks = []
    for _ in range(n_tok):
        t = synth.decode_step_inputs(dcfg, rng)
        toks.append({n: _to_dev(t[n], torch) for n in ("q", "k", "v", "g", "beta")})
    o_dec = torch.empty((dcfg.N, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream().cuda_stream
    K, W = args.steps, args.warmup
    evs = [Events(hip, 6) for _ in range(K)]

    def step(i, ev):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S_T, workspace=ws,
                      events=None if ev is None else ev.ev[:4], check=False)
        if ev is not None:
            ev.record(4, stream)
        tk = toks[i % n_tok]
        kda.recurrent_step(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S_dec, out=o_dec)
        if ev is not None:
            ev.record(5, stream)

    for i in range(W):
        step(i, None)
    dist = torch.distributed.is_available() and torch.distributed.is_initialized()
    if dist:
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, evs[i])
    if dist:
        torch.distributed.barrier()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / K
    kda.chunk_fwd_check(ws)  # the timed prefills ran to completion (no rejected offsets, no timed-out wait)

    # 64 decode steps back to back on one state (the serving pattern), each
    # timed, after the timed region: the step above follows a prefill, these
    # follow each other
    n_b2b = 64
    ev_b2b = Events(hip, n_b2b + 1)
    for i in range(3):
        tk = toks[i % n_tok]
        kda.recurrent_step(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S_dec, out=o_dec)
    ev_b2b.record(0, stream)
    for i in range(n_b2b):
        tk = toks[i % n_tok]
        kda.recurrent_step(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S_dec, out=o_dec)
        ev_b2b.record(i + 1, stream)
    torch.cuda.synchronize()
    b2b_ms = [ev_b2b.ms(i, i + 1) for i in range(n_b2b)]
    t_b2b = float(np.median(b2b_ms))

    prepath = time_prepath(kda, torch, hip, x, T, H, dk, stream, S_dec, toks)
    d64 = None if args.no_variants else time_d64_variant(kda, torch, hip, stream)
    c128 = None if args.no_variants else time_c128(kda, torch, hip, x, T, H, dk, dv, stream)
    longc = None if args.no_long_context else time_long_context(kda, torch, hip, stream,
                                                                  with_c128=not args.no_variants)
    bwd = None if args.no_backward else time_backward(kda, torch, hip, x, d, T, H, dk, dv, stream,
                                                      steps=args.backward_steps)

    avg = lambda i, j: float(np.mean([e.ms(i, j) for e in evs]))
    stats = lambda i, j: {"mean": avg(i, j), "median": float(np.median([e.ms(i, j) for e in evs])),
                          "min": float(np.min([e.ms(i, j) for e in evs]))}
    t_map, t_intra, t_walk = avg(0, 1), avg(1, 2), avg(2, 3)
    t_fwd, t_dec = avg(0, 3), avg(4, 5)
    ht = T * H
    tokens_per_s = T / (t_fwd * 1e-3)

    # the method's minimum bytes per launch: a prefill kernel is priced with
    # the whole path's 1282 B per head-token, the decode step with its own
    kern = {
        "kda::intra_chunk_kernel": (t_intra, PATH_MIN_BYTES_PER_HT * ht),
        "kda::seg_walk_kernel": (t_walk, PATH_MIN_BYTES_PER_HT * ht),
        "kda::decode_step_kernel": (t_dec, DECODE_BYTES_PER_STEP),
    }
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_bytes = kern[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    walk_bytes = (WALK_BYTES_PER_HT + SEG_PASS1_BYTES_PER_HT * (SEG_GROUPS_32K - 1) / SEG_GROUPS_32K) * ht
    inter = {"intra_chunk": {"ms": t_intra, "bytes": INTRA_BYTES_PER_HT * ht,
                             "GB_per_s": INTRA_BYTES_PER_HT * ht / (t_intra * 1e-3) / 1e9},
             "chunk_walk": {"ms": t_walk, "bytes": walk_bytes, "GB_per_s": walk_bytes / (t_walk * 1e-3) / 1e9,
                            "what": "segmented walk: pass 3 reads every chunk's operands and writes o, pass 1 "
                                    "re-reads W, KdT, U', Gn of the chunks outside the last segment"}}
    dec_gbs = DECODE_BYTES_PER_STEP / (t_dec * 1e-3) / 1e9
    path_gbs = PATH_MIN_BYTES_PER_HT * ht / (t_fwd * 1e-3) / 1e9
    path_tflops = PATH_FLOP_PER_HT * ht / (t_fwd * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_32k_bf16 prefill: B=1, T=32768, H=32, d_k=d_v=128, C=64, per-channel gate, "
                               "bf16 inputs, fp32 state; plus one decode step of decode_256x32: 256 sequences x "
                               "32 heads, d=128, fp32 state",
                   "global_batch": 1, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv, "chunk": 64},
        "prefill_ms": t_fwd,
        "prefill_ms_stats": stats(0, 3),
        "decode_us_stats": {k: v * 1e3 for k, v in stats(4, 5).items()},
        "kernels_ms": {"chunk_map": t_map, "intra_chunk": t_intra, "chunk_walk": t_walk, "decode_step": t_dec},
        "decode": {"us_per_step": t_dec * 1e3, "GB_per_s": dec_gbs, "frac_hbm_peak": dec_gbs / HBM_PEAK_GBS,
                   "tokens_per_s": dcfg.N / (t_dec * 1e-3), "bytes_per_step": DECODE_BYTES_PER_STEP,
                   "back_to_back": {"steps": n_b2b, "us_per_step_median": t_b2b * 1e3,
                                    "us_per_step_min": float(np.min(b2b_ms)) * 1e3,
                                    "GB_per_s": DECODE_BYTES_PER_STEP / (t_b2b * 1e-3) / 1e9,
                                    "frac_hbm_peak": DECODE_BYTES_PER_STEP / (t_b2b * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "tokens_per_s": dcfg.N / (t_b2b * 1e-3)}},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(dom),
                     "algorithmic_bytes": dom_bytes,
                     "what": "the method's minimum bytes per launch (1282 B per head-token for a prefill "
                             "kernel, the decode step's state and token bytes) over the dominant kernel's "
                             "HIP-event time"},
        "kernels_intermediate": inter,
        "path_roofline": {"what": "whole kda_chunk_fwd call vs the method's minimum bytes (1282 B/head-token) "
                                  "and algorithmic FLOPs (139136 /head-token)",
                          "GB_per_s": path_gbs, "frac_hbm_peak": path_gbs / HBM_PEAK_GBS,
                          "TFLOP_per_s": path_tflops, "frac_bf16_mfma_peak": path_tflops / BF16_MFMA_PEAK_TFLOPS},
    }
    res["prepath"] = prepath
    if longc is not None:
        res["long_context"] = longc
    if d64 is not None:
        res["variant_d64"] = d64
    if c128 is not None:
        res["variant_c128"] = c128
    if bwd is not None:
        res["backward"] = bwd
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_prefix)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
