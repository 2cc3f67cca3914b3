#!/usr/bin/env python3
"""Throughput of the SepLLM separator-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One JSON line on stdout.  The main workload is the Pythia-160m-shaped
training step of the attention: B=8, 12 heads, S=2048, d=64, bf16, separator
probability 0.08 over 9 ids, a=4 initial tokens, window n=64.  One step is
the whole prefill/training path over one batch: index build (separator flags,
anchors, tile schedule), forward, backward.  Inputs are seeded synthetic data
resident in HBM before the timed region.

value = kept-tile TFLOP/s of forward+backward, counted on the canonical
schedule the index defines (E = sum over query tiles of rows * 64 * kept
tiles; forward 4*d*E, backward 10*d*E, over batch x heads), divided by the
measured step time (index build included).  The useful-entry count
(visible mask entries) and the tile efficiency are reported beside it.

roofline: the kernel with the largest average duration (its duration measured
with HIP events on the launch stream during the timed steps), placed by its
algorithmic work on the kept-tile schedule: the GEMMs it computes per kept
entry (forward: S and PV, 4*d*E; backward dQ kernel: S, dP and dQ, 6*d*E;
backward main kernel, key-major: S, dP, dV and dK, 8*d*E) and the bytes of
every tensor it reads once and writes once.  Whichever takes longer at the
MI355X peak (bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s) is the bound reported;
the other view is given beside it.

other_configs: the d=128 shapes (Llama-3-8B-shaped prefill, B1 32/8 heads,
8192 tokens, n=256; 32768 tokens with bursty separators), whole steps timed,
then every kernel timed with events in a second pass; kept-tile TFLOP/s on
the same counting, and a roofline block for the step's dominant kernel and
one for the forward; reported beside the main workload, not part of its
value (--no-long skips them).

decode: the streaming SepCache workload (B=64, 32 q / 8 kv heads, d=128,
c=800 = 4 initial + 64 separator slots + a 256-token window, RoPE theta
500000 by slot), 4096 steps of update + decode; HBM GB/s of the decode kernel
over the steady state (steps 1024..4095), counting every cached K/V row read
once per step per kv head plus the queries.

cpu_baseline: the fp64 CPU oracle (plain numpy, materialised mask) timed on a
bounded sample of the same workload (whole sequences, all heads, until about
--cpu-seconds of work or the whole batch), scaled to the same unit, with the
thread count numpy's BLAS used; beside it the same oracle on one thread for
sequence 0.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Events:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch
    loaded), recorded by the library's profiled entry points."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
            self.made.append(e.value)
        return out

    def record(self, e, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


class EventRing:
    """Times many intervals with a fixed set of events: groups of `width`
    events are handed out until `depth` groups are in use, then the stream is
    synchronised, the recorded groups are read (the times of consecutive
    events of each group) and the groups are reused.  The number of live
    events stays at depth * width however many steps a pass runs (a pass of
    4096 steps with a new event pair per step kept ~13 000 events alive at
    once, and the process died under the counter profiler)."""

    def __init__(self, ev, width, depth=256):
        self.ev, self.width = ev, width
        self.groups = [ev.new(width) for _ in range(depth)]
        self.used = 0
        self.times = []  # per group: width - 1 intervals (ms)

    def take(self):
        if self.used == len(self.groups):
            self.harvest()
        g = self.groups[self.used]
        self.used += 1
        return g

    def harvest(self):
        import torch
        torch.cuda.synchronize()
        for g in self.groups[:self.used]:
            self.times.append([self.ev.ms(g[i], g[i + 1]) if g[i] and g[i + 1] else None
                               for i in range(self.width - 1)])
        self.used = 0

    def result(self):
        self.harvest()
        return self.times


def schedule_counts(qtile, sep_prefix, a, n, S, tk=64):
    """Kept-tile entries (total, anchor part, band part) and visible entries
    of one sequence, from its index (qtile fields and separator prefix)."""
    qt = qtile.astype(np.int64)
    rows, n_anchor, kb, ke, n_kept = qt[:, 5], qt[:, 1], qt[:, 2], qt[:, 3], qt[:, 4]
    E = int((rows * tk * n_kept).sum())
    Ea = int((rows * tk * ((n_anchor + tk - 1) // tk)).sum())
    Eb = int((rows * tk * (ke - kb + 1)).sum())
    i = np.arange(S, dtype=np.int64)
    lo = np.maximum(0, i - n + 1)
    nnz = int(((i - lo + 1) + np.minimum(a, lo) + sep_prefix.astype(np.int64)[lo]).sum())
    return E, Ea, Eb, nnz


TRAFFIC_SOURCE = ("profiles/traffic.json: FETCH_SIZE and WRITE_SIZE from two rocprofv3 --pmc runs of this bench, "
                  "scaled by a known-size copy; not measured in this run (reported only while the kernel's "
                  "source hash matches)")


def kernel_work(B, Hq, Hkv, S, d, E):
    """Algorithmic work of each kernel on the kept-tile schedule (bf16): the
    GEMMs it computes per kept entry (forward: S, PV; backward dQ kernel: S,
    dP, dQ; backward main kernel, key-major: S, dP, dV, dK) and every tensor
    it reads once and writes once."""
    q_bytes, kv_bytes, row_bytes = B * Hq * S * d * 2, B * Hkv * S * d * 2, B * Hq * S * 4
    ld_bytes = B * Hq * ((S + 63) // 64) * 64 * 2 * 4   # per-row (log2e LSE, -D) of the dQ kernel
    flops = {"fwd": 4 * d * E, "bwd_dq": 6 * d * E, "bwd_main": 8 * d * E}
    nbytes = {"fwd": 2 * q_bytes + 2 * kv_bytes + row_bytes,
              "bwd_dq": 4 * q_bytes + 2 * kv_bytes + row_bytes + ld_bytes,
              "bwd_main": 2 * q_bytes + 4 * kv_bytes + ld_bytes}
    return flops, nbytes


KERNEL_SYMBOL = {"fwd": "fwd_kernel", "bwd_dq": "bwd_dq_kernel", "bwd_main": "bwd_main_kernel"}


def roofline_block(kernel, avg_ms, flops, nbytes, traffic=None):
    """The kernel placed by its algorithmic work: whichever of its flops (at
    the bf16 MFMA peak) and bytes (at the HBM peak) takes longer is the
    bound; achieved = that work / the average launch time."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    tflops = flops / (avg_ms * 1e-3) / 1e12
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    mfma_view = dict(bound="mfma", achieved=round(tflops, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                     frac=round(tflops / PEAK_BF16_TFLOPS, 4))
    hbm_view = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(gbs / PEAK_HBM_GBS, 4))
    binding, other = (hbm_view, mfma_view) if t_hbm >= t_mfma else (mfma_view, hbm_view)
    return dict(kernel=KERNEL_SYMBOL[kernel], **binding, traffic=traffic,
                traffic_source=TRAFFIC_SOURCE if traffic else None,
                algorithmic_mb_per_launch=round(nbytes / 1e6, 3), algorithmic_gflop_per_launch=round(flops / 1e9, 3),
                time_at_peak_us=dict(hbm=round(t_hbm * 1e6, 2), mfma=round(t_mfma * 1e6, 2)),
                other_view=other, avg_launch_ms=round(avg_ms, 5))


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` (a synth.CONFIGS name)
    from the committed counter summary (FETCH_SIZE and WRITE_SIZE, scaled by
    a known-size copy), if it was taken on the current kernel sources; else
    None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        import hashlib
        with open(path) as f:
            rec = json.load(f).get(workload, {}).get(kernel)
        if not rec:
            return None
        h = hashlib.sha256()
        for src in rec["source"]:
            with open(os.path.join(ROOT, "sparse_attention_sepattn_amd", "csrc", src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


def prefill_leg(args, torch, sa, synth):
    cfg = synth.CONFIGS["pythia160m"]
    B, Hq, Hkv, S, d, a, n = (cfg[x] for x in ("B", "Hq", "Hkv", "S", "d", "a", "n"))
    inp = synth.prefill_inputs(cfg)
    dev = torch.device("cuda:0")

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = bf(inp["q"]), bf(inp["k"]), bf(inp["v"]), bf(inp["do"])
    tok = torch.from_numpy(inp["tok"]).to(dev)
    sep = inp["sep"]
    scale = float(inp["scale"])
    idx = sa.Index(B, S, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(sa.bwd_workspace_bytes(B, Hq, Hkv, S, d), dtype=torch.uint8, device=dev)
    ev = Events()
    stream = torch.cuda.current_stream().cuda_stream

    def step(marks=None):
        if marks is not None:
            ev.record(marks[0], stream)
        sa.build_index(tok, sep, a, n, index=idx)
        if marks is not None:
            ev.record(marks[1], stream)
        sa.fwd(q, k, v, idx, scale, o=o, lse=lse)
        if marks is not None:
            ev.record(marks[2], stream)
        sa.bwd(q, k, v, o, lse, do, idx, scale, dq=dq, dk=dk, dv=dv, ws=ws,
               events=None if marks is None else marks[3:7])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel breakdown (events between every kernel); not the timed region
    K = args.steps
    marks = [ev.new(7) for _ in range(K)]
    for s in range(K):
        step(marks[s])
    torch.cuda.synchronize()
    names = ["index", "fwd", "bwd_dq", "bwd_main", "bwd_finalize"]
    seg = {nm: [] for nm in names}
    for m in marks:
        seg["index"].append(ev.ms(m[0], m[1]))
        seg["fwd"].append(ev.ms(m[1], m[2]))
        seg["bwd_dq"].append(ev.ms(m[3], m[4]))
        seg["bwd_main"].append(ev.ms(m[4], m[5]))
        seg["bwd_finalize"].append(ev.ms(m[5], m[6]))
    avg = {nm: float(np.mean(x)) for nm, x in seg.items()}
    dominant = max(("fwd", "bwd_dq", "bwd_main"), key=lambda k_: avg[k_])

    # timed region: K whole steps; events only around the dominant kernel
    dom = [ev.new(2) for _ in range(K)]

    def timed_step(e2):
        sa.build_index(tok, sep, a, n, index=idx)
        if dominant == "fwd":
            ev.record(e2[0], stream)
        sa.fwd(q, k, v, idx, scale, o=o, lse=lse)
        if dominant == "fwd":
            ev.record(e2[1], stream)
            sa.bwd(q, k, v, o, lse, do, idx, scale, dq=dq, dk=dk, dv=dv, ws=ws)
        elif dominant == "bwd_dq":
            sa.bwd(q, k, v, o, lse, do, idx, scale, dq=dq, dk=dk, dv=dv, ws=ws, events=[e2[0], e2[1], None, None])
        else:
            sa.bwd(q, k, v, o, lse, do, idx, scale, dq=dq, dk=dk, dv=dv, ws=ws, events=[None, e2[0], e2[1], None])

    t_start, t_end = ev.new(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.record(t_start, stream)
    for s in range(K):
        timed_step(dom[s])
    ev.record(t_end, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev.ms(t_start, t_end)
    dom_ms = float(np.mean([ev.ms(e2[0], e2[1]) for e2 in dom]))
    ev.close()

    # work on the canonical schedule, from the index the step built
    qtile = idx.qtile.cpu().numpy()
    pref = idx.sep_prefix.cpu().numpy()
    E = Ea = Eb = nnz = 0
    E_seqs = []
    for b in range(B):
        e, ea, eb, nz = schedule_counts(qtile[b], pref[b], a, n, S)
        E_seqs.append(e)
        E += e * Hq
        Ea += ea * Hq
        Eb += eb * Hq
        nnz += nz * Hq
    fwd_flops, bwd_flops = 4 * d * E, 10 * d * E
    ms_step = total_ms / K
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    kernel_flops, kernel_bytes = kernel_work(B, Hq, Hkv, S, d, E)
    traffic = traffic_from_profiles(KERNEL_SYMBOL[dominant], "pythia160m")
    roof = roofline_block(dominant, dom_ms, kernel_flops[dominant], kernel_bytes[dominant], traffic)
    result = dict(
        metric="kept-tile TFLOP/s (fwd+bwd) and decode HBM GB/s; % of MI355X roofline",
        value=round(value, 3), unit="TFLOP/s", n_gpus=1, steps=K, warmup=args.warmup,
        ms_per_step=round(ms_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload="pythia160m-shaped SepLLM attention training step (index+fwd+bwd)",
                    B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, a=a, n=n, p_sep=cfg["p_sep"], n_sep_ids=9,
                    kept_tile_gflop_fwd=round(fwd_flops / 1e9, 3), kept_tile_gflop_bwd=round(bwd_flops / 1e9, 3),
                    useful_gflop_fwd_bwd=round(14 * d * nnz / 1e9, 3), tile_efficiency=round(nnz / E, 4),
                    wall_ms_per_step=round(wall / K * 1e3, 4)),
        kernels_ms_untimed_pass={nm: round(x, 5) for nm, x in avg.items()},
        roofline=roof,
    )
    if not args.no_dense:
        result["dense_layer"] = dense_layer(args, torch, sa, (q, k, v, do), tok, sep, scale, cfg, ev_cls=Events)
    return result, inp, E_seqs


def dense_layer(args, torch, sa, tensors, tok, sep, scale, cfg, ev_cls):
    """The same inputs with a window n = S: every earlier key visible (a dense
    causal layer, as the hybrid's first and last layers), whole steps timed."""
    q, k, v, do = tensors
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    a, n = cfg["a"], S
    dev = q.device
    idx = sa.Index(B, S, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(sa.bwd_workspace_bytes(B, Hq, Hkv, S, d), dtype=torch.uint8, device=dev)

    def step():
        sa.build_index(tok, sep, a, n, index=idx)
        sa.fwd(q, k, v, idx, scale, o=o, lse=lse)
        sa.bwd(q, k, v, o, lse, do, idx, scale, dq=dq, dk=dk, dv=dv, ws=ws)

    for _ in range(args.warmup):
        step()
    ev = ev_cls()
    stream = torch.cuda.current_stream().cuda_stream
    t0, t1 = ev.new(2)
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for _ in range(args.steps):
        step()
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / args.steps
    ev.close()
    qt = idx.qtile.cpu().numpy().astype(np.int64)
    E = int((qt[:, :, 5] * 64 * qt[:, :, 4]).sum()) * Hq
    causal = B * Hq * S * (S + 1) // 2
    return dict(workload=f"same shapes, window n = S = {S} (dense causal)", ms_per_step=round(ms, 4),
                kept_tile_TFLOPs=round(14 * d * E / (ms * 1e-3) / 1e12, 3),
                causal_TFLOPs=round(14 * d * causal / (ms * 1e-3) / 1e12, 3))


def tiny_config(torch, sa, synth, calls=50):
    """The fp32 parity configuration (B1 H1 S512 d64, forward only): a
    latency figure, the median over `calls` event-timed launches of the
    index and of the forward."""
    cfg = synth.CONFIGS["tiny_fp32"]
    B, Hq, Hkv, S, d, a, n = (cfg[x] for x in ("B", "Hq", "Hkv", "S", "d", "a", "n"))
    inp = synth.prefill_inputs(cfg)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(inp[x], dtype=np.float32)).to(dev) for x in ("q", "k", "v"))
    tok = torch.from_numpy(inp["tok"]).to(dev)
    idx = sa.Index(B, S, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    ev = Events()
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(5):
        sa.build_index(tok, inp["sep"], a, n, index=idx)
        sa.fwd(q, k, v, idx, inp["scale"], o=o, lse=lse)
    marks = [ev.new(3) for _ in range(calls)]
    for m in marks:
        ev.record(m[0], stream)
        sa.build_index(tok, inp["sep"], a, n, index=idx)
        ev.record(m[1], stream)
        sa.fwd(q, k, v, idx, inp["scale"], o=o, lse=lse)
        ev.record(m[2], stream)
    torch.cuda.synchronize()
    t_idx = float(np.median([ev.ms(m[0], m[1]) for m in marks])) * 1e3
    t_fwd = float(np.median([ev.ms(m[1], m[2]) for m in marks])) * 1e3
    ev.close()
    return dict(B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, a=a, n=n, dtype="f32", calls=calls,
                index_us=round(t_idx, 2), fwd_us=round(t_fwd, 2))


def long_configs(args, torch, sa, synth):
    """The d=128 prefill/training shapes (Llama-3-8B-shaped prefill at 8192
    tokens, and 32768 tokens with bursty separators): whole steps (index,
    forward, backward) timed with events, then the forward alone.  Reported
    beside the main workload, not part of its value."""
    out = {}
    for name, steps in (("llama3_8b_prefill", 10), ("long_context_32k", 4)):
        cfg = synth.CONFIGS[name]
        B, Hq, Hkv, S, d, a, n = (cfg[x] for x in ("B", "Hq", "Hkv", "S", "d", "a", "n"))
        inp = synth.prefill_inputs(cfg, with_grad=True)
        dev = torch.device("cuda:0")

        def bf(x):
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

        q, k, v, do = bf(inp["q"]), bf(inp["k"]), bf(inp["v"]), bf(inp["do"])
        tok = torch.from_numpy(inp["tok"]).to(dev)
        sep, scale = inp["sep"], float(inp["scale"])
        del inp
        idx = sa.Index(B, S, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(sa.bwd_workspace_bytes(B, Hq, Hkv, S, d), dtype=torch.uint8, device=dev)
        ev = Events()
        stream = torch.cuda.current_stream().cuda_stream

        def step(fe=None):
            sa.build_index(tok, sep, a, n, index=idx)
            if fe is not None:
                ev.record(fe[0], stream)
            sa.fwd(q, k, v, idx, scale, o=o, lse=lse)
            sa.bwd(q, k, v, o, lse, do, idx, scale, dq=dq, dk=dk, dv=dv, ws=ws,
                   events=None if fe is None else fe[1:5])

        for _ in range(3):
            step()
        t0, t1 = ev.new(2)
        torch.cuda.synchronize()
        ev.record(t0, stream)
        for _ in range(steps):
            step()
        ev.record(t1, stream)
        torch.cuda.synchronize()
        ms_step = ev.ms(t0, t1) / steps
        # per kernel: events before the forward and around the backward's
        # kernels (dQ, main, finalize) in a second pass, not the timed one
        fmarks = [ev.new(5) for _ in range(steps)]
        for fe in fmarks:
            step(fe)
        torch.cuda.synchronize()
        kms = {nm: float(np.mean([ev.ms(fe[i], fe[i + 1]) for fe in fmarks]))
               for i, nm in enumerate(("fwd", "bwd_dq", "bwd_main", "bwd_finalize"))}
        ev.close()
        qtile = idx.qtile.cpu().numpy()
        pref = idx.sep_prefix.cpu().numpy()
        E = sum(schedule_counts(qtile[b], pref[b], a, n, S)[0] for b in range(B)) * Hq
        flops, nbytes = kernel_work(B, Hq, Hkv, S, d, E)
        dominant = max(("fwd", "bwd_dq", "bwd_main"), key=lambda k_: kms[k_])
        ms_fwd = kms["fwd"]
        fwd_tf = 4 * d * E / (ms_fwd * 1e-3) / 1e12
        out[name] = dict(B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, a=a, n=n, bursty=bool(cfg.get("bursty")),
                         steps=steps, ms_per_step=round(ms_step, 4), fwd_ms=round(ms_fwd, 4),
                         kept_tile_TFLOPs_fwd_bwd=round(14 * d * E / (ms_step * 1e-3) / 1e12, 3),
                         fwd_TFLOPs=round(fwd_tf, 3), fwd_frac_of_mfma_peak=round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                         kernels_ms_untimed_pass={k_: round(v_, 5) for k_, v_ in kms.items()},
                         roofline=roofline_block(dominant, kms[dominant], flops[dominant], nbytes[dominant],
                                                 traffic_from_profiles(KERNEL_SYMBOL[dominant], name)),
                         fwd_roofline=roofline_block("fwd", ms_fwd, flops["fwd"], nbytes["fwd"],
                                                     traffic_from_profiles("fwd_kernel", name)))
        del q, k, v, do, o, lse, dq, dk, dv, ws, idx, tok
        torch.cuda.empty_cache()
    return out


def decode_leg(args, torch, sa, synth):
    cfg = synth.CONFIGS["sepcache_decode"]
    B, Hq, Hkv, d, c, a, s, w = (cfg[x] for x in ("B", "Hq", "Hkv", "d", "c", "a", "s", "w"))
    T = args.decode_steps
    dev = torch.device("cuda:0")
    r = synth.rng(cfg["seed"])
    sep = synth.separator_ids(r, cfg["vocab"])
    toks = torch.from_numpy(synth.token_ids_iid(r, (T, B), cfg["vocab"], sep, cfg["p_sep"])).to(dev)
    gen = torch.Generator(device=dev).manual_seed(cfg["seed"])
    qs = torch.randn((T, B, Hq, d), device=dev, generator=gen).to(torch.bfloat16)
    ks = torch.randn((T, B, Hkv, d), device=dev, generator=gen).to(torch.bfloat16)
    vs = torch.randn((T, B, Hkv, d), device=dev, generator=gen).to(torch.bfloat16)
    cos, sin = sa.rope_table(cfg["theta"], c, d)
    cos, sin = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    scale = d ** -0.5
    cache = sa.SepCache(B, Hkv, d, c, a, s, w, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(cache.workspace_bytes(Hq), dtype=torch.uint8, device=dev)

    # untimed pass: cache lengths after every update (for the byte count)
    lens = torch.empty((T, B, 4), dtype=torch.int32, device=dev)
    for t in range(T):
        if t and t % 1024 == 0:
            log(f"  decode length pass: step {t}")
        cache.update(ks[t], vs[t], toks[t], sep)
        lens[t].copy_(cache.state)
    L = lens[:, :, :3].sum(-1).cpu().numpy().astype(np.int64)  # [T, B]

    ev = Events()
    stream = torch.cuda.current_stream().cuda_stream

    # per-kernel breakdown (events between every kernel); not the timed region
    cache.init()
    only_flushed = args.decode_flushed_only
    nb = 0 if only_flushed else min(T, args.decode_breakdown_steps)
    ring = EventRing(ev, 4)
    for t in range(nb):
        if t and t % 1024 == 0:
            log(f"  decode breakdown pass: step {t}")
        m = ring.take()
        ev.record(m[0], stream)
        cache.update(ks[t], vs[t], toks[t], sep)
        cache.decode(qs[t], cos, sin, scale, o=out, ws=ws, events=m[1:4])
    bt = ring.result()
    lob = nb // 2
    upd = np.array([x[0] for x in bt][lob:])
    mrg = np.array([x[2] for x in bt][lob:])

    total_ms = dec = None
    if not only_flushed:
        # timed region: T update + decode steps, events only at its ends
        cache.init()
        t0, t1 = ev.new(2)
        torch.cuda.synchronize()
        ev.record(t0, stream)
        for t in range(T):
            cache.update(ks[t], vs[t], toks[t], sep)
            cache.decode(qs[t], cos, sin, scale, o=out, ws=ws)
        ev.record(t1, stream)
        torch.cuda.synchronize()
        total_ms = ev.ms(t0, t1)

        # the decode kernel alone, cache-warm: the same steps with an event pair
        # around every decode kernel (read back in groups, outside the kernels)
        log("  decode timed pass done")
        cache.init()
        ring = EventRing(ev, 2)
        for t in range(T):
            if t and t % 1024 == 0:
                log(f"  decode cache-warm pass: step {t}")
            cache.update(ks[t], vs[t], toks[t], sep)
            m = ring.take()
            cache.decode(qs[t], cos, sin, scale, o=out, ws=ws, events=[m[0], m[1], None])
        dec = np.array([x[0] for x in ring.result()])

    # flushed pass: at every 8th step of the steady state, reading 512 MB of
    # scratch evicts the K/V working set (at most ~210 MB here, below the
    # 256 MB Infinity Cache) before the decode kernel is timed, so those
    # launches read their K/V rows from HBM.  The flush reads (a sum) rather
    # than writes, so the caches hold clean lines and the timed kernel pays
    # for no write-backs of the flush.
    lo = min(1024, T // 4)
    flush_every = 8
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    cache.init()
    sampled = [t for t in range(lo, T) if (t - lo) % flush_every == 0]
    sampled_set = set(sampled)
    ring = EventRing(ev, 2, depth=64)
    torch.cuda.synchronize()
    for t in range(T):
        if t and t % 1024 == 0:
            log(f"  decode flushed pass: step {t}")
        cache.update(ks[t], vs[t], toks[t], sep)
        if t in sampled_set:
            torch.sum(scratch, dim=(0,), out=flush_sink)
            m = ring.take()
            cache.decode(qs[t], cos, sin, scale, o=out, ws=ws, events=[m[0], m[1], None])
        else:
            cache.decode(qs[t], cos, sin, scale, o=out, ws=ws)
    fdec = np.array([x[0] for x in ring.result()])
    del scratch, flush_sink
    ev.close()
    handoff = prefill_handoff(torch, sa, synth, cfg, sep, cos.device)

    kv_bytes = (L * Hkv * d * 2 * 2).sum(axis=1)          # K and V rows, every slot, every kv head
    q_bytes = B * Hq * d * 2
    table_bytes = c * (d // 2) * 4 * 2
    dec_bytes = kv_bytes + q_bytes + table_bytes            # per decode-kernel launch
    gbs = dec_bytes[sampled].sum() / (fdec.sum() * 1e-3) / 1e9   # flushed: the HBM figure
    step_bytes = kv_bytes + 2 * q_bytes + B * Hkv * d * 2 * 2 + B * 4
    rnd = lambda x, k: None if x is None else round(float(x), k)  # noqa: E731
    gbs_warm = None if dec is None else dec_bytes[lo:].sum() / (dec[lo:].sum() * 1e-3) / 1e9
    step_ms = None if total_ms is None else total_ms / T
    traffic = traffic_from_profiles("decode_kernel", "sepcache_decode")
    return dict(
        workload="SepCache streaming decode: B64, 32 q / 8 kv heads, d128, bf16, c=800 (a4 s64 w256), "
                 "RoPE theta 500000 by slot, p_sep 0.08; value: decode kernel after reading 512 MB (cache flush)",
        steps=T, steady_from=lo, mean_cached_slots=round(float(L[lo:].mean()), 1),
        decode_kernel_us_flushed=round(float(fdec.mean()) * 1e3, 3),
        flushed_launches=len(sampled),
        decode_kernel_us_cache_warm=None if dec is None else round(float(dec[lo:].mean()) * 1e3, 3),
        cache_warm_GBps=rnd(gbs_warm, 1),
        merge_kernel_us_untimed_pass=round(float(mrg.mean()) * 1e3, 3) if nb else None,
        update_kernel_us_untimed_pass=round(float(upd.mean()) * 1e3, 3) if nb else None,
        us_per_step=None if step_ms is None else round(step_ms * 1e3, 3), loop_ms_total=rnd(total_ms, 3),
        value=round(float(gbs), 1), unit="GB/s",
        prefill_handoff=handoff,
        step_GBps=None if total_ms is None else round(float(step_bytes.sum() / (total_ms * 1e-3) / 1e9), 1),
        roofline=dict(kernel="decode_kernel", bound="hbm", achieved=round(float(gbs), 1), peak=PEAK_HBM_GBS,
                      unit="GB/s", frac=round(float(gbs) / PEAK_HBM_GBS, 4), traffic=traffic,
                      traffic_source=TRAFFIC_SOURCE if traffic else None,
                      algorithmic_MB_per_launch=round(float(dec_bytes[sampled].mean()) / 1e6, 3)),
    )


def prefill_handoff(torch, sa, synth, cfg, sep, dev, P=4096, reps=20):
    """sepcache_prefill of a P-token prompt per sequence (its index built
    beforehand, as the prefill pass has it): time per call and the bytes it
    moves (each kept K/V row read once and written once, plus pos/tok)."""
    B, Hkv, d, c, a, s, w = (cfg[x] for x in ("B", "Hkv", "d", "c", "a", "s", "w"))
    r = synth.rng(cfg["seed"] + 100)
    tok = torch.from_numpy(synth.token_ids_iid(r, (B, P), cfg["vocab"], sep, cfg["p_sep"])).to(dev)
    gen = torch.Generator(device=dev).manual_seed(cfg["seed"] + 100)
    k = torch.randn((B, Hkv, P, d), device=dev, generator=gen).to(torch.bfloat16)
    v = torch.randn((B, Hkv, P, d), device=dev, generator=gen).to(torch.bfloat16)
    idx = sa.build_index(tok, sep, a, 64)
    cache = sa.SepCache(B, Hkv, d, c, a, s, w, device=dev)
    for _ in range(3):
        cache.prefill(k, v, tok, idx)
    ev = Events()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = ev.new(2)
    torch.cuda.synchronize()
    ev.record(e0, stream)
    for _ in range(reps):
        cache.prefill(k, v, tok, idx)
    ev.record(e1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(e0, e1) / reps
    ev.close()
    L = int(cache.state[:, :3].sum())
    moved = L * Hkv * d * 2 * 2 * 2 + B * c * 4 * 2
    del k, v
    return dict(prompt_tokens=P, sequences=B, cached_slots_total=L, us_per_call=round(ms * 1e3, 3),
                GBps=round(moved / (ms * 1e-3) / 1e9, 1))


def cpu_leg(args, inp, E_seqs):
    """The oracle's fwd+bwd over whole sequences (all heads), one sequence at
    a time, until about --cpu-seconds of work or the whole batch is done."""
    from oracle import attention
    cfg = inp["cfg"]
    a, n, d, Hq = cfg["a"], cfg["n"], cfg["d"], cfg["Hq"]
    try:
        from threadpoolctl import threadpool_info
        cores = max([x.get("num_threads", 1) for x in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()

    spent, flops, nb = 0.0, 0, 0
    for b in range(len(E_seqs)):
        sl = (slice(b, b + 1), slice(0, Hq))
        t = time.perf_counter()
        attention.attention_forward(inp["qf"][sl], inp["kf"][sl], inp["vf"][sl], inp["tok"][b:b + 1], inp["sep"],
                                    a, n, scale=inp["scale"])
        attention.attention_backward(inp["qf"][sl], inp["kf"][sl], inp["vf"][sl], inp["dof"][sl],
                                     inp["tok"][b:b + 1], inp["sep"], a, n, scale=inp["scale"])
        spent += time.perf_counter() - t
        flops += (4 + 10) * d * E_seqs[b] * Hq  # kept-tile work of this sequence
        nb += 1
        if spent >= args.cpu_seconds:
            break
    out = dict(value=round(flops / spent / 1e12, 6), unit="TFLOP/s", cores=int(cores), kind="oracle",
               sample=f"fp64 numpy oracle fwd+bwd of sequences 0..{nb - 1}, all {Hq} heads, of the same inputs "
                      f"({nb * Hq} of {cfg['B'] * Hq} (sequence, head) pairs), {spent:.1f} s",
               seconds=round(spent, 2))
    out["cpu_model"] = cpu_model()
    try:  # the same oracle on one thread, sequence 0
        from threadpoolctl import threadpool_limits
        sl = (slice(0, 1), slice(0, Hq))
        with threadpool_limits(limits=1):
            t = time.perf_counter()
            attention.attention_forward(inp["qf"][sl], inp["kf"][sl], inp["vf"][sl], inp["tok"][0:1], inp["sep"],
                                        a, n, scale=inp["scale"])
            attention.attention_backward(inp["qf"][sl], inp["kf"][sl], inp["vf"][sl], inp["dof"][sl],
                                         inp["tok"][0:1], inp["sep"], a, n, scale=inp["scale"])
            t1 = time.perf_counter() - t
        out["single_thread"] = dict(value=round((4 + 10) * d * E_seqs[0] * Hq / t1 / 1e12, 6), unit="TFLOP/s",
                                    cores=1, sample=f"sequence 0, all {Hq} heads, {t1:.1f} s")
        out["tiny_fp32_forward_single_thread"] = tiny_oracle_time(threadpool_limits)
    except ImportError:
        pass
    return out


def cpu_model():
    """The host CPU's model name (as lscpu reports it, from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def tiny_oracle_time(threadpool_limits, reps=5):
    """The fp32 parity configuration (B1 H1 S512 d64, forward) through the
    oracle on one thread: median wall time of `reps` runs."""
    import synth
    from oracle import attention
    cfg = synth.CONFIGS["tiny_fp32"]
    inp = synth.prefill_inputs(cfg)
    times = []
    with threadpool_limits(limits=1):
        for _ in range(reps):
            t = time.perf_counter()
            attention.attention_forward(inp["qf"], inp["kf"], inp["vf"], inp["tok"], inp["sep"], cfg["a"], cfg["n"],
                                        scale=inp["scale"])
            times.append(time.perf_counter() - t)
    return dict(ms=round(float(np.median(times)) * 1e3, 3), cores=1,
                sample=f"B1 H1 S512 d64 fp32 forward, median of {reps} runs")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--decode-breakdown-steps", type=int, default=1024,
                    help="steps of the untimed per-kernel breakdown pass of the decode leg (0: none)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-flushed-only", action="store_true",
                    help="decode leg: only the length pass and the flushed pass (for counter runs, whose "
                         "per-dispatch overhead makes every pass slow)")
    ap.add_argument("--no-long", action="store_true", help="skip the d=128 Llama-shaped and 32k-token steps")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-layer (window n = S) steps of the Pythia-shaped leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first launch one device-to-device copy of this many MiB (a known-size kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (every configuration of this "
              f"workload fits one MI355X; see DESIGN.md for how the path would shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_sepattn_amd as sa
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sa.load_library()
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: read {args.copy_mib} MiB, wrote {args.copy_mib} MiB")
        del src, dst
    log("prefill/training leg ...")
    result, inp, E_seqs = prefill_leg(args, torch, sa, synth)
    log(f"  {result['value']} TFLOP/s, {result['ms_per_step']} ms/step")
    if not args.no_long:
        log("d=128 prefill/training shapes ...")
        result["other_configs"] = long_configs(args, torch, sa, synth)
        for nm, r in result["other_configs"].items():
            log(f"  {nm}: {r['ms_per_step']} ms/step, forward {r['fwd_ms']} ms = {r['fwd_TFLOPs']} TFLOP/s")
        result["other_configs"]["tiny_fp32"] = tiny = tiny_config(torch, sa, synth)
        log(f"  tiny_fp32: index {tiny['index_us']} us, forward {tiny['fwd_us']} us")
    if not args.no_decode:
        log("decode leg ...")
        result["decode"] = decode_leg(args, torch, sa, synth)
        log(f"  {result['decode']['value']} GB/s decode kernel")
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_leg(args, inp, E_seqs)
        log(f"  {result['cpu_baseline']['value']} TFLOP/s on {result['cpu_baseline']['cores']} threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
