#!/usr/bin/env python3
"""Benchmark of the 2-bit draft head on one MI355X.

One step = one full call of the head (coarse scores + block top-KCAND, row
top-R + exact rerank, argmax) on one rank's vocabulary shard, x[M, 5120] @
W[5120, 124160] with M = 1 (one draft slot), KCAND = 8, R = 32, on seeded
synthetic inputs already resident in HBM.  Each timed step reads a different
one of `--copies` device copies of the weights, so no step finds its 178.8 MB
of packed weights in the 256 MB Infinity Cache left by the previous step.

Prints one JSON line:
  value        HBM GB/s of the call: 178,790,400 B (packed codes + scale pair,
               the page's "0.167 GiB") / measured time per call
  ms_per_step  time per call (calls with no per-call events)
  roofline     the coarse kernel: algorithmic bytes per launch / its average
               duration (HIP events set by the kernel's own dispatch on the
               launch stream, in a second pass of as many calls) vs 8 TB/s
  cpu_baseline the CPU oracle timed on this host, one full call each at
               M = 1, 8, 72 (value: M = 1), with the CPU model, the cores
               visible and the BLAS threads
  extra.parity the acceptance report on the same inputs: per M = 1, 8, 72
               the comparator's counts (tie rows, excused near-tie lists,
               final-id differences on tie rows, value errors) and the argmax
               agreement with the exact bf16 head; the recall-stress case
               (M = 32, KCAND = 8 and 1) with its argmax misses
  extra        per-M (1, 8, 72) times with the coarse kernel's p10/p50/p90 and
               its fractions of the HBM and bf16 MFMA peaks, the warm
               (cache-resident) figure, the time of the row handed to a
               top-k caller (draft_head_logits_row), the per-call time with
               the e4m3 and NVFP4 rerank sources, the per-call time of the call
               that also builds the caller's bf16 row (draft_head_forward_row,
               full and top-k only, beside the plain call), of forwards
               replayed from a HIP graph (launch gaps removed; not the
               headline), the 4-bit head's per-call time
               (KCAND = 1, 357,580,800 B of codes and pairs per call),
               and the device's achieved
               read rate (the library's streaming-read reference) and copy rate
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0     # dense
K, N, KCAND, R = 5120, 124160, 8, 32
NBLK = (N + 63) // 64
WEIGHT_BYTES = N * (K // 4) + 2 * 2 * N * (K // 128)       # 178,790,400


def coarse_kernel_name(m: int) -> str:
    """The coarse kernel one launch at M rows runs (K = 5120 and the 2-bit
    head; one row runs the two-row instance; from three row tiles on, the
    fp16 many-row kernel)."""
    if m <= 8:
        return f"coarse_resident_kernel<{2 if m <= 2 else 4 if m <= 4 else 8}, false>"
    mt = min((m + 15) // 16, 5)
    return f"coarse_h16_kernel<{mt}>" if mt >= 3 else f"coarse_mfma_kernel<{mt}, false>"


def coarse_alg_bytes(m: int) -> int:
    """Bytes the coarse pass must move: packed codes + scale pair + x + candidates."""
    return WEIGHT_BYTES + 2 * K * m + 8 * NBLK * KCAND * m


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "bit_quantized_lm_amd", "csrc", "device.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


class Rig:
    """Device copies of the head and preallocated outputs for every M."""

    def __init__(self, copies: int, max_m: int):
        import torch
        from bit_quantized_lm_amd import _binding as B
        from bit_quantized_lm_amd import workload
        self.torch, self.B = torch, B
        dev = torch.device("cuda:0")
        t0 = time.time()
        log("generating W (bf16, N(0, 0.02)) and x (N(0, 1), 1% channels x8)")
        self.x_host, w = workload.make_inputs(workload.CONFIGS["m72"])
        self.w_host = w
        log(f"host quantize_pack ({time.time() - t0:.1f}s)")
        tq = time.time()
        packed = B.draft_head_quantize_pack(w)
        self.quantize_s = time.time() - tq
        tiled, pairs = B.draft_head_tile(*packed)
        log(f"upload {copies} copies ({time.time() - t0:.1f}s)")
        t_tiled = torch.from_numpy(tiled).to(dev)
        t_pairs = torch.from_numpy(pairs.view(np.int32)).to(dev)
        t_w = torch.from_numpy(w.view(np.int16)).to(dev)
        self.heads = []
        for c in range(copies):
            if c == 0:
                self.heads.append(B.DraftHead(t_tiled, t_pairs, t_w, N, K, KCAND, R))
            else:
                self.heads.append(B.DraftHead(t_tiled.clone(), t_pairs.clone(), t_w.clone(),
                                              N, K, KCAND, R))
        self.x = torch.from_numpy(self.x_host[:max_m].view(np.int16)).to(dev)
        self.dev = dev
        self.stream = torch.cuda.current_stream().cuda_stream   # looked up once
        self.out = {}
        self.ws = {}
        torch.cuda.synchronize()
        log(f"ready ({time.time() - t0:.1f}s)")

    def buffers(self, m):
        if m not in self.out:
            self.out[m] = self.B.forward_buffers(m, N, KCAND, R, self.dev)
            self.ws[m] = self.B.workspace_for(m, K, self.dev)
        return self.out[m]

    def step(self, m, head, ev=None):
        """One full call through the library's one-call entry point; `ev` takes
        the coarse kernel's own dispatch timestamps."""
        out = self.buffers(m)
        head(self.x[:m], stream=self.stream, out=out, coarse_events=ev, workspace=self.ws[m])

    def timed(self, m, steps, warmup, copies=None):
        """(seconds per call, seconds per coarse launch, wall seconds).

        The calls are timed over `steps` calls with no per-call events (the
        coarse kernel's dispatch events cost the stream a few microseconds
        per call); the coarse kernel's duration comes from a second pass of
        `steps` calls that pass those events.  Warm-up runs first, at least
        0.2 s of calls, so that the clocks have ramped."""
        torch = self.torch
        heads = self.heads if copies is None else self.heads[:copies]
        t0 = time.perf_counter()
        i = 0
        while i < warmup or time.perf_counter() - t0 < 0.2:
            self.step(m, heads[i % len(heads)])
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            self.step(m, heads[i % len(heads)])
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = start.elapsed_time(end)

        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:      # torch creates an event on its first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(m, heads[i % len(heads)], evs[i])
        torch.cuda.synchronize()
        coarse_ms = np.array([a.elapsed_time(b) for a, b in evs])
        self.last_coarse_pct = {f"p{q}": round(float(np.percentile(coarse_ms, q)) * 1e3, 2) for q in (10, 50, 90)}
        return total_ms / 1e3 / steps, float(np.mean(coarse_ms)) / 1e3, wall

    def tiny_call_us(self, steps=500):
        """Per-call time of the tiny configuration (M = 1, K = 1024, N = 16384,
        KCAND = 8, R = 32): launch latency more than bandwidth (its 4.2 MB of
        codes and pairs stay in the Infinity Cache between calls)."""
        torch, B = self.torch, self.B
        from bit_quantized_lm_amd import workload
        cfg = workload.CONFIGS["tiny"]
        x_host, w = workload.make_inputs(cfg)
        head = B.DraftHead.from_weight(w, kcand=cfg.kcand, R=cfg.rerank, device=self.dev)
        x = torch.from_numpy(x_host.view(np.int16)).to(self.dev)
        out = B.forward_buffers(cfg.m, cfg.n, cfg.kcand, cfg.rerank, self.dev)
        ws = B.workspace_for(cfg.m, cfg.k, self.dev)
        for i in range(50):
            head(x, stream=self.stream, out=out, workspace=ws)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(steps):
            head(x, stream=self.stream, out=out, workspace=ws)
        e.record()
        torch.cuda.synchronize()
        return {"us_per_call": round(s.elapsed_time(e) / steps * 1e3, 2), "M": cfg.m, "K": cfg.k, "N": cfg.n}

    def e4m3_call_us(self, ms=(1, 8, 72), steps=200):
        """Per-call time with the rerank reading an e4m3 copy of the head
        (a synthetic per-channel FP8 head; coarse pass unchanged)."""
        torch, B = self.torch, self.B
        from bit_quantized_lm_amd import workload
        if not hasattr(self, "w8"):
            w8, wscale = workload.e4m3_head(self.w_host)
            self.w8 = torch.from_numpy(w8).to(self.dev)
            self.wscale = torch.from_numpy(wscale).to(self.dev)
        res = {}
        for m in ms:
            heads = [B.DraftHead(h.tiled, h.pairs, self.w8, N, K, KCAND, R, wscale=self.wscale) for h in self.heads]
            out = self.buffers(m)
            for i in range(20):
                heads[i % len(heads)](self.x[:m], stream=self.stream, out=out, workspace=self.ws[m])
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for i in range(steps):
                heads[i % len(heads)](self.x[:m], stream=self.stream, out=out, workspace=self.ws[m])
            e.record()
            torch.cuda.synchronize()
            res[str(m)] = round(s.elapsed_time(e) / steps * 1e3, 2)
        return res

    def nvfp4_call_us(self, ms=(1, 8, 72), steps=200):
        """Per-call time with the rerank reading an NVFP4 copy of the head (a
        synthetic two-level-scaled FP4 head; coarse pass unchanged)."""
        torch, B = self.torch, self.B
        from bit_quantized_lm_amd import workload
        w4, bs, g = workload.nvfp4_head(self.w_host)
        t_w4 = torch.from_numpy(w4).to(self.dev)
        t_bs = torch.from_numpy(bs).to(self.dev)
        t_g = torch.tensor([g], dtype=torch.float32, device=self.dev)
        res = {}
        for m in ms:
            heads = [B.DraftHead(h.tiled, h.pairs, t_w4, N, K, KCAND, R, bscale=t_bs, gscale=t_g) for h in self.heads]
            out = self.buffers(m)
            for i in range(20):
                heads[i % len(heads)](self.x[:m], stream=self.stream, out=out, workspace=self.ws[m])
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for i in range(steps):
                heads[i % len(heads)](self.x[:m], stream=self.stream, out=out, workspace=self.ws[m])
            e.record()
            torch.cuda.synchronize()
            res[str(m)] = round(s.elapsed_time(e) / steps * 1e3, 2)
        del t_w4, t_bs
        return res

    def int4_call_us(self, ms=(1, 8, 72), steps=200, copies=2):
        """Per-call time of the 4-bit head at KCAND = 1 (the page's 4-bit
        configuration), its own bytes and pairs (draft_head_tile_int4:
        N K/2 + 4 N K/128 = 337,715,200 bytes a call); weights rotated."""
        torch, B = self.torch, self.B
        packed4 = B.draft_head_quantize_pack_int4(self.w_host)
        tiled, pairs = B.draft_head_tile_int4(*packed4)
        t_t = torch.from_numpy(tiled).to(self.dev)
        t_p = torch.from_numpy(pairs.view(np.int32)).to(self.dev)
        heads = [B.DraftHead(t_t if c == 0 else t_t.clone(), t_p if c == 0 else t_p.clone(), self.heads[0].w,
                             N, K, 1, R, bits=4) for c in range(copies)]
        res = {}
        for m in ms:
            out = B.forward_buffers(m, N, 1, R, self.dev)
            ws = B.workspace_for(m, 2 * K, self.dev)
            for i in range(20):
                heads[i % copies](self.x[:m], stream=self.stream, out=out, workspace=ws)
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for i in range(steps):
                heads[i % copies](self.x[:m], stream=self.stream, out=out, workspace=ws)
            e.record()
            torch.cuda.synchronize()
            res[str(m)] = round(s.elapsed_time(e) / steps * 1e3, 2)
        del heads, t_t, t_p
        return res

    def graph_us(self, m=1, calls=8, reps=50):
        """Per-call time of `calls` forwards (weight copies rotated) captured in
        one HIP graph and replayed: the launch gaps between calls removed."""
        torch = self.torch
        out = self.buffers(m)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                self.heads[i % len(self.heads)](self.x[:m], out=out, workspace=self.ws[m])
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        return round(s.elapsed_time(e) / (reps * calls) * 1e3, 2)

    def forward_row_us(self, m, reps=100):
        """Per-call time of draft_head_forward_row (the call with the caller's
        bf16 row built inside it; full and top-k only) beside the plain call,
        weights rotated."""
        torch, B = self.torch, self.B
        out = self.buffers(m)
        row = torch.empty((m, N), dtype=torch.int16, device=self.dev)
        res = {}
        for name in ("plain", "full", "topk_only"):
            def call(i):
                h = self.heads[i % len(self.heads)]
                if name == "plain":
                    h(self.x[:m], stream=self.stream, out=out, workspace=self.ws[m])
                else:
                    h.logits_row(self.x[:m], topk_only=name == "topk_only", stream=self.stream, out=out, row=row,
                                 workspace=self.ws[m])
            for i in range(10):
                call(i)
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for i in range(reps):
                call(i)
            e.record()
            torch.cuda.synchronize()
            res[name] = round(s.elapsed_time(e) / reps * 1e3, 2)
        return res

    def logits_row_us(self, m, reps=50):
        """Time of draft_head_logits_row alone at M rows (full and top-k only)."""
        torch, B = self.torch, self.B
        coarse = torch.empty((m, N), dtype=torch.float32, device=self.dev)
        out = self.heads[0](self.x[:m], coarse_out=coarse, stream=self.stream)
        row = torch.empty((m, N), dtype=torch.int16, device=self.dev)
        res = {}
        for name, c, topk in (("full", coarse, False), ("topk_only", None, True)):
            for _ in range(3):
                B.draft_head_logits_row(out["rr_id"], out["rr_val"], N, coarse=c, topk_only=topk, out=row,
                                        stream=self.stream)
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                B.draft_head_logits_row(out["rr_id"], out["rr_val"], N, coarse=c, topk_only=topk, out=row,
                                        stream=self.stream)
            e.record()
            torch.cuda.synchronize()
            res[name] = round(s.elapsed_time(e) / reps * 1e3, 2)
        return res

    def read_bandwidth(self, reps=20):
        """The device's streaming read rate with the library's read reference
        (draft_head_stream_read): over four rotated buffers of the weights'
        size (no Infinity-Cache reuse) and over one 1 GiB buffer, in GB/s."""
        torch, B = self.torch, self.B
        res = {}
        for name, size, nbuf in (("weights_size_rotated", WEIGHT_BYTES, 4), ("1GiB", 1 << 30, 1)):
            bufs = [torch.ones(size // 4, dtype=torch.int32, device=self.dev) for _ in range(nbuf)]
            out = torch.empty(B.DH_READ_BLOCKS, dtype=torch.int32, device=self.dev)
            for i in range(4):
                B.draft_head_stream_read(bufs[i % nbuf], out=out, stream=self.stream)
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for i in range(reps):
                B.draft_head_stream_read(bufs[i % nbuf], out=out, stream=self.stream)
            e.record()
            torch.cuda.synchronize()
            res[name] = round(size / (s.elapsed_time(e) / 1e3 / reps) / 1e9, 1)
            del bufs
        return res

    def copy_bandwidth(self, mib=1024, reps=5):
        """Device-to-device copy of `mib` MiB: (read + write bytes) / time."""
        torch = self.torch
        a = torch.empty(mib << 20, dtype=torch.uint8, device=self.dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            b.copy_(a)
        e.record()
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / 1e3 / reps
        del a, b
        return 2 * (mib << 20) / t / 1e9


def host_cpu():
    """CPU model, cores visible to this process, logical CPUs of the host, and
    the BLAS thread count numpy runs with."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    return {"model": model or platform.machine(), "cores": len(os.sched_getaffinity(0)),
            "host_logical_cpus": os.cpu_count(), "blas_threads": blas}


def cpu_baseline(x_host, w_host):
    """The oracle, untuned, on one full call each at M = 1, 8 and 72 (dequantise
    from the packed arrays, float64 GEMV, block top-8, row top-32, exact
    rerank, argmax); the value is the M = 1 call's.  Also returns the oracle's
    packed arrays and its M = 72 outputs (the rows are independent, so M = 1
    and 8 are prefixes) for the acceptance report."""
    import oracle
    cpu = host_cpu()
    packed = oracle.quantize_pack(w_host)
    per_m = {}
    ref = None
    for m in (1, 8, 72):
        x = x_host[:m]
        t0 = time.perf_counter()
        c = oracle.coarse(x, *packed)
        cv, ci = oracle.block_topk(c, KCAND)
        rr_id, _ = oracle.row_topr(cv, ci, R)
        e = oracle.rerank_exact(x, w_host, rr_id)
        out_id, out_val = oracle.final_argmax(rr_id, e)
        per_m[str(m)] = round((time.perf_counter() - t0) * 1e6, 1)
        ref = {"coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": e,
               "out_id": out_id, "out_val": out_val, "tie_rows": oracle.tie_rows(e),
               "tied_ids": oracle.tied_ids(rr_id, e)}
    t = per_m["1"] / 1e6
    base = {"value": round(WEIGHT_BYTES / t / 1e9, 4), "unit": "GB/s", "us_per_call": per_m["1"],
            "us_per_call_per_m": per_m,
            "cores": int(cpu["blas_threads"] or cpu["cores"]), "cpu": cpu["model"],
            "host_cores_visible": cpu["cores"], "host_logical_cpus": cpu["host_logical_cpus"],
            "blas_threads": cpu["blas_threads"], "kind": "oracle",
            "sample": "one full call each at M=1, 8, 72, K=5120, N=124160 (dequantise + float64 GEMV + "
                      "selection + rerank + argmax); value from M=1; quantisation not timed; cores = the "
                      "BLAS threads the oracle's GEMV ran on"}
    return base, packed, ref


def _prefix(ref, m):
    return {k: (v[:m] if isinstance(v, (np.ndarray, list)) else v) for k, v in ref.items()}


def acceptance_report(rig, packed, ref):
    """The acceptance figures on the benchmark's own inputs (part of the CPU
    baseline leg: the oracle's outputs against the GPU's on the same seeded
    inputs).  Per M = 1, 8, 72: the comparator's counts (tie rows, near-tie
    block and rerank lists it excused, final-id differences on tie rows, the
    largest value errors) and the argmax agreement of the GPU and of the
    oracle with the exact bf16 head; then the recall-stress case (M = 32,
    planted same-block pairs with a 0.01 logit gap) at KCAND = 8 and 1: parity
    with the oracle and the argmax misses against the planted winners."""
    import oracle
    from oracle.acceptance import compare
    from bit_quantized_lm_amd import workload
    torch, B = rig.torch, rig.B
    x_host, w_host = rig.x_host, rig.w_host
    t0 = time.perf_counter()
    E = oracle.exact_head(x_host[:72], w_host)
    exact_id = np.argmax(E, axis=1)
    res = {"per_m": {}}
    head = rig.heads[0]
    for m in (1, 8, 72):
        coarse = torch.empty((m, N), dtype=torch.float32, device=rig.dev)
        out = head(rig.x[:m], coarse_out=coarse)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in out.items()}
        got["coarse"] = coarse.cpu().numpy()
        st = compare(_prefix(ref, m), got, N, KCAND)
        st["argmax_agree_exact_head_gpu"] = int(np.sum(got["out_id"] == exact_id[:m]))
        st["argmax_agree_exact_head_oracle"] = int(np.sum(ref["out_id"][:m] == exact_id[:m]))
        st["parity"] = "pass"
        res["per_m"][str(m)] = st
        log(f"acceptance M={m}: {st}")
    # recall stress: only the planted rows of W change, so the oracle quantises
    # those rows and keeps its own arrays for the rest (rows are independent)
    cfg = workload.CONFIGS["recall"]
    xr = x_host[:cfg.m]
    wp, pairs = workload.plant_recall_pairs(xr, w_host, target=12.0, gap=0.01)
    rows = sorted({c for p in pairs for c in p})
    opacked = [a.copy() for a in packed]
    for a, b in zip(opacked, oracle.quantize_pack(wp[rows])):
        a[rows] = b
    lpacked = B.draft_head_quantize_pack(wp)
    same_bytes = all(np.array_equal(a, b) for a, b in zip(lpacked, opacked))
    c = oracle.coarse(xr, *opacked)
    winners = np.array([p[0] for p in pairs])
    tiled, tpairs = B.draft_head_tile(*lpacked)
    t_t = torch.from_numpy(tiled).to(rig.dev)
    t_p = torch.from_numpy(tpairs.view(np.int32)).to(rig.dev)
    t_w = torch.from_numpy(wp.view(np.int16)).to(rig.dev)
    rec = {"rows": cfg.m, "quantiser_bytes_equal": bool(same_bytes)}
    for kc in (8, 1):
        h = B.DraftHead(t_t, t_p, t_w, N, K, kc, R)
        out = h(rig.x[:cfg.m])
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in out.items()}
        cv, ci = oracle.block_topk(c, kc)
        rr_id, _ = oracle.row_topr(cv, ci, R)
        e = oracle.rerank_exact(xr, wp, rr_id)
        out_id, out_val = oracle.final_argmax(rr_id, e)
        r = {"coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": e, "out_id": out_id,
             "out_val": out_val, "tie_rows": oracle.tie_rows(e), "tied_ids": oracle.tied_ids(rr_id, e)}
        st = compare(r, got, N, kc, check_coarse=False)
        rec[f"kcand{kc}"] = {"misses_gpu": int(np.sum(got["out_id"] != winners)),
                             "misses_oracle": int(np.sum(out_id != winners)),
                             "tie_rows": st["tie_rows"], "blocks_excused": st["blocks_excused"],
                             "rows_rr_excused": st["rows_rr_excused"],
                             "final_mismatch_on_tie_rows": st["final_mismatch_on_tie_rows"], "parity": "pass"}
    del t_t, t_p, t_w
    res["recall_stress"] = rec
    res["seconds"] = round(time.perf_counter() - t0, 1)
    log(f"acceptance recall stress: {rec}")
    return res


def load_traffic(m):
    """HBM bytes per coarse launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"coarse_m{m}_k5120_n124160_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("device_hip_sha256_16") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--m", type=int, default=1, help="rows (draft slots) of the headline line")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-M and warm figures")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run one device copy of this size (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the draft head runs on one "
              "rank's vocabulary shard, and the cross-rank exchange of the per-row results is not "
              "implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy_mib:
        a = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": args.calib_copy_mib << 20}), flush=True)
        return
    from bit_quantized_lm_amd import _binding as B
    if not os.path.exists(B.library_path()):
        import __graft_entry__
        __graft_entry__.build()

    rig = Rig(args.copies, max(72, args.m))
    m = args.m
    t_call, t_coarse, wall = rig.timed(m, args.steps, args.warmup)
    coarse_pct = rig.last_coarse_pct
    log(f"M={m}: {t_call * 1e6:.1f} us/call, coarse {t_coarse * 1e6:.1f} us {coarse_pct}, wall {wall:.3f}s")

    extra = {"quantize_pack_host_s": round(rig.quantize_s, 2), "copies_rotated": args.copies}
    if not args.no_extra:
        per_m = {}
        for mm in (1, 8, 72):
            tc, tk, _ = rig.timed(mm, max(20, args.steps // 2), 5)
            per_m[str(mm)] = {"us_per_call": round(tc * 1e6, 2), "coarse_us": round(tk * 1e6, 2),
                              "coarse_us_pct": rig.last_coarse_pct,
                              "GBps": round(WEIGHT_BYTES / tc / 1e9, 1),
                              "frac_hbm_peak": round(WEIGHT_BYTES / tc / 1e9 / HBM_PEAK_GBPS, 4),
                              "coarse_GBps": round(coarse_alg_bytes(mm) / tk / 1e9, 1),
                              "coarse_frac_hbm_peak": round(coarse_alg_bytes(mm) / tk / 1e9 / HBM_PEAK_GBPS, 4),
                              "coarse_TFLOPs": round(2.0 * mm * K * N / tk / 1e12, 2),
                              "coarse_frac_bf16_mfma_peak": round(2.0 * mm * K * N / tk / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
            log(f"M={mm}: {per_m[str(mm)]}")
        extra["per_m"] = per_m
        tw, tkw, _ = rig.timed(m, args.steps, args.warmup, copies=1)
        extra["warm_not_hbm"] = {"us_per_call": round(tw * 1e6, 2), "coarse_us": round(tkw * 1e6, 2),
                                 "note": "one weight copy reused back to back: Infinity-Cache resident"}
        extra["logits_row_us"] = {str(mm): rig.logits_row_us(mm) for mm in (1, 8, 72)}
        extra["forward_row_us_per_call"] = {str(mm): rig.forward_row_us(mm) for mm in (1, 8, 72)}
        log(f"one call with the caller's bf16 row built inside it: {extra['forward_row_us_per_call']}")
        extra["tiny_config_call"] = rig.tiny_call_us()
        log(f"one call of the tiny configuration: {extra['tiny_config_call']}")
        extra["e4m3_rerank_us_per_call"] = rig.e4m3_call_us()
        extra["graph_replay_us_per_call"] = {str(m): rig.graph_us(m) for m in (1, 8, 72)}
        log(f"one call inside a replayed HIP graph: {extra['graph_replay_us_per_call']}")
        extra["nvfp4_rerank_us_per_call"] = rig.nvfp4_call_us()
        log(f"one call with the NVFP4 rerank source: {extra['nvfp4_rerank_us_per_call']}")
        extra["int4_kcand1_us_per_call"] = rig.int4_call_us()
        extra["int4_bytes_per_call"] = N * K // 2 + 4 * N * (K // 128)
        log(f"one call of the 4-bit head at KCAND=1: {extra['int4_kcand1_us_per_call']}")
        log(f"one call with the e4m3 rerank source: {extra['e4m3_rerank_us_per_call']}")
        log(f"row for the caller (draft_head_logits_row alone): {extra['logits_row_us']}")
        extra["device_copy_GBps"] = round(rig.copy_bandwidth(), 1)
        extra["stream_read_GBps"] = rig.read_bandwidth()
        log(f"read reference: {extra['stream_read_GBps']}, copy {extra['device_copy_GBps']}")

    alg = coarse_alg_bytes(m)
    achieved = alg / t_coarse / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(m),
                "kernel": coarse_kernel_name(m), "alg_bytes_per_launch": alg,
                "avg_launch_us": round(t_coarse * 1e6, 2), "launch_us_pct": coarse_pct}
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (one full call at M = 1, 8, 72)")
        cpu, opacked, ref = cpu_baseline(rig.x_host, rig.w_host)
        log(f"cpu oracle: {cpu}")
        log("acceptance: the GPU's outputs against the oracle's on the same inputs")
        extra["parity"] = acceptance_report(rig, opacked, ref)

    line = {
        "metric": "us/call + HBM GB/s (% peak), 2-bit draft head K=5120 N=124160, M=1/8/72",
        "value": round(WEIGHT_BYTES / t_call / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_call * 1e3, 5),
        "us_per_call": round(t_call * 1e6, 2),
        "frac_hbm_peak": round(WEIGHT_BYTES / t_call / 1e9 / HBM_PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"2-bit draft head, one vocab shard: M={m} K={K} N={N} KCAND={KCAND} R={R}",
                   "M": m, "K": K, "N": N, "kcand": KCAND, "rerank": R,
                   "weights": "int2 g128 asym (bf16 scale pair), fp32 accumulation"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
