#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's layer share on one MI355X.

A step is one pass of the whole hot path over one synthetic batch of a
Llama3-70B-shaped TP=8 rank (4096 tokens, hidden 8192, bf16):

  forward   QKV projection (column-parallel [8192,1280]), input rows arriving
            as 8 sequence chunks from a side stream (stand-in for the
            all-gather); O projection (row-parallel [1024,8192]) -> partial;
            reduction of 8 partials onto this rank's 512-token slice;
            MLP (up [8192,3584] chunk-fed + GeLU, down [3584,8192] -> partial);
            reduction onto the slice.
  backward  MLP (dY arriving in chunks; dZ, dW_down, dW_up, dX partial);
            reduction of dX; O (dY arriving in chunks; dA, dW_o);
            QKV (dW_qkv, dX partial); reduction of dX.

The 8 partials of each reduction are this rank's own (written by the GEMM
into its slot) plus 7 seeded stand-ins for the peers' contributions.

value = algorithmic GEMM work of the step (12 GEMMs, 2*M*N*K each,
1907.0 GFLOP) / step time.  Extra lines: the same step with inputs resident
(no chunk arrival), the 8 x [8192,8192] -> [1024,8192] reduction (GB/s), and
the Llama3-70B (bf16) / 405B (fp8) shaped MLP forwards.

python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extra] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
FP8_PEAK_TFLOPS = 5033.2
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=512)
    ap.add_argument("--producer-cus", type=int, default=32,
                    help="CUs of the stream that writes arriving chunks in the arrival step (the others run the GEMMs)")
    ap.add_argument("--yardstick", action="store_true",
                    help="bf16 GEMM 8192^3 in three layouts, ours next to torch.matmul (hipBLASLt), and ours on "
                         "256 / 128 / 64 CUs (CU-masked streams); one JSON line")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: one line per (T, chunks) of the Llama3-70B MLP share "
                         "(8192 tokens, D 8192, F 28672), T in 1, 2, 4, 8 and chunks in T, 2T, 4T")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 256 MiB device copy first (reference for HBM byte counters)")
    return ap.parse_args()


class Layer:
    """Device buffers and the step of the C5 workload (one TP=8 rank)."""

    def __init__(self, torch, tpm, si, M=4096, D=8192, F=28672, T=8, rank=0, heads=8, kv=1, hd=128,
                 producer_cus=32):
        self.torch, self.tpm = torch, tpm
        self.M, self.D, self.T, self.rank = M, D, T, rank
        self.Ft = F // T
        self.Nqkv = (heads + 2 * kv) * hd            # 1280
        self.Dattn = heads * hd                      # 1024
        self.C = T
        dev = "cuda"
        bf = lambda x: si.to_bf16(x).to(dev)
        M, D, Ft, Nq, Da = self.M, self.D, self.Ft, self.Nqkv, self.Dattn
        # seeds follow the workload recipe: X 1, W_up 2, W_down 3, dY_mlp 4,
        # W_qkv 5, W_o 6, attention output 7, dY_qkv 8, dY_o 9
        x = bf(si.normal_f32((M, D), 1))
        self.x_src = x                                # the gathered rows as they land
        self.x_qkv = torch.empty_like(x)
        self.x_mlp = torch.empty_like(x)
        self.w_qkv = bf(si.normal_f32((D, Nq), 5, 0.02))
        self.w_up = bf(si.normal_f32((D, Ft), 2, 0.02))
        self.w_o = bf(si.normal_f32((Da, D), 6, 0.02))
        self.w_down = bf(si.normal_f32((Ft, D), 3, 0.02))
        self.attn = bf(si.normal_f32((M, Da), 7))
        self.dy_qkv = bf(si.normal_f32((M, Nq), 8))
        self.dy_mlp_src = bf(si.normal_f32((M, D), 4))
        self.dy_o_src = bf(si.normal_f32((M, D), 9))
        self.dy_mlp = torch.empty_like(self.dy_mlp_src)
        self.dy_o = torch.empty_like(self.dy_o_src)
        for dst, src in ((self.x_qkv, x), (self.x_mlp, x), (self.dy_mlp, self.dy_mlp_src),
                         (self.dy_o, self.dy_o_src)):
            dst.copy_(src)
        e = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
        self.qkv = e(M, Nq)
        self.z, self.h = e(M, Ft), e(M, Ft)
        self.d_attn = e(M, Da)
        self.g_qkv, self.g_up, self.g_o, self.g_down = e(D, Nq), e(D, Ft), e(Da, D), e(Ft, D)
        # partial stack: slot `rank` is written by the GEMMs, the other slots
        # hold the peers' stand-in partials (N(0,1), seeds 100 + t)
        self.stack = e(T, M, D)
        for t in range(T):
            if t != rank:
                self.stack[t] = bf(si.normal_f32((M, D), 100 + t))
        self.slice_o, self.slice_mlp, self.slice_dxm, self.slice_dxq = (e(M // T, D) for _ in range(4))
        self.ws_fwd = tpm.alloc_workspace(tpm.OP_MLP_FWD, M, D, F, T, self.C, tpm.BF16)
        self.ws_bwd = tpm.alloc_workspace(tpm.OP_MLP_BWD, M, D, F, T, self.C, tpm.BF16)
        # one workspace for all seq_chunk_gemm calls (stream-ordered): control
        # words plus the split-K scratch of the narrowest projections
        shapes = [(M, Nq, D, T), (M, D, Da, T), (M, Da, D, T), (Da, D, M, 1), (D, Nq, M, 1), (M, D, Nq, 1)]
        self.ws_g = torch.zeros(max(tpm.workspace_bytes(tpm.OP_SEQ_CHUNK_GEMM, m, n, k, 1, c) for m, n, k, c in shapes),
                                dtype=torch.uint8, device=dev)
        # and one for the paired backward launches of the two projections
        self.ws_l = torch.zeros(max(tpm.workspace_bytes(tpm.OP_LINEAR_BWD, M, n, k) for n, k in ((D, Da), (Nq, D))),
                                dtype=torch.uint8, device=dev)
        self.flags = torch.zeros(4, self.C, dtype=torch.int32, device=dev)
        self.counters = torch.zeros(4, self.C, dtype=torch.int32, device=dev)
        self.order = si.ring_chunk_order(T, self.C, rank)
        self.dest = si.dest_range_order(T, rank)
        self.producer_cus = producer_cus
        self.compute, self.side = tpm.masked_streams(producer_cus=producer_cus)
        self.gemm_events = []
        fl = lambda m, n, k: 2.0 * m * n * k
        self.flops = (3 * fl(M, Nq, D) + 3 * fl(M, Ft, D) + 3 * fl(M, D, Da) + 3 * fl(M, D, Ft))

    # -- chunk arrival: the producer stream writes the remote chunks in ring
    # order (one tpm_write_chunks launch, which publishes each chunk's ready
    # flag as soon as its rows are in place; the rank's own chunks are only
    # flagged).  The boundary event is recorded on the compute stream before
    # the chunk-fed GEMM is enqueued; the writer is enqueued after it (its
    # host-side launch cost overlaps the GEMM) but starts at the boundary.
    def _boundary(self):
        ev = self.torch.cuda.Event()
        ev.record(self.torch.cuda.current_stream())
        return ev

    def _arrive(self, which, dst, src, epoch, boundary):
        own = set(range(self.rank * (self.C // self.T), (self.rank + 1) * (self.C // self.T)))
        self.side.wait_event(boundary)            # communication starts at the layer boundary
        self.tpm.write_chunks(dst, src, self.C, self.order, self.flags[which], epoch, self.counters[which],
                              copy=[c not in own for c in range(self.C)], stream=self.side)

    def _timed(self, fn, record):
        if not record:
            fn()
            return
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.gemm_events.append((a, b))

    def _check(self, ws, check):
        if not check:
            return
        self.torch.cuda.synchronize()
        err = self.tpm.poll_device_error(ws)
        if err != 0:
            raise RuntimeError(f"device error {err} in a chunk-gated call (watchdog): the timing is invalid")

    def step(self, epoch: int, arrive: bool = True, record: bool = False, check: bool = False):
        torch, tpm = self.torch, self.tpm
        T, r, C = self.T, self.rank, self.C
        ready = (lambda i: self.flags[i]) if arrive else (lambda i: None)
        wsg = self.ws_g
        own_slot = self.stack[r]
        # ---- forward, attention projections
        b = self._boundary()
        self._timed(lambda: tpm.seq_chunk_gemm(self.x_qkv, self.w_qkv, self.qkv, num_chunks=C,
                                               chunk_order=self.order, chunk_ready=ready(0), epoch=epoch,
                                               workspace=wsg), record)
        if arrive:
            self._arrive(0, self.x_qkv, self.x_src, epoch, b)
        self._check(wsg, check)
        self._timed(lambda: tpm.seq_chunk_gemm(self.attn, self.w_o, own_slot, num_chunks=T,
                                               chunk_order=self.dest, workspace=wsg), record)
        tpm.partial_reduce_seqshard(self.stack, self.slice_o, T=T, rank=r)
        # ---- forward, MLP
        b = self._boundary()
        self._timed(lambda: tpm.tp_mlp_fwd(self.x_mlp, self.w_up, self.w_down, self.h, own_slot, T=T, rank=r,
                                           act=tpm.ACT_GELU_ERF, Z_t=self.z, num_chunks=C,
                                           chunk_order=self.order, chunk_ready=ready(1), epoch=epoch,
                                           workspace=self.ws_fwd), record)
        if arrive:
            self._arrive(1, self.x_mlp, self.x_src, epoch, b)
        self._check(self.ws_fwd, check)
        tpm.partial_reduce_seqshard(self.stack, self.slice_mlp, T=T, rank=r)
        # ---- backward, MLP
        b = self._boundary()
        self._timed(lambda: tpm.tp_mlp_bwd(self.x_mlp, self.w_up, self.w_down, self.z, self.h, self.dy_mlp,
                                           self.g_up, self.g_down, own_slot, T=T, rank=r,
                                           act=tpm.ACT_GELU_ERF, num_chunks=C, dy_chunk_order=self.order,
                                           dy_ready=ready(2), epoch=epoch, workspace=self.ws_bwd), record)
        if arrive:
            self._arrive(2, self.dy_mlp, self.dy_mlp_src, epoch, b)
        self._check(self.ws_bwd, check)
        tpm.partial_reduce_seqshard(self.stack, self.slice_dxm, T=T, rank=r)
        # ---- backward, O projection: dA = dY_o W_o^T, dW_o = A^T dY_o.  All of
        # dY_o resident: one paired launch (tp_linear_bwd); with dY_o's rows
        # arriving: dA chunk-fed, then dW_o (which needs every row)
        if not arrive:
            self._timed(lambda: tpm.tp_linear_bwd(self.attn, self.w_o, self.dy_o, self.g_o, self.d_attn,
                                                  workspace=self.ws_l), record)
        b = self._boundary() if arrive else None

        def o_bwd_dgrad():
            tpm.seq_chunk_gemm(self.dy_o, self.w_o, self.d_attn, trans_b=True, num_chunks=C,
                               chunk_order=self.order, chunk_ready=ready(3), epoch=epoch, workspace=wsg)

        def o_bwd_wgrad():
            tpm.seq_chunk_gemm(self.attn, self.dy_o, self.g_o, trans_a=True, workspace=wsg)
        if arrive and check:
            o_bwd_dgrad()
            self._arrive(3, self.dy_o, self.dy_o_src, epoch, b)
            self._check(wsg, check)
            o_bwd_wgrad()
        elif arrive:
            self._timed(lambda: (o_bwd_dgrad(), o_bwd_wgrad()), record)
            self._arrive(3, self.dy_o, self.dy_o_src, epoch, b)

        # ---- backward, QKV projection: dW_qkv = X^T dQKV, dX = dQKV W_qkv^T
        # (partial), one paired launch
        self._timed(lambda: tpm.tp_linear_bwd(self.x_qkv, self.w_qkv, self.dy_qkv, self.g_qkv, own_slot,
                                              workspace=self.ws_l), record)
        tpm.partial_reduce_seqshard(self.stack, self.slice_dxq, T=T, rank=r)
        if arrive:
            done = torch.cuda.Event()
            done.record(self.side)
            torch.cuda.current_stream().wait_event(done)


def time_steps(torch, layer, steps, warmup, arrive, epoch0):
    """Warm-up, then `steps` timed steps on the compute stream (the CU-masked
    one when chunks arrive from the producer stream, the default stream with
    every CU when all chunks are resident)."""
    stream = layer.compute if arrive else torch.cuda.default_stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            layer.step(epoch0 + i, arrive=arrive)
        torch.cuda.synchronize()
        layer.gemm_events = []
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            layer.step(epoch0 + warmup + i, arrive=arrive, record=True)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(stop) / steps
        gemm_ms = sum(a.elapsed_time(b) for a, b in layer.gemm_events) / steps
        # one more step that synchronises after every chunk-gated call and
        # reads its device error word: a wait that ran into the watchdog would
        # have made the timed steps meaningless
        if arrive:
            layer.step(epoch0 + warmup + steps, arrive=arrive, check=True)
    return ms, gemm_ms, wall


def time_steps_graph(torch, layer, steps, warmup):
    """The resident step captured once in a HIP graph and replayed: the same
    kernels with the same arguments, without the host launching each of
    them.  Returns ms per step."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step(0, arrive=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(0, arrive=False)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def arrival_step(torch, layer, args, ms_resident):
    """The same step with the chunk-fed GEMMs (QKV, MLP up, dZ, dA) gated on
    chunks that a producer stream writes in ring order while they run, the
    producer confined to `producer_cus` CUs (32 by default: about 0.67 TB/s
    of chunk writes, the order of a rank's ingress over 7 xGMI links) and
    the GEMMs to the others.  Reports the writer's time alone (4 launches of
    7 x 8 MB) and the overlap efficiency
    (t_resident + t_copy - t_overlap) / min(t_resident, t_copy)."""
    ms, gemm_ms, _ = time_steps(torch, layer, args.steps, args.warmup, arrive=True, epoch0=1000)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    epoch = 5000
    for rep in range(2):
        a.record(layer.side)
        for which, (dst, src) in enumerate(((layer.x_qkv, layer.x_src), (layer.x_mlp, layer.x_src),
                                            (layer.dy_mlp, layer.dy_mlp_src), (layer.dy_o, layer.dy_o_src))):
            layer._arrive(which, dst, src, epoch + rep, a)
        b.record(layer.side)
        torch.cuda.synchronize()
    t_copy = a.elapsed_time(b)
    eff = (ms_resident + t_copy - ms) / min(ms_resident, t_copy)
    return {"ms": round(ms, 4), "TFLOPS": round(layer.flops / (ms * 1e-3) / 1e12, 2),
            "gemm_TFLOPS": round(layer.flops / (gemm_ms * 1e-3) / 1e12, 2),
            "writer_only_ms": round(t_copy, 4), "overlap_efficiency": round(eff, 3),
            "producer_cus": layer.producer_cus}


def bench_reduce(torch, tpm, si, iters=40):
    """8 bf16 partials [8192, 8192] -> rank slice [1024, 8192]; the rank
    rotates 0..7 so each launch reads a different 134 MB (the 1 GiB stack
    does not fit the 256 MB last-level cache).  Launches are timed back to
    back (one event pair around all of them), so the per-launch figure is
    the kernel's duration plus the gap between consecutive kernels; the
    single-launch median (one event pair per launch) is reported beside it."""
    T, M, D = 8, 8192, 8192
    P = torch.empty(T, M, D, dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        P[t] = si.to_bf16(si.normal_f32((M, D), 100 + t)).cuda()
    out = torch.empty(M // T, D, dtype=torch.bfloat16, device="cuda")
    for r in range(T):
        tpm.partial_reduce_seqshard(P, out, T=T, rank=r)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        tpm.partial_reduce_seqshard(P, out, T=T, rank=i % T)
    b.record()
    torch.cuda.synchronize()
    per_launch = a.elapsed_time(b) / iters
    evs = []
    for i in range(iters):
        x, y = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        x.record()
        tpm.partial_reduce_seqshard(P, out, T=T, rank=i % T)
        y.record()
        evs.append((x, y))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in evs)
    med = ms[len(ms) // 2]
    nbytes = T * (M // T) * D * 2 + (M // T) * D * 2
    del P
    return dict(bytes=nbytes, ms_back_to_back=per_launch, GBs=nbytes / (per_launch * 1e-3) / 1e9,
                frac_hbm_peak=nbytes / (per_launch * 1e-3) / 1e9 / HBM_PEAK_GBS,
                ms_single_launch_median=med, GBs_single_launch=nbytes / (med * 1e-3) / 1e9)


def bench_mlp_fwd(torch, tpm, si, M, D, F, T, C, fp8, iters=10):
    Ft = F // T
    dev = "cuda"
    x = si.normal_f32((M, D), 1)
    wu = si.normal_f32((D, Ft), 2, 0.02)
    wd = si.normal_f32((Ft, D), 3, 0.02)
    H = torch.empty(M, Ft, dtype=torch.bfloat16, device=dev)
    P = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    if fp8:
        import numpy as np
        xq, sx = si.to_e4m3_current(x)
        wuq, su = si.to_e4m3_current(np.ascontiguousarray(wu.T))
        wdq, sd = si.to_e4m3_current(np.ascontiguousarray(wd.T))
        X, WU, WD = xq.to(dev), wuq.to(dev), wdq.to(dev)
        scales = torch.tensor([sx, su, sd], dtype=torch.float32, device=dev)
        ws = tpm.alloc_workspace(tpm.OP_MLP_FWD, M, D, F, T, C, tpm.FP8_E4M3)
        call = lambda: tpm.tp_mlp_fwd(X, WU, WD, H, P, T=T, rank=0, act=tpm.ACT_GELU_ERF, scales=scales,
                                      num_chunks=C, workspace=ws)
    else:
        X, WU, WD = si.to_bf16(x).to(dev), si.to_bf16(wu).to(dev), si.to_bf16(wd).to(dev)
        call = lambda: tpm.tp_mlp_fwd(X, WU, WD, H, P, T=T, rank=0, act=tpm.ACT_GELU_ERF, num_chunks=C)
    del x, wu, wd
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[iters // 2]
    flops = 2.0 * M * Ft * D * 2
    peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    tf = flops / (ms * 1e-3) / 1e12
    return dict(M=M, D=D, F=F, T=T, chunks=C, dtype="fp8_e4m3" if fp8 else "bf16", ms=ms, TFLOPS=tf,
                frac_mfma_peak=tf / peak)


def sweep_point(torch, tpm, si, M, D, F, T, C, iters=10):
    """Rank 0's MLP share at tensor-parallel degree T with its X (and dY)
    cut into C sequence chunks, chunk-gated with every flag already set:
    forward (GEMM1 + GeLU, GEMM2) and backward (dZ, dW_down, dW_up, dX) timed
    separately with events, bf16."""
    Ft = F // T
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(1000 * T + C)
    rnd = lambda *shape, s=1.0: (torch.randn(*shape, generator=g, device=dev) * s).to(torch.bfloat16)
    X, Wu, Wd, dY = rnd(M, D), rnd(D, Ft, s=0.02), rnd(Ft, D, s=0.02), rnd(M, D)
    Z = torch.empty(M, Ft, dtype=torch.bfloat16, device=dev)
    H, P, dX = torch.empty_like(Z), torch.empty(M, D, dtype=torch.bfloat16, device=dev), torch.empty_like(X)
    dWu, dWd = torch.empty_like(Wu), torch.empty_like(Wd)
    flags = torch.full((C,), 1, dtype=torch.int32, device=dev)
    order = si.ring_chunk_order(T, C, 0)
    wsf = tpm.alloc_workspace(tpm.OP_MLP_FWD, M, D, F, T, C, tpm.BF16)
    wsb = tpm.alloc_workspace(tpm.OP_MLP_BWD, M, D, F, T, C, tpm.BF16)
    fwd = lambda: tpm.tp_mlp_fwd(X, Wu, Wd, H, P, T=T, rank=0, act=tpm.ACT_GELU_ERF, Z_t=Z, num_chunks=C,
                                 chunk_order=order, chunk_ready=flags, epoch=1, workspace=wsf)
    bwd = lambda: tpm.tp_mlp_bwd(X, Wu, Wd, Z, H, dY, dWu, dWd, dX, T=T, rank=0, act=tpm.ACT_GELU_ERF,
                                 num_chunks=C, dy_chunk_order=order, dy_ready=flags, epoch=1, workspace=wsb)
    out = {}
    for name, fn, gemms in (("fwd", fwd, 2), ("bwd", bwd, 4)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)[iters // 2]
        tf = gemms * 2.0 * M * Ft * D / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "TFLOPS": round(tf, 1), "frac_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    assert tpm.poll_device_error(wsf) == 0 and tpm.poll_device_error(wsb) == 0
    ms = out["fwd"]["ms"] + out["bwd"]["ms"]
    return {"sweep": "tp_degree_and_chunks", "M": M, "D": D, "F": F, "T": T, "F_t": Ft, "chunks": C,
            "chunk_rows": M // C, "dtype": "bf16", **out, "ms_fwd_bwd": round(ms, 4),
            "TFLOPS_fwd_bwd": round(6 * 2.0 * M * Ft * D / (ms * 1e-3) / 1e12, 1)}


def run_yardstick(torch, tpm):
    """Yardsticks for the GEMM kernel on one square bf16 product (M = N = K =
    8192, random normal operands): ours and torch.matmul (hipBLASLt) in the
    three operand layouts (A and B row-major; B stored [N, K]; A stored
    [K, M]), then ours on streams restricted to a half and a quarter of the
    CUs (128 and 64 on MI355X), which shows
    how the per-CU rate depends on how many CUs share the L2s and the
    fabric.  Median of 10 calls each, HIP events; prints one JSON line."""
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    at, bt = a.t().contiguous(), b.t().contiguous()
    y = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    fl = 2.0 * n ** 3

    def med(fn, reps=10, stream=None):
        stream = stream or torch.cuda.current_stream()
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[reps // 2]

    out = {"shape": [n, n, n], "dtype": "bf16", "unit": "TFLOP/s"}
    layouts = {"NN": (lambda: tpm.seq_chunk_gemm(a, b, y), lambda: torch.matmul(a, b, out=y)),
               "NT": (lambda: tpm.seq_chunk_gemm(a, bt, y, trans_b=True), lambda: torch.matmul(a, bt.t(), out=y)),
               "TN": (lambda: tpm.seq_chunk_gemm(at, b, y, trans_a=True), lambda: torch.matmul(at.t(), b, out=y))}
    for name, (ours, blas) in layouts.items():
        out[f"ours_{name}"] = round(fl / (med(ours) * 1e-3) / 1e12, 1)
        out[f"hipblaslt_{name}"] = round(fl / (med(blas) * 1e-3) / 1e12, 1)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    for keep in (ncu // 2, ncu // 4):
        comp, _ = tpm.masked_streams(producer_cus=ncu - keep)
        with torch.cuda.stream(comp):
            t = med(lambda: tpm.seq_chunk_gemm(a, b, y), reps=6, stream=comp)
        out[f"ours_NN_{keep}cus"] = round(fl / (t * 1e-3) / 1e12, 1)
        out[f"ours_NN_{keep}cus_per_cu_as_{ncu}"] = round(fl / (t * 1e-3) / 1e12 * ncu / keep, 1)
    print(json.dumps({"yardstick": out}), flush=True)


def run_sweep(torch, tpm, si):
    M, D, F = 8192, 8192, 28672
    for T in (1, 2, 4, 8):
        for C in (T, 2 * T, 4 * T):
            print(json.dumps(sweep_point(torch, tpm, si, M, D, F, T, C)), flush=True)
            torch.cuda.empty_cache()


def bench_mlp_fwd_delayed(torch, tpm, si, M=8192, D=16384, F=53248, T=8, C=16, iters=10):
    """The fp8 configuration's MLP forward under delayed scaling: H's scale
    comes from the amax history (updated on the device after each call), so
    GEMM1 writes e4m3 H directly; inputs resident (no chunk flags, every CU)."""
    import numpy as np
    Ft = F // T
    dev = "cuda"
    xq, sx = si.to_e4m3_current(si.normal_f32((M, D), 1))
    wuq, su = si.to_e4m3_current(np.ascontiguousarray(si.normal_f32((D, Ft), 2, 0.02).T))
    wdq, sd = si.to_e4m3_current(np.ascontiguousarray(si.normal_f32((Ft, D), 3, 0.02).T))
    X, WU, WD = xq.to(dev), wuq.to(dev), wdq.to(dev)
    scales = torch.tensor([sx, su, sd], dtype=torch.float32, device=dev)
    hist = torch.zeros(16, dtype=torch.float32, device=dev)
    hs = torch.ones(1, dtype=torch.float32, device=dev)
    H = torch.empty(M, Ft, dtype=torch.uint8, device=dev)
    P = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    ws = tpm.alloc_workspace(tpm.OP_FP8_DELAYED_MLP_FWD, M, D, F, T, C, tpm.FP8_E4M3)
    order = si.ring_chunk_order(T, C, 0)
    step = [0]

    def call():
        k = step[0] % hist.numel()
        tpm.tp_mlp_fwd_delayed(X, WU, WD, H, P, T=T, rank=0, scales=scales, h_scale=hs,
                               h_amax_out=hist[k:k + 1], act=tpm.ACT_GELU_ERF, num_chunks=C, chunk_order=order,
                               workspace=ws)
        tpm.fp8_delayed_scale(hist, hs)
        step[0] += 1
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    assert tpm.poll_device_error(ws) == 0
    ms = sorted(a.elapsed_time(b) for a, b in evs)[iters // 2]
    tf = 2.0 * M * Ft * D * 2 / (ms * 1e-3) / 1e12
    return dict(M=M, D=D, F=F, T=T, chunks=C, dtype="fp8_e4m3 (delayed scaling, history 16)", ms=ms, TFLOPS=tf,
                frac_mfma_peak=tf / FP8_PEAK_TFLOPS)


def bench_mlp_bwd_fp8(torch, tpm, M=8192, D=16384, F=53248, T=8, iters=10):
    """The fp8 configuration's MLP backward in fp8 (e5m2 gradients with
    current scaling, e4m3 activations and weights): the casts of dY, H and X
    and the four GEMMs, timed with events.  Inputs drawn on the device (N(0,1)
    activations and gradients, N(0, 0.02) weights) and cast with the
    library's own current-scaling cast."""
    Ft = F // T
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rnd = lambda r, c, s=1.0: (torch.randn(r, c, generator=g, device=dev) * s).to(torch.bfloat16)

    def fp8(x):
        q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
        sc = torch.empty(1, dtype=torch.float32, device=dev)
        tpm.cast_fp8(x, tpm.FP8_E4M3, q=q, scale_out=sc)
        return q, sc
    X, sx = fp8(rnd(M, D))
    WU, su = fp8(rnd(D, Ft, 0.02))
    WD, sd = fp8(rnd(Ft, D, 0.02))
    scales = torch.cat([sx, su, sd])
    Z, H, dY = rnd(M, Ft), rnd(M, Ft).abs(), rnd(M, D)
    dWu = torch.empty(D, Ft, dtype=torch.bfloat16, device=dev)
    dWd = torch.empty(Ft, D, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    ws = tpm.alloc_workspace(tpm.OP_MLP_BWD_FP8, M, D, F, T, 1, tpm.FP8_E4M3)
    call = lambda: tpm.tp_mlp_bwd_fp8(X, WU, WD, Z, H, dY, dWu, dWd, dX, T=T, rank=0, scales=scales,
                                      act=tpm.ACT_GELU_ERF, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[iters // 2]
    tf = 4 * 2.0 * M * Ft * D / (ms * 1e-3) / 1e12
    return dict(M=M, D=D, F=F, T=T, dtype="fp8 (e4m3 activations / weights, e5m2 gradients)", ms=ms, TFLOPS=tf,
                frac_mfma_peak=tf / FP8_PEAK_TFLOPS)


def bench_mlp_fwd_mx(torch, tpm, si, M=8192, D=16384, F=53248, T=8, C=16, iters=10):
    """The fp8 configuration's MLP forward under MXFP8 block scaling (inputs
    and weights MXFP8 along their contraction axes, H requantised to MXFP8 in
    GEMM1's epilogue), inputs resident (no chunk flags, every CU); events."""
    Ft = F // T
    dev = "cuda"
    def mx(x, k):
        c, e = si.to_mxfp8(x)
        return c.to(dev), tpm.mx_swizzle_scales(e.to(dev), k)
    X, Xs = mx(si.normal_f32((M, D), 1), D)
    WU, WUs = mx(si.normal_f32((Ft, D), 2, 0.02), D)
    WD, WDs = mx(si.normal_f32((D, Ft), 3, 0.02), Ft)
    H = torch.empty(M, Ft, dtype=torch.uint8, device=dev)
    Hs = torch.zeros(tpm.mx_scales_bytes(M, Ft), dtype=torch.uint8, device=dev)
    P = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    ws = tpm.alloc_workspace(tpm.OP_MX_MLP_FWD, M, D, F, T, C, tpm.FP8_E4M3)
    order = si.ring_chunk_order(T, C, 0)
    call = lambda: tpm.tp_mlp_fwd_mx(X, Xs, WU, WUs, WD, WDs, H, Hs, P, T=T, rank=0, act=tpm.ACT_GELU_ERF,
                                     num_chunks=C, chunk_order=order, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    assert tpm.poll_device_error(ws) == 0
    ms = sorted(a.elapsed_time(b) for a, b in evs)[iters // 2]
    tf = 2.0 * M * Ft * D * 2 / (ms * 1e-3) / 1e12
    return dict(M=M, D=D, F=F, T=T, chunks=C, dtype="mxfp8 (e4m3, 32-element E8M0 blocks)", ms=ms, TFLOPS=tf,
                frac_mfma_peak=tf / FP8_PEAK_TFLOPS)


def bench_gated_mlp(torch, tpm, si, M=8192, D=4096, F=16384, T=4, C=4, iters=10):
    """The worked example's gated MLP share (X [8192, 4096], F = 16384, T = 4:
    gate and up shards [4096, 4096] each, contraction shard [4096, 4096]),
    SwiGLU, bf16, rank 0, inputs resident (no chunk flags, every CU): forward
    and backward timed separately with events."""
    import numpy as np
    Ft = F // T
    dev = "cuda"
    X = si.to_bf16(si.normal_f32((M, D), 1)).to(dev)
    WGU = si.to_bf16(np.concatenate([si.normal_f32((D, Ft), 2, 0.02), si.normal_f32((D, Ft), 5, 0.02)],
                                    axis=1)).to(dev)
    WD = si.to_bf16(si.normal_f32((Ft, D), 3, 0.02)).to(dev)
    dY = si.to_bf16(si.normal_f32((M, D), 4)).to(dev)
    GU = torch.empty(M, 2 * Ft, dtype=torch.bfloat16, device=dev)
    H, P = torch.empty(M, Ft, dtype=torch.bfloat16, device=dev), torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    dWgu, dWd, dX = torch.empty_like(WGU), torch.empty_like(WD), torch.empty_like(X)
    order = si.ring_chunk_order(T, C, 0)
    wsf = tpm.alloc_workspace(tpm.OP_GATED_MLP_FWD, M, D, F, T, C, tpm.BF16)
    wsb = tpm.alloc_workspace(tpm.OP_GATED_MLP_BWD, M, D, F, T, C, tpm.BF16)
    fwd = lambda: tpm.tp_gated_mlp_fwd(X, WGU, WD, H, P, T=T, rank=0, act=tpm.ACT_SILU, GU_t=GU, num_chunks=C,
                                       chunk_order=order, workspace=wsf)
    bwd = lambda: tpm.tp_gated_mlp_bwd(X, WGU, WD, GU, H, dY, dWgu, dWd, dX, T=T, rank=0, act=tpm.ACT_SILU,
                                       num_chunks=C, dy_chunk_order=order, workspace=wsb)
    out = {"M": M, "D": D, "F": F, "T": T, "chunks": C, "act": "silu (SwiGLU)", "dtype": "bf16"}
    for name, fn, units in (("fwd", fwd, 3), ("bwd", bwd, 6)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)[iters // 2]
        tf = units * 2.0 * M * Ft * D / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "TFLOPS": round(tf, 1), "frac_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    assert tpm.poll_device_error(wsf) == 0 and tpm.poll_device_error(wsb) == 0
    ms = out["fwd"]["ms"] + out["bwd"]["ms"]
    out["TFLOPS_fwd_bwd"] = round(9 * 2.0 * M * Ft * D / (ms * 1e-3) / 1e12, 1)
    return out


def recorded_traffic():
    """HBM bytes per step of the GEMM launches, as measured with rocprofv3
    FETCH_SIZE / WRITE_SIZE (profiles/gemm_traffic.md), or None when the GEMM
    sources (kernel file and the two headers it includes) have changed since
    the counters were taken."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", "gemm_traffic.md")).read()
        src = b"".join(open(os.path.join(ROOT, "sequence_transformer_gemms_amd", "csrc", f), "rb").read()
                       for f in ("gemm_mfma.hip", "tpm_device.hpp", "tpm_internal.hpp"))
    except OSError:
        return None
    m_b = re.search(r"traffic_bytes_per_step:\s*(\d+)", text)
    m_h = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
    if not m_b or not m_h or m_h.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return int(m_b.group(1))


def cpu_baseline(sample_tokens: int, target_s: float = 20.0):
    """The fp64 oracle, as it stands, on the first m tokens of the same layer
    (all weights, D = 8192, F/T = 3584): the 12 GEMMs of the step at M = m.
    A calibration run on `sample_tokens` tokens sets m so that the timed run
    takes about `target_s` seconds (at most the full 4096 tokens).  Reported
    in the step metric's unit."""
    cal = _cpu_oracle_run(sample_tokens)
    per_token_s = cal["seconds"] / sample_tokens
    m = int(min(4096, max(256, (target_s / per_token_s) // 256 * 256)))
    r = _cpu_oracle_run(m)
    return dict(value=r["flops"] / r["seconds"] / 1e12, unit="TFLOPS", cores=r["threads"], kind="oracle",
                sample=f"fp64 oracle, the 12 GEMMs + GeLU of the layer step on {m} of 4096 tokens "
                       f"({r['flops'] / 1e9:.1f} GFLOP in {r['seconds']:.1f} s)")


def _cpu_oracle_run(sample_tokens: int):
    import numpy as np  # noqa: F401
    from threadpoolctl import threadpool_info

    import synthetic_inputs as si
    from oracle import ops
    m, D, Ft, Nq, Da = sample_tokens, 8192, 3584, 1280, 1024
    f64 = lambda a: si.to_bf16(a).to(dtype=__import__("torch").float64).numpy()
    x = f64(si.normal_f32((4096, D), 1)[:m])
    w_qkv = f64(si.normal_f32((D, Nq), 5, 0.02))
    w_up = f64(si.normal_f32((D, Ft), 2, 0.02))
    w_o = f64(si.normal_f32((Da, D), 6, 0.02))
    w_down = f64(si.normal_f32((Ft, D), 3, 0.02))
    attn = f64(si.normal_f32((4096, Da), 7)[:m])
    dy_qkv = f64(si.normal_f32((4096, Nq), 8)[:m])
    dy_mlp = f64(si.normal_f32((4096, D), 4)[:m])
    dy_o = f64(si.normal_f32((4096, D), 9)[:m])
    t0 = time.perf_counter()
    ops.seq_chunk_gemm(x, w_qkv)
    ops.seq_chunk_gemm(attn, w_o)
    fw = ops.tp_mlp_fwd(x, w_up, w_down, ops.ACT_GELU_ERF, store="bf16")
    ops.tp_mlp_bwd(x, w_up, w_down, fw["Z"], fw["H"], dy_mlp, ops.ACT_GELU_ERF, store="bf16")
    ops.linear_bwd(attn, w_o, dy_o)
    ops.linear_bwd(x, w_qkv, dy_qkv)
    dt = time.perf_counter() - t0
    flops = 2.0 * m * (3 * D * Nq + 3 * D * Ft + 3 * Da * D + 3 * Ft * D)
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    if threads == 0:
        threads = len(os.sched_getaffinity(0))
    return dict(seconds=dt, flops=flops, threads=threads)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU runs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import sequence_transformer_gemms_amd as tpm
    import synthetic_inputs as si
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep:
        run_sweep(torch, tpm, si)
        return
    if args.yardstick:
        run_yardstick(torch, tpm)
        return
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    layer = Layer(torch, tpm, si, producer_cus=args.producer_cus)
    torch.cuda.synchronize()
    # headline: the rank's step with every chunk already in place (flags
    # not consulted), on the default stream with every CU
    ms_eager, gemm_ms, wall = time_steps(torch, layer, args.steps, args.warmup, arrive=False, epoch0=0)
    ms = time_steps_graph(torch, layer, args.steps, args.warmup)
    flops = layer.flops
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    rec = {
        "metric": "TFLOPS/GPU on TP-rank MLP fwd+bwd (% of MFMA peak); reduce GB/s",
        "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama3-70B-shaped TP=8 rank layer share fwd+bwd: QKV [8192,1280], O [1024,8192], "
                               "MLP up [8192,3584] + GeLU, down [3584,8192]; 4096 tokens; 4 sequence-sharded "
                               "reductions of 8 partials; inputs resident in HBM; the step's kernels replayed from "
                               "one HIP graph (the step with the 8 sequence chunks arriving from a producer stream "
                               "is extra.arrival_step)",
                   "tokens": 4096, "hidden": 8192, "ffn": 28672, "tp": 8, "chunks": 8,
                   "gflop_per_step": round(flops / 1e9, 1), "frac_mfma_peak": round(value / BF16_PEAK_TFLOPS, 4),
                   "launch": "hip_graph", "ms_per_step_eager": round(ms_eager, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": recorded_traffic(),
                     "traffic_unit": "bytes per step (the 12 GEMMs in 10 launches + split-K finalisation)",
                     "kernel": "gemm_kernel / gemm_pair_kernel (bf16 MFMA): the step's 12 GEMMs in 10 launches "
                               "(each projection backward's dW and dX paired in one)",
                     "gemm_ms_per_step": round(gemm_ms, 4)},
    }
    if not args.no_extra:
        extra = {"arrival_step": arrival_step(torch, layer, args, ms_eager)}
        del layer
        torch.cuda.empty_cache()
        extra["reduce_c3"] = bench_reduce(torch, tpm, si)
        torch.cuda.empty_cache()
        extra["mlp_fwd_c3_bf16"] = bench_mlp_fwd(torch, tpm, si, 8192, 8192, 28672, 8, 8, False)
        torch.cuda.empty_cache()
        extra["mlp_fwd_c4_fp8"] = bench_mlp_fwd(torch, tpm, si, 8192, 16384, 53248, 8, 16, True)
        torch.cuda.empty_cache()
        extra["mlp_fwd_c4_mxfp8"] = bench_mlp_fwd_mx(torch, tpm, si)
        torch.cuda.empty_cache()
        extra["mlp_fwd_c4_fp8_delayed"] = bench_mlp_fwd_delayed(torch, tpm, si)
        torch.cuda.empty_cache()
        extra["mlp_bwd_c4_fp8"] = bench_mlp_bwd_fp8(torch, tpm)
        torch.cuda.empty_cache()
        extra["gated_mlp_worked_example"] = bench_gated_mlp(torch, tpm, si)
        rec["extra"] = extra
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.cpu_sample_tokens)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
