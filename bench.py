#!/usr/bin/env python3
"""Benchmark of the routed MoE layer (Beam: H=5120, E=256, top-8, I=1536) on one MI355X.

One step = one whole layer (router GEMM + top-k, permute, grouped SwiGLU expert
GEMMs, finalize) over one batch of synthetic input already resident in HBM.
The headline workload is decode (T=128 tokens, bf16 weights, near-uniform
routing), bound by streaming the touched experts' weights from HBM; prefill
(T=16384 = 8 x 2048 tokens, Zipf(1.1) expert load) is reported beside it
against the bf16 MFMA peak, and the NVFP4-weight layer (T=4096) against the
bound it is closer to (HBM bytes or bf16 MFMA).

Beside the headline line's `roofline` and `cpu_baseline` (the oracle on a
token sample of the same workload, on the host's cores), the line carries the
small-batch decode record (T = 1, 8, 32 at I = 1536 and 2560, eager and graph
replay), the layer ending in the fused finalize + norms (moe_forward_norm), and
the oracle's rate on prefill and NVFP4 samples.

Prints one JSON line. Options: --gpus N (only 1 is supported), --steps K,
--warmup W, --workload decode|prefill (headline), --no-prefill, --no-quant,
--no-cpu, --no-small.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (H5120,E256,k8) + % peak HBM BW decode / % MFMA prefill"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=["decode", "prefill", "small"], default="decode",
                   help="small: only the small-batch decode records (T = 1, 8, 32), one JSON line "
                        "(for kernel traces of those batches)")
    p.add_argument("--no-prefill", action="store_true", help="skip the secondary prefill line")
    p.add_argument("--no-quant", action="store_true", help="skip the secondary NVFP4 line")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--no-small", action="store_true",
                   help="skip the small-batch decode record (T = 1, 8, 32)")
    p.add_argument("--hbm-probe", action="store_true",
                   help="time a plain 4 GiB device copy (the reference kernel for HBM counters) and exit")
    p.add_argument("--gemm-probe", action="store_true",
                   help="time the vendor library's dense bf16 GEMMs (torch.matmul) on shapes with "
                        "the prefill expert GEMMs' FLOPs, for comparison, and exit")
    return p.parse_args()


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Workload:
    """Device-resident inputs, outputs and workspace of one configuration."""

    def __init__(self, cfg, moe, torch, dev_weights=None):
        import synth
        self.cfg, self.moe, self.torch = cfg, moe, torch
        T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
        self.x_host = synth.gen_x(cfg)
        self.wr_host, self.bias_host = synth.gen_router(cfg)
        self.x = moe.to_device_bf16(self.x_host)
        self.wr = torch.from_numpy(self.wr_host).cuda()
        self.bias = None if self.bias_host is None else torch.from_numpy(self.bias_host).cuda()
        if dev_weights is None:
            self.w_host = synth.gen_experts(cfg)
            dev_weights = moe.experts_to_device(self.w_host)
        self.w = dev_weights
        P = T * k
        dt = torch.bfloat16
        self.out = torch.empty((T, H), dtype=dt, device="cuda")
        self.logits = torch.empty((T, E), dtype=dt, device="cuda")
        self.ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        self.tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        self.ws = moe.workspace(moe.moe_forward_workspace_size(T, H, I, E, k, self.w))
        # stage-by-stage buffers
        self.rws = moe.workspace(moe.moe_route_workspace_size(T, H, E))
        self.counts = torch.empty(E, dtype=torch.int32, device="cuda")
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.sp = torch.empty(P, dtype=torch.int32, device="cuda")
        self.pp = torch.empty(P, dtype=torch.int32, device="cuda")
        self.y = torch.empty((P, H), dtype=torch.float32, device="cuda")
        self.ews = moe.workspace(moe.moe_experts_workspace_size(T, H, I, E, k, self.w))
        # compact expert rows where the library supports them: moe_forward then
        # runs those kernels, so the stage timing does too
        self.y16 = torch.empty((P, H), dtype=torch.int16, device="cuda")
        self.ysc = torch.empty((P, H // 64), dtype=torch.uint8, device="cuda")
        self.rows16 = True
        # finalize fused with the sandwich norms (timed beside the plain finalize)
        self.res = torch.randn((T, H), generator=torch.Generator("cuda").manual_seed(cfg.seed),
                               device="cuda").to(dt)
        self.gamma = torch.ones(H, dtype=dt, device="cuda")
        self.res_out = torch.empty_like(self.res)
        self.normed = torch.empty_like(self.res)

    def forward(self):
        c = self.cfg
        self.moe.moe_forward(self.x, self.wr, self.bias, self.w, c.I, c.k, self.out, self.ws,
                             logits=self.logits, topk_ids=self.ids, topk_w=self.tw)

    def forward_norm(self):
        """The layer ending in the fused finalize + sandwich norms (moe_forward_norm)."""
        c = self.cfg
        self.moe.moe_forward_norm(self.x, self.wr, self.bias, self.w, c.I, c.k, self.res,
                                  self.gamma, self.gamma, 1e-6, self.res_out, self.normed,
                                  self.ws, logits=self.logits, topk_ids=self.ids, topk_w=self.tw)

    def stage_calls(self):
        c, m = self.cfg, self.moe
        return [
            ("route", lambda: m.moe_route(self.x, self.wr, self.bias, c.k, m.MOE_BF16, self.logits,
                                          None, self.ids, self.tw, self.rws)),
            ("permute", lambda: m.moe_permute(self.ids, c.E, self.counts, self.offsets, self.sp,
                                              self.pp)),
            ("experts", lambda: m.moe_experts_rows16(self.x, c.I, c.E, c.k, self.offsets, self.sp,
                                                     self.w, self.y16, self.ysc, self.ews)
             if self.rows16 else m.moe_experts(self.x, c.I, c.E, c.k, self.offsets, self.sp,
                                               self.w, self.y, self.ews)),
            ("finalize", lambda: m.moe_finalize_rows16(self.y16, self.ysc, self.pp, self.tw,
                                                       self.out)
             if self.rows16 else m.moe_finalize(self.y, self.pp, self.tw, self.out)),
            # the fused finalize + norms on the same rows (moe_forward_norm's last step)
            ("finalize_norm", lambda: m.moe_finalize_norm_rows16(
                self.y16, self.ysc, self.pp, self.tw, self.res, self.gamma, self.gamma, 1e-6,
                self.res_out, self.normed)
             if self.rows16 else m.moe_finalize_norm(self.y, self.pp, self.tw, self.res,
                                                     self.gamma, self.gamma, 1e-6, self.res_out,
                                                     self.normed)),
        ]

    def time_forward(self, steps, warmup, fn=None):
        torch = self.torch
        fn = fn or self.forward
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def iter_spread(self, n=50):
        """Per-call times (ms) of n more forward calls, each bracketed by events
        with a synchronisation after it: median and the p10 / p90 spread."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(n):
            e0.record()
            self.forward()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        q = np.percentile(ts, [10, 50, 90])
        return {"n": n, "p10": round(float(q[0]), 4), "median": round(float(q[1]), 4),
                "p90": round(float(q[2]), 4)}

    def time_stages(self, steps):
        """Per-stage average durations (ms) from events recorded between the stage
        calls on the stream the kernels run on."""
        torch, c, m = self.torch, self.cfg, self.moe
        calls = self.stage_calls()
        calls[0][1]()
        calls[1][1]()
        try:  # compact rows unless the library does not support them here
            calls[2][1]()
        except m.MoEError as err:
            if err.status != 2:
                raise
            self.rows16 = False
            del self.y16, self.ysc
        for _, f in calls[2:]:
            f()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
               for _ in range(steps)]
        for s in range(steps):
            evs[s][0].record()
            for i, (_, f) in enumerate(calls):
                f()
                evs[s][i + 1].record()
        torch.cuda.synchronize()
        out = {}
        for i, (name, _) in enumerate(calls):
            out[name] = float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]))
        return out

    def touched(self):
        self.torch.cuda.synchronize()
        return self.counts.cpu().numpy()


CSRC = os.path.join(ROOT, "sparse_moe_layer_gemm_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_t128_moe_experts_hbm_traffic.md")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_t16384_zipf_moe_experts_hbm_traffic.md")
# Each counter record is keyed to the device source of the kernels it measured: the kernel
# file and the device headers it includes (host-side declarations are not part of it).
STREAM_SRC = [os.path.join(CSRC, f) for f in ("expert_stream.hip", "stream_common.h", "device_common.h")]
STREAM_Q_SRC = [os.path.join(CSRC, f) for f in ("expert_stream_q.hip", "stream_common.h", "device_common.h")]
TILE_SRC = [os.path.join(CSRC, f) for f in ("expert_tile.hip", "tile_common.h", "device_common.h")]
TILE_Q_SRC = [os.path.join(CSRC, f) for f in ("expert_tile_q.hip", "tile_common.h", "device_common.h")]


def source_sha256(paths):
    """sha256 of one file, or of the concatenated bytes of several, in the order given."""
    import hashlib
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "nvfp4_moe_experts_counters.md")


def measured_traffic(path=TRAFFIC_FILE, src=STREAM_SRC, key=None):
    """HBM bytes per expert stage (moe_experts launch), from a committed rocprofv3 counter
    summary (its "TRAFFIC_JSON:" line, or "TRAFFIC_JSON[key]:" for one of several
    workloads), or None when it is missing or the kernel source changed since."""
    tag = "TRAFFIC_JSON:" if key is None else f"TRAFFIC_JSON[{key}]:"
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(tag):
                    d = json.loads(line[len(tag):])
                    if d.get("source_sha256") == source_sha256(src):
                        return d["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def hbm_probe(torch):
    """Plain device copy of 4 GiB: reads and writes a known number of bytes."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    nbytes = n * 4
    print(json.dumps({"probe": "device copy", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "ms_per_launch": ms,
                      "GB/s (read+write)": 2 * nbytes / (ms / 1e3) / 1e9}), flush=True)


def gemm_probe(torch):
    """torch.matmul / torch.bmm in bf16 (the vendor GEMM library) at the prefill expert shapes,
    then this library's grouped GEMMs on the batched one.

    Dense: all T*k = 131072 routed rows as one [131072, K] x [K, N] product (gate/up: K = 5120,
    N = 3072; down: K = 1536, N = 5120), i.e. the grouped GEMMs' FLOPs with no grouping and no
    gather. Batched: 256 experts x 512 rows each, the same FLOPs at perfectly uniform load.
    Operands are contiguous; inputs N(0,1) in bf16.
    """
    g = torch.Generator(device="cuda").manual_seed(0)
    P, H, I, E = 131072, 5120, 1536, 256
    cases = [("dense gate/up", (P, H), (H, 2 * I)), ("dense down", (P, I), (I, H)),
             ("batched gate/up", (E, P // E, H), (E, H, 2 * I)),
             ("batched down", (E, P // E, I), (E, I, H))]
    for name, sa, sb in cases:
        a = torch.randn(sa, generator=g, device="cuda").to(torch.bfloat16).contiguous()
        b = torch.randn(sb, generator=g, device="cuda").to(torch.bfloat16).contiguous()
        f = torch.matmul if a.dim() == 2 else torch.bmm
        c = f(a, b)
        for _ in range(3):
            f(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            f(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        flops = 2.0 * P * sa[-1] * sb[-1]
        print(json.dumps({"probe": f"torch bf16 {name}", "a": list(sa), "b": list(sb),
                          "ms_per_launch": round(ms, 4),
                          "TFLOP/s": round(flops / (ms / 1e3) / 1e12, 1),
                          "frac_of_2.5_PFLOPs": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 3)}),
              flush=True)
        del a, b, c
    # this library's grouped GEMMs on the batched shape (moe_experts with compact rows, as
    # moe_forward runs them at prefill): 256 experts x 512 rows, the rows gathered through a
    # random permutation of the 131072 (token, slot) pairs; weights N(0, 1/fan_in)
    import sparse_moe_layer_gemm_amd as moe
    k = 8
    T = P // k
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    wgu = torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device="cuda")
    wdn = torch.empty((E, I, H), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        wgu[e] = torch.randn((H, 2 * I), generator=g, device="cuda") * H ** -0.5
        wdn[e] = torch.randn((I, H), generator=g, device="cuda") * I ** -0.5
    w = moe.ExpertWeights(moe.MOE_BF16, wgu, wdn)
    offsets = (torch.arange(E + 1, device="cuda", dtype=torch.int32) * (P // E)).contiguous()
    sorted_pair = torch.randperm(P, generator=g, device="cuda").to(torch.int32)
    y16 = torch.empty((P, H), dtype=torch.int16, device="cuda")
    ysc = torch.empty((P, H // 64), dtype=torch.uint8, device="cuda")
    ws = moe.workspace(moe.moe_experts_workspace_size(T, H, I, E, k, w))

    def run():
        moe.moe_experts_rows16(x, I, E, k, offsets, sorted_pair, w, y16, ysc, ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 2.0 * P * H * 2 * I + 2.0 * P * I * H
    print(json.dumps({"probe": "moe_experts_rows16, 256 experts x 512 gathered rows (gate/up + down)",
                      "ms_per_launch": round(ms, 4),
                      "TFLOP/s": round(flops / (ms / 1e3) / 1e12, 1),
                      "frac_of_2.5_PFLOPs": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 3)}),
          flush=True)


def hbm_ceiling(torch, moe, nbytes=4 << 30, reps=10):
    """The library's own streaming read (moe_hbm_read) over a 4 GiB buffer: the
    measured HBM read ceiling of this chip."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        moe.moe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_hbm_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    return {"kernel": "moe_hbm_read (16-byte nontemporal loads)", "bytes": nbytes,
            "ms": round(ms, 4), "GB/s": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}


LAYERS_PER_GRAPH = 16  # layer calls per captured graph in the small-batch record


def decode_small(torch, moe, dec, reps=200):
    """Small-batch decode (H=5120, E=256, k=8): T in {1, 8, 32} at I = 1536 (the decode
    layer's weights) and I = 2560 (the width the checkpoint sizes imply; only the routed
    experts' weights are generated, the rest is never read). Per case: moe_forward back to
    back (events around `reps` calls) on distinct inputs in turn (so consecutive calls read
    mostly different experts, as consecutive layers do); the same sequence captured as
    LAYERS_PER_GRAPH calls in one HIP graph and replayed back to back (per-layer time, the
    way a model's captured decode step runs its layers), and, for reference, one call per
    graph (which adds a graph launch to every layer); weight GB/s counts the touched
    experts' bytes (mean over the inputs)."""
    import synth
    base = synth.CONFIGS["decode_t128"]
    E, H, k = base.E, base.H, base.k
    out = []
    for I in (base.I, 2560):
        if I == base.I:
            dw = dec.w
        else:
            x32 = moe.to_device_bf16(dec.x_host[:32])
            ids = torch.empty((32, k), dtype=torch.int32, device="cuda")
            tw = torch.empty((32, k), dtype=torch.float32, device="cuda")
            lg = torch.empty((32, E), dtype=torch.bfloat16, device="cuda")
            moe.moe_route(x32, dec.wr, None, k, moe.MOE_BF16, lg, None, ids, tw,
                          moe.workspace(moe.moe_route_workspace_size(32, H, E)))
            touched = np.unique(ids.cpu().numpy())
            cfg = base.with_(name="decode_i2560", I=I)
            sub = synth.gen_experts(cfg, experts=touched)
            gu = torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device="cuda")
            dn = torch.empty((E, I, H), dtype=torch.bfloat16, device="cuda")
            idx = torch.from_numpy(touched).cuda()
            gu[idx] = moe.to_device_bf16(sub["gate_up"])
            dn[idx] = moe.to_device_bf16(sub["down"])
            del sub
            dw = moe.ExpertWeights(moe.MOE_BF16, gu, dn)
        for T in (1, 8, 32):
            cfg = base.with_(name=f"decode_t{T}_i{I}", T=T, I=I)
            # R distinct inputs (consecutive T-token slices of the first 32 tokens,
            # whose experts the I = 2560 case generates), used in turn, so that
            # consecutive calls mostly read different experts, as consecutive
            # layers do
            R = max(1, min(LAYERS_PER_GRAPH, 32 // T))
            xs = [moe.to_device_bf16(dec.x_host[r * T:(r + 1) * T]) for r in range(R)]
            ids = [torch.empty((T, k), dtype=torch.int32, device="cuda") for _ in range(R)]
            o = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            ws = moe.workspace(moe.moe_forward_workspace_size(T, H, I, E, k, dw))

            def fwd(i):
                moe.moe_forward(xs[i % R], dec.wr, None, dw, I, k, o, ws, topk_ids=ids[i % R])
            for i in range(10 * R):
                fwd(i)
            torch.cuda.synchronize()
            n_touched = float(np.mean([np.unique(t.cpu().numpy()).size for t in ids]))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fwd(i)
            e1.record()
            torch.cuda.synchronize()
            eager_ms = e0.elapsed_time(e1) / reps

            def graph_ms_per_layer(layers):
                # `layers` consecutive calls captured in one graph, replayed back to back
                g = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    fwd(0)
                torch.cuda.current_stream().wait_stream(side)
                with torch.cuda.graph(g):
                    for i in range(layers):
                        fwd(i)
                for _ in range(3):
                    g.replay()
                torch.cuda.synchronize()
                n = max(1, reps // layers)
                e0.record()
                for _ in range(n):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / (n * layers)
                del g
                return ms
            graph1_ms = graph_ms_per_layer(1)
            graph_ms = graph_ms_per_layer(LAYERS_PER_GRAPH)
            wbytes = n_touched * expert_bytes(cfg)
            out.append({"T": T, "I": I, "touched_experts": round(n_touched, 2), "distinct_inputs": R,
                        "ms_per_step": round(eager_ms, 4), "graph_replay_ms": round(graph_ms, 4),
                        "graph_replay_one_layer_ms": round(graph1_ms, 4),
                        "tokens_per_s": round(T / (graph_ms / 1e3), 1),
                        "weight_GBps": round(wbytes / (graph_ms / 1e3) / 1e9, 1),
                        "weight_frac_of_peak_hbm": round(wbytes / (graph_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)})
        if I != base.I:
            del dw, gu, dn
    return out


def expert_bytes(cfg):
    """Bytes of one expert's weights: gate/up [H, 2I] + down [I, H] (with scales)."""
    n = cfg.H * 2 * cfg.I + cfg.I * cfg.H
    if cfg.w_dtype == "fp4":
        return n // 2 + n // 16 + 2 * 4  # E2M1 codes, one E4M3 scale per 16, two global scales
    if cfg.w_dtype == "fp8":
        return n + 4 * (2 * cfg.I + cfg.H)  # E4M3 codes, one fp32 scale per output channel
    return 2 * n


def cpu_baseline(wl, budget_s=10.0, qmode="w", one_thread=True):
    """Oracle (fp64, OpenMP) on a bounded sample of the workload's tokens: the whole
    layer per token (qmode "f8": the oracle's fp8-MFMA-mode layer)."""
    import oracle
    c = wl.cfg
    sel = c.logits_dtype

    def run(rows):
        oracle.layer(wl.x_host, wl.wr_host, wl.bias_host, wl.w_host, c.I, c.k, sel, rows=rows,
                     qmode=qmode)
    n = 8
    t = time.perf_counter()
    run(np.arange(n))
    dt = time.perf_counter() - t
    n2 = int(min(c.T, max(n, n * budget_s / max(dt, 1e-3))))
    rows = np.linspace(0, c.T - 1, n2).astype(np.int64)
    # whole passes over the sample until about budget_s of oracle work has run
    t = time.perf_counter()
    passes = 0
    while True:
        run(rows)
        passes += 1
        dt = time.perf_counter() - t
        if dt >= budget_s or passes >= 50:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    value = round(passes * n2 / dt, 3)
    # the same oracle on one thread, over 8 tokens
    one = None
    try:
        if not one_thread:
            raise OSError
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        rows1 = rows[:8]
        t = time.perf_counter()
        run(rows1)
        one = round(rows1.size / (time.perf_counter() - t), 3)
        gomp.omp_set_num_threads(cores)
    except OSError:
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} pass(es) over {n2} of the {c.T} {c.name} tokens (whole layer per "
                      f"token, fp64{', fp8-MFMA-mode encodings' if qmode == 'f8' else ''}), "
                      f"{dt:.1f} s",
            "value_1_thread": one,
            "host": {"cpu_model": model, "os_cpu_count": os.cpu_count(),
                     "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the layer is measured "
              f"unsharded on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.hbm_probe:
        hbm_probe(torch)
        return
    if a.gemm_probe:
        gemm_probe(torch)
        return
    import sparse_moe_layer_gemm_amd as moe
    import synth

    dec_cfg = synth.CONFIGS["decode_t128"]
    pre_cfg = synth.CONFIGS["prefill_t16384_zipf"]
    if a.workload == "small":
        progress("generating decode inputs (T=128, bf16 experts) for the small batches")
        dec = Workload(dec_cfg, moe, torch)
        print(json.dumps({"decode_small": decode_small(torch, moe, dec)}), flush=True)
        return
    dec_line = pre_line = dec = pre = None
    if a.workload == "decode":
        progress("generating decode inputs (T=128, bf16 experts)")
        dec = Workload(dec_cfg, moe, torch)
        progress("timing decode")
        dec_ms = dec.time_forward(a.steps, a.warmup)
        dec_stage = dec.time_stages(a.steps)
        counts = dec.touched()
        n_touched = int((counts > 0).sum())
        wbytes = n_touched * expert_bytes(dec_cfg)
        layer_bytes = wbytes + dec_cfg.H * dec_cfg.E * 4 + 2 * dec_cfg.T * dec_cfg.H * 2
        dec_line = {
            "value": dec_cfg.T / (dec_ms / 1e3),
            "ms_per_step": dec_ms,
            "stages_ms": dec_stage,
            "touched_experts": n_touched,
            "layer_hbm_frac": layer_bytes / (dec_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "roofline": {"bound": "hbm", "kernel": "moe_experts (gate/up + down stream GEMMs)",
                         "achieved": wbytes / (dec_stage["experts"] / 1e3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": measured_traffic()},
        }
        dec_line["roofline"]["frac"] = dec_line["roofline"]["achieved"] / HBM_PEAK_GBS
        dec_line["iter_ms"] = dec.iter_spread()
        dec_line["forward_norm_ms"] = dec.time_forward(a.steps, a.warmup, dec.forward_norm)
        if not a.no_small:
            progress("timing small-batch decode (T = 1, 8, 32 at I = 1536 and 2560)")
            dec_line["decode_small"] = decode_small(torch, moe, dec)
        progress("measuring the HBM read ceiling (4 GiB)")
        ceil = hbm_ceiling(torch, moe)
        ceil["decode_experts_frac_of_ceiling"] = round(
            dec_line["roofline"]["achieved"] / ceil["GB/s"], 4)
        dec_line["hbm_ceiling"] = ceil

    if a.workload == "prefill" or not a.no_prefill:
        progress("generating prefill inputs (T=16384, Zipf load)")
        pre = Workload(pre_cfg, moe, torch, dev_weights=None if dec is None else dec.w)
        if dec is not None:
            pre.w_host = dec.w_host  # the same expert weights (same seed)
        progress("timing prefill")
        psteps = a.steps if a.workload == "prefill" else max(3, a.steps // 2)
        pre_ms = pre.time_forward(psteps, max(1, a.warmup // 2))
        pre_stage = pre.time_stages(psteps)
        P = pre_cfg.T * pre_cfg.k
        flops = 2.0 * P * (pre_cfg.H * 2 * pre_cfg.I + pre_cfg.I * pre_cfg.H)
        router_flops = 2.0 * pre_cfg.T * pre_cfg.H * pre_cfg.E
        pc = pre.touched()
        pre_line = {
            "value": pre_cfg.T / (pre_ms / 1e3),
            "ms_per_step": pre_ms,
            "stages_ms": pre_stage,
            "expert_load": {"max": int(pc.max()), "median": float(np.median(pc)), "min": int(pc.min())},
            "expert_rows": "fp16, power-of-two scale per 64 columns" if pre.rows16 else "fp32",
            "layer_mfma_frac": (flops + router_flops) / (pre_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "moe_experts (gate/up + down grouped GEMMs)",
                         "achieved": flops / (pre_stage["experts"] / 1e3) / 1e12,
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "traffic": measured_traffic(PREFILL_TRAFFIC_FILE, TILE_SRC)
                         if pre.rows16 else None},
        }
        pre_line["roofline"]["frac"] = pre_line["roofline"]["achieved"] / BF16_PEAK_TFLOPS
        pre_line["iter_ms"] = pre.iter_spread(20)
        pre_line["forward_norm_ms"] = pre.time_forward(psteps, 1, pre.forward_norm)
        if not a.no_cpu:
            progress("timing the CPU oracle on a prefill token sample")
            pre_line["cpu_baseline"] = cpu_baseline(pre, budget_s=8.0, one_thread=False)

    q_cfg = synth.CONFIGS["nvfp4_t4096"]
    q_line = None
    if a.workload == "decode" and not a.no_quant:
        progress("generating NVFP4 inputs (T=4096)")
        qw = Workload(q_cfg, moe, torch)
        progress("timing NVFP4")
        qsteps = max(3, a.steps // 2)
        q_ms = qw.time_forward(qsteps, max(1, a.warmup // 2))
        q_stage = qw.time_stages(qsteps)
        qc = qw.touched()
        P = q_cfg.T * q_cfg.k
        flops = 2.0 * P * 3 * q_cfg.H * q_cfg.I
        wbytes = int((qc > 0).sum()) * expert_bytes(q_cfg)
        tb = wbytes / (q_stage["experts"] / 1e3) / 1e9
        tf = flops / (q_stage["experts"] / 1e3) / 1e12
        hbm_frac, mfma_frac = tb / HBM_PEAK_GBS, tf / BF16_PEAK_TFLOPS
        q_line = {"workload": q_cfg.name, "value": round(q_cfg.T / (q_ms / 1e3), 1),
                  "unit": "tokens/s", "ms_per_step": round(q_ms, 4),
                  "stages_ms": {k: round(v, 4) for k, v in q_stage.items()},
                  "roofline": {"bound": "hbm" if hbm_frac >= mfma_frac else "mfma",
                               "kernel": "moe_experts (NVFP4 weights, bf16 MFMA)",
                               "achieved": tb if hbm_frac >= mfma_frac else tf,
                               "peak": HBM_PEAK_GBS if hbm_frac >= mfma_frac else BF16_PEAK_TFLOPS,
                               "unit": "GB/s" if hbm_frac >= mfma_frac else "TFLOP/s",
                               "frac": max(hbm_frac, mfma_frac),
                               "traffic": measured_traffic(QUANT_TRAFFIC_FILE, TILE_Q_SRC, "nvfp4_t4096_w"),
                               "weight_GBps": round(tb, 1), "TFLOPs": round(tf, 1)}}
        if not a.no_cpu:
            progress("timing the CPU oracle on an NVFP4 token sample")
            q_line["cpu_baseline"] = cpu_baseline(qw, budget_s=8.0, one_thread=False)
        # the same layer in the fp8-MFMA mode (activations quantised in-kernel)
        progress("timing NVFP4, fp8-MFMA mode")
        import dataclasses
        qw.w = dataclasses.replace(qw.w, qmode=moe.MOE_QMODE_F8)
        qw.ws = moe.workspace(moe.moe_forward_workspace_size(q_cfg.T, q_cfg.H, q_cfg.I, q_cfg.E,
                                                             q_cfg.k, qw.w))
        qw.ews = moe.workspace(moe.moe_experts_workspace_size(q_cfg.T, q_cfg.H, q_cfg.I, q_cfg.E,
                                                              q_cfg.k, qw.w))
        f_ms = qw.time_forward(qsteps, max(1, a.warmup // 2))
        f_stage = qw.time_stages(qsteps)
        tb8 = wbytes / (f_stage["experts"] / 1e3) / 1e9
        tf8 = flops / (f_stage["experts"] / 1e3) / 1e12
        h8, m8 = tb8 / HBM_PEAK_GBS, tf8 / FP8_PEAK_TFLOPS
        q_line["fp8_mfma_mode"] = {
            "value": round(q_cfg.T / (f_ms / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(f_ms, 4),
            "stages_ms": {k: round(v, 4) for k, v in f_stage.items()},
            "roofline": {"bound": "hbm" if h8 >= m8 else "mfma",
                         "kernel": "moe_experts (NVFP4 weights, fp8 MFMA)",
                         "achieved": tb8 if h8 >= m8 else tf8,
                         "peak": HBM_PEAK_GBS if h8 >= m8 else FP8_PEAK_TFLOPS,
                         "unit": "GB/s" if h8 >= m8 else "TFLOP/s",
                         "frac": max(h8, m8),
                         "traffic": measured_traffic(QUANT_TRAFFIC_FILE, TILE_Q_SRC, "nvfp4_t4096_f8"),
                         "weight_GBps": round(tb8, 1), "TFLOPs": round(tf8, 1)}}
        if not a.no_cpu:
            progress("timing the CPU oracle (fp8-MFMA mode) on an NVFP4 token sample")
            q_line["fp8_mfma_mode"]["cpu_baseline"] = cpu_baseline(qw, budget_s=8.0, qmode="f8",
                                                                   one_thread=False)
        # NVFP4 decode (T=128, exact dequantisation): the streaming kernels on the same weights
        progress("timing NVFP4 decode (T=128)")
        qd_cfg = q_cfg.with_(name="nvfp4_t128", T=128)
        qd = Workload(qd_cfg, moe, torch, dev_weights=dataclasses.replace(qw.w, qmode=moe.MOE_QMODE_W))
        d_ms = qd.time_forward(a.steps, a.warmup)
        d_stage = qd.time_stages(a.steps)
        d_bytes = int((qd.touched() > 0).sum()) * expert_bytes(qd_cfg)
        d_gbs = d_bytes / (d_stage["experts"] / 1e3) / 1e9
        q_line["decode_t128"] = {
            "value": round(qd_cfg.T / (d_ms / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(d_ms, 4),
            "stages_ms": {k: round(v, 4) for k, v in d_stage.items()},
            "roofline": {"bound": "hbm", "kernel": "moe_experts (NVFP4 weights, stream, bf16 MFMA)",
                         "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(QUANT_TRAFFIC_FILE, STREAM_Q_SRC, "nvfp4_t128")}}
        del qw, qd

    head, head_cfg = (dec_line, dec_cfg) if a.workload == "decode" else (pre_line, pre_cfg)
    cpu = None
    if not a.no_cpu:
        progress("timing the CPU oracle on a token sample")
        cpu = cpu_baseline(dec if a.workload == "decode" else pre)

    line = {
        "metric": METRIC,
        "value": round(head["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head_cfg.name, "T": head_cfg.T, "H": head_cfg.H, "E": head_cfg.E,
                   "k": head_cfg.k, "I": head_cfg.I, "expert_weights": head_cfg.w_dtype,
                   "routing": "zipf(1.1)" if head_cfg.zipf_s else "near-uniform",
                   "parallelism": "single GPU, one unsharded layer"},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "stages_ms": {k: round(v, 4) for k, v in head["stages_ms"].items()},
        "iter_ms": head["iter_ms"],
    }
    if a.workload == "decode":
        line["touched_experts"] = dec_line["touched_experts"]
        line["layer_hbm_frac"] = round(dec_line["layer_hbm_frac"], 4)
        line["hbm_ceiling"] = dec_line["hbm_ceiling"]
        line["forward_norm_ms"] = round(dec_line["forward_norm_ms"], 4)
        if "decode_small" in dec_line:
            line["decode_small"] = dec_line["decode_small"]
        if pre_line is not None:
            line["prefill"] = {"workload": pre_cfg.name, "value": round(pre_line["value"], 1),
                               "unit": "tokens/s", "ms_per_step": round(pre_line["ms_per_step"], 4),
                               "layer_mfma_frac": round(pre_line["layer_mfma_frac"], 4),
                               "roofline": pre_line["roofline"],
                               "stages_ms": {k: round(v, 4) for k, v in pre_line["stages_ms"].items()},
                               "iter_ms": pre_line["iter_ms"],
                               "forward_norm_ms": round(pre_line["forward_norm_ms"], 4),
                               "expert_load": pre_line["expert_load"],
                               "cpu_baseline": pre_line.get("cpu_baseline")}
        if q_line is not None:
            line["quantised"] = q_line
    else:
        line["expert_load"] = pre_line["expert_load"]
        line["layer_mfma_frac"] = round(pre_line["layer_mfma_frac"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
