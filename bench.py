#!/usr/bin/env python3
"""Benchmark of the chunked Gated Delta Product prefill forward on one MI355X.

One step = the whole hot path over one batch of synthetic input, all on the
GPU through the C ABI of libgdp.so:
    gdp_prefill_fwd_scan     (default, --path prefill-scan: recompute_w_u
                              with the prefill prepare (split /
                              GQA-expand / Householder-fold / gate) done
                              inside it; the affine state map of each of 16
                              segments, composed in parallel; a scan over
                              the segments for the state entering each;
                              chunk_h over all segments at once; chunk_o.
                              The value copies and beta, which no stage after
                              WY reads, are not stored unless --store-v-beta)
 or gdp_prefill_prepare then gdp_chunk_fwd_scan (--path scan: the same with
                              prepare as its own launch)
 or gdp_prefill_prepare then gdp_chunk_fwd_pipelined (--path pipelined:
                              recompute_w_u -> chunk_h -> chunk_o over 3
                              segments: chunk_h runs the segments in order,
                              handing its fp32 state on, while recompute_w_u
                              of later segments and chunk_o of finished ones
                              run on side streams)
Workload: the long single-sequence prefill, B=1, T=32768 tokens, 16 heads
(query/key groups = value heads = 16), K=V=128, M=2 Householder copies, chunk
64, bf16 activations with fp32 gates, state and accumulation.  Inputs are
drawn once (seeded, synthetic) and resident in HBM before timing starts.

Prints one JSON line: tokens/s over the timed steps, the roofline of the
dominant kernel (the one with the longest launch: algorithmic bytes per
launch / its average launch duration from HIP events recorded on its stream
around every launch, vs 8 TB/s HBM; the events record without a
system-scope fence, so they do not slow the step they time) and the
oracle's throughput on the host cores as a reported baseline.  --stages adds a sequential (not overlapped) pass that
times each stage on its own.

    python bench.py [--steps K] [--warmup W] [--path prefill-scan|scan|pipelined] [--segments S] [--stages]
                    [--no-cpu-baseline] [--copy-mib N] [--store-v-beta]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDP prefill forward tokens/s (T=32k, H=16, K=V=128, M=2) + % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
WORKLOAD = dict(workload="long_prefill_32k", B=1, T=32768, H=16, HV=16, G=16, K=128, V=128, M=2, chunk=64,
                dtype="bf16", path="prepare+pipelined(recompute_w_u,chunk_h,chunk_o)")
SEGMENTS = 3
SCAN_SEGMENTS = 16
# A serving decode step of the same layer: 256 requests, one token each
# (no draft tokens), the fp32 state of every request read and written once.
DECODE = dict(workload="decode_step", n=256, S=1, H=16, HV=16, G=16, K=128, V=128, M=2, dtype="bf16")
KERNELS = ["gdp_prefill_prepare", "gdp_recompute_w_u", "gdp_chunk_h", "gdp_chunk_o"]


class TimingEvent:
    """A HIP timing event that records without a system-scope fence
    (hipEventDisableSystemFence).  A default event writes back and
    invalidates the caches when it records, which slows the work around it:
    with one such event before and after each kernel the step took about
    40 us longer.  Read elapsed_time only after the device is synchronised.
    The interface is the part of torch.cuda.Event the benchmark uses
    (record, elapsed_time, and cuda_event, the raw handle)."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        h = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
        self.cuda_event = h.value

    def record(self, stream):
        rc = self._runtime().hipEventRecord(self.cuda_event, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        if self._hip is not None and self.cuda_event:
            self._hip.hipEventDestroy(self.cuda_event)


def algorithmic_bytes(w, T=None, es=2):
    """HBM bytes each stage must move at minimum (inputs read once, outputs
    written once), per launch over T tokens (default: the whole workload).
    es = 2 (bf16); beta, g, k_rnorm, gcum and kdecay are fp32.
      prepare  x, ba -> q, k, v, beta, g
      WY       k, v, beta, g -> w, u, k_rnorm, gcum, kdecay
      chunk_h  k, kdecay, gcum, w, u -> v_new, h (one state per 64-row chunk;
               the segment-parallel forms write one per 64-token chunk)
      chunk_o  q, k, k_rnorm, v_new, h (one per 64-token chunk), g -> o"""
    T = w["T"] * w["B"] if T is None else T
    M, H, HV, G, K, V = w["M"], w["H"], w["HV"], w["G"], w["K"], w["V"]
    P, N = V, K
    TM = T * M
    nte = math.ceil(T * M / 64)
    ntok_chunks = math.ceil(T / 64)
    prep = T * (M * H * P + M * G * N + G * N) * es + T * (M * H + H) * es \
        + T * H * N * es + TM * H * N * es + TM * H * P * es + TM * H * 4 + T * H * 4
    wy = TM * H * K * es + TM * HV * V * es + TM * HV * 4 + T * HV * 4 \
        + TM * HV * K * es + TM * HV * V * es + TM * H * 4 + TM * HV * 8
    ch = TM * H * K * es + TM * HV * 8 + TM * HV * K * es + TM * HV * V * es \
        + TM * HV * V * es + nte * HV * V * K * es
    co = T * H * K * es + TM * H * K * es + TM * H * 4 + TM * HV * V * es + ntok_chunks * HV * V * K * es \
        + T * HV * 4 + T * HV * V * es
    return {"gdp_prefill_prepare": prep, "gdp_recompute_w_u": wy, "gdp_chunk_h": ch, "gdp_chunk_o": co}


def scan_bytes(w, segments, nseg, mapped_tokens=None, nstates=None):
    """Algorithmic bytes per launch of the segment-parallel stages over the
    whole workload (one sequence, es = 2).
      wy_fused  the prepare's reads (x, ba) and writes (q, k, g; v and beta
                are not stored) plus WY's writes (w, u, k_rnorm, gcum,
                kdecay): the key and value copies, beta and g stay on chip
      map       k, kdecay, gcum, w, u of every segment but the last, read
                once; one fp32 K x (K + V) map per segment and head written
      scan      the maps read, one fp32 state per segment and head written
      chunk_h   as algorithmic_bytes, with one state per 64-token chunk
      chunk_ho  chunk_h and chunk_o as one pass: k, kdecay, gcum, w, u,
                k_rnorm, q and g read once, o written
    Packed requests give mapped_tokens (the tokens of every segment but the
    last of each request) and nstates (the segments) instead of nseg."""
    T, M, H, HV, G, K, V = w["T"] * w["B"], w["M"], w["H"], w["HV"], w["G"], w["K"], w["V"]
    ab = algorithmic_bytes(w)
    TM = T * M
    wy_fused = ab["gdp_prefill_prepare"] + ab["gdp_recompute_w_u"] - (TM * HV * (K + V) * 2 + TM * HV * 4 + T * HV * 4) \
        - TM * HV * (V * 2 + 4)
    seg_tok = math.ceil(math.ceil(T / 64) / segments) * 64
    if mapped_tokens is None:
        mapped_tokens, nstates = (nseg - 1) * seg_tok, nseg
    TMm = mapped_tokens * M
    maps = mapped_tokens // seg_tok * HV * K * (K + V) * 4
    mapb = TMm * H * K * 2 + TMm * HV * 8 + TMm * HV * (K + V) * 2 + maps
    scanb = maps + nstates * HV * V * K * 4
    ch = ab["gdp_chunk_h"] - (math.ceil(T * M / 64) - math.ceil(T / 64)) * HV * V * K * 2
    # one pass: k, kdecay, gcum, w, u, k_rnorm, q, g in; o out
    ho = TM * H * K * 2 + TM * HV * 8 + TM * HV * (K + V) * 2 + TM * H * 4 + T * H * K * 2 + T * HV * 4 \
        + T * HV * V * 2
    return {"wy_fused": wy_fused, "map": mapb, "scan": scanb, "chunk_h": ch, "chunk_ho": ho}


def decode_bytes(c):
    """Minimum HBM bytes of gdp_decode_update: the fp32 state read and
    written once, the q, k, v rows and fp32 beta, g read, o written."""
    n, L, es = c["n"], c["S"] * c["M"], 2
    return (2 * n * c["HV"] * c["V"] * c["K"] * 4 + n * L * (2 * c["H"] * c["K"] + c["HV"] * c["V"]) * es
            + n * L * c["HV"] * 8 + n * L * c["HV"] * c["V"] * es)


def measured_traffic(kernel, segments, path):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    the same chunk-forward path, if it was taken on the current kernel source
    with the same segments (the launch sizes); else None."""
    from gated_delta_product_amd import profiling
    name = {"scan": "traffic_long_prefill_32k_scan.json", "prefill-scan": "traffic_long_prefill_32k_prefill_scan.json"}.get(
        path, "traffic_long_prefill_32k.json")
    fn = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        t = json.load(f)
    e = t.get(kernel)
    if not e or e.get("src_digest") != profiling.src_digest(kernel) or t.get("_segments") != segments:
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(d, w, threads):
    """The oracle (numpy prepare + C recurrence and WY) on the same workload,
    timed on the host cores."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from oracle import prepare as OP

    T, M, H, K, V = w["T"], w["M"], w["H"], w["K"], w["V"]
    Ts = int(os.environ.get("GDP_BENCH_CPU_TOKENS", T))
    x = d["x"][:, :Ts].float().numpy()
    ba = d["ba"][:, :Ts].float().numpy()
    oracle.lib()
    t0 = time.perf_counter()
    q, k, v, beta, g = OP.prefill_prepare(x, ba, d["A_log"].numpy(), d["dt_bias"].numpy(), M, H, w["G"], V, K)

    def head(hv):
        qh = np.ascontiguousarray(q[0, :, hv])
        kh = np.ascontiguousarray(k[0, :, hv])
        vh = np.ascontiguousarray(v[0, :, hv])
        bh = np.ascontiguousarray(beta[0, :, hv])
        gh = np.ascontiguousarray(g[0, :, hv])
        oracle.recurrence(qh, kh, vh, bh, gh, M, scale=1.0 / math.sqrt(K))
        oracle.wy(kh, vh, bh, gh, M)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(head, range(w["HV"])))
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": Ts / dt, "unit": "tokens/s", "cores": threads, "host_cores": os.cpu_count(),
            "cpu_model": model, "kind": "oracle",
            "sample": "%d tokens x %d heads of the same workload (prepare, serial fp64 recurrence "
                      "-> o, v_new, h, and per-chunk WY -> w, u); %.1f s wall" % (Ts, w["HV"], dt)}


def decode_step(G, torch, dev, stream, steps):
    """Time gdp_decode_prepare + gdp_decode_update on the DECODE workload
    (inputs resident; the state pool advanced in place every step)."""
    from gated_delta_product_amd import synth
    c = DECODE
    n, S, M, H, Gq, P, N = c["n"], c["S"], c["M"], c["H"], c["G"], c["V"], c["K"]
    d = synth.prepare_draws(n, S, M, H, Gq, P, N, "bf16", synth.seed_of(4) + 200)
    x, ba = d["x"].to(dev), d["ba"].to(dev)
    A_log, dt_bias = d["A_log"].to(dev), d["dt_bias"].to(dev)
    gen = torch.Generator(device=dev).manual_seed(synth.seed_of(4) + 201)
    state = torch.randn((n, c["HV"], c["V"], c["K"]), generator=gen, device=dev) * 0.1
    rows = G.decode_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N)
    o = torch.empty((n, S * M, c["HV"], c["V"]), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        G.decode_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N, out=rows)
        G.decode_update(*rows, state, M, o=o)
    ev = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        G.decode_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N, out=rows)
        e[1].record(stream)
        G.decode_update(*rows, state, M, o=o)
        e[2].record(stream)
    torch.cuda.synchronize()
    prep_us = sum(e[0].elapsed_time(e[1]) for e in ev) / steps * 1e3
    upd_us = sum(e[1].elapsed_time(e[2]) for e in ev) / steps * 1e3
    ub = decode_bytes(c)
    return {"config": dict(c), "tokens_per_s": round(n * S / ((prep_us + upd_us) / 1e6), 1),
            "gdp_decode_prepare_us": round(prep_us, 2),
            "gdp_decode_update": {"us": round(upd_us, 2), "alg_bytes": ub, "GB/s": round(ub / upd_us / 1e3, 1),
                                  "hbm_frac": round(ub / upd_us / 1e3 / HBM_PEAK_GBS, 4)}}


def varlen_segments(cu, segments):
    """Segments the packed scan form cuts each request into (host copy of
    the device plan): seg_tok from the packed total, ceil(len / seg_tok) per
    request."""
    T = int(cu[-1])
    seg_tok = math.ceil(math.ceil(T / 64) / segments) * 64
    return seg_tok, [math.ceil((int(cu[i + 1]) - int(cu[i])) / seg_tok) for i in range(len(cu) - 1)]


def stage_record(torch, stream, n):
    evs = [TimingEvent() for _ in range(n)]
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    return evs


def time_stages(torch, stream, fn, n_ev, reps=10, warmup=3):
    """Mean time (us) between consecutive events of fn(events) over reps
    calls; fn records events[0] first and fills the rest."""
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    evs = [stage_record(torch, stream, n_ev) for _ in range(reps)]
    for e in evs:
        fn(e)
    torch.cuda.synchronize()
    return [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps * 1e3 for i in range(n_ev - 1)]


def roofline_of(kern):
    dom = max(kern, key=lambda kk: kern[kk]["us"])
    return {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dom]["hbm_frac"]}


def kernel_entry(us, alg):
    return {"us": round(us, 2), "alg_bytes": int(alg), "GB/s": round(alg / us / 1e3, 1),
            "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)}


def chunk_fwd_line(G, torch, dev, stream, cfg_id, reps):
    """gdp_chunk_fwd (its three stages in order, each bracketed by events) on
    one of the equal-length workloads, inputs drawn on the device: q, k on the
    unit sphere, v, b, a ~ N(0, 1) (a scaled by the workload's sigma), A_log =
    log U[1, 16], dt_bias ~ U[-1, 1]; beta and g from them by the gate
    formulas, outside the timed region."""
    from gated_delta_product_amd import synth
    c = synth.CONFIGS[cfg_id]
    B, T, H, HV, K, V, M = c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], c["M"]
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(synth.seed_of(cfg_id) + 500)

    def sphere(shape):
        x = torch.randn(shape, generator=gen, device=dev)
        return (x / x.norm(dim=-1, keepdim=True)).to(dt)

    q, k = sphere((B, T, H, K)), sphere((B, T * M, H, K))
    v = torch.randn((B, T * M, HV, V), generator=gen, device=dev).to(dt)
    b = torch.randn((B, T * M, HV), generator=gen, device=dev)
    a = torch.randn((B, T, HV), generator=gen, device=dev) * c.get("a_sigma", 1.0)
    A_log = torch.log(torch.rand(HV, generator=gen, device=dev) * 15 + 1)
    dt_bias = torch.rand(HV, generator=gen, device=dev) * 2 - 1
    beta = torch.sigmoid(b)
    g = -torch.exp(A_log) * torch.nn.functional.softplus(a + dt_bias)
    buf = G.ChunkBuffers(q, k, v, beta, g)

    def run(ev):
        if ev:
            ev[0].record(stream)
        buf.recompute_w_u()
        if ev:
            ev[1].record(stream)
        buf.chunk_h()
        if ev:
            ev[2].record(stream)
        buf.chunk_o()
        if ev:
            ev[3].record(stream)

    us = time_stages(torch, stream, run, 4, reps)
    w = dict(B=B, T=T, H=H, HV=HV, G=H, K=K, V=V, M=M)
    ab = algorithmic_bytes(w, es=2 if dt == torch.bfloat16 else 4)
    kern = {"gdp_recompute_w_u": kernel_entry(us[0], ab["gdp_recompute_w_u"]),
            "gdp_chunk_h": kernel_entry(us[1], ab["gdp_chunk_h"]),
            "gdp_chunk_o": kernel_entry(us[2], ab["gdp_chunk_o"])}
    tot = sum(us)
    out = {"workload": c["name"], "shape": dict(w, dtype=c["dtype"]), "path": "gdp_chunk_fwd",
           "us": round(tot, 1), "tokens_per_s": round(B * T / (tot / 1e6), 1), "kernels": kern,
           "roofline": roofline_of(kern)}
    if dt == torch.bfloat16 and M >= 2 and K in (64, 128) and V in (64, 128, 256):
        # the output-only form: v_new and h NULL, chunk_h and chunk_o as one
        # pass; its pass time is the whole call less WY alone, both timed here
        def run_wy(ev):
            ev[0].record(stream) if ev else None
            buf.recompute_w_u()
            ev[1].record(stream) if ev else None

        def run_fused(ev):
            ev[0].record(stream) if ev else None
            buf.forward(store_vnew_h=False)
            ev[1].record(stream) if ev else None

        wy_us = time_stages(torch, stream, run_wy, 2, reps)[0]
        fz_us = time_stages(torch, stream, run_fused, 2, reps)[0]
        kf = {"gdp_recompute_w_u": kernel_entry(wy_us, ab["gdp_recompute_w_u"]),
              "gdp_chunk_ho": dict(kernel_entry(fz_us - wy_us, scan_bytes(w, 1, 1)["chunk_ho"]),
                                   note="the call less WY alone")}
        out["fused"] = {"path": "gdp_chunk_fwd with v_new and h NULL (WY, then chunk_h and chunk_o as one pass)",
                        "us": round(fz_us, 1), "tokens_per_s": round(B * T / (fz_us / 1e6), 1), "kernels": kf,
                        "roofline": roofline_of(kf)}
    del buf, q, k, v, b, a, beta, g
    torch.cuda.empty_cache()
    return out


def varlen_line(G, torch, dev, stream, reps, segments=16):
    """The GVA varlen prefill workload: 8 packed requests (lengths drawn in
    [64, 4096]), prepare with 16 heads from 4 groups (timed on its own), then
    the segment-parallel chunk forward with GVA (4 key heads for 16 value
    heads); and the fused form, gdp_prefill_fwd_scan on the expanded heads,
    end to end."""
    from gated_delta_product_amd import synth
    c = synth.CONFIGS[3]
    p = c["prep"]
    M = c["M"]
    d = synth.varlen_prepare_draws(3)
    cu = d["cu_seqlens"]
    T = int(cu[-1])
    x, ba, A_log, dt_bias = d["x"].to(dev), d["ba"].to(dev), d["A_log"].to(dev), d["dt_bias"].to(dev)
    cu_d = torch.as_tensor(cu, dtype=torch.int32).to(dev)
    pre = G.prefill_prepare(x, ba, A_log, dt_bias, M, p["H"], p["G"], p["P"], p["N"])

    def run_prep(ev):
        if ev:
            ev[0].record(stream)
        G.prefill_prepare(x, ba, A_log, dt_bias, M, p["H"], p["G"], p["P"], p["N"], out=pre)
        if ev:
            ev[1].record(stream)

    prep_us = time_stages(torch, stream, run_prep, 2, reps)[0]
    q, k, v, beta, g = pre
    hpg = p["H"] // p["G"]
    gva = G.ChunkBuffers(q[:, :, ::hpg].contiguous(), k[:, :, ::hpg].contiguous(), v, beta, g, cu_seqlens=cu_d,
                         cu_seqlens_host=cu)

    def run_scan(ev):
        if ev:
            ev[0].record(stream)
        gva.forward_scan(segments, stage_events=ev[1:] if ev else None, store_vnew_h=False)

    us = time_stages(torch, stream, run_scan, 6, reps)
    seq = G.ChunkBuffers(gva.q, gva.k, v, beta, g, cu_seqlens=cu_d, cu_seqlens_host=cu)

    def run_seq(ev):
        if ev:
            ev[0].record(stream)
        seq.forward(store_vnew_h=False)
        if ev:
            ev[1].record(stream)

    seq_us = time_stages(torch, stream, run_seq, 2, reps)[0]
    fz = G.ChunkBuffers(*[torch.empty_like(t) for t in pre], cu_seqlens=cu_d, cu_seqlens_host=cu)

    def run_fused(ev):
        if ev:
            ev[0].record(stream)
        fz.prefill_scan(x, ba, A_log, dt_bias, p["G"], segments, stage_events=ev[1:] if ev else None,
                        store_v_beta=False, store_vnew_h=False, store_qk=False)

    fus = time_stages(torch, stream, run_fused, 6, reps)

    def run_fused1(ev):  # every request one segment: no maps
        if ev:
            ev[0].record(stream)
        fz.prefill_scan(x, ba, A_log, dt_bias, p["G"], 1, stage_events=ev[1:] if ev else None,
                        store_v_beta=False, store_vnew_h=False, store_qk=False)

    fus1 = time_stages(torch, stream, run_fused1, 6, reps)
    # algorithmic bytes: the chunk stages at H = 4 key heads, HV = 16
    w = dict(B=1, T=T, H=c["H"], HV=c["HV"], G=c["H"], K=c["K"], V=c["V"], M=M)
    ab = algorithmic_bytes(w)
    wp = dict(B=1, T=T, H=p["H"], HV=p["H"], G=p["G"], K=p["N"], V=p["P"], M=M)
    prep_b = algorithmic_bytes(wp)["gdp_prefill_prepare"]
    seg_tok, nsegs = varlen_segments(cu, segments)
    mapped = sum((n - 1) * seg_tok for n in nsegs if n > 1)
    sb = scan_bytes(w, segments, None, mapped_tokens=mapped, nstates=sum(nsegs))
    kern = {"gdp_recompute_w_u": kernel_entry(us[0], ab["gdp_recompute_w_u"]),
            "gdp_seg_map": kernel_entry(us[1], sb["map"]), "gdp_seg_scan": kernel_entry(us[2], sb["scan"]),
            "gdp_chunk_ho": kernel_entry(us[3] + us[4], sb["chunk_ho"])}
    tot = sum(us)
    sbf = scan_bytes(wp, segments, None, mapped_tokens=mapped, nstates=sum(nsegs))
    wyb = sbf["wy_fused"] - (T * (p["G"] + p["H"]) * p["N"] * 2 + T * M * p["H"] * p["N"] * 2)  # no q, k stores
    kf = {"gdp_recompute_w_u (prepare fused)": kernel_entry(fus[0], wyb),
          "gdp_seg_map": kernel_entry(fus[1], sbf["map"]), "gdp_seg_scan": kernel_entry(fus[2], sbf["scan"]),
          "gdp_chunk_ho": kernel_entry(fus[3] + fus[4], sbf["chunk_ho"])}
    out = {"workload": c["name"], "T": T, "cu_seqlens": [int(t) for t in cu], "segments_per_request": nsegs,
           "seg_tok": seg_tok,
           "prepare": dict(kernel_entry(prep_us, prep_b), tokens_per_s=round(T / (prep_us / 1e6), 1),
                           shape=dict(H=p["H"], G=p["G"], P=p["P"], N=p["N"], M=M)),
           "chunk_fwd_scan_gva": {"path": "gdp_chunk_fwd_scan, H=4 key heads, HV=16, v_new and h not stored "
                                          "(chunk_h and chunk_o as one pass)", "us": round(tot, 1),
                                  "tokens_per_s": round(T / (tot / 1e6), 1), "kernels": kern,
                                  "roofline": roofline_of(kern)},
           "chunk_fwd_sequential_gva": {"path": "gdp_chunk_fwd, unsegmented, v_new and h not stored",
                                        "us": round(seq_us, 1),
                                        "tokens_per_s": round(T / (seq_us / 1e6), 1)},
           "prefill_fwd_scan": {"path": "gdp_prefill_fwd_scan (prepare inside WY, H=HV=16 expanded, v, beta, "
                                        "q, k, v_new and h not stored)", "us": round(sum(fus), 1),
                                "tokens_per_s": round(T / (sum(fus) / 1e6), 1), "kernels": kf,
                                "roofline": roofline_of(kf)},
           "prefill_fwd_scan_1seg": {"path": "gdp_prefill_fwd_scan with num_segments=1 (no request split, no "
                                             "maps; v, beta, q, k, v_new and h not stored)", "us": round(sum(fus1), 1),
                                     "tokens_per_s": round(T / (sum(fus1) / 1e6), 1),
                                     "stage_us": [round(u, 1) for u in fus1]}}
    del gva, seq, fz, pre, x, ba
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--path", choices=["pipelined", "scan", "prefill-scan"], default="prefill-scan",
                    help="gdp_chunk_fwd_pipelined or gdp_chunk_fwd_scan after gdp_prefill_prepare, or "
                         "gdp_prefill_fwd_scan (prepare inside the WY stage)")
    ap.add_argument("--segments", type=int, default=None,
                    help="segments of the chunk forward (default %d pipelined, %d scan)" % (SEGMENTS, SCAN_SEGMENTS))
    ap.add_argument("--stages", action="store_true", help="also time each stage sequentially (not overlapped)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--store-v-beta", action="store_true",
                    help="prefill-scan: also store the value copies and beta (no later stage reads them)")
    ap.add_argument("--store-qk", action="store_true",
                    help="prefill-scan: also store q and k (otherwise the later stages read their rows from x)")
    ap.add_argument("--store-vnew-h", action="store_true",
                    help="scan paths: store v_new and h, i.e. run chunk_h and chunk_o as two launches (by default "
                         "they run as one pass that stores neither)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (tiny, Householder-copy, GVA varlen prefill, wide-head stress)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB (untimed), "
                         "the known-size kernel that calibrates rocprofv3 byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU hot path only; --gpus %d (WORLD_SIZE %d) is not supported: "
              "this build has no multi-GPU path." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_product_amd import binding as G
    from gated_delta_product_amd import synth

    w = dict(WORKLOAD)
    fused = args.path == "prefill-scan"
    scan = args.path == "scan" or fused
    if args.segments is None:
        args.segments = SCAN_SEGMENTS if scan else SEGMENTS
    ho = "chunk_h,chunk_o" if args.store_vnew_h else "chunk_h+o in one pass"
    if args.store_vnew_h:
        args.store_qk = True  # q and k from x only with the one-pass form
    if fused:
        w["path"] = "prefill_scan(recompute_w_u with prepare,seg_map,seg_scan,%s)" % ho + (
            "" if args.store_v_beta else "; v, beta not stored") + ("" if args.store_vnew_h else "; v_new, h not stored") \
            + ("" if args.store_qk else "; q, k not stored (read from x)")
    elif scan:
        w["path"] = "prepare+scan(recompute_w_u,seg_map,seg_scan,%s)" % ho
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synth.prepare_draws(1, w["T"], w["M"], w["H"], w["G"], w["V"], w["K"], "bf16", synth.seed_of(4) + 100)
    x, ba = d["x"].to(dev), d["ba"].to(dev)
    A_log, dt_bias = d["A_log"].to(dev), d["dt_bias"].to(dev)
    M, H, Gq, P, N = w["M"], w["H"], w["G"], w["V"], w["K"]
    prep_out = G.prefill_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N)
    buf = G.ChunkBuffers(*prep_out)
    stream = torch.cuda.current_stream(dev)
    nseg = G.scan_segments(w["T"], args.segments) if scan else G.pipeline_segments(w["T"], args.segments)
    # events: [0] step start, [1] after prepare (its own launch), then the
    # scan forms' five stage events (after WY, the maps, the scan, chunk_h,
    # chunk_o) or a pair around each pipelined chunk_h launch
    nev = 2 + (5 if scan else 2 * nseg)

    def new_events(n):
        evs = [TimingEvent() for _ in range(n)]
        for e in evs:
            e.record(stream)  # instantiate the handles
        return evs

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        if fused:
            if ev:
                ev[1].record(stream)
            buf.prefill_scan(x, ba, A_log, dt_bias, Gq, args.segments, stage_events=ev[2:] if ev else None,
                             store_v_beta=args.store_v_beta, store_vnew_h=args.store_vnew_h,
                             store_qk=args.store_qk)
            return
        G.prefill_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N, out=prep_out)
        if ev:
            ev[1].record(stream)
        if scan:
            buf.forward_scan(args.segments, stage_events=ev[2:] if ev else None, store_vnew_h=args.store_vnew_h)
        else:
            buf.forward_pipelined(nseg, chunk_h_events=ev[2:] if ev else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [new_events(nev) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens = w["B"] * w["T"]
    value = tokens / (ms_per_step / 1e3)

    def span_us(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in evs) / args.steps * 1e3

    ab = algorithmic_bytes(w)
    kern = {}

    def add(name, us, alg, launches=1, note=None):
        kern[name] = {"us": round(us, 2), "launches_per_step": launches, "alg_bytes": int(alg),
                      "GB/s": round(alg / us / 1e3, 1), "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)}
        if note:
            kern[name]["note"] = note

    if scan:
        sb = scan_bytes(w, args.segments, nseg)
        if fused:
            wyb = sb["wy_fused"] if not args.store_v_beta else sb["wy_fused"] + w["T"] * w["M"] * w["HV"] * (w["V"] * 2 + 4)
            if not args.store_qk:  # no q read, no q or k stored
                wyb -= w["T"] * (w["G"] + w["H"]) * w["K"] * 2 + w["T"] * w["M"] * w["H"] * w["K"] * 2
            add("gdp_recompute_w_u (prepare fused)", span_us(1, 2), wyb)
        else:
            add("gdp_prefill_prepare", span_us(0, 1), ab["gdp_prefill_prepare"])
            add("gdp_recompute_w_u", span_us(1, 2), ab["gdp_recompute_w_u"])
        add("gdp_seg_map", span_us(2, 3), sb["map"])
        add("gdp_seg_scan", span_us(3, 4), sb["scan"])
        if args.store_vnew_h:
            add("gdp_chunk_h", span_us(4, 5), sb["chunk_h"], note="all %d segments in one launch" % nseg)
            add("gdp_chunk_o", span_us(5, 6), ab["gdp_chunk_o"])
        else:
            add("gdp_chunk_ho", span_us(4, 6), sb["chunk_ho"],
                note="chunk_h and chunk_o as one pass over all %d segments (v_new and h not stored)" % nseg)
    else:
        add("gdp_prefill_prepare", span_us(0, 1), ab["gdp_prefill_prepare"])
        # chunk_h: every segment launch, bracketed on its own stream
        seg_ms = [e[2 + 2 * j].elapsed_time(e[3 + 2 * j]) for e in evs for j in range(nseg)]
        starts = G.pipeline_plan(w["T"], args.segments)
        seg_tokens = [starts[j + 1] - starts[j] for j in range(nseg)]
        ch_bytes = sum(algorithmic_bytes(w, t)["gdp_chunk_h"] for t in seg_tokens) / nseg  # per launch
        add("gdp_chunk_h", sum(seg_ms) / len(seg_ms) * 1e3, ch_bytes, launches=nseg,
            note="per segment launch, overlapped with the side streams' WY and chunk_o")
    # the roofline is reported for the kernel that takes the longest per launch
    dom = max(kern, key=lambda kk: kern[kk]["us"])
    kd = kern[dom]
    roof = {"kernel": dom, "bound": "hbm", "achieved": kd["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kd["GB/s"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom.split(" ")[0], nseg, args.path)}

    stages = None
    if args.stages:  # each stage alone, whole workload, for reference
        torch.cuda.synchronize()
        se = [new_events(5) for _ in range(3)]
        for e in se:
            e[0].record(stream)
            G.prefill_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N, out=prep_out)
            e[1].record(stream)
            buf.recompute_w_u()
            e[2].record(stream)
            buf.chunk_h()
            e[3].record(stream)
            buf.chunk_o()
            e[4].record(stream)
        torch.cuda.synchronize()
        stages = {}
        for i, k in enumerate(KERNELS):
            ms = sum(e[i].elapsed_time(e[i + 1]) for e in se) / len(se)
            stages[k] = {"us": round(ms * 1e3, 2), "GB/s": round(ab[k] / (ms / 1e3) / 1e9, 1),
                         "hbm_frac": round(ab[k] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    dec = None
    if not args.no_decode:
        dec = decode_step(G, torch, dev, stream, max(args.steps, 20))

    cfgs = None
    if not args.no_configs:
        cfgs = {"tiny_f32": chunk_fwd_line(G, torch, dev, stream, 1, 10),
                "householder_m2": chunk_fwd_line(G, torch, dev, stream, 2, 10),
                "gva_varlen_prepare": varlen_line(G, torch, dev, stream, 10),
                "wide_head_stress": chunk_fwd_line(G, torch, dev, stream, 5, 5)}

    if args.copy_mib > 0:
        n = args.copy_mib * 1024 * 1024 // 2
        src = torch.ones(n, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(d, w, threads)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": dict(w, segments=nseg), "roofline": roof, "cpu_baseline": cpu, "kernels": kern,
        "kernels_sum_us": round(sum(k["us"] * (1 if k["launches_per_step"] == 1 or scan else 0) for k in kern.values()), 1),
    }
    if stages:
        out["stages_sequential"] = stages
    if dec:
        out["decode"] = dec
    if cfgs:
        out["configs"] = cfgs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
