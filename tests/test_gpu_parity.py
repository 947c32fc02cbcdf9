"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Small workloads are compared on every (sequence, value head); the long and
wide workloads on sampled heads that the oracle runs end to end.  Tolerances:
prepare copies bit-exact and gates within BETA_ULPS / G_ULPS; chunk outputs within relative
L2 5e-3 and max-abs 2e-2 (bf16 inputs, fp32 accumulation) -- raw for o, and
beyond each element's half-ulp bf16 storage quantum for the bf16 intermediates
w, u, v_new and h, whose values reach ~10."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prepare as OP
from gated_delta_product_amd import binding as G
from gated_delta_product_amd import synth
from helpers import TOL, Acc, f32, gates, log, metrics, oracle_pair, run_pairs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# The gates are the eager tensor expressions of the prepare page (which asks
# for bitwise equality with the eager path), so they use the device's float32
# exp and log1p, each within 1 ulp of the exact value, where the oracle
# rounds exactly rounded functions per operation.  beta has one such function
# in its chain (exp, then 1 + e and 1 / d): within 2 ulp of the oracle.  g has
# three (exp(A_log), exp(s), log1p) and a product: within 4 ulp.  Equality
# with torch's eager expressions on the device is checked separately
# (test_gpu_eager_gates).
BETA_ULPS, G_ULPS = 2, 4


def _ulps(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


# ---------------------------------------------------------------------- chunk

def _seqs_equal(B, T, M):
    nte = math.ceil(T * M / 64)
    return [(b, 0, T, b * nte) for b in range(B)]


def _seqs_varlen(cu, M):
    out, base = [], 0
    for i in range(len(cu) - 1):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        out.append((0, t0, t1, base))
        base += math.ceil((t1 - t0) * M / 64)
    return out


def check_chunk(q, k, v, beta, g, seqs, hv_list, M, scale=None, cu=None, cu_host=None, tag="",
                want_wu=True, buf=None, h0=None, hstep=1):
    """Run the GPU forward (unless buf is given) and compare o, v_new, h, w, u
    (and the final state when an initial state h0 [nseq,HV,V,K] is given)
    with the oracle on the listed (sequence, value head) pairs.  g may be
    None (ungated).  hstep > 1 compares only the states entering chunks
    c % hstep == 0 (the ones the segment-parallel forward writes)."""
    dt = q.dtype
    tol = TOL[dt]
    H, HV, K = q.shape[2], v.shape[2], q.shape[3]
    if buf is None:
        buf = G.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), None if g is None else g.to(DEV),
                          scale=scale,
                          cu_seqlens=None if cu is None else torch.as_tensor(cu, dtype=torch.int32).to(DEV),
                          cu_seqlens_host=cu_host, initial_state=None if h0 is None else h0.to(DEV),
                          output_final_state=h0 is not None)
        torch.cuda.synchronize()
    sc = scale if scale is not None else 1.0 / math.sqrt(K)
    items = [(si, s, hv) for si, s in enumerate(seqs) for hv in hv_list if s[2] > s[1]]
    log("%s: %d (seq, head) pairs" % (tag, len(items)))

    def one(item):
        si, (b, t0, t1, hbase), hv = item
        hk = hv // (HV // H)
        qn = f32(q[b, t0:t1, hk])
        kn = f32(k[b, t0 * M:t1 * M, hk])
        vn = f32(v[b, t0 * M:t1 * M, hv])
        bn = f32(beta[b, t0 * M:t1 * M, hv])
        gn = None if g is None else f32(g[b, t0:t1, hv])
        h0n = None if h0 is None else h0[si, hv].double().numpy()
        return oracle_pair(qn, kn, vn, bn, gn, M, sc, want_wu, h0=h0n)

    refs = run_pairs(one, items)
    names = ["o", "v_new", "h"] + (["w", "u"] if want_wu else []) + (["ht"] if h0 is not None else [])
    # the final state is fp32 on both sides: judged raw
    accs = {n: Acc(n, raw_max_abs=(n in ("o", "ht"))) for n in names}
    bf = dt == torch.bfloat16
    vn_rows = G.slices_to_rows(buf.v_new)
    u_rows = G.slices_to_rows(buf.u) if want_wu else None
    for (si, (b, t0, t1, hbase), hv), r in zip(items, refs):
        nc = math.ceil((t1 - t0) * M / 64)
        accs["o"].add(f32(buf.o[b, t0:t1, hv]), r["o"], bf)
        accs["v_new"].add(f32(vn_rows[b, t0 * M:t1 * M, hv]), r["v_new"], bf)
        accs["h"].add(f32(buf.h[hbase:hbase + nc:hstep, hv]), r["h"][::hstep], bf)
        if want_wu:
            accs["w"].add(f32(buf.w[b, t0 * M:t1 * M, hv]), r["w"], bf)
            accs["u"].add(f32(u_rows[b, t0 * M:t1 * M, hv]), r["u"], bf)
        if h0 is not None:
            accs["ht"].add(f32(buf.ht[si, hv]), r["h_final"], False)
    for a in accs.values():
        a.check(tol)
    return buf


def _cfg_inputs(cfg):
    d = synth.config_chunk_draws(cfg)
    beta, g = gates(d)
    c = synth.CONFIGS[cfg]
    beta = beta.reshape(c["B"], c["T"] * c["M"], c["HV"])
    return d, beta, g


def test_chunk_tiny_f32():
    """B=1, T=128, H=HV=2, K=V=64, M=1, float32: every output, every head."""
    c = synth.CONFIGS[1]
    d, beta, g = _cfg_inputs(1)
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(c["B"], c["T"], c["M"]), range(c["HV"]),
                c["M"], tag="tiny_f32")


@pytest.mark.parametrize("M", [2, 4])
def test_chunk_f32_wide_value_many_copies(M):
    """float32, K=64, V=128 with M = 2 (one 128-column output slab) and M = 4
    (two 64-column slabs, so the V slab of all copies fits the output stage's
    LDS), ragged T: every output, every head."""
    B_, T, H, HV, K, V = 1, 100, 2, 2, 64, 128
    d = synth.chunk_draws(B_, T, H, HV, K, V, M, "f32", synth.seed_of(1) + M)
    beta, g = gates(d)
    beta = beta.reshape(B_, T * M, HV)
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(B_, T, M), range(HV), M, tag="f32 V=128 M=%d" % M)


def test_chunk_householder_m2():
    """B=2, T=1024, H=HV=8, K=V=128, M=2, bf16: every output, every head."""
    c = synth.CONFIGS[2]
    d, beta, g = _cfg_inputs(2)
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(c["B"], c["T"], c["M"]), range(c["HV"]),
                c["M"], tag="householder_m2")


def test_chunk_long_prefill_sampled():
    """B=1, T=32768, H=HV=16, K=V=128, M=2 (the timed workload): the whole
    sequence on sampled heads."""
    c = synth.CONFIGS[4]
    d, beta, g = _cfg_inputs(4)
    log("long_prefill: inputs drawn")
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(c["B"], c["T"], c["M"]), [0, 9, 15],
                c["M"], tag="long_prefill_32k")


def test_chunk_wide_head_stress_sampled():
    """B=4, T=8192, H=HV=32, K=128, V=256, M=3, extreme gates (planted on
    batch 0 / head 0): sampled (batch row, head) pairs."""
    c = synth.CONFIGS[5]
    d, beta, g = _cfg_inputs(5)
    log("wide_head: inputs drawn; g range [%.1f, %.1f]" % (float(g.min()), float(g.max())))
    seqs = _seqs_equal(c["B"], c["T"], c["M"])
    buf = None
    for srow, hvs in ((0, [0]), (3, [31]), (1, [17])):
        buf = check_chunk(d["q"], d["k"], d["v"], beta, g, [seqs[srow]], hvs, c["M"], tag="wide_head",
                          buf=buf)


def test_chunk_ragged_and_degenerate():
    """Ragged tails (T*M not a multiple of 64), M=3 and M=4, T=1, and the
    degenerate gates: beta=0 (no writes: v_new = 0, o = 0), g=0 (no decay),
    long memory (|g| ~ 1e-3) so the state carries over many chunks."""
    cases = [
        dict(B=2, T=100, H=2, HV=4, K=64, V=128, M=3, seed=11),
        dict(B=1, T=1, H=1, HV=1, K=128, V=64, M=2, seed=12),
        dict(B=1, T=77, H=2, HV=2, K=128, V=256, M=4, seed=13),
        dict(B=1, T=300, H=1, HV=2, K=64, V=64, M=1, seed=14),
    ]
    for cs in cases:
        d = synth.chunk_draws(cs["B"], cs["T"], cs["H"], cs["HV"], cs["K"], cs["V"], cs["M"], "bf16",
                              cs["seed"])
        beta, g = gates(d)
        check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(cs["B"], cs["T"], cs["M"]), range(cs["HV"]),
                    cs["M"], tag="ragged %s" % cs)
    # degenerate gates on one shape
    B_, T, H, HV, K, V, M = 1, 200, 2, 2, 128, 128, 2
    d = synth.chunk_draws(B_, T, H, HV, K, V, M, "bf16", 21)
    beta, g = gates(d)
    buf = G.chunk_fwd(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), torch.zeros_like(beta).to(DEV),
                      g.to(DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf.v_new).item() == 0 and torch.count_nonzero(buf.o).item() == 0
    check_chunk(d["q"], d["k"], d["v"], beta, torch.zeros_like(g), _seqs_equal(B_, T, M), range(HV), M,
                tag="no decay")
    dl = synth.chunk_draws(B_, T, H, HV, K, V, M, "bf16", 22)
    dl["dt_bias"] = torch.empty(HV).uniform_(-9, -7, generator=torch.Generator().manual_seed(5))
    beta, g = gates(dl)
    check_chunk(dl["q"], dl["k"], dl["v"], beta, g, _seqs_equal(B_, T, M), range(HV), M, tag="long memory")


def test_chunk_determinism():
    c = synth.CONFIGS[2]
    d, beta, g = _cfg_inputs(2)
    args = [t.to(DEV) for t in (d["q"], d["k"], d["v"], beta, g)]
    b1 = G.chunk_fwd(*args)
    b2 = G.chunk_fwd(*args)
    torch.cuda.synchronize()
    for n in ("o", "w", "u", "v_new", "h", "k_rnorm"):
        assert torch.equal(getattr(b1, n), getattr(b2, n)), n


def test_stages_match_fused_call():
    """Calling recompute_w_u, chunk_h and chunk_o one by one gives the same
    bytes as gdp_chunk_fwd."""
    d = synth.chunk_draws(2, 200, 2, 4, 128, 128, 2, "bf16", 31)
    beta, g = gates(d)
    args = [t.to(DEV) for t in (d["q"], d["k"], d["v"], beta, g)]
    b1 = G.chunk_fwd(*args)
    b2 = G.ChunkBuffers(*args)
    b2.recompute_w_u()
    b2.chunk_h()
    b2.chunk_o()
    torch.cuda.synchronize()
    for n in ("o", "w", "u", "v_new", "h"):
        assert torch.equal(getattr(b1, n), getattr(b2, n)), n


def test_chunk_o_alone_on_oracle_state():
    """chunk_o fed with the oracle's own boundary states and corrected values
    (rounded to bf16) reproduces the oracle output: isolates the output stage."""
    B_, T, H, HV, K, V, M = 1, 256, 2, 2, 128, 128, 3
    d = synth.chunk_draws(B_, T, H, HV, K, V, M, "bf16", 41)
    beta, g = gates(d)
    args = [t.to(DEV) for t in (d["q"], d["k"], d["v"], beta, g)]
    buf = G.ChunkBuffers(*args)
    buf.recompute_w_u()  # k_rnorm
    sc = 1.0 / math.sqrt(K)
    h_ref = torch.empty_like(buf.h, device="cpu")
    vn_ref = torch.empty((B_, T * M, HV, V), dtype=torch.bfloat16)
    refs = []
    for hv in range(HV):
        hk = hv // (HV // H)
        r = oracle.recurrence(f32(d["q"][0, :, hk]), f32(d["k"][0, :, hk]), f32(d["v"][0, :, hv]),
                              f32(beta[0, :, hv]), f32(g[0, :, hv]), M, scale=sc)
        h_ref[:, hv] = torch.from_numpy(r["h"]).to(torch.bfloat16)
        vn_ref[0, :, hv] = torch.from_numpy(r["v_new"]).to(torch.bfloat16)
        refs.append(r)
    buf.set(h=h_ref.to(DEV), v_new=G.rows_to_slices(vn_ref).to(DEV))
    buf.chunk_o()
    torch.cuda.synchronize()
    acc = Acc("o", raw_max_abs=True)
    for hv in range(HV):
        acc.add(f32(buf.o[0, :, hv]), refs[hv]["o"])
    acc.check(TOL[torch.bfloat16])


# ---------------------------------------------------------------------- prepare

def _prepare_check(x, ba, A_log, dt_bias, M, H, G_, P, N, tag):
    q, k, v, beta, g = G.prefill_prepare(x.to(DEV) if not x.is_cuda else x, ba.to(DEV) if not ba.is_cuda else ba,
                                         A_log.to(DEV), dt_bias.to(DEV), M, H, G_, P, N)
    torch.cuda.synchronize()
    rq, rk, rv, rb, rg = OP.prefill_prepare(f32(x), f32(ba), A_log.numpy(), dt_bias.numpy(), M, H, G_, P, N)
    dt = q.dtype
    assert torch.equal(q.cpu(), torch.from_numpy(rq).to(dt)), tag + " q"
    assert torch.equal(k.cpu(), torch.from_numpy(rk).to(dt)), tag + " k"
    assert torch.equal(v.cpu(), torch.from_numpy(rv).to(dt)), tag + " v"
    ub = _ulps(beta.cpu().numpy(), rb)
    ug = _ulps(g.cpu().numpy(), rg)
    log("%s: beta max ulp %d (%d differ), g max ulp %d (%d differ)" % (
        tag, ub.max(), (ub > 0).sum(), ug.max(), (ug > 0).sum()))
    assert ub.max() <= BETA_ULPS and ug.max() <= G_ULPS
    return q, k, v, beta, g


def test_prepare_varlen_prefill():
    """The packed n == 1 prefill of 8 requests (H=16, G=4, P=N=128, M=2)."""
    d = synth.varlen_prepare_draws(3)
    p = synth.CONFIGS[3]["prep"]
    log("varlen prepare: T=%d, cu_seqlens=%s" % (int(d["cu_seqlens"][-1]), list(d["cu_seqlens"])))
    _prepare_check(d["x"], d["ba"], d["A_log"], d["dt_bias"], synth.CONFIGS[3]["M"], p["H"], p["G"], p["P"],
                   p["N"], "varlen_prepare")


def test_prepare_gate_edges_planted():
    """a + dt_bias hits 20 (log1p side), nextafter(20) (identity side), 25,
    88, -16, -30, -90, -104; b hits 0, 17, 100, -104 and large negatives."""
    M, H, G_, P, N, T = 2, 2, 1, 8, 8, 8
    width = M * H * P + M * G_ * N + G_ * N
    for dtype in (torch.bfloat16, torch.float32):
        x = torch.randn(1, T, width, generator=torch.Generator().manual_seed(1)).to(dtype)
        ba = torch.zeros(1, T, M * H + H)
        a_vals = torch.tensor([20.0, 20.0, 25.0, 88.0, -16.0, -30.0, -90.0, -104.0])
        ba[0, :, M * H + 0] = a_vals            # head 0: dt_bias 0 -> s = a
        ba[0, :, M * H + 1] = 20.0               # head 1: dt_bias 2^-19 -> s = nextafter(20)
        b_vals = torch.tensor([0.0, 17.0, 100.0, -104.0, -20.0, 1.5, -0.75, 88.0])
        for j in range(M * H):
            ba[0, :, j] = b_vals
        ba = ba.to(dtype)
        A_log = torch.tensor([0.0, math.log(16.0)], dtype=torch.float32)
        dt_bias = torch.tensor([0.0, 2.0 ** -19], dtype=torch.float32)
        _, _, _, beta, g = _prepare_check(x, ba, A_log, dt_bias, M, H, G_, P, N, "edges %s" % dtype)
        s1 = np.float32(20.0) + np.float32(2.0 ** -19)
        assert s1 == np.nextafter(np.float32(20), np.float32(30))
        assert g[0, 0, 0].item() == -20.0 and beta[0, 0, 0].item() == 0.5


def test_prepare_strided_rows_and_scalar_path():
    """x as a row-strided view (wider parent rows) and ba as a column slice of
    a wider tensor give the same results; odd head dims take the element-wise
    copy path."""
    M, H, G_, P, N, T = 3, 4, 2, 16, 24, 37
    width = M * H * P + M * G_ * N + G_ * N
    gen = torch.Generator().manual_seed(3)
    parent = torch.randn(2, T, width + 40, generator=gen).to(torch.bfloat16).to(DEV)
    x = parent[:, :, 8:8 + width]
    bparent = torch.randn(2, T, M * H + H + 5, generator=gen).to(torch.bfloat16).to(DEV)
    ba = bparent[:, :, 2:2 + M * H + H]
    A_log = torch.log(torch.rand(H, generator=gen) * 15 + 1)
    dt_bias = torch.rand(H, generator=gen) * 2 - 1
    _prepare_check(x, ba, A_log, dt_bias, M, H, G_, P, N, "strided")
    P2, N2 = 12, 20  # not multiples of 8 elements: per-element path
    width2 = M * H * P2 + M * G_ * N2 + G_ * N2
    x2 = torch.randn(1, T, width2, generator=gen).to(torch.bfloat16)
    ba2 = torch.randn(1, T, M * H + H, generator=gen).to(torch.bfloat16)
    _prepare_check(x2, ba2, A_log, dt_bias, M, H, G_, P2, N2, "scalar path")


# ---------------------------------------------------------------------- end to end

def test_varlen_gva_end_to_end():
    """Packed 8-request prefill: GPU prepare then GPU chunk forward with GVA
    (H=4 query/key heads for HV=16 value heads) against the oracle on every
    (request, head); the GVA run equals the run on head-expanded q/k, and the
    packed run equals each request run on its own, bit for bit."""
    c = synth.CONFIGS[3]
    p = c["prep"]
    M = c["M"]
    d = synth.varlen_prepare_draws(3)
    cu = d["cu_seqlens"]
    q, k, v, beta, g = _prepare_check(d["x"], d["ba"], d["A_log"], d["dt_bias"], M, p["H"], p["G"], p["P"],
                                      p["N"], "e2e prepare")
    hpg = p["H"] // p["G"]
    qg = q[:, :, ::hpg].contiguous()   # heads 0, 4, 8, 12 = the G groups
    kg = k[:, :, ::hpg].contiguous()
    cu_d = torch.as_tensor(cu, dtype=torch.int32).to(DEV)
    seqs = _seqs_varlen(cu, M)
    buf = check_chunk(qg.cpu(), kg.cpu(), v.cpu(), beta.cpu(), g.cpu(), seqs, range(c["HV"]), M, cu=cu,
                      cu_host=cu, tag="varlen_gva")
    full = G.chunk_fwd(q, k, v, beta, g, cu_seqlens=cu_d, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    for n in ("o", "w", "u", "v_new", "h"):
        assert torch.equal(getattr(buf, n), getattr(full, n)), "GVA vs expanded: " + n
    for i, (b, t0, t1, hbase) in enumerate(seqs):
        one = G.chunk_fwd(qg[:, t0:t1].contiguous(), kg[:, t0 * M:t1 * M].contiguous(),
                          v[:, t0 * M:t1 * M].contiguous(), beta[:, t0 * M:t1 * M].contiguous(),
                          g[:, t0:t1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(one.o, buf.o[:, t0:t1]), "request %d o" % i
        nc = one.h.shape[0]
        assert torch.equal(one.h, buf.h[hbase:hbase + nc]), "request %d h" % i


def test_varlen_empty_and_tiny_requests():
    """Requests of length 0, 1, 63, 64, 65 packed together (ragged chunks at
    every request boundary)."""
    lens = [0, 1, 63, 0, 64, 65, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    M, H, HV, K, V = 3, 2, 4, 64, 64
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", 51)
    beta, g = gates(d)
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_varlen(cu, M), range(HV), M, cu=cu, cu_host=cu,
                tag="tiny requests")


def test_long_prefill_path_with_prepare():
    """The timed workload's launch configuration: prepare (H=G=16,
    P=N=128, M=2) feeding the chunk forward at T=32768; the output of
    sampled heads against the oracle run on the oracle's prepare output."""
    c = synth.CONFIGS[4]
    M, H, T = c["M"], c["HV"], c["T"]
    d = synth.prepare_draws(1, T, M, H, H, c["V"], c["K"], "bf16", synth.seed_of(4) + 100)
    log("long prepare: inputs drawn")
    x = d["x"].to(DEV)
    ba = d["ba"].to(DEV)
    q, k, v, beta, g = G.prefill_prepare(x, ba, d["A_log"].to(DEV), d["dt_bias"].to(DEV), M, H, H, c["V"], c["K"])
    buf = G.chunk_fwd(q, k, v, beta, g)
    torch.cuda.synchronize()
    # oracle prepare on the sampled heads' slices only
    xs = f32(d["x"][0])
    bas = f32(d["ba"][0])
    P_, N_ = c["V"], c["K"]
    heads = [0, 13]
    for hv in heads:
        vh = np.ascontiguousarray(xs[:, : M * H * P_].reshape(T, M, H, P_)[:, :, hv].reshape(T * M, P_))
        kh = np.ascontiguousarray(xs[:, M * H * P_: M * H * P_ + M * H * N_].reshape(T, M, H, N_)[:, :, hv]
                                  .reshape(T * M, N_))
        qh = np.ascontiguousarray(xs[:, M * H * P_ + M * H * N_:].reshape(T, H, N_)[:, hv])
        bh = OP.sigmoid_rn32(bas[:, : M * H].reshape(T, M, H)[:, :, hv].reshape(T * M))
        gh = OP.decay_rn32(bas[:, M * H + hv], d["A_log"].numpy()[hv], d["dt_bias"].numpy()[hv])
        r = oracle.recurrence(qh, kh, vh, bh, np.ascontiguousarray(gh), M, scale=1.0 / math.sqrt(N_))
        a = Acc("o[%d]" % hv, raw_max_abs=True)
        a.add(f32(buf.o[0, :, hv]), r["o"])
        a.check(TOL[torch.bfloat16])


# ------------------------------------------------- ungated rule, state chaining

def test_ungated_matches_oracle_and_zero_decay():
    """g = None (the pages' ungated call) against the oracle's ungated
    recurrence, with GVA and a ragged tail; bit for bit the run with g = 0."""
    B, T, H, HV, K, V, M = 2, 300, 2, 4, 128, 128, 2
    d = synth.chunk_draws(B, T, H, HV, K, V, M, "bf16", synth.seed_of(2) + 7)
    beta, _ = gates(d)
    beta = beta.reshape(B, T * M, HV)
    q, k, v = d["q"], d["k"], d["v"]
    buf = check_chunk(q, k, v, beta, None, _seqs_equal(B, T, M), range(HV), M, tag="ungated")
    zero = G.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), torch.zeros(B, T, HV, device=DEV))
    torch.cuda.synchronize()
    for n in ("o", "w", "u", "v_new", "h"):
        assert torch.equal(getattr(buf, n), getattr(zero, n)), n


def test_initial_and_final_state_varlen():
    """A given initial state per request and the final state, against the
    oracle (which starts its recurrence from h0), on packed requests that
    include an empty one (its final state is its initial state) and ragged
    tails."""
    M, H, HV, K, V = 2, 2, 4, 128, 128
    cu = [0, 70, 70, 200, 457]
    T = cu[-1]
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", synth.seed_of(3) + 11)
    beta, g = gates(d)
    beta = beta.reshape(1, T * M, HV)
    h0 = synth.initial_state_draws(len(cu) - 1, HV, V, K, synth.seed_of(3) + 12)
    buf = check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_varlen(cu, M), range(HV), M, cu=cu, cu_host=cu,
                      tag="h0/ht varlen", h0=h0)
    assert torch.equal(buf.ht[1].cpu(), h0[1]), "empty request: ht must equal h0"


def test_state_chaining_is_exact():
    """Running a sequence in two calls -- the second starting from the first
    call's final state -- reproduces the single call bit for bit (the split
    is on a 64-token boundary, so every chunk is the same)."""
    B, T, H, HV, K, V, M = 1, 512, 2, 2, 128, 128, 2
    d = synth.chunk_draws(B, T, H, HV, K, V, M, "bf16", synth.seed_of(2) + 13)
    beta, g = gates(d)
    beta = beta.reshape(B, T * M, HV).to(DEV)
    q, k, v, g = d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), g.to(DEV)
    full = G.chunk_fwd(q, k, v, beta, g, output_final_state=True)
    s = 192
    a = G.chunk_fwd(q[:, :s].contiguous(), k[:, :s * M].contiguous(), v[:, :s * M].contiguous(),
                    beta[:, :s * M].contiguous(), g[:, :s].contiguous(), output_final_state=True)
    b = G.chunk_fwd(q[:, s:].contiguous(), k[:, s * M:].contiguous(), v[:, s * M:].contiguous(),
                    beta[:, s * M:].contiguous(), g[:, s:].contiguous(), initial_state=a.ht,
                    output_final_state=True)
    torch.cuda.synchronize()
    nc = s * M // 64
    assert torch.equal(full.o, torch.cat([a.o, b.o], 1))
    assert torch.equal(full.v_new, torch.cat([a.v_new, b.v_new], 3))  # slice-major: rows are dim 3
    assert torch.equal(full.h, torch.cat([a.h, b.h], 0)) and a.h.shape[0] == nc
    assert torch.equal(full.ht, b.ht)


def test_pipelined_forward_is_bit_identical():
    """gdp_chunk_fwd_pipelined (segments chained through the fp32 state, with
    the parallel stages on side streams) gives exactly the outputs of
    gdp_chunk_fwd, for several segment counts, with an initial state, a
    ragged last chunk and the ungated rule."""
    B, T, H, HV, K, V, M = 1, 1000, 2, 4, 128, 128, 2
    d = synth.chunk_draws(B, T, H, HV, K, V, M, "bf16", synth.seed_of(2) + 17)
    beta, g = gates(d)
    beta = beta.reshape(B, T * M, HV).to(DEV)
    q, k, v, g = d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), g.to(DEV)
    h0 = synth.initial_state_draws(1, HV, V, K, synth.seed_of(2) + 18).to(DEV)
    for gg in (g, None):
        ref = G.ChunkBuffers(q, k, v, beta, gg, initial_state=h0, output_final_state=True)
        ref.forward()
        for nseg in (1, 3, 7, 64):
            pip = G.ChunkBuffers(q, k, v, beta, gg, initial_state=h0, output_final_state=True)
            n = G.pipeline_segments(T, nseg)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            for e in evs:
                e.record()
            pip.forward_pipelined(nseg, chunk_h_events=evs)
            torch.cuda.synchronize()
            for nm in ("o", "w", "u", "v_new", "h", "ht"):
                assert torch.equal(getattr(ref, nm), getattr(pip, nm)), (nseg, gg is None, nm)
            assert all(evs[2 * i].elapsed_time(evs[2 * i + 1]) > 0 for i in range(n))


def test_prefill_pipelined_is_bit_identical():
    """gdp_prefill_fwd_pipelined (each segment's prepare on the WY side stream)
    gives exactly the outputs of gdp_prefill_prepare then gdp_chunk_fwd, for
    several segment counts and a ragged last chunk."""
    T, M, H, G_, P, N = 1000, 2, 4, 2, 128, 128
    d = synth.prepare_draws(1, T, M, H, G_, P, N, "bf16", synth.seed_of(4) + 90)
    x, ba, A_log, dt_bias = d["x"].to(DEV), d["ba"].to(DEV), d["A_log"].to(DEV), d["dt_bias"].to(DEV)
    pre = G.prefill_prepare(x, ba, A_log, dt_bias, M, H, G_, P, N)
    h0 = synth.initial_state_draws(1, H, P, N, synth.seed_of(4) + 91).to(DEV)
    ref = G.ChunkBuffers(*pre, initial_state=h0, output_final_state=True)
    ref.forward()
    torch.cuda.synchronize()
    for nseg in (1, 3, 5):
        log("prefill pipelined, %d segments" % nseg)
        outs = [torch.full_like(t, 7) for t in pre]  # prepare must overwrite all of them
        pip = G.ChunkBuffers(*outs, initial_state=h0, output_final_state=True)
        pip.prefill_pipelined(x, ba, A_log, dt_bias, G_, nseg)
        torch.cuda.synchronize()
        for a, b, nm in zip(outs, pre, ("q", "k", "v", "beta", "g")):
            assert torch.equal(a, b), nm
        for nm in ("o", "w", "u", "v_new", "h", "ht"):
            assert torch.equal(getattr(pip, nm), getattr(ref, nm)), nm


# ---------------------------------------------------------------------- decode

def test_decode_prepare_matches_oracle():
    """gdp_decode_prepare: key, value and the query copies bit-exact, the
    query only on each token's last copy and the decay only on its first
    (exact zeros elsewhere), gates within BETA_ULPS / G_ULPS; bf16 and f32, M = 2 and 3."""
    cases = (("bf16", 5, 3, 2, 16, 4, 128, 128), ("f32", 3, 2, 3, 4, 2, 64, 64), ("bf16", 64, 1, 4, 16, 16, 128, 128))
    for i, (dt, n, S, M, H, G_, P, N) in enumerate(cases):
        d = synth.prepare_draws(n, S, M, H, G_, P, N, dt, synth.seed_of(3) + 50 + i)
        log("decode prepare case %d: %s n=%d S=%d M=%d H=%d G=%d P=%d N=%d" % (i, dt, n, S, M, H, G_, P, N))
        q, k, v, beta, g = G.decode_prepare(d["x"].to(DEV), d["ba"].to(DEV), d["A_log"].to(DEV),
                                            d["dt_bias"].to(DEV), M, H, G_, P, N)
        torch.cuda.synchronize()
        rq, rk, rv, rb, rg = OP.decode_prepare(f32(d["x"]), f32(d["ba"]), d["A_log"].numpy(), d["dt_bias"].numpy(),
                                               M, H, G_, P, N)
        t = q.dtype
        assert torch.equal(q.cpu(), torch.from_numpy(rq).to(t)), "q"
        assert torch.equal(k.cpu(), torch.from_numpy(rk).to(t)), "k"
        assert torch.equal(v.cpu(), torch.from_numpy(rv).to(t)), "v"
        gc = g.cpu().numpy()
        assert np.all(gc[:, [e for e in range(S * M) if e % M]] == 0.0)
        assert _ulps(beta.cpu().numpy(), rb).max() <= BETA_ULPS and _ulps(gc, rg).max() <= G_ULPS


def _decode_oracle(q, k, v, beta, g, state, slots, scale=None):
    """The per-row gated delta rule of each request from its slot's state,
    by oracle.recurrence with one copy per row.  Returns (o [n,L,HV,V],
    state after the step [pool,HV,V,K]) in float64."""
    n, L, H, _ = q.shape
    HV = v.shape[2]
    o = np.zeros((n, L, HV, v.shape[3]))
    st = state.astype(np.float64).copy()
    for i in range(n):
        s = int(slots[i])
        if s < 0 or s >= state.shape[0]:
            continue
        for hv in range(HV):
            hk = hv // (HV // H)
            r = oracle.recurrence(q[i, :, hk], k[i, :, hk], v[i, :, hv], beta[i, :, hv],
                                  None if g is None else g[i, :, hv], 1, scale=scale, h0=state[s, hv],
                                  want_vnew=False, want_h=False)
            o[i, :, hv] = r["o"]
            st[s, hv] = r["h_final"]
    return o, st


DECODE_CASES = [
    # dtype, n, S, M, H, HV, K, V, pool, slots (None = request i -> slot i), gated
    ("bf16", 5, 3, 2, 2, 4, 128, 128, 7, [6, -1, 0, 3, 7], True),
    ("f32", 3, 2, 3, 1, 2, 64, 256, 3, None, True),
    ("bf16", 4, 5, 1, 2, 2, 64, 64, 4, [2, 3, 1, 0], False),
    ("bf16", 2, 1, 4, 1, 2, 128, 256, 2, None, True),
    ("f32", 2, 7, 2, 2, 2, 128, 64, 9, [8, 4], True),
    ("bf16", 1, 1024, 4, 1, 1, 64, 64, 1, None, True),   # the longest step: S*M = 4096 rows
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=["%s-K%dV%d-M%d" % (c[0], c[6], c[7], c[3]) for c in DECODE_CASES])
def test_decode_update_matches_oracle(case):
    """gdp_decode_update against the oracle's serial recurrence: every row has
    its own query, key, beta and decay; states come from a pool through
    slots (negative and out-of-pool slots skip their request: o rows zero,
    no state touched); unnamed slots keep their bits."""
    dt, n, S, M, H, HV, K, V, pool, slots, gated = case
    L = S * M
    log("decode update: %s n=%d S=%d M=%d H=%d HV=%d K=%d V=%d pool=%d slots=%s gated=%s" % case)
    d = synth.chunk_draws(n, L, H, HV, K, V, 1, dt, synth.seed_of(2) + 60 + K + V + M)
    beta, g = gates(d)
    beta = beta.reshape(n, L, HV)
    g = g if gated else None
    st0 = synth.initial_state_draws(pool, HV, V, K, synth.seed_of(2) + 61, sigma=0.2)
    state = st0.to(DEV)
    sl = None if slots is None else torch.tensor(slots, dtype=torch.int32, device=DEV)
    o = G.decode_update(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), beta.to(DEV),
                        None if g is None else g.to(DEV), state, M, slots=sl)
    torch.cuda.synchronize()
    slots_h = list(range(n)) if slots is None else slots
    ro, rst = _decode_oracle(f32(d["q"]), f32(d["k"]), f32(d["v"]), beta.numpy(), None if g is None else g.numpy(),
                             st0.numpy(), slots_h)
    tol = TOL[d["q"].dtype]
    mo, ro_l2, fin = metrics(f32(o), ro)
    ms, rs_l2, fin_s = metrics(state.cpu().numpy(), rst)
    log("  o: max_abs %.3g rel_l2 %.3g; state: max_abs %.3g rel_l2 %.3g" % (mo, ro_l2, ms, rs_l2))
    assert fin and fin_s
    assert mo <= tol["max_abs"] and ro_l2 <= tol["rel_l2"]
    assert ms <= TOL[torch.float32]["max_abs"] and rs_l2 <= TOL[torch.float32]["rel_l2"]
    used = {s for s in slots_h if 0 <= s < pool}
    for s in range(pool):
        if s not in used:
            assert torch.equal(state[s].cpu(), st0[s]), "slot %d touched" % s
    for i, s in enumerate(slots_h):
        if not 0 <= s < pool:
            assert torch.count_nonzero(o[i]) == 0, "skipped request %d wrote o" % i


def test_decode_continues_chunked_prefill():
    """A prompt run through gdp_prefill_prepare + gdp_chunk_fwd, then S tokens
    through gdp_decode_prepare + gdp_decode_update from its final state, gives
    the outputs (read on each token's last copy) and final state of the
    chunked forward over prompt plus the S tokens; and S one-token decode
    calls equal one S-token call bit for bit."""
    n, T0, S, M, H, G_, P, N = 3, 200, 3, 2, 4, 2, 128, 128
    d = synth.prepare_draws(n, T0 + S, M, H, G_, P, N, "bf16", synth.seed_of(3) + 70)
    x, ba, A_log, dt_bias = d["x"].to(DEV), d["ba"].to(DEV), d["A_log"].to(DEV), d["dt_bias"].to(DEV)
    full = G.chunk_fwd(*G.prefill_prepare(x, ba, A_log, dt_bias, M, H, G_, P, N), output_final_state=True)
    pre = G.chunk_fwd(*G.prefill_prepare(x[:, :T0], ba[:, :T0], A_log, dt_bias, M, H, G_, P, N),
                      output_final_state=True)
    state = pre.ht.clone()
    o = G.decode_update(*G.decode_prepare(x[:, T0:], ba[:, T0:], A_log, dt_bias, M, H, G_, P, N), state, M)
    state1 = pre.ht.clone()
    o1 = [G.decode_update(*G.decode_prepare(x[:, T0 + t:T0 + t + 1], ba[:, T0 + t:T0 + t + 1], A_log, dt_bias,
                                            M, H, G_, P, N), state1, M) for t in range(S)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(o1, 1), o) and torch.equal(state1, state)
    tol = TOL[torch.bfloat16]
    mo, ro, fin = metrics(f32(o[:, M - 1::M]), f32(full.o[:, T0:]))
    ms, rs, fin_s = metrics(state.cpu().numpy(), full.ht.cpu().numpy())
    log("decode after prefill: o max_abs %.3g rel_l2 %.3g; state max_abs %.3g rel_l2 %.3g" % (mo, ro, ms, rs))
    assert fin and fin_s and mo <= tol["max_abs"] and ro <= tol["rel_l2"] and rs <= tol["rel_l2"]
    assert torch.count_nonzero(o.reshape(n, S, M, -1)[:, :, :M - 1]) == 0


# ---------------------------------------------------------------------- graphs

def test_hip_graph_capture_replays():
    """Prefill prepare, the chunk forward (one stream, pipelined over the
    library's side streams, and segment-parallel) and a decode step from the
    prefill's final state, captured into one HIP graph over static buffers.  Before each replay the
    inputs are rewritten in place by eager work; every replay equals the
    eager calls on the same inputs bit for bit."""
    T, S, M, H, G_, P, N = 700, 2, 2, 4, 2, 128, 128
    draws = [synth.prepare_draws(1, T + S, M, H, G_, P, N, "bf16", synth.seed_of(4) + 80 + i) for i in range(3)]
    A_log, dt_bias = draws[0]["A_log"].to(DEV), draws[0]["dt_bias"].to(DEV)
    x, ba = draws[0]["x"].to(DEV), draws[0]["ba"].to(DEV)
    xp, bap, xd, bad = x[:, :T], ba[:, :T], x[:, T:], ba[:, T:]
    pre = G.prefill_prepare(xp, bap, A_log, dt_bias, M, H, G_, P, N)
    seq = G.ChunkBuffers(*pre, output_final_state=True)
    pip = G.ChunkBuffers(*pre, output_final_state=True)
    scn = G.ChunkBuffers(*pre, output_final_state=True)
    dec = G.decode_prepare(xd, bad, A_log, dt_bias, M, H, G_, P, N)
    dec_o = torch.empty((1, S * M, H, P), dtype=torch.bfloat16, device=DEV)
    # warm-up outside capture: the pipelined call creates its streams and events here
    seq.forward()
    pip.forward_pipelined(3)
    scn.forward_scan(4)  # and the scan workspace is allocated here
    G.decode_update(*dec, seq.ht, M, o=dec_o)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.prefill_prepare(xp, bap, A_log, dt_bias, M, H, G_, P, N, out=pre)
        seq.forward()
        pip.forward_pipelined(3)
        scn.forward_scan(4)
        G.decode_prepare(xd, bad, A_log, dt_bias, M, H, G_, P, N, out=dec)
        G.decode_update(*dec, seq.ht, M, o=dec_o)   # continues from the prefill state, in place
    for i in (1, 2, 0, 1):
        log("graph replay on draw %d" % i)
        x.copy_(draws[i]["x"].to(DEV))
        ba.copy_(draws[i]["ba"].to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        pre_ref = G.prefill_prepare(xp, bap, A_log, dt_bias, M, H, G_, P, N)
        ref_scn = G.ChunkBuffers(*pre_ref, output_final_state=True)
        ref_scn.forward_scan(4)
        ref = G.chunk_fwd(*pre_ref, output_final_state=True)
        ref_ht = ref.ht.clone()
        ref_o = G.decode_update(*G.decode_prepare(xd, bad, A_log, dt_bias, M, H, G_, P, N), ref.ht, M)
        torch.cuda.synchronize()
        for nm in ("o", "w", "u", "v_new", "h"):
            assert torch.equal(getattr(seq, nm), getattr(ref, nm)), "sequential " + nm
            assert torch.equal(getattr(pip, nm), getattr(ref, nm)), "pipelined " + nm
            got, want = getattr(scn, nm), getattr(ref_scn, nm)
            if nm == "h":  # the scan form writes only the states entering chunks c % M == 0
                got, want = got[::M], want[::M]
            assert torch.equal(got, want), "scan " + nm
        assert torch.equal(pip.ht, ref_ht), "pipelined ht"
        assert torch.equal(scn.ht, ref_scn.ht), "scan ht"
        assert torch.equal(dec_o, ref_o) and torch.equal(seq.ht, ref.ht), "decode"


# --------------------------------------------- segment-parallel state recurrence

H_MARK = 7.0  # a bf16 value no snapshot of these draws takes in every element


def _check_unwritten_h(buf, M, seqs=None):
    """The segment-parallel forward writes only the states entering chunks
    c % M == 0 of each sequence (c counted from the sequence's first chunk);
    every other slot must still hold the mark put there before.  seqs: the
    (batch, t0, t1, first chunk) list of packed requests (default: one
    sequence)."""
    if M == 1:
        return
    keep = torch.ones(buf.h.shape[0], dtype=torch.bool, device=buf.h.device)
    if seqs is None:
        keep[::M] = False
    else:
        for (_, t0, t1, hbase) in seqs:
            nc = math.ceil((t1 - t0) * M / 64)
            keep[hbase:hbase + nc:M] = False
    rest = buf.h[keep]
    assert bool((rest == H_MARK).all()), "a skipped state slot was written"
    written = buf.h[~keep]
    assert written.numel() == 0 or not bool((written == H_MARK).all()), "the written state slots were not written"


def _stage_events():
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for e in evs:
        e.record()  # creates the HIP event
    return evs


def _scan_buf(q, k, v, beta, g, nseg, h0=None, cu=None, seqs=None):
    buf = G.ChunkBuffers(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), None if g is None else g.to(DEV),
                         cu_seqlens=None if cu is None else torch.as_tensor(cu, dtype=torch.int32).to(DEV),
                         cu_seqlens_host=cu,
                         initial_state=None if h0 is None else h0.to(DEV), output_final_state=h0 is not None)
    buf.h.fill_(H_MARK)
    evs = _stage_events()
    buf.forward_scan(nseg, stage_events=evs)
    torch.cuda.synchronize()
    # the stages in order (a map stage with no map to compose may take ~0)
    assert all(evs[i].elapsed_time(evs[i + 1]) >= 0 for i in range(4))
    assert evs[2].elapsed_time(evs[3]) > 0 and evs[3].elapsed_time(evs[4]) > 0
    _check_unwritten_h(buf, buf.dims["M"], seqs)
    return buf


SCAN_CASES = [
    # B, T, H, HV, K, V, M, segments, seed, gated, long memory, h0
    (1, 1000, 2, 4, 128, 128, 2, 5, 31, True, False, True),
    (1, 1000, 2, 4, 128, 128, 2, 7, 32, True, True, True),
    (1, 1000, 2, 4, 128, 128, 2, 3, 33, False, False, False),
    (1, 700, 1, 2, 64, 128, 3, 4, 34, True, False, False),
    (1, 513, 2, 2, 128, 64, 1, 3, 35, True, True, True),
    (1, 300, 2, 2, 64, 64, 2, 64, 36, True, True, False),
    (1, 64, 1, 1, 128, 128, 4, 8, 37, True, False, True),
    # shorter than a chunk, one token past one, and a 1-token last segment
    (1, 1, 1, 1, 64, 64, 2, 4, 38, True, False, True),
    (1, 65, 2, 2, 128, 128, 2, 4, 39, True, True, True),
    (1, 129, 1, 2, 64, 128, 3, 3, 40, True, False, False),
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=["T%d-K%dV%d-M%d-s%d%s%s" % (c[1], c[4], c[5], c[6], c[7],
                                                                            "-long" if c[10] else "",
                                                                            "" if c[9] else "-ungated")
                                                  for c in SCAN_CASES])
def test_scan_forward_matches_oracle(case):
    """gdp_chunk_fwd_scan: every output of every head against the oracle
    (o, v_new, h, w, u and the final state), including long memory (|g| ~
    1e-3, so each segment's state depends on the composed maps of all earlier
    ones), M = 1, 3, 4, ragged tails, more segments asked than chunks, the
    ungated rule and an initial state; w, u and the per-row intermediates
    bit-identical to gdp_chunk_fwd, and so are h, v_new and o over the first
    segment."""
    B_, T, H, HV, K, V, M, nseg, seed, gated, longmem, with_h0 = case
    d = synth.chunk_draws(B_, T, H, HV, K, V, M, "bf16", seed)
    if longmem:
        d["dt_bias"] = torch.empty(HV).uniform_(-9, -7, generator=torch.Generator().manual_seed(seed))
    beta, g = gates(d)
    beta = beta.reshape(B_, T * M, HV)
    g = g if gated else None
    h0 = synth.initial_state_draws(1, HV, V, K, seed + 100) if with_h0 else None
    n = G.scan_segments(T, nseg)
    log("scan %s: %d segments" % (case, n))
    buf = _scan_buf(d["q"], d["k"], d["v"], beta, g, nseg, h0)
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(B_, T, M), range(HV), M, tag="scan", buf=buf, h0=h0,
                hstep=M)
    ref = G.chunk_fwd(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), beta.to(DEV),
                      None if g is None else g.to(DEV), initial_state=None if h0 is None else h0.to(DEV),
                      output_final_state=h0 is not None)
    torch.cuda.synchronize()
    for nm in ("w", "u", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(getattr(ref, nm), getattr(buf, nm)), nm
    seg_tok = ((T + 63) // 64 + nseg - 1) // nseg * 64
    t1 = min(T, seg_tok)
    c1 = (t1 * M + 63) // 64
    assert torch.equal(ref.o[:, :t1], buf.o[:, :t1])
    assert torch.equal(ref.h[:c1:M], buf.h[:c1:M])
    assert torch.equal(ref.v_new[..., :t1 * M, :], buf.v_new[..., :t1 * M, :])


@pytest.mark.parametrize("case", [(1000, 2, 4, 128, 128, 2, 7, 32), (700, 1, 2, 64, 128, 3, 4, 34),
                                  (700, 1, 2, 128, 128, 3, 4, 34), (300, 2, 2, 64, 64, 2, 64, 36)],
                         ids=lambda c: "T%d-K%dV%d-M%d-s%d" % (c[0], c[3], c[4], c[5], c[6]))
def test_scan_adds_no_error_long_memory(case):
    """Long memory (|g| ~ 1e-3): each segment's entering state comes from the
    composed maps of every earlier segment.  Against the oracle, o, h and
    v_new of both gdp_chunk_fwd and gdp_chunk_fwd_scan meet the tolerance
    (rel-L2 <= 5e-3, o max-abs <= 2e-2) and o's rel-L2 stays at or below
    4.2e-3, and the scan's error stays within 2% (plus 1e-5) of the
    sequential path's: composing the maps adds nothing measurable to the
    bf16 path's own error."""
    T, H, HV, K, V, M, nseg, seed = case
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", seed)
    d["dt_bias"] = torch.empty(HV).uniform_(-9, -7, generator=torch.Generator().manual_seed(seed))
    beta, g = gates(d)
    beta = beta.reshape(1, T * M, HV)
    args = [t.to(DEV) for t in (d["q"], d["k"], d["v"], beta, g)]
    seq = G.chunk_fwd(*args)
    sc = _scan_buf(d["q"], d["k"], d["v"], beta, g, nseg)
    err = {"seq": {}, "scan": {}}
    r2 = {}
    o_max = {"seq": 0.0, "scan": 0.0}
    nc = math.ceil(T * M / 64)
    for hv in range(HV):
        hk = hv // (HV // H)
        r = oracle_pair(f32(d["q"][0, :, hk]), f32(d["k"][0, :, hk]), f32(d["v"][0, :, hv]), f32(beta[0, :, hv]),
                        f32(g[0, :, hv]), M, 1.0 / math.sqrt(K), False)
        for nm in ("o", "h", "v_new"):
            r2[nm] = r2.get(nm, 0.0) + float(((r[nm][::M] if nm == "h" else r[nm]) ** 2).sum())
        for tag, b in (("seq", seq), ("scan", sc)):
            got = {"o": f32(b.o[0, :, hv]), "h": f32(b.h[:nc:M, hv]), "v_new": f32(G.slices_to_rows(b.v_new)[0, :, hv])}
            for nm, x in got.items():
                e = x.astype(np.float64) - (r[nm][::M] if nm == "h" else r[nm])
                err[tag][nm] = err[tag].get(nm, 0.0) + float((e * e).sum())
                if nm == "o":
                    o_max[tag] = max(o_max[tag], float(np.abs(e).max()))
    for nm in ("o", "h", "v_new"):
        es, ec = math.sqrt(err["seq"][nm] / r2[nm]), math.sqrt(err["scan"][nm] / r2[nm])
        log("  %-6s rel_l2 sequential %.4e scan %.4e" % (nm, es, ec))
        assert es <= TOL[torch.bfloat16]["rel_l2"] and ec <= TOL[torch.bfloat16]["rel_l2"], (nm, es, ec)
        assert ec <= 1.02 * es + 1e-5, (nm, ec, es)
        if nm == "o":
            assert es <= 4.2e-3 and ec <= 4.2e-3, ("o margin", es, ec)
    log("  o max_abs sequential %.3e scan %.3e" % (o_max["seq"], o_max["scan"]))
    assert o_max["seq"] <= TOL[torch.bfloat16]["max_abs"] and o_max["scan"] <= TOL[torch.bfloat16]["max_abs"]


def test_scan_long_prefill_sampled():
    """The timed workload (B=1, T=32768, H=HV=16, K=V=128, M=2) through
    gdp_chunk_fwd_scan with 16 segments, the launch configuration the
    benchmark times: the whole sequence on sampled heads against the oracle."""
    c = synth.CONFIGS[4]
    d, beta, g = _cfg_inputs(4)
    log("long_prefill scan: inputs drawn")
    buf = _scan_buf(d["q"], d["k"], d["v"], beta, g, 16)
    check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_equal(c["B"], c["T"], c["M"]), [0, 9, 15], c["M"],
                tag="long_prefill_32k scan", buf=buf, hstep=c["M"])


VARLEN_SCAN_CASES = [
    # lengths, H, HV, K, V, M, segments, seed, long memory, h0
    ([1000, 0, 1, 64, 65, 2500, 130, 700], 2, 4, 128, 128, 2, 8, 61, False, True),
    ([3000, 17, 1500], 1, 2, 64, 128, 3, 6, 62, True, False),
    ([200, 300, 129], 2, 2, 128, 64, 1, 4, 63, False, True),
    ([50, 60, 70], 1, 1, 64, 64, 2, 2, 64, False, True),  # every request shorter than a segment: no map
]


@pytest.mark.parametrize("case", VARLEN_SCAN_CASES, ids=lambda c: "n%d-K%dV%d-M%d-s%d%s" % (
    len(c[0]), c[3], c[4], c[5], c[6], "-long" if c[8] else ""))
def test_scan_varlen_matches_oracle(case):
    """gdp_chunk_fwd_scan on packed requests (cu_seqlens): each long request
    cut into segments on the device, short, 1-token and empty requests kept
    whole, GVA, M = 1..3, long memory, per-request initial and final states.
    Every output of every (request, head) against the oracle; w, u and the
    per-row intermediates bit-identical to gdp_chunk_fwd, and so are o and
    v_new over the first segment of each request."""
    lens, H, HV, K, V, M, nseg, seed, longmem, with_h0 = case
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", seed)
    if longmem:
        d["dt_bias"] = torch.empty(HV).uniform_(-9, -7, generator=torch.Generator().manual_seed(seed))
    beta, g = gates(d)
    beta = beta.reshape(1, T * M, HV)
    h0 = synth.initial_state_draws(len(lens), HV, V, K, seed + 100) if with_h0 else None
    seqs = _seqs_varlen(cu, M)
    seg_tok = ((T + 63) // 64 + nseg - 1) // nseg * 64 if T else 64
    log("varlen scan %s: T=%d, seg_tok %d, segments %s" % (lens, T, seg_tok, [-(-n // seg_tok) for n in lens]))
    buf = _scan_buf(d["q"], d["k"], d["v"], beta, g, nseg, h0, cu=cu, seqs=seqs)
    check_chunk(d["q"], d["k"], d["v"], beta, g, seqs, range(HV), M, cu=cu, cu_host=cu, tag="varlen scan",
                buf=buf, h0=h0, hstep=M)
    cu_d = torch.as_tensor(cu, dtype=torch.int32).to(DEV)
    ref = G.chunk_fwd(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), beta.to(DEV), g.to(DEV), cu_seqlens=cu_d,
                      cu_seqlens_host=cu, initial_state=None if h0 is None else h0.to(DEV),
                      output_final_state=h0 is not None)
    torch.cuda.synchronize()
    for nm in ("w", "u", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(ref.__dict__[nm], buf.__dict__[nm]), nm
    vn_ref, vn = G.slices_to_rows(ref.v_new), G.slices_to_rows(buf.v_new)
    for (_, t0, t1, _) in seqs:
        t1s = min(t1, t0 + seg_tok)
        assert torch.equal(ref.o[:, t0:t1s], buf.o[:, t0:t1s]), ("first segment o", t0)
        assert torch.equal(vn_ref[:, t0 * M:t1s * M], vn[:, t0 * M:t1s * M]), ("first segment v_new", t0)


def test_prefill_scan_varlen_workload():
    """The GVA varlen prefill workload (8 packed requests, lengths in [64,
    4096], prepare with 16 heads from 4 groups, M = 2) through
    gdp_prefill_fwd_scan: prepare's outputs and every chunk output
    bit-identical to gdp_prefill_prepare then gdp_chunk_fwd_scan on the same
    cu_seqlens, o against the oracle on sampled heads of every request, and
    the GVA form (H = 4 key heads, the pre-expansion groups) of
    gdp_chunk_fwd_scan equal to the expanded run."""
    c = synth.CONFIGS[3]
    p = c["prep"]
    M, nseg = c["M"], 16
    d = synth.varlen_prepare_draws(3)
    cu = d["cu_seqlens"]
    T = int(cu[-1])
    x, ba, A_log, dt_bias = d["x"].to(DEV), d["ba"].to(DEV), d["A_log"].to(DEV), d["dt_bias"].to(DEV)
    cu_d = torch.as_tensor(cu, dtype=torch.int32).to(DEV)
    pre = G.prefill_prepare(x, ba, A_log, dt_bias, M, p["H"], p["G"], p["P"], p["N"])
    ref = G.ChunkBuffers(*pre, cu_seqlens=cu_d, cu_seqlens_host=cu)
    ref.h.fill_(H_MARK)
    ref.forward_scan(nseg)
    outs = [torch.full_like(t, 7) for t in pre]
    fz = G.ChunkBuffers(*outs, cu_seqlens=cu_d, cu_seqlens_host=cu)
    fz.h.fill_(H_MARK)
    fz.prefill_scan(x, ba, A_log, dt_bias, p["G"], nseg, stage_events=_stage_events())
    torch.cuda.synchronize()
    for a_, b_, nm in zip(outs, pre, ("q", "k", "v", "beta", "g")):
        assert torch.equal(a_, b_), nm
    for nm in ("o", "w", "u", "v_new", "h", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(getattr(fz, nm), getattr(ref, nm)), nm
    seqs = _seqs_varlen(cu, M)
    _check_unwritten_h(fz, M, seqs)
    hpg = p["H"] // p["G"]
    q, k, v, beta, g = pre
    gva = G.ChunkBuffers(q[:, :, ::hpg].contiguous(), k[:, :, ::hpg].contiguous(), v, beta, g, cu_seqlens=cu_d,
                         cu_seqlens_host=cu)
    gva.forward_scan(nseg)
    torch.cuda.synchronize()
    for nm in ("o", "w", "u", "v_new"):
        assert torch.equal(getattr(gva, nm), getattr(ref, nm)), "GVA vs expanded: " + nm
    check_chunk(q.cpu(), k.cpu(), v.cpu(), beta.cpu(), g.cpu(), seqs, [0, 7, 15], M, cu=cu, cu_host=cu,
                tag="varlen prefill scan", buf=fz, hstep=M, want_wu=False)


def check_o(buf, q, k, v, beta, g, seqs, hv_list, M, tag, h0=None, scale=None):
    """o (and the final state when h0 is given) of every listed (sequence,
    value head) against the oracle, to the bf16 tolerance."""
    H, HV, K = q.shape[2], v.shape[2], q.shape[3]
    sc = scale if scale is not None else 1.0 / math.sqrt(K)
    items = [(si, s_, hv) for si, s_ in enumerate(seqs) for hv in hv_list if s_[2] > s_[1]]
    log("%s: %d (seq, head) pairs" % (tag, len(items)))

    def one(item):
        si, (b, t0, t1, _), hv = item
        hk = hv // (HV // H)
        return oracle_pair(f32(q[b, t0:t1, hk]), f32(k[b, t0 * M:t1 * M, hk]), f32(v[b, t0 * M:t1 * M, hv]),
                           f32(beta[b, t0 * M:t1 * M, hv]), None if g is None else f32(g[b, t0:t1, hv]), M, sc,
                           False, h0=None if h0 is None else h0[si, hv].double().numpy())

    refs = run_pairs(one, items)
    ao, ah = Acc("o", raw_max_abs=True), Acc("ht", raw_max_abs=True)
    for (si, (b, t0, t1, _), hv), r in zip(items, refs):
        ao.add(f32(buf.o[b, t0:t1, hv]), r["o"], True)
        if h0 is not None:
            ah.add(f32(buf.ht[si, hv]), r["h_final"], False)
    ao.check(TOL[torch.bfloat16])
    if h0 is not None:
        ah.check(TOL[torch.bfloat16])
    return ao.rel()


FUSED_CASES = [
    # lengths (None: one sequence of T), T, H, HV, K, V, M, segments, seed, gated, long memory, h0
    (None, 1000, 2, 4, 128, 128, 2, 5, 71, True, False, True),
    (None, 700, 1, 2, 64, 128, 3, 4, 72, True, True, False),
    (None, 513, 2, 2, 128, 64, 4, 3, 73, True, False, True),
    (None, 65, 2, 2, 128, 128, 2, 4, 74, True, True, True),
    (None, 300, 1, 2, 64, 64, 2, 64, 75, False, False, False),
    (None, 1, 1, 1, 64, 64, 3, 4, 79, True, False, True),
    ([1000, 0, 1, 64, 65, 2500, 130, 700], None, 2, 4, 128, 128, 2, 8, 76, True, False, True),
    ([3000, 17, 1500], None, 1, 2, 64, 128, 3, 6, 77, True, True, True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "%s-K%dV%d-M%d-s%d%s%s" % (
    "n%d" % len(c[0]) if c[0] else "T%d" % c[1], c[4], c[5], c[6], c[7], "-long" if c[10] else "",
    "" if c[9] else "-ungated"))
def test_scan_fused_output_matches_oracle(case):
    """gdp_chunk_fwd_scan with v_new and h passed as NULL: chunk_h and chunk_o
    as one pass.  o and the final states against the oracle on every
    (sequence, head); the final states bit-identical to the two-stage scan
    form (the fused pass runs the same state arithmetic), w, u and the per-row
    intermediates too, and v_new and h left untouched."""
    lens, T, H, HV, K, V, M, nseg, seed, gated, longmem, with_h0 = case
    cu = None
    if lens is not None:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(cu[-1])
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", seed)
    if longmem:
        d["dt_bias"] = torch.empty(HV).uniform_(-9, -7, generator=torch.Generator().manual_seed(seed))
    beta, g = gates(d)
    beta = beta.reshape(1, T * M, HV)
    g = g if gated else None
    nseq = 1 if cu is None else len(lens)
    h0 = synth.initial_state_draws(nseq, HV, V, K, seed + 100) if with_h0 else None
    seqs = _seqs_equal(1, T, M) if cu is None else _seqs_varlen(cu, M)
    cu_d = None if cu is None else torch.as_tensor(cu, dtype=torch.int32).to(DEV)
    mk = lambda: G.ChunkBuffers(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), beta.to(DEV),
                                None if g is None else g.to(DEV), cu_seqlens=cu_d, cu_seqlens_host=cu,
                                initial_state=None if h0 is None else h0.to(DEV), output_final_state=h0 is not None)
    fz, ref = mk(), mk()
    fz.h.fill_(H_MARK)
    fz.v_new.fill_(H_MARK)
    fz.forward_scan(nseg, stage_events=_stage_events(), store_vnew_h=False)
    ref.forward_scan(nseg)
    torch.cuda.synchronize()
    assert bool((fz.h == H_MARK).all()) and bool((fz.v_new == H_MARK).all()), "v_new or h was written"
    for nm in ("w", "u", "k_rnorm", "gcum", "kdecay") + (("ht",) if h0 is not None else ()):
        assert torch.equal(getattr(fz, nm), getattr(ref, nm)), nm
    rel = check_o(fz, d["q"], d["k"], d["v"], beta, g, seqs, range(HV), M, "fused scan", h0=h0)
    if longmem:
        assert rel <= 4.2e-3, rel
    # the two-stage form's o, for scale: the two differ by rounding only
    diff = (fz.o.float() - ref.o.float()).norm() / ref.o.float().norm()
    log("  fused vs two-stage o: rel-L2 %.3e" % float(diff))
    assert float(diff) <= 5e-3


@pytest.mark.parametrize("B_,T,H,HV,K,V,M,seed", [(2, 600, 2, 4, 128, 256, 3, 81), (3, 200, 1, 1, 64, 256, 2, 82),
                                                  (2, 300, 2, 2, 128, 64, 4, 83)])
def test_chunk_fwd_fused_output_matches_oracle(B_, T, H, HV, K, V, M, seed):
    """gdp_chunk_fwd with v_new and h passed as NULL (B > 1 rows, V = 256):
    o and the final states against the oracle, the final states and w, u
    bit-identical to the two-stage call."""
    d = synth.chunk_draws(B_, T, H, HV, K, V, M, "bf16", seed, a_sigma=3.0 if seed == 81 else 1.0,
                          plant_edges=seed == 81)
    beta, g = gates(d)
    beta = beta.reshape(B_, T * M, HV)
    h0 = synth.initial_state_draws(B_, HV, V, K, seed + 100)
    mk = lambda: G.ChunkBuffers(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), beta.to(DEV), g.to(DEV),
                                initial_state=h0.to(DEV), output_final_state=True)
    fz, ref = mk(), mk()
    fz.forward(store_vnew_h=False)
    ref.forward()
    torch.cuda.synchronize()
    for nm in ("w", "u", "ht"):
        assert torch.equal(getattr(fz, nm), getattr(ref, nm)), nm
    check_o(fz, d["q"], d["k"], d["v"], beta, g, _seqs_equal(B_, T, M), range(HV), M, "fused chunk_fwd", h0=h0)


def test_prefill_scan_fused_long_prefill_sampled():
    """The timed configuration: gdp_prefill_fwd_scan at B=1, T=32768,
    H=HV=16, K=V=128, M=2, 16 segments, with v, beta, v_new and h all NULL
    (prepare in WY, chunk_h and chunk_o in one pass): prepare's stored outputs
    equal gdp_prefill_prepare's, the final state equals the two-stage scan's
    bit for bit, and o of sampled heads against the oracle run on the
    oracle's prepare output."""
    c = synth.CONFIGS[4]
    M, H, T = c["M"], c["HV"], c["T"]
    d = synth.prepare_draws(1, T, M, H, H, c["V"], c["K"], "bf16", synth.seed_of(4) + 100)
    x, ba, A_log, dt_bias = d["x"].to(DEV), d["ba"].to(DEV), d["A_log"].to(DEV), d["dt_bias"].to(DEV)
    pre = G.prefill_prepare(x, ba, A_log, dt_bias, M, H, H, c["V"], c["K"])
    h0 = synth.initial_state_draws(1, H, c["V"], c["K"], 91).to(DEV)
    ref = G.ChunkBuffers(*pre, initial_state=h0, output_final_state=True)
    ref.forward_scan(16)
    fz = G.ChunkBuffers(*[torch.full_like(t, 7) for t in pre], initial_state=h0, output_final_state=True)
    fz.prefill_scan(x, ba, A_log, dt_bias, H, 16, store_v_beta=False, store_vnew_h=False)
    torch.cuda.synchronize()
    for nm in ("q", "k", "g"):
        assert torch.equal(getattr(fz, nm), getattr(ref, nm)), nm
    for nm in ("w", "u", "ht", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(getattr(fz, nm), getattr(ref, nm)), nm
    xs, bas = f32(d["x"][0]), f32(d["ba"][0])
    P_, N_ = c["V"], c["K"]
    for hv in (0, 11):
        vh = np.ascontiguousarray(xs[:, : M * H * P_].reshape(T, M, H, P_)[:, :, hv].reshape(T * M, P_))
        kh = np.ascontiguousarray(xs[:, M * H * P_: M * H * P_ + M * H * N_].reshape(T, M, H, N_)[:, :, hv]
                                  .reshape(T * M, N_))
        qh = np.ascontiguousarray(xs[:, M * H * P_ + M * H * N_:].reshape(T, H, N_)[:, hv])
        bh = OP.sigmoid_rn32(bas[:, : M * H].reshape(T, M, H)[:, :, hv].reshape(T * M))
        gh = OP.decay_rn32(bas[:, M * H + hv], d["A_log"].numpy()[hv], d["dt_bias"].numpy()[hv])
        r = oracle.recurrence(qh, kh, vh, bh, np.ascontiguousarray(gh), M, scale=1.0 / math.sqrt(N_),
                              h0=h0[0, hv].double().cpu().numpy())
        a = Acc("o[%d]" % hv, raw_max_abs=True)
        a.add(f32(fz.o[0, :, hv]), r["o"])
        a.check(TOL[torch.bfloat16])


@pytest.mark.parametrize("K,V,M,n", [(128, 128, 2, 64), (64, 256, 3, 64), (128, 64, 1, 64), (128, 128, 2, 12)])
def test_chunk_h_two_pairs_per_block(K, V, M, n):
    """With many chains (packed requests x 16 value heads) chunk_h runs
    several 16-column slices per block: two (two waves per slice, one per K
    half) for V = 64 and for 12 requests at V = 128, four (one wave per
    slice holding the whole K) for 64 requests at V >= 128.  Its outputs are
    bit-identical to the same requests run one call each (one slice per
    block), and match the oracle on every (request, head), final states
    included; every request starts from a given state; the requests include
    empty and one-token ones and ragged tails."""
    H, HV = 4, 16
    rng = np.random.default_rng(900 + K + V + M)
    lens = rng.integers(1, 90, size=n)
    lens[[3, 17 if n > 17 else n - 2]] = 0
    lens[5] = 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", synth.seed_of(3) + K + V + M)
    beta, g = gates(d)
    beta = beta.reshape(1, T * M, HV)
    h0 = synth.initial_state_draws(n, HV, V, K, synth.seed_of(3) + K + V + M + 1)
    buf = check_chunk(d["q"], d["k"], d["v"], beta, g, _seqs_varlen(cu, M), range(HV), M, cu=cu, cu_host=cu,
                      tag="two pairs K%d V%d M%d" % (K, V, M), h0=h0)
    vn_rows = G.slices_to_rows(buf.v_new)
    hbase = 0
    for i in range(n):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        if t1 == t0:
            continue
        one = G.chunk_fwd(d["q"][:, t0:t1].contiguous().to(DEV), d["k"][:, t0 * M:t1 * M].contiguous().to(DEV),
                          d["v"][:, t0 * M:t1 * M].contiguous().to(DEV),
                          beta[:, t0 * M:t1 * M].contiguous().to(DEV), g[:, t0:t1].contiguous().to(DEV),
                          initial_state=h0[i:i + 1].contiguous().to(DEV), output_final_state=True)
        torch.cuda.synchronize()
        nc = math.ceil((t1 - t0) * M / 64)
        assert torch.equal(one.ht[0], buf.ht[i]), i
        assert torch.equal(one.o[0], buf.o[0, t0:t1]), i
        assert torch.equal(G.slices_to_rows(one.v_new)[0], vn_rows[0, t0 * M:t1 * M]), i
        assert torch.equal(one.h, buf.h[hbase:hbase + nc]), i
        hbase += nc


@pytest.mark.parametrize("case", [(1000, 2, 4, 2, 128, 128, 5), (700, 3, 2, 1, 64, 64, 4), (513, 1, 4, 4, 128, 64, 3),
                                  (1, 2, 2, 1, 64, 64, 4), (65, 4, 2, 2, 128, 128, 2),
                                  (32768, 2, 16, 16, 128, 128, 16)],
                         ids=lambda c: "T%d-M%d-H%d-G%d-P%d-N%d-s%d" % c)
def test_prefill_scan_is_bit_identical(case):
    """gdp_prefill_fwd_scan (prepare done inside the WY stage) gives exactly
    the outputs of gdp_prefill_prepare then gdp_chunk_fwd_scan: q, k, v, beta,
    g and every chunk output, with an initial state, ragged tails, M = 1..3,
    GQA groups, and the timed workload (T = 32768, 16 heads, 16 segments).
    With v and beta passed as NULL they stay untouched and nothing else
    changes; in the one chunk_h + chunk_o pass the same holds for q and k,
    whose rows the later stages then read from x."""
    T, M, H, G_, P, N, nseg = case
    d = synth.prepare_draws(1, T, M, H, G_, P, N, "bf16", synth.seed_of(4) + 300 + T % 97)
    x, ba, A_log, dt_bias = d["x"].to(DEV), d["ba"].to(DEV), d["A_log"].to(DEV), d["dt_bias"].to(DEV)
    pre = G.prefill_prepare(x, ba, A_log, dt_bias, M, H, G_, P, N)
    h0 = synth.initial_state_draws(1, H, P, N, synth.seed_of(4) + 301).to(DEV)
    ref = G.ChunkBuffers(*pre, initial_state=h0, output_final_state=True)
    ref.h.fill_(H_MARK)
    ref.forward_scan(nseg)
    outs = [torch.full_like(t, 7) for t in pre]  # the fused prepare must overwrite all of them
    fz = G.ChunkBuffers(*outs, initial_state=h0, output_final_state=True)
    fz.h.fill_(H_MARK)  # the slots neither call writes then match as well
    fz.prefill_scan(x, ba, A_log, dt_bias, G_, nseg, stage_events=_stage_events())
    torch.cuda.synchronize()
    for a_, b_, nm in zip(outs, pre, ("q", "k", "v", "beta", "g")):
        assert torch.equal(a_, b_), nm
    for nm in ("o", "w", "u", "v_new", "h", "ht", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(getattr(fz, nm), getattr(ref, nm)), nm
    _check_unwritten_h(fz, M)
    # v and beta passed as NULL: not stored, every other output unchanged
    outs2 = [torch.full_like(t, 7) for t in pre]
    nv = G.ChunkBuffers(*outs2, initial_state=h0, output_final_state=True)
    nv.h.fill_(H_MARK)
    nv.prefill_scan(x, ba, A_log, dt_bias, G_, nseg, store_v_beta=False)
    torch.cuda.synchronize()
    for a_, b_, nm in zip(outs2, pre, ("q", "k", "v", "beta", "g")):
        if nm in ("v", "beta"):
            assert bool((a_ == 7).all()), nm + " was written"
        else:
            assert torch.equal(a_, b_), nm
    for nm in ("o", "w", "u", "v_new", "h", "ht", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(getattr(nv, nm), getattr(ref, nm)), "without v, beta: " + nm
    if M < 2:
        return  # the one-pass chunk_h + chunk_o form needs M >= 2
    # one chunk_h + chunk_o pass: with q and k not stored (their rows read
    # from x by the later stages) every output equals the run that stores
    # them, and q and k stay untouched
    runs = []
    for store_qk in (True, False):
        o3 = [torch.full_like(t, 7) for t in pre]
        b3 = G.ChunkBuffers(*o3, initial_state=h0, output_final_state=True)
        b3.prefill_scan(x, ba, A_log, dt_bias, G_, nseg, store_v_beta=False, store_vnew_h=False, store_qk=store_qk)
        torch.cuda.synchronize()
        runs.append((o3, b3))
    (oq, bq), (ox, bx) = runs
    for a_, b_, nm in zip(ox, pre, ("q", "k", "v", "beta", "g")):
        if nm in ("q", "k", "v", "beta"):
            assert bool((a_ == 7).all()), nm + " was written"
        else:
            assert torch.equal(a_, b_), nm
    assert torch.equal(oq[0], pre[0]) and torch.equal(oq[1], pre[1]), "q, k stored"
    for nm in ("o", "w", "u", "ht", "k_rnorm", "gcum", "kdecay"):
        assert torch.equal(getattr(bx, nm), getattr(bq, nm)), "q, k read from x: " + nm
