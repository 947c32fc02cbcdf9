// api.cpp -- the C ABI declared in include/gdp.h: argument validation,
// error reporting and kernel launches on the caller's stream.  No device
// memory allocation and no synchronisation with the host; the pipelined
// forward creates two side streams and its events once per device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "gdp_internal.h"

namespace {

thread_local std::string g_err;

gdp_status fail(gdp_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

gdp_status ok() {
    g_err.clear();
    return GDP_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t dsize(gdp_dtype d) { return d == GDP_BF16 ? 2 : 4; }

gdp_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(GDP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Stage masks for validation.
// stages of a call; ST_WYP is WY with the prepare fused in, which takes its
// values and beta from the activations, so it needs neither tensor
// ST_HO is chunk_h and chunk_o as one pass, which stores neither v_new nor h
// ST_QKX: q and k are read from the activations (the fused prefill that
// does not store them), so neither tensor is needed
enum : unsigned { ST_WY = 1u, ST_H = 2u, ST_O = 4u, ST_WYP = 8u, ST_HO = 16u, ST_QKX = 32u };

gdp_status check_chunk(const gdp_chunk_args *a, unsigned stages, gdp::ChunkParams *out) {
    if (!a) return fail(GDP_ERR_INVALID, "args is NULL");
    if (a->dtype != GDP_F32 && a->dtype != GDP_BF16) return fail(GDP_ERR_INVALID, "unknown dtype %d", (int)a->dtype);
    if (a->B < 0 || a->T < 0) return fail(GDP_ERR_INVALID, "B and T must be >= 0 (B=%lld T=%lld)",
                                          (long long)a->B, (long long)a->T);
    if (a->H < 1 || a->HV < 1) return fail(GDP_ERR_INVALID, "H and HV must be >= 1");
    if (a->HV % a->H) return fail(GDP_ERR_INVALID, "HV (%d) must be a multiple of H (%d)", a->HV, a->H);
    if (a->HV > 65535) return fail(GDP_ERR_UNSUPPORTED, "HV > 65535");
    if (a->M < 1 || a->M > 4) return fail(GDP_ERR_UNSUPPORTED, "num_householder M=%d not in [1, 4]", a->M);
    if (a->chunk_size != 64) return fail(GDP_ERR_UNSUPPORTED, "chunk_size %d: only 64 is built", a->chunk_size);
    if (a->dtype == GDP_BF16) {
        if (!(a->K == 64 || a->K == 128)) return fail(GDP_ERR_UNSUPPORTED, "K=%d: bf16 supports 64, 128", a->K);
        if (!(a->V == 64 || a->V == 128 || a->V == 256))
            return fail(GDP_ERR_UNSUPPORTED, "V=%d: bf16 supports 64, 128, 256", a->V);
    } else {
        if (a->K != 64 || !(a->V == 64 || a->V == 128))
            return fail(GDP_ERR_UNSUPPORTED, "f32 supports K=64 with V in {64, 128} (K=%d V=%d)", a->K, a->V);
    }
    if (!std::isfinite(a->scale)) return fail(GDP_ERR_INVALID, "scale is not finite");
    if (a->cu_seqlens) {
        if (a->B != 1) return fail(GDP_ERR_INVALID, "cu_seqlens requires B == 1 (got %lld)", (long long)a->B);
        if (a->num_seqs < 0) return fail(GDP_ERR_INVALID, "num_seqs < 0");
    }
    if (a->h_chunks < 0) return fail(GDP_ERR_INVALID, "h_chunks < 0");

    const int64_t T = a->T;
    const int64_t nseq = a->cu_seqlens ? a->num_seqs : a->B;
    const int64_t per_seq = cdiv(T * a->M, 64);
    const int64_t max_items = a->cu_seqlens ? (nseq > 0 ? per_seq + nseq : 0) : a->B * per_seq;
    const int64_t max_tok = a->cu_seqlens ? (nseq > 0 ? cdiv(T, 64) + nseq : 0) : a->B * cdiv(T, 64);
    if (max_items > 0x7fffffff || max_tok > 0x7fffffff || nseq * a->HV * 16 > 0x7fffffff)
        return fail(GDP_ERR_UNSUPPORTED, "problem too large for one launch");
    if (!a->cu_seqlens && (stages & (ST_H | ST_O)) && a->h_chunks < a->B * per_seq)
        return fail(GDP_ERR_INVALID, "h_chunks %lld < required %lld", (long long)a->h_chunks,
                    (long long)(a->B * per_seq));

    const bool empty = (T == 0 || nseq == 0);
    struct Need {
        unsigned stages;
        const void *p;
        const char *name;
        bool qk;  // q or k
    } needs[] = {
        {ST_O | ST_HO, a->q, "q", true},   {ST_WY | ST_WYP | ST_H | ST_O | ST_HO, a->k, "k", true},
        {ST_WY, a->v, "v", false},         {ST_WY, a->beta, "beta", false},
        {ST_WY | ST_WYP | ST_O | ST_HO, a->k_rnorm, "k_rnorm", false},
        {ST_WY | ST_WYP | ST_H | ST_HO, a->gcum, "gcum", false},
        {ST_WY | ST_WYP | ST_H | ST_HO, a->kdecay, "kdecay", false},
        {ST_WY | ST_WYP | ST_H | ST_HO, a->w, "w", false},   {ST_WY | ST_WYP | ST_H | ST_HO, a->u, "u", false},
        {ST_H | ST_O, a->v_new, "v_new", false},
        {ST_H | ST_O, a->h, "h", false},    {ST_O | ST_HO, a->o, "o", false},
    };
    if (!empty) {
        for (const Need &n : needs) {
            if (!(n.stages & stages)) continue;
            if ((stages & ST_QKX) && n.qk) continue;  // read from the activations
            if (!n.p) return fail(GDP_ERR_INVALID, "%s is NULL", n.name);
            if (!aligned16(n.p)) return fail(GDP_ERR_INVALID, "%s is not 16-byte aligned", n.name);
        }
    }
    // optional tensors: g (NULL = ungated), h0, ht
    const struct {
        const void *p;
        const char *name;
    } opt[] = {{a->g, "g"}, {a->h0, "h0"}, {a->ht, "ht"}};
    for (const auto &o : opt)
        if (o.p && !aligned16(o.p)) return fail(GDP_ERR_INVALID, "%s is not 16-byte aligned", o.name);
    out->a = *a;
    if (!(out->a.scale > 0.f)) out->a.scale = 1.0f / std::sqrt((float)a->K);
    out->nseq = empty ? 0 : nseq;
    out->max_items = empty ? 0 : max_items;
    out->max_tok_chunks = empty ? 0 : max_tok;
    out->uv_ss = T * a->M * 16;
    out->qk = gdp::QKRows{a->k, a->q, (int64_t)a->M * a->H * a->K, (int64_t)a->H * a->K, (int64_t)a->H * a->K,
                          (int64_t)a->K, 1};
    return ok();
}

}  // namespace

namespace gdp {

// Side streams and events of the pipelined forward, created once per device
// and kept for the life of the process.
struct PipeCtx {
    hipStream_t side[2] = {nullptr, nullptr};  // [0]: recompute_w_u, [1]: chunk_o
    std::vector<hipEvent_t> ev;
};
static std::mutex g_pipe_mu;
static PipeCtx g_pipe[64];

static hipError_t pipe_ctx(int dev, size_t nev, PipeCtx *&out) {
    PipeCtx &c = g_pipe[dev];
    for (int i = 0; i < 2; ++i)
        if (!c.side[i]) {
            hipError_t e = hipStreamCreateWithFlags(&c.side[i], hipStreamNonBlocking);
            if (e != hipSuccess) return e;
        }
    while (c.ev.size() < nev) {
        hipEvent_t ev;
        // every consumer is on this device: a device-scope release suffices,
        // and skips the system-scope cache writeback of a default event
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventReleaseToDevice);
        if (e != hipSuccess) return e;
        c.ev.push_back(ev);
    }
    out = &c;
    return hipSuccess;
}

}  // namespace gdp

extern "C" {

// Validates the arguments of a prepare call; on GDP_OK, *out holds the launch
// parameters (out->n == 0 or out->T == 0: nothing to launch).
static gdp_status prepare_check(const char *name, bool decode, const void *x, int64_t x_n_stride,
                                int64_t x_t_stride, const void *ba, int64_t ba_n_stride, int64_t ba_t_stride,
                                const float *A_log, const float *dt_bias, int64_t n, int64_t T, int32_t M,
                                int32_t H, int32_t G, int32_t P, int32_t N, gdp_dtype dtype, void *q, void *k,
                                void *v, float *beta, float *g, gdp::PrepareParams *out,
                                bool vb_optional = false, bool qk_optional = false) {
    *out = gdp::PrepareParams{};
    if (dtype != GDP_F32 && dtype != GDP_BF16) return fail(GDP_ERR_INVALID, "%s: unknown dtype %d", name, (int)dtype);
    if (n < 0 || T < 0) return fail(GDP_ERR_INVALID, "%s: n and T must be >= 0", name);
    if (M < 1 || H < 1 || G < 1 || P < 1 || N < 1) return fail(GDP_ERR_INVALID, "%s: M, H, G, P, N must be >= 1", name);
    if (H % G) return fail(GDP_ERR_INVALID, "%s: num_heads H=%d must be a multiple of num_groups G=%d", name, H, G);
    if (n > 65535 || T > 0x7fffffff) return fail(GDP_ERR_UNSUPPORTED, "%s: n or T too large for one launch", name);
    const int64_t width = (int64_t)M * H * P + (int64_t)M * G * N + (int64_t)G * N;
    if (width * M > 0x7fffffff) return fail(GDP_ERR_UNSUPPORTED, "%s: rows too wide", name);
    if (x_t_stride < 0 || x_n_stride < 0 || ba_t_stride < 0 || ba_n_stride < 0)
        return fail(GDP_ERR_INVALID, "%s: strides must be >= 0", name);
    if (n == 0 || T == 0) return ok();  // *out stays empty
    if (!x || !ba || !A_log || !dt_bias || (!q && !qk_optional) || (!k && !qk_optional) || (!v && !vb_optional) ||
        (!beta && !vb_optional) || !g)
        return fail(GDP_ERR_INVALID, "%s: a tensor pointer is NULL", name);
    if (T > 1 && x_t_stride < width) return fail(GDP_ERR_INVALID, "%s: x rows overlap (t stride %lld < width %lld)",
                                                 name, (long long)x_t_stride, (long long)width);
    if (T > 1 && ba_t_stride < (int64_t)M * H + H) return fail(GDP_ERR_INVALID, "%s: ba rows overlap", name);
    const size_t es = dsize(dtype);
    const bool vec16 = aligned16(x) && aligned16(q) && aligned16(k) && aligned16(v) &&
                       ((x_t_stride * es) % 16 == 0) && ((x_n_stride * es) % 16 == 0) &&
                       ((P * es) % 16 == 0) && ((N * es) % 16 == 0);
    *out = gdp::PrepareParams{x, x_n_stride, x_t_stride, ba, ba_n_stride, ba_t_stride, A_log, dt_bias, n, T,
                              M, H, G, P, N, dtype, decode, vec16, q, k, v, beta, g};
    return ok();
}

static gdp_status prepare_common(const char *name, bool decode, const void *x, int64_t x_n_stride,
                                 int64_t x_t_stride, const void *ba, int64_t ba_n_stride, int64_t ba_t_stride,
                                 const float *A_log, const float *dt_bias, int64_t n, int64_t T, int32_t M,
                                 int32_t H, int32_t G, int32_t P, int32_t N, gdp_dtype dtype, void *q, void *k,
                                 void *v, float *beta, float *g, void *stream) {
    gdp::PrepareParams p;
    const gdp_status st = prepare_check(name, decode, x, x_n_stride, x_t_stride, ba, ba_n_stride, ba_t_stride,
                                        A_log, dt_bias, n, T, M, H, G, P, N, dtype, q, k, v, beta, g, &p);
    if (st != GDP_OK || p.n == 0 || p.T == 0) return st;
    return hip_status(gdp::launch_prepare(p, (hipStream_t)stream), name);
}

gdp_status gdp_prefill_prepare(const void *x, int64_t x_n_stride, int64_t x_t_stride, const void *ba,
                               int64_t ba_n_stride, int64_t ba_t_stride, const float *A_log,
                               const float *dt_bias, int64_t n, int64_t T, int32_t M, int32_t H, int32_t G,
                               int32_t P, int32_t N, gdp_dtype dtype, void *q, void *k, void *v, float *beta,
                               float *g, void *stream) {
    return prepare_common("gdp_prefill_prepare", false, x, x_n_stride, x_t_stride, ba, ba_n_stride, ba_t_stride,
                          A_log, dt_bias, n, T, M, H, G, P, N, dtype, q, k, v, beta, g, stream);
}

gdp_status gdp_decode_prepare(const void *x, int64_t x_n_stride, int64_t x_t_stride, const void *ba,
                              int64_t ba_n_stride, int64_t ba_t_stride, const float *A_log,
                              const float *dt_bias, int64_t n, int64_t S, int32_t M, int32_t H, int32_t G,
                              int32_t P, int32_t N, gdp_dtype dtype, void *q, void *k, void *v, float *beta,
                              float *g, void *stream) {
    return prepare_common("gdp_decode_prepare", true, x, x_n_stride, x_t_stride, ba, ba_n_stride, ba_t_stride,
                          A_log, dt_bias, n, S, M, H, G, P, N, dtype, q, k, v, beta, g, stream);
}

gdp_status gdp_decode_update(const gdp_decode_args *a, void *stream) {
    if (!a) return fail(GDP_ERR_INVALID, "args is NULL");
    if (a->dtype != GDP_F32 && a->dtype != GDP_BF16) return fail(GDP_ERR_INVALID, "unknown dtype %d", (int)a->dtype);
    if (a->n < 0 || a->S < 0) return fail(GDP_ERR_INVALID, "n and S must be >= 0");
    if (a->H < 1 || a->HV < 1 || a->HV % a->H) return fail(GDP_ERR_INVALID, "HV must be a positive multiple of H");
    if (a->M < 1 || a->M > 4) return fail(GDP_ERR_UNSUPPORTED, "num_householder M=%d not in [1, 4]", a->M);
    if (!(a->K == 64 || a->K == 128) || !(a->V == 64 || a->V == 128 || a->V == 256))
        return fail(GDP_ERR_UNSUPPORTED, "head dims K=%d, V=%d not built (K in {64, 128}, V in {64, 128, 256})",
                    a->K, a->V);
    if (!std::isfinite(a->scale)) return fail(GDP_ERR_INVALID, "scale is not finite");
    if (a->n > 0x7fffffff || a->HV > 65535 || a->S * a->M > 4096)
        return fail(GDP_ERR_UNSUPPORTED, "decode step too large (n, HV or S*M)");
    if (a->pool < 0 || (!a->slots && a->pool < a->n)) return fail(GDP_ERR_INVALID, "state pool too small");
    if (a->n == 0 || a->S == 0) return ok();
    const struct {
        const void *p;
        const char *name;
    } need[] = {{a->q, "q"}, {a->k, "k"}, {a->v, "v"}, {a->beta, "beta"}, {a->state, "state"}, {a->o, "o"}};
    for (const auto &t : need) {
        if (!t.p) return fail(GDP_ERR_INVALID, "%s is NULL", t.name);
        if (!aligned16(t.p)) return fail(GDP_ERR_INVALID, "%s is not 16-byte aligned", t.name);
    }
    gdp_decode_args d = *a;
    if (!(d.scale > 0.f)) d.scale = 1.0f / std::sqrt((float)a->K);
    return hip_status(gdp::launch_decode(d, (hipStream_t)stream), "gdp_decode_update launch");
}

gdp_status gdp_recompute_w_u(const gdp_chunk_args *a, void *stream) {
    gdp::ChunkParams p;
    gdp_status st = check_chunk(a, ST_WY, &p);
    if (st != GDP_OK) return st;
    return hip_status(gdp::launch_wy(p, (hipStream_t)stream), "gdp_recompute_w_u launch");
}

gdp_status gdp_chunk_h(const gdp_chunk_args *a, void *stream) {
    gdp::ChunkParams p;
    gdp_status st = check_chunk(a, ST_H, &p);
    if (st != GDP_OK) return st;
    return hip_status(gdp::launch_chunk_h(p, (hipStream_t)stream), "gdp_chunk_h launch");
}

gdp_status gdp_chunk_o(const gdp_chunk_args *a, void *stream) {
    gdp::ChunkParams p;
    gdp_status st = check_chunk(a, ST_O, &p);
    if (st != GDP_OK) return st;
    return hip_status(gdp::launch_chunk_o(p, (hipStream_t)stream), "gdp_chunk_o launch");
}

gdp_status gdp_chunk_fwd(const gdp_chunk_args *a, void *stream) {
    gdp::ChunkParams p;
    hipStream_t s = (hipStream_t)stream;
    if (a && a->v_new == nullptr && a->h == nullptr) {  // chunk_h and chunk_o as one pass
        gdp_status st = check_chunk(a, ST_WY | ST_HO, &p);
        if (st != GDP_OK || p.nseq == 0) return st;  // (nothing to launch for an empty problem)
        if (a->M < 2 || a->dtype != GDP_BF16)
            return fail(GDP_ERR_UNSUPPORTED, "gdp_chunk_fwd: v_new and h may be NULL only for bf16 with M >= 2");
        if ((st = hip_status(gdp::launch_wy(p, s), "gdp_chunk_fwd: recompute_w_u launch")) != GDP_OK) return st;
        return hip_status(gdp::launch_chunk_ho(p, s), "gdp_chunk_fwd: chunk_h+o launch");
    }
    gdp_status st = check_chunk(a, ST_WY | ST_H | ST_O, &p);
    if (st != GDP_OK) return st;
    if ((st = hip_status(gdp::launch_wy(p, s), "gdp_chunk_fwd: recompute_w_u launch")) != GDP_OK) return st;
    if ((st = hip_status(gdp::launch_chunk_h(p, s), "gdp_chunk_fwd: chunk_h launch")) != GDP_OK) return st;
    return hip_status(gdp::launch_chunk_o(p, s), "gdp_chunk_fwd: chunk_o launch");
}

// Segment plan of the pipelined forward: num_segments equal shares of the
// 64-token chunks, each boundary rounded to a whole chunk, empty segments
// dropped.  (Shorter first and last segments, whose recompute_w_u and chunk_o
// overlap nothing, measured no faster: the step is bound by the memory
// traffic of all stages together.)  Fills starts[0..n] (token offsets,
// starts[n] = T) when starts is not NULL and returns n, the segment count.
static int32_t segment_plan(int64_t T, int32_t num_segments, int64_t *starts) {
    const int64_t nch = cdiv(T, 64);
    int32_t n = 0;
    int64_t prev = 0;
    if (starts) starts[0] = 0;
    for (int64_t i = 1; i <= num_segments; ++i) {
        const int64_t end = (nch * i + num_segments / 2) / num_segments;  // in chunks, rounded
        if (end <= prev) continue;
        prev = end;
        ++n;
        if (starts) starts[n] = end * 64 < T ? end * 64 : T;
    }
    return n;
}

int32_t gdp_pipeline_segments(int64_t T, int32_t num_segments) {
    if (T < 0 || num_segments < 1) return -1;
    return segment_plan(T, num_segments, nullptr);
}

int32_t gdp_pipeline_plan(int64_t T, int32_t num_segments, int64_t *starts) {
    if (T < 0 || num_segments < 1 || !starts) return -1;
    return segment_plan(T, num_segments, starts);
}

// The pipelined chunk forward; with prep, each segment's prepare runs right
// before that segment's WY, on the same stream.
static gdp_status pipelined_impl(const gdp_chunk_args *a, const gdp::PrepareParams *prep, int32_t num_segments,
                                 float *state_workspace, void *const *chunk_h_events, void *stream) {
    gdp::ChunkParams p;
    gdp_status st = check_chunk(a, ST_WY | ST_H | ST_O, &p);
    if (st != GDP_OK) return st;
    if (a->cu_seqlens) return fail(GDP_ERR_INVALID, "gdp_chunk_fwd_pipelined: cu_seqlens must be NULL");
    if (a->B != 1) return fail(GDP_ERR_INVALID, "gdp_chunk_fwd_pipelined: B must be 1 (got %lld)", (long long)a->B);
    if (num_segments < 1) return fail(GDP_ERR_INVALID, "num_segments must be >= 1");
    if (a->T == 0) return ok();
    if (!state_workspace || !aligned16(state_workspace))
        return fail(GDP_ERR_INVALID, "state_workspace must be a 16-byte aligned device pointer");
    std::vector<int64_t> starts((size_t)num_segments + 1);
    const int64_t nseg = segment_plan(a->T, num_segments, starts.data());
    const size_t es = dsize(a->dtype);
    const int64_t state_elems = (int64_t)a->HV * a->V * a->K;
    hipStream_t s0 = (hipStream_t)stream;

    std::lock_guard<std::mutex> lock(gdp::g_pipe_mu);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(GDP_ERR_UNSUPPORTED, "device index %d", dev);
    // every segment's arguments are checked before anything is enqueued
    std::vector<gdp::ChunkParams> sps((size_t)nseg);
    std::vector<gdp::PrepareParams> pps(prep ? (size_t)nseg : 0);
    for (int64_t sidx = 0; sidx < nseg; ++sidx) {
        const int64_t t0 = starts[sidx], Tn = starts[sidx + 1] - t0;
        const int64_t r0 = t0 * a->M;      // first expanded row
        const int64_t c0 = r0 / 64;        // first state chunk (t0 is a multiple of 64)
        gdp_chunk_args sa = *a;
        sa.T = Tn;
        sa.h_chunks = a->h_chunks - c0;
        sa.q = (const char *)a->q + t0 * a->H * a->K * es;
        sa.k = (const char *)a->k + r0 * a->H * a->K * es;
        sa.v = (const char *)a->v + r0 * a->HV * a->V * es;
        sa.beta = a->beta + r0 * a->HV;
        sa.g = a->g ? a->g + t0 * a->HV : nullptr;
        sa.k_rnorm = a->k_rnorm + r0 * a->H;
        sa.gcum = a->gcum + r0 * a->HV;
        sa.kdecay = a->kdecay + r0 * a->HV;
        sa.w = (char *)a->w + r0 * a->HV * a->K * es;
        sa.u = (char *)a->u + r0 * 16 * es;          // row r0 of every 16-column slice
        sa.v_new = (char *)a->v_new + r0 * 16 * es;
        sa.h = (char *)a->h + c0 * state_elems * es;
        sa.o = (char *)a->o + t0 * a->HV * a->V * es;
        sa.h0 = sidx == 0 ? a->h0 : state_workspace + ((sidx - 1) & 1) * state_elems;
        sa.ht = sidx == nseg - 1 ? a->ht : state_workspace + (sidx & 1) * state_elems;
        if ((st = check_chunk(&sa, ST_WY | ST_H | ST_O, &sps[sidx])) != GDP_OK) return st;
        sps[sidx].uv_ss = a->T * a->M * 16;  // slices keep the whole sequence's stride
        if (prep) {  // tokens [t0, t0 + Tn) of the one sequence
            gdp::PrepareParams &pp = pps[sidx];
            pp = *prep;
            const int64_t pes = (int64_t)dsize(prep->dtype);
            pp.x = (const char *)prep->x + t0 * prep->x_t_stride * pes;
            pp.ba = (const char *)prep->ba + t0 * prep->ba_t_stride * pes;
            pp.T = Tn;
            pp.q = (char *)prep->q + t0 * prep->H * prep->N * pes;
            pp.k = (char *)prep->k + t0 * prep->M * prep->H * prep->N * pes;
            pp.v = (char *)prep->v + t0 * prep->M * prep->H * prep->P * pes;
            pp.beta = prep->beta + t0 * prep->M * prep->H;
            pp.g = prep->g + t0 * prep->H;
        }
    }

    gdp::PipeCtx *ctx = nullptr;
    if ((e = gdp::pipe_ctx(dev, (size_t)(2 * nseg + 2), ctx)) != hipSuccess)
        return hip_status(e, "gdp_chunk_fwd_pipelined: stream/event creation");
    hipStream_t sw = ctx->side[0], so = ctx->side[1];
    hipEvent_t ev_end = ctx->ev[1];
    auto ev_w = [&](int64_t sidx) { return ctx->ev[2 + 2 * sidx]; };  // segment's WY done
    auto ev_h = [&](int64_t sidx) { return ctx->ev[3 + 2 * sidx]; };  // segment's chunk_h done
#define GDP_TRY(call, what)                                      \
    do {                                                         \
        hipError_t e_ = (call);                                  \
        if (e_ != hipSuccess) return hip_status(e_, what);       \
    } while (0)
    // Order of work.  Every cross-stream wait costs the serial chain about
    // 10-15 us, so the chain on `stream` holds only the waits it needs:
    //   stream: [prepare 0] WY 0, chunk_h 0, (wait WY 1) chunk_h 1, ...,
    //           chunk_h n-1, chunk_o n-1, (wait the last side chunk_o)
    //   side 0: [prepare s] WY s for s >= 1, back to back once WY 0 is done
    //           (they all overlap the first chunk_h or two: spreading them
    //           one per chunk_h measured slower, as each chunk_h then
    //           shares the memory system with a WY and a chunk_o)
    //   side 1: chunk_o s after chunk_h s, for s < n-1
    // A side stream's first operation waits on an event of `stream`, and
    // its last is waited on by `stream`, so a capture takes both in.
    if (prep) GDP_TRY(gdp::launch_prepare(pps[0], s0), "gdp_prefill_fwd_pipelined: prepare launch");
    GDP_TRY(gdp::launch_wy(sps[0], s0), "gdp_chunk_fwd_pipelined: recompute_w_u launch");
    if (nseg > 1) {
        GDP_TRY(hipEventRecord(ev_w(0), s0), "hipEventRecord");
        GDP_TRY(hipStreamWaitEvent(sw, ev_w(0), 0), "hipStreamWaitEvent");
    }
    for (int64_t sidx = 0; sidx < nseg; ++sidx) {
        const bool last = sidx == nseg - 1;
        if (!last) {  // the next segment's WY
            if (prep) GDP_TRY(gdp::launch_prepare(pps[sidx + 1], sw), "gdp_prefill_fwd_pipelined: prepare launch");
            GDP_TRY(gdp::launch_wy(sps[sidx + 1], sw), "gdp_chunk_fwd_pipelined: recompute_w_u launch");
            GDP_TRY(hipEventRecord(ev_w(sidx + 1), sw), "hipEventRecord");
        }
        if (sidx >= 1) GDP_TRY(hipStreamWaitEvent(s0, ev_w(sidx), 0), "hipStreamWaitEvent");
        if (chunk_h_events) GDP_TRY(hipEventRecord((hipEvent_t)chunk_h_events[2 * sidx], s0), "hipEventRecord");
        GDP_TRY(gdp::launch_chunk_h(sps[sidx], s0), "gdp_chunk_fwd_pipelined: chunk_h launch");
        if (chunk_h_events) GDP_TRY(hipEventRecord((hipEvent_t)chunk_h_events[2 * sidx + 1], s0), "hipEventRecord");
        if (!last) {
            GDP_TRY(hipEventRecord(ev_h(sidx), s0), "hipEventRecord");
            GDP_TRY(hipStreamWaitEvent(so, ev_h(sidx), 0), "hipStreamWaitEvent");
            GDP_TRY(gdp::launch_chunk_o(sps[sidx], so), "gdp_chunk_fwd_pipelined: chunk_o launch");
        } else {
            GDP_TRY(gdp::launch_chunk_o(sps[sidx], s0), "gdp_chunk_fwd_pipelined: chunk_o launch");
        }
    }
    if (nseg > 1) {
        GDP_TRY(hipEventRecord(ev_end, so), "hipEventRecord");
        GDP_TRY(hipStreamWaitEvent(s0, ev_end, 0), "hipStreamWaitEvent");
    }
#undef GDP_TRY
    return ok();
}

// Plan of the segment-parallel forward: segments of seg_tok tokens (equal
// shares of the 64-token chunks, rounded up), the last one possibly shorter.
// For packed requests seg_tok comes from the packed total T the same way and
// every request is cut at multiples of it on the device (launch_seg_plan);
// the return value is then the number of plan slots, an upper bound on the
// segments: ceil(T / seg_tok) + num_seqs.
static int64_t scan_plan(int64_t T, int32_t num_segments, int64_t num_seqs, bool packed, int64_t *seg_tok) {
    const int64_t nch = cdiv(T, 64);
    const int64_t per = cdiv(nch, num_segments) * 64;
    *seg_tok = per;
    if (T <= 0) return 0;
    return packed ? cdiv(T, per) + num_seqs : cdiv(T, per);
}

// Byte offsets of the regions of the scan workspace (each 256-byte aligned):
// maps, entering states, segment offsets, and for packed requests the plan's
// per-slot last flags and per-request first slot and count.
struct ScanLayout {
    int64_t maps, hstart, cu, seg_last, req_first, req_nseg, total;
};
static ScanLayout scan_layout(int64_t nslot, bool packed, int64_t num_seqs, int64_t HV, int64_t K, int64_t V) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t nmaps = packed ? nslot : (nslot > 1 ? nslot - 1 : 0);
    ScanLayout L;
    L.maps = 0;
    L.hstart = up(nmaps * HV * K * (K + V) * 4);
    L.cu = L.hstart + up(nslot * HV * V * K * 4);
    L.seg_last = L.cu + up((nslot + 1) * 4);
    L.req_first = L.seg_last + (packed ? up(nslot * 4) : 0);
    L.req_nseg = L.req_first + (packed ? up(num_seqs * 4) : 0);
    L.total = L.req_nseg + (packed ? up(num_seqs * 4) : 0);
    return L;
}

int32_t gdp_scan_segments(int64_t T, int32_t num_segments) {
    if (T < 0 || num_segments < 1 || num_segments > GDP_SCAN_MAX_SEGMENTS) return -1;
    int64_t st;
    return (int32_t)scan_plan(T, num_segments, 0, false, &st);
}

int64_t gdp_scan_workspace_bytes(int64_t T, int32_t HV, int32_t K, int32_t V, int32_t num_segments) {
    if (T < 0 || HV < 1 || K < 1 || V < 1 || num_segments < 1 || num_segments > GDP_SCAN_MAX_SEGMENTS) return -1;
    int64_t st;
    const int64_t nseg = scan_plan(T, num_segments, 0, false, &st);
    return scan_layout(nseg, false, 0, HV, K, V).total;
}

int64_t gdp_scan_workspace_bytes_varlen(int64_t T, int64_t num_seqs, int32_t HV, int32_t K, int32_t V,
                                        int32_t num_segments) {
    if (T < 0 || num_seqs < 0 || HV < 1 || K < 1 || V < 1 || num_segments < 1 ||
        num_segments > GDP_SCAN_MAX_SEGMENTS)
        return -1;
    int64_t st;
    const int64_t nslot = scan_plan(T, num_segments, num_seqs, true, &st);
    return scan_layout(nslot, true, num_seqs, HV, K, V).total;
}

// The segment-parallel forward; with prep, WY also does the prepare of its
// rows (launch_wy_prepare).  With scratch_base set, `workspace` is not the
// caller's: it is the library's scratch array (gdp_chunk_fwd_scan_noalloc),
// looked up by scratch_base() only once every argument, the plan and its
// size have been checked, so a rejected call makes no HIP call at all.
static gdp_status scan_impl(const char *name, const gdp_chunk_args *a, const gdp::PrepareParams *prep,
                            int32_t num_segments, void *workspace, int64_t workspace_bytes,
                            void *const *stage_events, void *stream, gdp_status (*scratch_base)(void **) = nullptr) {
    if (!a) return fail(GDP_ERR_INVALID, "%s: args is NULL", name);
    // v_new and h both NULL: chunk_h and chunk_o run as one pass that stores
    // neither (launch_chunk_ho)
    const bool fused = a->v_new == nullptr && a->h == nullptr;
    // q and k not stored (the fused prefill only): the later stages read
    // their rows from the activations
    const bool qkx = prep != nullptr && a->q == nullptr && a->k == nullptr;
    const unsigned qks = qkx ? ST_QKX : 0u;
    gdp::ChunkParams p;
    gdp_status st = check_chunk(a, (prep ? ST_WYP : ST_WY) | (fused ? ST_HO : ST_H | ST_O) | qks, &p);
    if (st != GDP_OK) return st;
    if (qkx) {  // x row: [values (M, H, P) | keys (M, G, N) | queries (G, N)] (bf16 here)
        const int64_t ko = (int64_t)prep->M * prep->H * prep->P, qo = ko + (int64_t)prep->M * prep->G * prep->N;
        const char *x = (const char *)prep->x;
        p.qk = gdp::QKRows{x + 2 * ko, x + 2 * qo, prep->x_t_stride, (int64_t)prep->G * prep->N, prep->x_t_stride,
                           (int64_t)prep->N, prep->H / prep->G};
    }
    if (fused && a->M < 2 && p.nseq > 0)
        return fail(GDP_ERR_UNSUPPORTED, "%s: v_new and h may be NULL (one chunk_h and chunk_o pass) only for M >= 2",
                    name);
    const bool packed = a->cu_seqlens != nullptr;
    if (a->B != 1)
        return fail(GDP_ERR_INVALID, "%s: B must be 1 (got %lld; packed requests go through cu_seqlens)", name,
                    (long long)a->B);
    if (num_segments < 1 || num_segments > GDP_SCAN_MAX_SEGMENTS)
        return fail(GDP_ERR_INVALID, "%s: num_segments %d not in [1, %d]", name, num_segments,
                    GDP_SCAN_MAX_SEGMENTS);
    if (a->dtype != GDP_BF16 || !((a->K == 64 || a->K == 128) && (a->V == 64 || a->V == 128)))
        return fail(GDP_ERR_UNSUPPORTED, "%s: bf16 with K, V in {64, 128} only (K=%d V=%d)", name, a->K,
                    a->V);
    if (p.nseq == 0) return ok();  // T == 0 or no requests: nothing to launch
    if (a->T * a->M * a->V * 2 >= ((int64_t)1 << 31))
        return fail(GDP_ERR_UNSUPPORTED, "%s: T*M*V*2 must stay below 2^31 (T=%lld)", name, (long long)a->T);
    int64_t seg_tok = 0;
    const int64_t nslot = scan_plan(a->T, num_segments, p.nseq, packed, &seg_tok);
    if (nslot * a->HV > 0x7fffffff || nslot >= 0x7fffffff / 8)
        return fail(GDP_ERR_UNSUPPORTED, "%s: too many segments for one launch", name);
    const ScanLayout L = scan_layout(nslot, packed, p.nseq, a->HV, a->K, a->V);
    if (scratch_base) {
        if (L.total > workspace_bytes)
            return fail(GDP_ERR_UNSUPPORTED,
                        "%s: this call needs %lld bytes of scratch, more than the %lld bytes of the library's own "
                        "(GDP_NOALLOC_SCRATCH_BYTES); use gdp_chunk_fwd_scan with a workspace, or fewer segments",
                        name, (long long)L.total, (long long)workspace_bytes);
        gdp_status st2 = scratch_base(&workspace);
        if (st2 != GDP_OK) return st2;
    }
    if (!workspace || ((uintptr_t)workspace & 255u))
        return fail(GDP_ERR_INVALID, "%s: workspace must be a 256-byte aligned device pointer", name);
    if (workspace_bytes < L.total)
        return fail(GDP_ERR_INVALID, "%s: workspace of %lld bytes, %lld needed", name,
                    (long long)workspace_bytes, (long long)L.total);
    char *ws = (char *)workspace;
    gdp::ScanParams sp{p,
                       nslot,
                       seg_tok,
                       (float *)(ws + L.maps),
                       (float *)(ws + L.hstart),
                       (int32_t *)(ws + L.cu),
                       packed ? (int32_t *)(ws + L.seg_last) : nullptr,
                       packed ? (int32_t *)(ws + L.req_first) : nullptr,
                       packed ? (int32_t *)(ws + L.req_nseg) : nullptr};
    // the chunk_h pass: the segments as packed sequences, each from its
    // entering state, whose final states replace it in place
    gdp_chunk_args ha = *a;
    ha.cu_seqlens = sp.cu;
    ha.num_seqs = nslot;
    ha.h0 = sp.hstart;
    ha.ht = sp.hstart;
    gdp::ChunkParams hp;
    if ((st = check_chunk(&ha, (fused ? ST_HO : ST_H) | qks, &hp)) != GDP_OK) return st;
    hp.qk = p.qk;
    // only the states chunk_o reads: the one entering each 64-token chunk.
    // Every segment starts on a 64-token boundary of its sequence, so
    // counting chunks per segment keeps the sequence's own c % M.
    hp.hstep = a->M;
    hipStream_t s = (hipStream_t)stream;
    auto mark = [&](int i) {
        return stage_events ? hip_status(hipEventRecord((hipEvent_t)stage_events[i], s), "hipEventRecord") : ok();
    };
    auto run = [&](hipError_t e, const char *what) { return hip_status(e, what); };
    if (!packed && p.nseq == 1 && nslot > 1) {  // WY in the order the segment maps read it
        p.seg_nch = seg_tok * a->M / 64;
        p.seg_n = nslot;
    }
    if ((st = run(prep ? gdp::launch_wy_prepare(p, *prep, s) : gdp::launch_wy(p, s),
                  "gdp_chunk_fwd_scan: recompute_w_u launch")) != GDP_OK)
        return st;
    if (packed && (st = run(gdp::launch_seg_plan(sp, s), "gdp_chunk_fwd_scan: segment plan launch")) != GDP_OK)
        return st;
    if ((st = mark(0)) != GDP_OK) return st;
    if ((st = run(gdp::launch_seg_map(sp, s), "gdp_chunk_fwd_scan: segment map launch")) != GDP_OK) return st;
    if ((st = mark(1)) != GDP_OK) return st;
    if ((st = run(gdp::launch_seg_scan(sp, s), "gdp_chunk_fwd_scan: segment scan launch")) != GDP_OK) return st;
    if ((st = mark(2)) != GDP_OK) return st;
    if (fused) {  // chunk_h and chunk_o in one pass: events 3 and 4 bracket nothing
        if ((st = run(gdp::launch_chunk_ho(hp, s), "gdp_chunk_fwd_scan: chunk_h+o launch")) != GDP_OK) return st;
        if ((st = mark(3)) != GDP_OK) return st;
        if ((st = mark(4)) != GDP_OK) return st;
    } else {
        if ((st = run(gdp::launch_chunk_h(hp, s), "gdp_chunk_fwd_scan: chunk_h launch")) != GDP_OK) return st;
        if ((st = mark(3)) != GDP_OK) return st;
        if ((st = run(gdp::launch_chunk_o(p, s), "gdp_chunk_fwd_scan: chunk_o launch")) != GDP_OK) return st;
        if ((st = mark(4)) != GDP_OK) return st;
    }
    if (a->ht) {
        if (packed) {
            if ((st = run(gdp::launch_seg_final(sp, s), "gdp_chunk_fwd_scan: final state launch")) != GDP_OK)
                return st;
        } else {
            const size_t bytes = (size_t)a->HV * a->V * a->K * sizeof(float);
            if ((st = run(hipMemcpyAsync(a->ht, sp.hstart + (nslot - 1) * a->HV * a->V * a->K, bytes,
                                         hipMemcpyDeviceToDevice, s),
                          "gdp_chunk_fwd_scan: final state copy")) != GDP_OK)
                return st;
        }
    }
    return ok();
}

gdp_status gdp_chunk_fwd_scan(const gdp_chunk_args *a, int32_t num_segments, void *workspace,
                              int64_t workspace_bytes, void *const *stage_events, void *stream) {
    return scan_impl("gdp_chunk_fwd_scan", a, nullptr, num_segments, workspace, workspace_bytes, stage_events,
                     stream);
}

gdp_status gdp_prefill_fwd_scan(const gdp_prepare_args *pa, const gdp_chunk_args *a, int32_t num_segments,
                                void *workspace, int64_t workspace_bytes, void *const *stage_events, void *stream) {
    if (!pa || !a) return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_scan: args is NULL");
    if (a->HV != a->H)
        return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_scan: prepare makes H value heads (HV=%d, H=%d)", a->HV, a->H);
    if (!a->g && a->T > 0) return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_scan: g is NULL (prepare writes it)");
    if ((a->q == nullptr) != (a->k == nullptr))
        return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_scan: q and k must both be given or both be NULL");
    if (a->q == nullptr && (a->v_new != nullptr || a->h != nullptr))
        return fail(GDP_ERR_UNSUPPORTED,
                    "gdp_prefill_fwd_scan: q and k may be NULL only with v_new and h NULL (one chunk_h + chunk_o pass)");
    gdp::PrepareParams pp;
    const gdp_status st = prepare_check("gdp_prefill_fwd_scan", false, pa->x, pa->x_n_stride, pa->x_t_stride, pa->ba,
                                        pa->ba_n_stride, pa->ba_t_stride, pa->A_log, pa->dt_bias, a->B, a->T, a->M,
                                        a->H, pa->G, a->V, a->K, a->dtype, (void *)a->q, (void *)a->k,
                                        (void *)a->v, (float *)a->beta, (float *)a->g, &pp, true, true);
    if (st != GDP_OK) return st;
    if (pp.T > 0 && !pp.vec16)
        return fail(GDP_ERR_UNSUPPORTED, "gdp_prefill_fwd_scan: x rows and outputs must be 16-byte aligned");
    return scan_impl("gdp_prefill_fwd_scan", a, pp.T > 0 ? &pp : nullptr, num_segments, workspace,
                     workspace_bytes, stage_events, stream);
}

}  // extern "C"

// ---- the allocation-free form of gdp_chunk_fwd_scan
// The workspace of the segment-parallel forward (segment maps, entering
// states, segment offsets) as a device array of the library's own, so the
// caller allocates nothing.  In host code `scratch` names a host-side
// stand-in, not device memory: every use below goes through the per-device
// address hipGetSymbolAddress gives (each GPU holds its own copy of the
// array, for the life of the process).  Nothing in it needs to start at
// zero: each call writes every byte it reads first.
static __device__ __align__(256) char scratch[GDP_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[64];  // the array's device address, per device (null until first use)

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
gdp_status scratch_base(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "gdp_chunk_fwd_scan_noalloc: hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(GDP_ERR_UNSUPPORTED, "gdp_chunk_fwd_scan_noalloc: device index %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "gdp_chunk_fwd_scan_noalloc: hipGetSymbolAddress(scratch)");
        if (!p || ((uintptr_t)p & 255u))
            return fail(GDP_ERR_HIP, "gdp_chunk_fwd_scan_noalloc: scratch address %p is not 256-byte aligned", p);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return ok();
}
}  // namespace

extern "C" {

gdp_status gdp_chunk_fwd_scan_noalloc(const gdp_chunk_args *a, int32_t num_segments, void *const *stage_events,
                                      void *stream) {
    return scan_impl("gdp_chunk_fwd_scan_noalloc", a, nullptr, num_segments, nullptr, GDP_NOALLOC_SCRATCH_BYTES,
                     stage_events, stream, scratch_base);
}

gdp_status gdp_chunk_fwd_pipelined(const gdp_chunk_args *a, int32_t num_segments, float *state_workspace,
                                   void *const *chunk_h_events, void *stream) {
    return pipelined_impl(a, nullptr, num_segments, state_workspace, chunk_h_events, stream);
}

gdp_status gdp_prefill_fwd_pipelined(const gdp_prepare_args *pa, const gdp_chunk_args *a, int32_t num_segments,
                                     float *state_workspace, void *const *chunk_h_events, void *stream) {
    if (!pa || !a) return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_pipelined: args is NULL");
    if (a->HV != a->H)
        return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_pipelined: prepare makes H value heads (HV=%d, H=%d)", a->HV,
                    a->H);
    if (!a->g && a->T > 0) return fail(GDP_ERR_INVALID, "gdp_prefill_fwd_pipelined: g is NULL (prepare writes it)");
    gdp::PrepareParams pp;
    const gdp_status st = prepare_check("gdp_prefill_fwd_pipelined", false, pa->x, pa->x_n_stride, pa->x_t_stride,
                                        pa->ba, pa->ba_n_stride, pa->ba_t_stride, pa->A_log, pa->dt_bias, a->B,
                                        a->T, a->M, a->H, pa->G, a->V, a->K, a->dtype, (void *)a->q, (void *)a->k,
                                        (void *)a->v, (float *)a->beta, (float *)a->g, &pp);
    if (st != GDP_OK) return st;
    return pipelined_impl(a, pp.T > 0 ? &pp : nullptr, num_segments, state_workspace, chunk_h_events, stream);
}

int64_t gdp_num_state_chunks(const int32_t *cu_seqlens_host, int64_t num_seqs, int64_t B, int64_t T, int32_t M,
                             int32_t chunk_size) {
    if (T < 0 || B < 0 || M < 1 || chunk_size < 1) return -1;
    if (!cu_seqlens_host) return B * cdiv(T * M, chunk_size);
    if (num_seqs < 0) return -1;
    int64_t total = 0;
    for (int64_t i = 0; i < num_seqs; ++i) {
        int64_t a = cu_seqlens_host[i], b = cu_seqlens_host[i + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        total += cdiv((b - a) * M, chunk_size);
    }
    return total;
}

const char *gdp_last_error(void) { return g_err.c_str(); }

const char *gdp_version(void) { return "gdp-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
