// chunk_h.hip -- inter-chunk state recurrence of the Gated Delta Product
// (the chunk_h stage whose outputs core.ssm.ops.gdp.chunk_o consumes: the
// state at each chunk boundary and the corrected values).
//
// For one sequence and one value head, serially over its 64-row chunks c of
// the expanded stream, with h the K x V transpose of the state S entering c:
//   snapshot  h[c] = h                     (stored as S = h^T, V x K)
//   v_new     = u - w h                    (corrected values of the chunk)
//   h         = exp2(gl) h + K^T diag(kdecay) v_new
// where gl is the chunk's total decay in log2 units (the within-chunk
// cumulative decay gcum on its last row) and kdecay = rnorm(k) exp2(gl - gcum)
// per row, both precomputed by the WY stage.
//
// Work split: one block of two waves per (sequence, value head, 16 value
// columns).  Wave k owns rows [k K/2, (k+1) K/2) of the fp32 state slice,
// which stays in its registers for the whole sequence.  Per chunk each wave
// forms its partial w h over its half of K; the halves are summed through
// LDS (one barrier), both waves form v_new, and each wave updates its half
// of h with its half of K.  Result tiles of the matrix cores feed the next
// product directly: a result tile gives a lane four consecutive rows of one
// column, a valid operand fragment once the other operand reads its
// contraction index in the same order -- w is read with its K columns
// permuted to match h, and K^T (transposed on the fly by ds_read_b64_tr_b16)
// with its rows permuted to match v_new.
//
// Memory: every wave streams its own w and K half tiles, the u slice,
// kdecay and gcum straight from HBM into a three-stage LDS ring (buffer
// loads with the LDS destination, two chunks ahead; no staging registers).
// Tile rows are XOR-swizzled in 16-byte units so the fragment reads of both
// products avoid bank conflicts.  The only cross-wave barrier is the
// partial-sum exchange, and it waits on LDS only, so the stream stays in
// flight across it.
#include "gdp_common.h"
#include "gdp_internal.h"

#include <type_traits>

namespace gdp {

namespace {
constexpr int C = 64;
}  // namespace

template <typename T, int KD>
struct HStage {
    T w[C * (KD / 2)];  // w half tile, swizzled rows
    T k[C * (KD / 2)];  // K half tile, swizzled rows
    T u[C * 16];        // u slice, plain rows of 16 elements
    float kd[C];        // key decay factor per row (0 past the end)
    float gc[C];        // cumulative log2 decay per row
};

template <typename T, int KD, int VD>
__global__ void __launch_bounds__(128)
gdp_chunk_h_k(const T *__restrict__ k, const float *__restrict__ kdecay, const T *__restrict__ w,
              const T *__restrict__ u, const float *__restrict__ gcum, const int32_t *__restrict__ cu,
              int64_t nseq, int64_t Ttok, int H, int HV, int M, int64_t h_chunks,
              T *__restrict__ v_new, T *__restrict__ hout) {
    typedef typename Frag<T>::type FragT;
    typedef typename Frag<T>::half HalfT;
    constexpr int ES = (int)sizeof(T);
    constexpr int KH = KD / 2;                 // state rows per wave
    constexpr int RB = KH * ES;                // bytes per half-tile row
    constexpr int UPR = RB / 16;               // 16-byte units per half-tile row
    constexpr int RPI = 64 / UPR;              // half-tile rows per DMA instruction
    constexpr int UUPR = 16 * ES / 16;         // 16-byte units per u row
    constexpr int NU = C * UUPR / 64;          // DMA instructions for the u slice
    constexpr int NDMA = 2 * UPR + NU + 2;     // DMA instructions per wave per chunk
    constexpr int NS = 3;                      // ring stages (prefetch distance 2)
    constexpr int NKT = KH / 16;               // 16-row state tiles per wave
    constexpr int NKS = KH / 32;               // phase-1 contraction steps per wave
    constexpr int LDT = 64 + 32 / ES;          // row stride of the v_new transpose
    constexpr int S = VD / 16;                 // column slices per head
    constexpr int SB = (int)sizeof(HStage<T, KD>);
    static_assert(NKS >= 1 && (UPR & (UPR - 1)) == 0, "tile shape");
    static_assert(2 * NDMA + 12 < 64, "in-flight DMA count must fit the vector memory counter");
    static_assert(SB % 16 == 0, "stage size");

    __shared__ __attribute__((aligned(16))) HStage<T, KD> ring[2][NS];   // [wave][stage]
    __shared__ __attribute__((aligned(16))) T Vt[2][16 * LDT];            // [wave] v_new transpose
    __shared__ __attribute__((aligned(16))) f32x4 Xs[NS][2][4][64];       // [stage][wave][row tile][lane]

    // ---- block -> (sequence, value head, slice); slices of one head share an XCD
    const int64_t P = nseq * HV;
    const int64_t id = blockIdx.x;
    const int64_t slot = id / 8, xcd = id % 8;
    const int64_t pair = (slot / S) * 8 + xcd;
    const int sl = (int)(slot % S);
    if (pair >= P) return;
    const int64_t seq = pair / HV;
    const int hv = (int)(pair % HV);
    const int hk = hv / (HV / H);
    int64_t bos, eos;
    seq_bounds(cu, Ttok, seq, bos, eos);
    const int64_t rows = (eos - bos) * M;
    const int nch = (int)ceil_div64(rows, C);
    const int64_t cbase = items_before(cu, Ttok, M, C, seq);
    if (nch == 0) return;

    const int lane = lane_id(), kw = wave_id();
    const int lg = lane >> 4, lc = lane & 15;
    const int ldk = H * KD, ldw = HV * KD, ldv = HV * VD;  // global row strides (elements)
    const int64_t r0 = bos * M;  // first expanded row of the sequence
    // chunks whose state snapshot fits below h_chunks
    const int64_t hroom = h_chunks - cbase;
    const int hlim = hroom < 0 ? 0 : (hroom > nch ? nch : (int)hroom);

    // byte offset of element column `col` of half-tile row r (swizzled)
    auto swz = [&](int r, int col) {
        const int b = col * ES;
        return r * RB + ((((b >> 4) ^ ((r >> 1) & (UPR - 1)))) << 4) + (b & 15);
    };
    // bytes a buffer resource must cover for n rows of `width` elements
    auto span = [](int n, int stride_b, int width_b) { return (uint32_t)(n > 0 ? (n - 1) * stride_b + width_b : 0); };
    auto clamp_rows = [](int r) { return r < 0 ? 0 : (r < C ? r : C); };

    // Per-lane DMA source offsets inside a chunk (fixed for the whole loop).
    uint32_t ow[UPR], ok[UPR], ou[NU];
#pragma unroll
    for (int i = 0; i < UPR; ++i) {
        const int r = i * RPI + lane / UPR;
        const int unit = (lane % UPR) ^ ((r >> 1) & (UPR - 1));
        ow[i] = (uint32_t)((r * ldw) * ES + unit * 16);
        ok[i] = (uint32_t)((r * ldk) * ES + unit * 16);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) ou[i] = (uint32_t)(((i * (64 / UUPR) + lane / UUPR) * ldv) * ES + (lane % UUPR) * 16);
    const uint32_t okd = (uint32_t)(lane * HV * 4), ogc = okd;

    // Streams advance by one chunk per issue.
    const char *pw = (const char *)(w + (r0 * HV + hv) * KD + kw * KH);
    const char *pk = (const char *)(k + (r0 * H + hk) * KD + kw * KH);
    const char *pu = (const char *)(u + (r0 * HV + hv) * VD + 16 * sl);
    const char *pd = (const char *)(kdecay + r0 * HV + hv);
    const char *pg = (const char *)(gcum + r0 * HV + hv);
    const int64_t stw = (int64_t)C * ldw * ES, stk = (int64_t)C * ldk * ES, stu = (int64_t)C * ldv * ES,
                  std_ = (int64_t)C * HV * 4;
    int rem_issue = (int)rows;  // rows left from the next chunk to issue
    const uint32_t ring_base = lds_addr(&ring[kw][0]);

    // Stream the next chunk into stage st: exactly NDMA DMA instructions.
    auto issue = [&](int st) {
        const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem_issue));
        const uint32_t sb = ring_base + st * SB;
        if (n < C) {  // tail or padding chunk: zero the stage first
            HStage<T, KD> &Sg = ring[kw][st];
            for (int i = lane; i < SB / 16; i += 64) ((uint4 *)&Sg)[i] = make_uint4(0, 0, 0, 0);
            wait_lgkm0();
        }
        const rsrc_t rw = make_rsrc(pw, span(n, ldw * ES, RB));
        const rsrc_t rk_ = make_rsrc(pk, span(n, ldk * ES, RB));
        const rsrc_t ru = make_rsrc(pu, span(n, ldv * ES, 16 * ES));
        const rsrc_t rd = make_rsrc(pd, span(n, HV * 4, 4));
        const rsrc_t rg = make_rsrc(pg, span(n, HV * 4, 4));
#pragma unroll
        for (int i = 0; i < UPR; ++i) {
            dma16_at(rw, ow[i], sb, (int)__builtin_offsetof(HStage<T, KD>, w) + i * 1024);
            dma16_at(rk_, ok[i], sb, (int)__builtin_offsetof(HStage<T, KD>, k) + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) dma16_at(ru, ou[i], sb, (int)__builtin_offsetof(HStage<T, KD>, u) + i * 1024);
        dma4_at(rd, okd, sb, (int)__builtin_offsetof(HStage<T, KD>, kd));
        dma4_at(rg, ogc, sb, (int)__builtin_offsetof(HStage<T, KD>, gc));
        pw += stw;
        pk += stk;
        pu += stu;
        pd += std_;
        pg += std_;
        rem_issue -= C;
    };

    // State slice of this wave, in a permuted K order: hs[kt][q] holds h at
    // K index kw*KH + kperm(kt, 4lg + q), column 16sl + lc, with
    //   kperm(kt, i) = 32(kt/2) + 8(i/4) + 4(kt%2) + i%4,
    // so that hb[ks] (tiles 2ks, 2ks+1 as bf16) holds 8 consecutive K
    // indices 32ks + 8lg .. +7: the phase-1 operand matches a plain 16-byte
    // row read of w and the snapshot is one 16-byte store.  K^T is read with
    // the same permutation.
    f32x4 hs[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) hs[kt] = zero4();
    FragT hb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) hb[ks] = FragT{};

    char *ph = (char *)(hout + (cbase * HV + hv) * (int64_t)VD * KD);
    char *pv = (char *)(v_new + (r0 * HV + hv) * VD + 16 * sl);
    const int64_t sth = (int64_t)HV * VD * KD * ES;
    int rem = (int)rows;  // rows left from the current chunk

    // One chunk on ring stage ST (a compile-time constant, so every LDS
    // address below is a fixed offset from a per-lane base).
    auto step = [&](int c, auto stc) {
        constexpr int ST = decltype(stc)::value;
        issue((ST + 2) % NS);
        wait_vmcnt<2 * NDMA>();  // chunk c landed (issued two steps ago)
        const HStage<T, KD> &Sg = ring[kw][ST];
        const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem));  // uniform

        // snapshot of the state entering chunk c (S = h^T, V x K); dropped
        // past h_chunks
        {
            const rsrc_t rh = make_rsrc(ph, c < hlim ? (uint32_t)(VD * KD * ES) : 0u);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const uint32_t off = (uint32_t)(((16 * sl + lc) * KD + kw * KH + 32 * ks + 8 * lg) * ES);
                if constexpr (ES == 2) {
                    buf_store16(rh, off, __builtin_bit_cast(uint4, hb[ks]));
                } else {
                    HalfT lo, hi;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        lo[q] = hb[ks][q];
                        hi[q] = hb[ks][4 + q];
                    }
                    buf_store16(rh, off, __builtin_bit_cast(uint4, lo));
                    buf_store16(rh, off + 16, __builtin_bit_cast(uint4, hi));
                }
            }
        }

        // phase 1: partial w h over this wave's half of K (w columns
        // 32ks + 8lg .. +7, the order of hb)
        f32x4 acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            acc[rt] = zero4();
            const int r = 16 * rt + lc;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const char *wb = (const char *)Sg.w;
                FragT a;
                if constexpr (ES == 2) {
                    a = *(const FragT *)(wb + swz(r, 32 * ks + 8 * lg));
                } else {
                    a = join<T>(*(const HalfT *)(wb + swz(r, 32 * ks + 8 * lg)),
                                *(const HalfT *)(wb + swz(r, 32 * ks + 8 * lg + 4)));
                }
                acc[rt] = mma(a, hb[ks], acc[rt]);
            }
        }

        // wave-private reads that need no barrier: u, key decays, K^T
        HalfT uu[4];
        f32x4 kd4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            uu[rt] = lds_col4<T>(Sg.u, 16, 16 * rt + 4 * lg, 0);
            kd4[rt] = *(const f32x4 *)(&Sg.kd[16 * rt + 4 * lg]);
        }
        const float glast = Sg.gc[n > 0 ? n - 1 : 0];
        FragT ka[NKT][2];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                HalfT x0, x1;
                const char *kb = (const char *)Sg.k;
                const int kbase = 32 * (kt >> 1) + 4 * (kt & 1);  // kperm(kt, 0)
                if constexpr (ES == 2) {
                    // transposed read: source lane j of the 16-lane group
                    // points at row rowA + j/4 and the 4 K indices
                    // kperm(kt, 4(j%4) .. +3); output lane i then holds
                    // K index kperm(kt, i) of rows rowA .. rowA+3
                    const int j = lane & 15;
                    const int ra = 32 * s + 4 * lg + (j >> 2), rb = ra + 16;
                    const int col = kbase + 8 * (j & 3);
                    x0 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swz(ra, col)))));
                    x1 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swz(rb, col)))));
                } else {
                    const int col = kbase + 8 * (lc >> 2) + (lc & 3);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x0[i] = *(const float *)(kb + swz(32 * s + 4 * lg + i, col));
                        x1[i] = *(const float *)(kb + swz(32 * s + 16 + 4 * lg + i, col));
                    }
                }
                ka[kt][s] = join<T>(x0, x1);
            }

        // exchange partials (one buffer per ring stage: one barrier)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Xs[ST][kw][rt][lane] = acc[rt];
        lds_barrier();

        // gl <= 0, and rows past the end carry decay factor 0
        const float gl = n > 0 ? __builtin_amdgcn_exp2f(glast) : 1.0f;
        FragT vb[2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 other = Xs[ST][kw ^ 1][rt][lane];
            HalfT v4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float vn = to_f32(uu[rt][q]) - acc[rt][q] - other[q];
                v4[q] = from_f32<T>(vn);
                vb[rt >> 1][4 * (rt & 1) + q] = from_f32<T>(vn * kd4[rt][q]);
            }
            *(HalfT *)(&Vt[kw][lc * LDT + 16 * rt + 4 * lg]) = v4;
        }

        // phase 2: h = exp2(gl) h + K^T (kd * v_new), this wave's K half
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) hs[kt][q] *= gl;
#pragma unroll
            for (int s = 0; s < 2; ++s) hs[kt] = mma(ka[kt][s], vb[s], hs[kt]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hb[ks][q] = from_f32<T>(hs[2 * ks][q]);
                hb[ks][4 + q] = from_f32<T>(hs[2 * ks + 1][q]);
            }

        // v_new rows [32kw, 32kw + 32) of this wave: 4 columns of a row per lane
        const rsrc_t rv = make_rsrc(pv, span(n, ldv * ES, 16 * ES));
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const HalfT o4 = lds_col4<T>(Vt[kw], LDT, 4 * lg, 32 * kw + 16 * r2);
            const uint32_t off = (uint32_t)(((32 * kw + 16 * r2 + lc) * ldv + 4 * lg) * ES);
            if constexpr (ES == 2)
                buf_store8(rv, off, __builtin_bit_cast(uint2, o4));
            else
                buf_store16(rv, off, __builtin_bit_cast(uint4, o4));
        }
        ph += sth;
        pv += stu;
        rem -= C;
    };

    issue(0);
    issue(1);
    static_assert(NS == 3, "the loop below is unrolled over three ring stages");
    for (int c = 0; c < nch; c += 3) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>{});
        if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>{});
    }
    wait_vmcnt<0>();  // no DMA may still target LDS when the block retires
}

template <typename T, int KD, int VD>
static hipError_t launch_chunk_h_t(const ChunkParams &p, hipStream_t stream) {
    const gdp_chunk_args &a = p.a;
    const int64_t P = p.nseq * a.HV;
    const int64_t S = VD / 16;
    const int64_t nblk = ((P + 7) / 8) * 8 * S;
    hipLaunchKernelGGL((gdp_chunk_h_k<T, KD, VD>), dim3((unsigned)nblk), dim3(128), 0, stream,
                       (const T *)a.k, a.kdecay, (const T *)a.w, (const T *)a.u, a.gcum, a.cu_seqlens,
                       p.nseq, a.T, a.H, a.HV, a.M, a.h_chunks, (T *)a.v_new, (T *)a.h);
    return hipGetLastError();
}

// bf16: K in {64, 128} x V in {64, 128, 256}; f32 (small-case reference
// precision): K = 64, V in {64, 128}.
static hipError_t launch_chunk_h_bf16(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_h_t<bf16, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_chunk_h_t<bf16, 64, 128>(p, stream);
    if (K == 64 && V == 256) return launch_chunk_h_t<bf16, 64, 256>(p, stream);
    if (K == 128 && V == 64) return launch_chunk_h_t<bf16, 128, 64>(p, stream);
    if (K == 128 && V == 128) return launch_chunk_h_t<bf16, 128, 128>(p, stream);
    if (K == 128 && V == 256) return launch_chunk_h_t<bf16, 128, 256>(p, stream);
    return hipErrorInvalidValue;
}
static hipError_t launch_chunk_h_f32(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_h_t<float, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_chunk_h_t<float, 64, 128>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_h(const ChunkParams &p, hipStream_t stream) {
    if (p.nseq == 0 || p.a.T == 0) return hipSuccess;
    return p.a.dtype == GDP_BF16 ? launch_chunk_h_bf16(p, stream) : launch_chunk_h_f32(p, stream);
}

}  // namespace gdp
