// chunk_h.hip -- inter-chunk state recurrence of the Gated Delta Product
// (the chunk_h stage whose outputs core.ssm.ops.gdp.chunk_o consumes: the
// state at each chunk boundary and the corrected values).
//
// For one sequence and one value head, serially over its 64-row chunks c of
// the expanded stream, with h the K x V transpose of the state S entering c:
//   snapshot  h[c] = h                     (stored as S = h^T, V x K)
//   v_new     = u - w h                    (corrected values of the chunk)
//   h         = exp2(gl) h + Khat^T diag(exp2(gl - gcum)) v_new
// where gcum is the within-chunk cumulative decay in log2 units (decay on
// the first copy of each token, precomputed by the WY stage) and gl its
// value on the chunk's last row.
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
// Memory: every wave streams its own w and K half tiles, the u slice, the
// key norms and gcum straight from HBM into a three-stage LDS ring (buffer
// loads with the LDS destination, two chunks ahead; no staging registers).
// Tile rows are XOR-swizzled in 16-byte units so the fragment reads of both
// products avoid bank conflicts.  The only cross-wave barrier is the
// partial-sum exchange, and it waits on LDS only, so the stream stays in
// flight across it.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

namespace {
constexpr int C = 64;
}  // namespace

template <typename T, int KD>
struct HStage {
    T w[C * (KD / 2)];  // w half tile, swizzled rows
    T k[C * (KD / 2)];  // K half tile, swizzled rows
    T u[C * 16];        // u slice, plain rows of 16 elements
    float rk[C];        // key inverse norms per row (0 past the end)
    float gc[C];        // cumulative log2 decay per row
};

template <typename T, int KD, int VD>
__global__ void __launch_bounds__(128)
gdp_chunk_h_k(const T *__restrict__ k, const float *__restrict__ k_rnorm, const T *__restrict__ w,
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
    static_assert(NKS >= 1 && (UPR & (UPR - 1)) == 0, "tile shape");
    static_assert(2 * NDMA + 12 < 64, "in-flight DMA count must fit the vector memory counter");

    __shared__ __attribute__((aligned(16))) HStage<T, KD> ring[2][NS];   // [wave][stage]
    __shared__ __attribute__((aligned(16))) T Vt[2][16 * LDT];            // [wave] v_new transpose
    __shared__ __attribute__((aligned(16))) f32x4 Xs[2][2][4][64];        // [parity][wave][row tile][lane]

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
    const int32_t rows32 = (int32_t)rows;
    const int64_t r0 = bos * M;  // first expanded row of the sequence
    const T *w0 = w + (r0 * HV + hv) * KD + kw * KH;
    const T *k0 = k + (r0 * H + hk) * KD + kw * KH;
    const T *u0 = u + (r0 * HV + hv) * VD + 16 * sl;
    T *vn0 = v_new + (r0 * HV + hv) * VD + 16 * sl;
    const float *rk0 = k_rnorm + r0 * H + hk;
    const float *gc0 = gcum + r0 * HV + hv;
    T *h0 = hout + (cbase * HV + hv) * (int64_t)VD * KD;

    // rows of chunk c (0 past the end: its loads are out of range)
    auto rows_in = [&](int c) {
        const int r = rows32 - C * c;
        return r < 0 ? 0 : (r < C ? r : C);
    };
    auto span = [&](int n, int stride, int width, int es) {
        return (uint32_t)(n > 0 ? ((n - 1) * stride + width) * es : 0);
    };
    // byte offset of element column `col` of half-tile row r (swizzled)
    auto swz = [&](int r, int col) {
        const int b = col * ES;
        return r * RB + ((((b >> 4) ^ ((r >> 1) & (UPR - 1)))) << 4) + (b & 15);
    };

    // Stream chunk c into stage st: exactly NDMA DMA instructions.
    auto issue = [&](int c, int st) {
        HStage<T, KD> &Sg = ring[kw][st];
        const int n = rows_in(c);
        if (n < C) {  // tail or padding chunk: zero the stage first
            for (int i = lane; i < (int)(sizeof(HStage<T, KD>) / 16); i += 64)
                ((uint4 *)&Sg)[i] = make_uint4(0, 0, 0, 0);
            wait_lgkm0();
        }
        const int64_t cr = (int64_t)C * c;
        const rsrc_t rw = make_rsrc(w0 + cr * ldw, span(n, ldw, KH, ES));
        const rsrc_t rk_ = make_rsrc(k0 + cr * ldk, span(n, ldk, KH, ES));
        const rsrc_t ru = make_rsrc(u0 + cr * ldv, span(n, ldv, 16, ES));
        const rsrc_t rr = make_rsrc(rk0 + cr * H, span(n, H, 1, 4));
        const rsrc_t rg = make_rsrc(gc0 + cr * HV, span(n, HV, 1, 4));
#pragma unroll
        for (int i = 0; i < UPR; ++i) {
            const int r = i * RPI + lane / UPR;
            const int unit = (lane % UPR) ^ ((r >> 1) & (UPR - 1));
            dma16(rw, (uint32_t)((r * ldw) * ES + unit * 16), lds_addr(Sg.w) + i * 1024);
            dma16(rk_, (uint32_t)((r * ldk) * ES + unit * 16), lds_addr(Sg.k) + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int r = i * (64 / UUPR) + lane / UUPR;
            dma16(ru, (uint32_t)((r * ldv) * ES + (lane % UUPR) * 16), lds_addr(Sg.u) + i * 1024);
        }
        dma4(rr, (uint32_t)(lane * H * 4), lds_addr(Sg.rk));
        dma4(rg, (uint32_t)(lane * HV * 4), lds_addr(Sg.gc));
    };

    // state: hs[kt] holds h[kw*KH + 16kt + 4lg + q][16sl + lc]
    f32x4 hs[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) hs[kt] = zero4();
    FragT hb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) hb[ks] = FragT{};

    issue(0, 0);
    issue(1, 1);
    int st = 0;
    for (int c = 0; c < nch; ++c) {
        issue(c + 2, st == 0 ? 2 : st - 1);
        wait_vmcnt<2 * NDMA>();  // chunk c landed (issued two steps ago)
        const HStage<T, KD> &Sg = ring[kw][st];
        const int n = rows_in(c);

        // snapshot of the state entering chunk c (S = h^T, V x K); dropped
        // past h_chunks
        {
            const rsrc_t rh = make_rsrc(h0 + (int64_t)c * HV * VD * KD,
                                        (cbase + c < h_chunks) ? (uint32_t)(VD * KD * ES) : 0u);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                HalfT h4;
#pragma unroll
                for (int q = 0; q < 4; ++q) h4[q] = from_f32<T>(hs[kt][q]);
                const uint32_t off = (uint32_t)(((16 * sl + lc) * KD + kw * KH + 16 * kt + 4 * lg) * ES);
                if constexpr (ES == 2)
                    buf_store8(rh, off, __builtin_bit_cast(uint2, h4));
                else
                    buf_store16(rh, off, __builtin_bit_cast(uint4, h4));
            }
        }

        // phase 1: partial w h over this wave's half of K; the w fragment
        // reads K columns {32ks + 4lg .. +3} then {32ks + 16 + 4lg .. +3},
        // the order of the h result tiles
        f32x4 acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            acc[rt] = zero4();
            const int r = 16 * rt + lc;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const char *wb = (const char *)Sg.w;
                const HalfT a0 = *(const HalfT *)(wb + swz(r, 32 * ks + 4 * lg));
                const HalfT a1 = *(const HalfT *)(wb + swz(r, 32 * ks + 16 + 4 * lg));
                acc[rt] = mma(join<T>(a0, a1), hb[ks], acc[rt]);
            }
        }

        // wave-private reads that need no barrier: u, norms, decays, K^T
        HalfT uu[4];
        f32x4 rk4[4], gc4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            uu[rt] = lds_col4<T>(Sg.u, 16, 16 * rt + 4 * lg, 0);
            rk4[rt] = *(const f32x4 *)(&Sg.rk[16 * rt + 4 * lg]);
            gc4[rt] = *(const f32x4 *)(&Sg.gc[16 * rt + 4 * lg]);
        }
        const float glast = Sg.gc[n > 0 ? n - 1 : 0];
        FragT ka[NKT][2];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                HalfT x0, x1;
                const char *kb = (const char *)Sg.k;
                if constexpr (ES == 2) {
                    // transposed read: source lane j of the 16-lane group
                    // points at row rowA + j/4, columns 16kt + 4(j%4) .. +3
                    const int j = lane & 15;
                    const int ra = 32 * s + 4 * lg + (j >> 2), rb = ra + 16;
                    const int col = 16 * kt + 4 * (j & 3);
                    x0 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swz(ra, col)))));
                    x1 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swz(rb, col)))));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x0[i] = *(const float *)(kb + swz(32 * s + 4 * lg + i, 16 * kt + lc));
                        x1[i] = *(const float *)(kb + swz(32 * s + 16 + 4 * lg + i, 16 * kt + lc));
                    }
                }
                ka[kt][s] = join<T>(x0, x1);
            }

        // exchange partials (double-buffered by chunk parity: one barrier)
        const int par = c & 1;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Xs[par][kw][rt][lane] = acc[rt];
        lds_barrier();

        const float gl = n > 0 ? exp2f(glast) : 1.0f;
        FragT vb[2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 other = Xs[par][kw ^ 1][rt][lane];
            HalfT v4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float vn = to_f32(uu[rt][q]) - acc[rt][q] - other[q];
                const float f = rk4[rt][q] * exp2f(glast - gc4[rt][q]);  // rk is 0 past the end
                v4[q] = from_f32<T>(vn);
                vb[rt >> 1][4 * (rt & 1) + q] = from_f32<T>(vn * f);
            }
            *(HalfT *)(&Vt[kw][lc * LDT + 16 * rt + 4 * lg]) = v4;
        }

        // phase 2: h = exp2(gl) h + K^T (f * v_new), this wave's K half
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
        const rsrc_t rv = make_rsrc(vn0 + (int64_t)C * c * ldv, span(n, ldv, 16, ES));
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const HalfT o4 = lds_col4<T>(Vt[kw], LDT, 4 * lg, 32 * kw + 16 * r2);
            const uint32_t off = (uint32_t)(((32 * kw + 16 * r2 + lc) * ldv + 4 * lg) * ES);
            if constexpr (ES == 2)
                buf_store8(rv, off, __builtin_bit_cast(uint2, o4));
            else
                buf_store16(rv, off, __builtin_bit_cast(uint4, o4));
        }
        st = st == NS - 1 ? 0 : st + 1;
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
                       (const T *)a.k, a.k_rnorm, (const T *)a.w, (const T *)a.u, a.gcum, a.cu_seqlens,
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
