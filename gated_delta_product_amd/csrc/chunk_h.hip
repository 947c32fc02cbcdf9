// chunk_h.hip -- inter-chunk state recurrence of the Gated Delta Product
// (the chunk_h stage whose outputs core.ssm.ops.gdp.chunk_o consumes: the
// state at each chunk boundary and the corrected values).
//
// For one sequence and one value head, serially over its 64-row chunks c of
// the expanded stream, with h the K x V transpose of the state S entering c:
//   snapshot  h[c] = h                     (stored as S = h^T, V x K)
//   v_new     = u - w h                    (corrected values of the chunk)
//   h         = exp(gamma_last) h + Khat^T diag(exp(gamma_last - gamma)) v_new
// where gamma is the within-chunk cumulative log decay (decay on copy 0).
//
// Work split: one wave per (sequence, value head, 16 value columns).  The
// fp32 state slice (K x 16) lives in registers for the whole sequence.  Both
// products run on the matrix cores and hand their result tiles straight to
// the next product as operands: a result tile gives each lane 4 consecutive
// rows of one column, which is a valid operand fragment once the other
// operand reads its contraction index in the same order.  So w is read with
// its K columns permuted to match h, and K^T (from LDS, transposed on the fly
// by ds_read_b64_tr_b16) with its rows permuted to match v_new.  w tiles go
// straight from HBM into operand registers; K and u are staged in LDS.  The
// next chunk is fetched while the current one is computed.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

namespace {
constexpr int C = 64;
template <typename T> struct PadH { static constexpr int value = 32 / (int)sizeof(T); };
}  // namespace

template <typename T, int KD, int VD>
__global__ void __launch_bounds__(64)
gdp_chunk_h_k(const T *__restrict__ k, const float *__restrict__ k_rnorm, const T *__restrict__ w,
              const T *__restrict__ u, const float *__restrict__ g, const int32_t *__restrict__ cu,
              int64_t nseq, int64_t Ttok, int H, int HV, int M, int64_t h_chunks,
              T *__restrict__ v_new, T *__restrict__ hout) {
    typedef typename Frag<T>::type FragT;
    typedef typename Frag<T>::half HalfT;
    constexpr int E = 16 / sizeof(T);          // elements per 16-byte unit
    constexpr int LDK = KD + PadH<T>::value;   // K tile row stride (elements)
    constexpr int LDU = 16 + PadH<T>::value;   // u tile row stride
    constexpr int NKT = KD / 16;               // 16-row tiles of h (K dim)
    constexpr int NKS = KD / 32;               // contraction steps over K
    constexpr int KUNITS = C * KD / E / 64;    // 16-byte K units per lane
    constexpr int UUNITS = C * 16 / E / 64;    // 16-byte u units per lane
    constexpr int S = VD / 16;                 // column slices per head

    __shared__ __attribute__((aligned(16))) T Ks[2][C * LDK];
    __shared__ __attribute__((aligned(16))) T Us[2][C * LDU];
    __shared__ __attribute__((aligned(16))) float Fs[2][C];  // rk * exp(gamma_last - gamma), 0 past the end
    __shared__ float Gl[2];                                   // exp(gamma_last)

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
    const int64_t nch = ceil_div64(rows, C);
    const int64_t cbase = items_before(cu, Ttok, M, C, seq);
    if (nch == 0) return;

    const int lane = lane_id();
    const int lg = lane >> 4, lc = lane & 15;
    const int64_t ldk_g = (int64_t)H * KD;    // global row stride of k
    const int64_t ldw_g = (int64_t)HV * KD;   // of w
    const int64_t ldv_g = (int64_t)HV * VD;   // of u / v_new

    // ---- prefetch registers for one chunk
    HalfT wn[4][NKS][2];   // w operand fragments: [row tile][k step][half]
    uint4 kn[KUNITS];
    uint4 un[UUNITS];
    float rkn, gn;
    int nn;  // rows of the prefetched chunk

    auto fetch = [&](int64_t c) {
        const int64_t e0 = bos * M + C * c;
        const int n = (int)((rows - C * c) < C ? (rows - C * c) : C);
        nn = n;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = 16 * rt + lc;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    HalfT val;
                    if (r < n)
                        val = *(const HalfT *)(w + (e0 + r) * ldw_g + hv * (int64_t)KD + 32 * ks + 16 * hf + 4 * lg);
                    else
                        val = HalfT{};
                    wn[rt][ks][hf] = val;
                }
        }
#pragma unroll
        for (int i = 0; i < KUNITS; ++i) {
            const int uidx = lane + 64 * i;
            const int r = uidx / (KD / E), cu_ = uidx % (KD / E);
            kn[i] = r < n ? *(const uint4 *)(k + (e0 + r) * ldk_g + hk * (int64_t)KD + cu_ * E)
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < UUNITS; ++i) {
            const int uidx = lane + 64 * i;
            const int r = uidx / (16 / E), cu_ = uidx % (16 / E);
            un[i] = r < n ? *(const uint4 *)(u + (e0 + r) * ldv_g + hv * (int64_t)VD + 16 * sl + cu_ * E)
                          : make_uint4(0, 0, 0, 0);
        }
        const int64_t e = e0 + lane;
        rkn = lane < n ? k_rnorm[e * H + hk] : 0.f;
        gn = (lane < n && (e % M) == 0) ? g[(e / M) * HV + hv] : 0.f;
    };

    auto commit = [&](int st) {
#pragma unroll
        for (int i = 0; i < KUNITS; ++i) {
            const int uidx = lane + 64 * i;
            const int r = uidx / (KD / E), cu_ = uidx % (KD / E);
            *(uint4 *)(&Ks[st][r * LDK + cu_ * E]) = kn[i];
        }
#pragma unroll
        for (int i = 0; i < UUNITS; ++i) {
            const int uidx = lane + 64 * i;
            const int r = uidx / (16 / E), cu_ = uidx % (16 / E);
            *(uint4 *)(&Us[st][r * LDU + cu_ * E]) = un[i];
        }
        const float gam = wave_inclusive_sum(gn);
        const float glast = __shfl(gam, 63, 64);
        Fs[st][lane] = lane < nn ? rkn * __expf(glast - gam) : 0.f;
        if (lane == 0) Gl[st] = __expf(glast);
    };

    // ---- state: h tiles [kt] hold h[16kt + 4lg + q][16sl + lc]
    f32x4 hs[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) hs[kt] = zero4();
    FragT hb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) hb[ks] = FragT{};

    fetch(0);
    HalfT wc[4][NKS][2];
    commit(0);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            wc[rt][ks][0] = wn[rt][ks][0];
            wc[rt][ks][1] = wn[rt][ks][1];
        }
    int ncur = nn;

    for (int64_t c = 0; c < nch; ++c) {
        const int st = (int)(c & 1);
        const int64_t e0 = bos * M + C * c;
        if (c + 1 < nch) fetch(c + 1);
        __syncthreads();  // stage st written by commit() of the previous step

        // snapshot of the state entering chunk c (S = h^T, V x K)
        if (cbase + c < h_chunks) {
            T *dst = hout + (((cbase + c) * HV + hv) * (int64_t)VD + 16 * sl + lc) * KD + 4 * lg;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                HalfT hv4;
#pragma unroll
                for (int q = 0; q < 4; ++q) hv4[q] = from_f32<T>(hs[kt][q]);
                *(HalfT *)(dst + 16 * kt) = hv4;
            }
        }

        // phase 1: acc = w h  (64 x 16)
        f32x4 acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            acc[rt] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                acc[rt] = mma(join<T>(wc[rt][ks][0], wc[rt][ks][1]), hb[ks], acc[rt]);
        }
        const float gl = Gl[st];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q) hs[kt][q] *= gl;

        // v_new = u - w h ; scaled copy feeds the state update
        FragT vb[2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const HalfT uu = lds_col4<T>(Us[st], LDU, 16 * rt + 4 * lg, 0);
            const f32x4 fr = *(const f32x4 *)(&Fs[st][16 * rt + 4 * lg]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 16 * rt + 4 * lg + q;
                const float vn = to_f32(uu[q]) - acc[rt][q];
                if (r < ncur) v_new[(e0 + r) * ldv_g + hv * (int64_t)VD + 16 * sl + lc] = from_f32<T>(vn);
                vb[rt >> 1][4 * (rt & 1) + q] = from_f32<T>(vn * fr[q]);
            }
        }

        // phase 2: h = exp(gamma_last) h + K^T (f * v_new)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                FragT a = lds_col8<T>(Ks[st], LDK, 32 * s + 4 * lg, 32 * s + 16 + 4 * lg, 16 * kt);
                hs[kt] = mma(a, vb[s], hs[kt]);
            }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hb[ks][q] = from_f32<T>(hs[2 * ks][q]);
                hb[ks][4 + q] = from_f32<T>(hs[2 * ks + 1][q]);
            }

        if (c + 1 < nch) {
            commit(st ^ 1);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    wc[rt][ks][0] = wn[rt][ks][0];
                    wc[rt][ks][1] = wn[rt][ks][1];
                }
            ncur = nn;
        }
    }
}

template <typename T, int KD, int VD>
static hipError_t launch_chunk_h_t(const ChunkParams &p, hipStream_t stream) {
    const gdp_chunk_args &a = p.a;
    const int64_t P = p.nseq * a.HV;
    const int64_t S = VD / 16;
    const int64_t nblk = ((P + 7) / 8) * 8 * S;
    hipLaunchKernelGGL((gdp_chunk_h_k<T, KD, VD>), dim3((unsigned)nblk), dim3(64), 0, stream,
                       (const T *)a.k, a.k_rnorm, (const T *)a.w, (const T *)a.u, a.g, a.cu_seqlens,
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
