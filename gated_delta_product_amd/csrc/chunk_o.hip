// chunk_o.hip -- output of the Gated Delta Product
// (core.ssm.ops.gdp.chunk_o: module description,
// chunk_gated_delta_product_fwd_o).
//
// One block (4 waves) per (64-token chunk i of a sequence, value head).  The
// queries are one per token; keys and corrected values live on the expanded
// stream, copy j of token s at row s*M + j.  With G the within-chunk
// cumulative log decay of the tokens and S the V x K state entering the
// chunk (the chunk_h snapshot at expanded chunk i*M):
//   o_t = scale * [ exp(G_t) S qhat_t
//                   + sum_j sum_{s <= t} exp(G_t - G_s) (qhat_t . khat_{sM+j}) v_new_{sM+j} ]
// computed transposed, O^T = S Q^T + sum_j V_j^T P_j^T, so a result lane
// holds four consecutive output columns of one token.  The score tile
// S_j^T = K_j Q^T comes out of the matrix cores with each lane holding four
// consecutive key rows of one query column -- exactly the B-operand layout the
// P V product needs once V_j^T is read with the same row order (LDS transpose
// reads).  Norms enter as fp32 scales on the scores and on the inter term.
// Wave w owns tokens [16w, 16w + 16) and skips the key tiles past them.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

namespace {
constexpr int C = 64;
template <typename T> struct PadO { static constexpr int value = 32 / (int)sizeof(T); };
}  // namespace

template <typename T, int KD, int VD>
__global__ void __launch_bounds__(256)
gdp_chunk_o_k(const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ k_rnorm,
              const T *__restrict__ v_new, const T *__restrict__ hst, const float *__restrict__ g,
              const int32_t *__restrict__ cu, int64_t nseq, int64_t Ttok, int H, int HV, int M,
              int64_t h_chunks, float scale, T *__restrict__ o) {
    typedef typename Frag<T>::type FragT;
    constexpr int LDK = KD + PadO<T>::value;
    constexpr int LDV = VD + PadO<T>::value;
    constexpr int NVT = VD / 16;
    constexpr int NKS = KD / 32;
    __shared__ __attribute__((aligned(16))) T Qs[C * LDK];
    __shared__ __attribute__((aligned(16))) T Ss[VD * LDK];
    __shared__ __attribute__((aligned(16))) T Kj[C * LDK];
    __shared__ __attribute__((aligned(16))) T Vj[C * LDV];
    __shared__ float s_rq[C], s_G[C], s_rk[C];

    const ChunkLoc loc = find_chunk(cu, nseq, Ttok, 1, C, blockIdx.x);
    if (loc.seq < 0) return;
    const int hv = blockIdx.y;
    const int hk = hv / (HV / H);
    const int64_t t0 = loc.bos + C * loc.c;  // first token (flattened)
    const int nt = (int)((loc.eos - t0) < C ? (loc.eos - t0) : C);
    const int64_t hidx = items_before(cu, Ttok, M, C, loc.seq) + loc.c * M;
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int lg = lane >> 4, lc = lane & 15;

    // ---- stage Q (with norms), the boundary state S, decays
    stage_tile<T, C, KD, LDK, 256>(Qs, q + (t0 * H + hk) * (int64_t)KD, (int64_t)H * KD, nt, s_rq);
    stage_tile<T, VD, KD, LDK, 256>(Ss, hst + (hidx * HV + hv) * (int64_t)VD * KD, (int64_t)KD,
                                    hidx < h_chunks ? VD : 0, nullptr);
    if (wv == 0) {
        const float gt = lane < nt ? g[(t0 + lane) * HV + hv] : 0.f;
        s_G[lane] = wave_inclusive_sum(gt);
    }
    __syncthreads();
    if (wv == 0) s_rq[lane] = 1.0f / sqrtf(s_rq[lane] + 1e-6f);
    __syncthreads();

    const int tt = wv;                 // token tile of this wave
    const int t_loc = 16 * tt + lc;    // token whose column this lane holds
    const float Gt = s_G[t_loc];

    // ---- inter-chunk term: O^T[vt] = S[16vt.., :] Q^T[:, t]
    f32x4 acc[NVT];
    {
        FragT qb[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qb[ks] = lds_row8<T>(Qs + t_loc * LDK + 32 * ks + 8 * lg);
        const float f = scale * s_rq[t_loc] * __expf(Gt);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            f32x4 a4 = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                a4 = mma(lds_row8<T>(Ss + (16 * vt + lc) * LDK + 32 * ks + 8 * lg), qb[ks], a4);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[vt][i] = a4[i] * f;
        }
    }

    // ---- intra-chunk attention, one Householder copy at a time
    const float fq = scale * s_rq[t_loc];
    for (int j = 0; j < M; ++j) {
        __syncthreads();  // previous copy's tiles are no longer read
        const int64_t r0 = t0 * M + j;  // expanded row of copy j of token t0
        stage_tile<T, C, KD, LDK, 256>(Kj, k + (r0 * H + hk) * (int64_t)KD, (int64_t)M * H * KD, nt, nullptr);
        stage_tile<T, C, VD, LDV, 256>(Vj, v_new + (r0 * HV + hv) * (int64_t)VD, (int64_t)M * HV * VD, nt,
                                       nullptr);
        if (wv == 0) s_rk[lane] = lane < nt ? k_rnorm[(r0 + (int64_t)lane * M) * H + hk] : 0.f;
        __syncthreads();

        // scores P^T tiles for key tiles st <= tt: lane holds s = 16st + 4lg + i, t = t_loc
        FragT qb[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qb[ks] = lds_row8<T>(Qs + t_loc * LDK + 32 * ks + 8 * lg);
        f32x4 p[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            p[st] = zero4();
            if (st <= tt) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    p[st] = mma(lds_row8<T>(Kj + (16 * st + lc) * LDK + 32 * ks + 8 * lg), qb[ks], p[st]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * st + 4 * lg + i;
                    p[st][i] = (s <= t_loc && s < nt) ? p[st][i] * fq * s_rk[s] * __expf(Gt - s_G[s]) : 0.f;
                }
            }
        }
        // O^T[vt] += V_j^T[vt, s] P^T[s, t]; contraction slot m <-> s = 32ks + 16(m/4) + 4lg + m%4
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (2 * ks <= tt) {
                FragT pb;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pb[i] = from_f32<T>(p[2 * ks][i]);
                    pb[4 + i] = from_f32<T>(p[2 * ks + 1][i]);
                }
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    FragT a = lds_col8<T>(Vj, LDV, 32 * ks + 4 * lg, 32 * ks + 16 + 4 * lg, 16 * vt);
                    acc[vt] = mma(a, pb, acc[vt]);
                }
            }
        }
    }

    // ---- store: lane holds o[t_loc][16vt + 4lg + i]
    if (t_loc < nt) {
        T *dst = o + ((t0 + t_loc) * HV + hv) * (int64_t)VD + 4 * lg;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            typename Frag<T>::half o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) o4[i] = from_f32<T>(acc[vt][i]);
            *(typename Frag<T>::half *)(dst + 16 * vt) = o4;
        }
    }
}

template <typename T, int KD, int VD>
static hipError_t launch_chunk_o_t(const ChunkParams &p, hipStream_t stream) {
    const gdp_chunk_args &a = p.a;
    dim3 grid((unsigned)p.max_tok_chunks, (unsigned)a.HV);
    hipLaunchKernelGGL((gdp_chunk_o_k<T, KD, VD>), grid, dim3(256), 0, stream,
                       (const T *)a.q, (const T *)a.k, a.k_rnorm, (const T *)a.v_new, (const T *)a.h, a.g,
                       a.cu_seqlens, p.nseq, a.T, a.H, a.HV, a.M, a.h_chunks, a.scale, (T *)a.o);
    return hipGetLastError();
}

// bf16: K in {64, 128} x V in {64, 128, 256}; f32 (small-case reference
// precision): K = 64, V in {64, 128}.
static hipError_t launch_chunk_o_bf16(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_o_t<bf16, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_chunk_o_t<bf16, 64, 128>(p, stream);
    if (K == 64 && V == 256) return launch_chunk_o_t<bf16, 64, 256>(p, stream);
    if (K == 128 && V == 64) return launch_chunk_o_t<bf16, 128, 64>(p, stream);
    if (K == 128 && V == 128) return launch_chunk_o_t<bf16, 128, 128>(p, stream);
    if (K == 128 && V == 256) return launch_chunk_o_t<bf16, 128, 256>(p, stream);
    return hipErrorInvalidValue;
}
static hipError_t launch_chunk_o_f32(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_o_t<float, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_chunk_o_t<float, 64, 128>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_o(const ChunkParams &p, hipStream_t stream) {
    if (p.max_tok_chunks == 0) return hipSuccess;
    return p.a.dtype == GDP_BF16 ? launch_chunk_o_bf16(p, stream) : launch_chunk_o_f32(p, stream);
}

}  // namespace gdp
