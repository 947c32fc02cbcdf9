// prepare.hip -- fused prefill and decode prepare for the Gated Delta Product
// (core.ssm.ops.gdp.prepare: module description, gdp_prefill_prepare and
// gdp_decode_prepare).
//
// One block per (token, batch row).  The block writes every output of its
// token: the value copies, the GQA-expanded key copies and query, beta for
// each (copy, head) and g for each head.  Copies move in 16-byte vectors when
// the rows allow it.  HBM-bound: each x row is read once (key/query groups are
// re-read from cache once per head sharing them) and every output is written
// once.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

// Copy unit: a 16-byte vector when VEC16, else one element.  (A native
// vector type, so arrays of units stay in registers.)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <typename T, bool VEC16>
struct Unit {
    typedef typename std::conditional<VEC16, u32x4_t, T>::type type;
    static constexpr int elems = VEC16 ? (int)(16 / sizeof(T)) : 1;
};

// DECODE: the query goes to the last copy of its token and g to the first,
// zeros elsewhere (q [n, T*M, H, N], g [n, T*M, H]); otherwise both stay
// one per token.
template <typename T, bool VEC16, bool DECODE>
__device__ __forceinline__ void
prepare_body(const T *__restrict__ x, int64_t xns, int64_t xts,
             const T *__restrict__ ba, int64_t bns, int64_t bts,
             const float *__restrict__ A_log, const float *__restrict__ dt_bias,
             int64_t T_, int M, int H, int G, int P, int N,
             T *__restrict__ q, T *__restrict__ k, T *__restrict__ v,
             float *__restrict__ beta, float *__restrict__ g) {
    typedef typename Unit<T, VEC16>::type U;
    constexpr int E = Unit<T, VEC16>::elems;
    const int64_t t = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t tok = b * T_ + t;  // flattened token index
    const T *xr = x + b * xns + t * xts;
    const T *br = ba + b * bns + t * bts;
    const int hpg = H / G;
    const int HN = H * N;

    const int nv = M * H * P / E;  // value units
    const int nk = M * HN / E;     // key units (expanded)
    const int nq = (DECODE ? M : 1) * HN / E;  // query units (expanded; all copies in decode)
    const int ntot = nv + nk + nq;
    const int kbase = M * H * P;   // key segment offset in x
    const int qbase = kbase + M * G * N;

    U *vo = (U *)(v + tok * (int64_t)M * H * P);
    U *ko = (U *)(k + tok * (int64_t)M * HN);
    U *qo = (U *)(q + tok * (int64_t)(DECODE ? M : 1) * HN);
    const U *xv = (const U *)xr;

    // Batches of UB units per thread: all loads of a batch are issued before
    // its stores, so each thread keeps UB 16-byte reads in flight.
    constexpr int UB = 8;
    for (int base = 0; base < ntot; base += UB * 256) {
        U val[UB];
#pragma unroll
        for (int it = 0; it < UB; ++it) {
            const int i = base + (int)threadIdx.x + 256 * it;
            if (i < nv) {
                // value copies are already in (copy, head, dim) order
                val[it] = xv[i];
            } else if (i < nv + nk) {
                const int e = (i - nv) * E;  // element within the token's key copies
                const int j = e / HN;
                const int rem = e - j * HN;
                const int h = rem / N, n = rem - h * N;
                val[it] = *(const U *)(xr + kbase + j * G * N + (h / hpg) * N + n);
            } else if (i < ntot) {
                int e = (i - nv - nk) * E;
                bool copy_q = true;
                if constexpr (DECODE) {  // element within the token's M query rows
                    const int j = e / HN;
                    copy_q = j == M - 1;
                    e -= j * HN;
                }
                const int h = e / N, n = e - h * N;
                if (copy_q)
                    val[it] = *(const U *)(xr + qbase + (h / hpg) * N + n);
                else
                    val[it] = U{};
            }
        }
#pragma unroll
        for (int it = 0; it < UB; ++it) {
            const int i = base + (int)threadIdx.x + 256 * it;
            if (i < nv)
                vo[i] = val[it];
            else if (i < nv + nk)
                ko[i - nv] = val[it];
            else if (i < ntot)
                qo[i - nv - nk] = val[it];
        }
    }
    // gates: beta for (copy, head) = M*H values, then g for H heads (for
    // every copy in decode, zero past the first)
    const int ng = (DECODE ? M : 1) * H;
    for (int i = threadIdx.x; i < M * H + ng; i += blockDim.x) {
        if (i < M * H) {
            beta[tok * (int64_t)M * H + i] = gate_beta(to_f32(br[i]));
        } else {
            const int c = i - M * H, h = c % H;
            g[tok * (int64_t)ng + c] = c < H ? gate_g(to_f32(br[M * H + h]), A_log[h], dt_bias[h]) : 0.0f;
        }
    }
}

// The prefill and decode forms are separate kernels so that profiles tell
// them apart.
#define GDP_PREPARE_PARAMS                                                                          \
    const T *__restrict__ x, int64_t xns, int64_t xts, const T *__restrict__ ba, int64_t bns,       \
        int64_t bts, const float *__restrict__ A_log, const float *__restrict__ dt_bias, int64_t T_, \
        int M, int H, int G, int P, int N, T *__restrict__ q, T *__restrict__ k, T *__restrict__ v,  \
        float *__restrict__ beta, float *__restrict__ g
template <typename T, bool VEC16>
__global__ void __launch_bounds__(256) gdp_prepare_k(GDP_PREPARE_PARAMS) {
    prepare_body<T, VEC16, false>(x, xns, xts, ba, bns, bts, A_log, dt_bias, T_, M, H, G, P, N, q, k, v, beta, g);
}
template <typename T, bool VEC16>
__global__ void __launch_bounds__(256) gdp_decode_prepare_k(GDP_PREPARE_PARAMS) {
    prepare_body<T, VEC16, true>(x, xns, xts, ba, bns, bts, A_log, dt_bias, T_, M, H, G, P, N, q, k, v, beta, g);
}
#undef GDP_PREPARE_PARAMS

template <typename T, bool VEC16, bool DECODE>
static hipError_t launch_prepare_t(const PrepareParams &p, hipStream_t stream) {
    dim3 grid((unsigned)p.T, (unsigned)p.n);
    hipLaunchKernelGGL((DECODE ? gdp_decode_prepare_k<T, VEC16> : gdp_prepare_k<T, VEC16>), grid, dim3(256), 0, stream,
                       (const T *)p.x, p.x_n_stride, p.x_t_stride,
                       (const T *)p.ba, p.ba_n_stride, p.ba_t_stride,
                       p.A_log, p.dt_bias, p.T, p.M, p.H, p.G, p.P, p.N,
                       (T *)p.q, (T *)p.k, (T *)p.v, p.beta, p.g);
    return hipGetLastError();
}

template <bool DECODE>
static hipError_t launch_prepare_d(const PrepareParams &p, hipStream_t stream) {
    if (p.dtype == GDP_BF16)
        return p.vec16 ? launch_prepare_t<bf16, true, DECODE>(p, stream) : launch_prepare_t<bf16, false, DECODE>(p, stream);
    return p.vec16 ? launch_prepare_t<float, true, DECODE>(p, stream) : launch_prepare_t<float, false, DECODE>(p, stream);
}

hipError_t launch_prepare(const PrepareParams &p, hipStream_t stream) {
    if (p.n == 0 || p.T == 0) return hipSuccess;
    return p.decode ? launch_prepare_d<true>(p, stream) : launch_prepare_d<false>(p, stream);
}

}  // namespace gdp
