// decode.hip -- one decode step of the Gated Delta Product: the recurrence
// over each request's S*M rows, row by row, with the state kept in registers
// between the state-pool load and store (the fused recurrent update that the
// prepare page names as the consumer of gdp_decode_prepare's interleaved
// rows; core.ssm.ops.gdp.prepare, module description, decode bullet).
//
// Per row e:  delta = beta (v - exp(g) S khat),  S <- exp(g) S + delta khat^T,
//             o = scale * S qhat,
// the corrected-value form of S <- exp(g) S (I - beta khat khat^T) + beta v khat^T.
//
// One block of NT threads per (request, value head).  Each state row (K fp32
// entries) is spread over TPR = K/4 consecutive lanes, 4 entries per lane,
// so one wave-wide 16-byte load or store covers whole contiguous rows; the
// block covers NT/TPR rows per pass and each thread holds RPT rows spaced by
// that stride.  The row dot products reduce over the TPR lanes of a row
// (DPP within 16 lanes, one swizzle beyond); the rank-1 update is local.
// The step is bound by moving the state (read and written once per step).
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

template <typename T> __device__ __forceinline__ f32x4 load4(const T *p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float *p) { return *(const f32x4 *)p; }
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16 *p) {
    const uint2 u = *(const uint2 *)p;
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

template <typename T, int KD, int VD, int NT>
__global__ void __launch_bounds__(NT)
gdp_decode_k(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
             const float *__restrict__ beta, const float *__restrict__ g, float *__restrict__ state,
             const int32_t *__restrict__ slots, int64_t pool, int L, int H, int HV, float scale,
             T *__restrict__ o) {
    constexpr int TPR = KD / 4;      // lanes per state row
    constexpr int RSTEP = NT / TPR;  // rows covered per pass of the block
    constexpr int RPT = VD / RSTEP;  // rows per thread
    static_assert(64 % TPR == 0 && VD % RSTEP == 0 && RPT >= 1, "state split");
    const int64_t req = blockIdx.x;
    const int hv = blockIdx.y, hk = hv / (HV / H);
    const int tid = threadIdx.x, p = tid % TPR, r0 = tid / TPR;
    const int64_t slot = slots ? (int64_t)slots[req] : req;

    if (slot < 0 || slot >= pool) {  // skipped request: its rows are zero
        for (int i = tid; i < L * VD; i += NT)
            o[((req * L + i / VD) * HV + hv) * (int64_t)VD + i % VD] = from_f32<T>(0.f);
        return;
    }
    float *st = state + (slot * HV + hv) * (int64_t)VD * KD + 4 * p;
    f32x4 s[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) s[j] = *(const f32x4 *)(st + (int64_t)(r0 + j * RSTEP) * KD);

    for (int e = 0; e < L; ++e) {
        const int64_t row = req * L + e;
        const f32x4 kr = load4<T>(k + (row * H + hk) * (int64_t)KD + 4 * p);
        const f32x4 qr = load4<T>(q + (row * H + hk) * (int64_t)KD + 4 * p);
        const T *vp = v + (row * HV + hv) * (int64_t)VD + r0;
        float vv[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j) vv[j] = to_f32(vp[j * RSTEP]);
        const float b = beta[row * HV + hv];
        const float alpha = g ? __expf(g[row * HV + hv]) : 1.0f;
        const float rk = 1.0f / sqrtf(group_sum<TPR>(dot4(kr, kr)) + 1e-6f);
        const float rq = 1.0f / sqrtf(group_sum<TPR>(dot4(qr, qr)) + 1e-6f);
        T *op = o + (row * HV + hv) * (int64_t)VD + r0;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const float sk = group_sum<TPR>(dot4(s[j], kr));
            const float dk = b * (vv[j] - alpha * (sk * rk)) * rk;
            s[j] = alpha * s[j] + dk * kr;
            const float so = group_sum<TPR>(dot4(s[j], qr));
            if (p == 0) op[j * RSTEP] = from_f32<T>(scale * rq * so);
        }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) *(f32x4 *)(st + (int64_t)(r0 + j * RSTEP) * KD) = s[j];
}

template <typename T, int KD, int VD>
static hipError_t launch_decode_t(const gdp_decode_args &a, hipStream_t stream) {
    constexpr int NT = KD * VD / 32 < 256 ? 256 : (KD * VD / 32 > 1024 ? 1024 : KD * VD / 32);
    dim3 grid((unsigned)a.n, (unsigned)a.HV);
    hipLaunchKernelGGL((gdp_decode_k<T, KD, VD, NT>), grid, dim3(NT), 0, stream, (const T *)a.q, (const T *)a.k,
                       (const T *)a.v, a.beta, a.g, a.state, a.slots, a.pool, (int)(a.S * a.M), a.H, a.HV,
                       a.scale, (T *)a.o);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dims(const gdp_decode_args &a, hipStream_t stream) {
    switch (a.K * 1000 + a.V) {
    case 64064: return launch_decode_t<T, 64, 64>(a, stream);
    case 64128: return launch_decode_t<T, 64, 128>(a, stream);
    case 64256: return launch_decode_t<T, 64, 256>(a, stream);
    case 128064: return launch_decode_t<T, 128, 64>(a, stream);
    case 128128: return launch_decode_t<T, 128, 128>(a, stream);
    case 128256: return launch_decode_t<T, 128, 256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const gdp_decode_args &a, hipStream_t stream) {
    if (a.n == 0 || a.S == 0) return hipSuccess;
    return a.dtype == GDP_BF16 ? launch_decode_dims<bf16>(a, stream) : launch_decode_dims<float>(a, stream);
}

}  // namespace gdp
