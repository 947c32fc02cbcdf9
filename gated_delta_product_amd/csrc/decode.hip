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
// One block of NT threads per (request, value head), NT sized so that each
// thread holds at most 32 state entries.  The V x K fp32 state is split into
// runs of EPT consecutive K entries of one row: thread t holds row t / TPR,
// entries (t % TPR) * EPT .. +EPT.  The two matrix-vector
// products of a row reduce over the TPR consecutive lanes of a row with
// cross-lane adds; the rank-1 update is local.  The step is bound by moving
// the state (read and written once per step).
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

template <typename T, int KD, int VD, int NT>
__global__ void __launch_bounds__(NT)
gdp_decode_k(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
             const float *__restrict__ beta, const float *__restrict__ g, float *__restrict__ state,
             const int32_t *__restrict__ slots, int64_t pool, int L, int H, int HV, float scale,
             T *__restrict__ o) {
    constexpr int EPT = KD * VD / NT;   // state entries per thread
    constexpr int TPR = KD / EPT;       // threads per state row
    constexpr int E = 16 / (int)sizeof(T);
    static_assert(EPT % 4 == 0 && EPT % E == 0 && TPR >= 1 && TPR <= 64 && (TPR & (TPR - 1)) == 0,
                  "state split");
    const int64_t req = blockIdx.x;
    const int hv = blockIdx.y, hk = hv / (HV / H);
    const int tid = threadIdx.x;
    const int vr = tid / TPR, k0 = (tid % TPR) * EPT;
    const bool writer = (tid % TPR) == 0;
    const int64_t slot = slots ? (int64_t)slots[req] : req;

    if (slot < 0 || slot >= pool) {  // skipped request: its rows are zero
        for (int e = 0; e < L; ++e)
            if (writer) o[((req * L + e) * HV + hv) * (int64_t)VD + vr] = from_f32<T>(0.f);
        return;
    }
    float *st = state + ((slot * HV + hv) * (int64_t)VD + vr) * KD + k0;
    float s[EPT];
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
        const f32x4 x = *(const f32x4 *)(st + i);
        s[i] = x[0], s[i + 1] = x[1], s[i + 2] = x[2], s[i + 3] = x[3];
    }
    // sum over the TPR lanes of one state row
    auto row_sum = [](float x) {
#pragma unroll
        for (int d = 1; d < TPR; d <<= 1) x += __shfl_xor(x, d, 64);
        return x;
    };

    for (int e = 0; e < L; ++e) {
        const int64_t row = req * L + e;
        float kr[EPT], qr[EPT];
        const T *kp = k + (row * H + hk) * (int64_t)KD + k0;
        const T *qp = q + (row * H + hk) * (int64_t)KD + k0;
#pragma unroll
        for (int i = 0; i < EPT; i += E) {
            const uint4 ku = *(const uint4 *)(kp + i), qu = *(const uint4 *)(qp + i);
            const T *ke = (const T *)&ku, *qe = (const T *)&qu;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                kr[i + j] = to_f32(ke[j]);
                qr[i + j] = to_f32(qe[j]);
            }
        }
        const float vv = to_f32(v[(row * HV + hv) * (int64_t)VD + vr]);
        const float b = beta[row * HV + hv];
        const float alpha = g ? __expf(g[row * HV + hv]) : 1.0f;
        float ssk = 0.f, ssq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            ssk += kr[i] * kr[i];
            ssq += qr[i] * qr[i];
            sk += s[i] * kr[i];
        }
        ssk = row_sum(ssk);
        ssq = row_sum(ssq);
        sk = row_sum(sk);
        const float rk = 1.0f / sqrtf(ssk + 1e-6f), rq = 1.0f / sqrtf(ssq + 1e-6f);
        const float delta = b * (vv - alpha * (sk * rk));
        const float dk = delta * rk;
        float so = 0.f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            s[i] = alpha * s[i] + dk * kr[i];
            so += s[i] * qr[i];
        }
        so = row_sum(so);
        if (writer) o[(row * HV + hv) * (int64_t)VD + vr] = from_f32<T>(scale * rq * so);
    }
#pragma unroll
    for (int i = 0; i < EPT; i += 4) *(f32x4 *)(st + i) = f32x4{s[i], s[i + 1], s[i + 2], s[i + 3]};
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
