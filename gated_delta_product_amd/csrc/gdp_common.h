// gdp_common.h -- device helpers shared by the gfx950 GDP kernels.
//
// Matrix-core conventions (16x16 output tiles, one wave64):
//   A operand (16 rows x 32 contraction): lane l holds A[l%16][8*(l/16) + i]
//   B operand (32 contraction x 16 cols): lane l holds B[8*(l/16) + i][l%16]
//   result    (16 x 16, f32):              lane l holds D[4*(l/16) + i][l%16]
// For bf16 one v_mfma_f32_16x16x32_bf16 consumes a fragment pair; for f32
// eight v_mfma_f32_16x16x4_f32 do (call i contracts slot i of every lane).
// The contraction order inside a fragment is free as long as the A and B
// fragments agree, which several kernels use to feed a result tile straight
// back as an operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; typedef bf16x4 half; };
template <> struct Frag<float> { typedef f32x8 type; typedef f32x4 half; };

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// ---------------------------------------------------------------- LDS fragments
// 8 consecutive elements of one row of a row-major LDS tile (16-byte aligned).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_row8(const T *p) {
    return *(const typename Frag<T>::type *)p;
}

// Four consecutive rows of one column: lane (g = l/16, c = l%16) receives
// X[rowA + r][col0 + c] for r = 0..3, where rowA may differ between the four
// 16-lane groups but is uniform inside one.  X is row-major in LDS with
// `stride` elements per row.  For bf16 this is one ds_read_b64_tr_b16: in a
// 16-lane group, source lane s points at X[rowA + s/4][col0 + 4*(s%4)] and
// output lane i slot r comes from source lane 4r + i/4, slot i%4.
template <typename T>
__device__ __forceinline__ typename Frag<T>::half lds_col4(const T *X, int stride, int rowA, int col0);

template <>
__device__ __forceinline__ bf16x4 lds_col4<bf16>(const bf16 *X, int stride, int rowA, int col0) {
    const int s = lane_id() & 15;
    const bf16 *p = X + (rowA + (s >> 2)) * stride + col0 + 4 * (s & 3);
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)p));
    return __builtin_bit_cast(bf16x4, r);
}
template <>
__device__ __forceinline__ f32x4 lds_col4<float>(const float *X, int stride, int rowA, int col0) {
    const int c = lane_id() & 15;
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = X[(rowA + i) * stride + col0 + c];
    return r;
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::type join(typename Frag<T>::half a, typename Frag<T>::half b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Fragment of 8 rows (rowA..rowA+3, rowB..rowB+3) at column col0 + l%16.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_col8(const T *X, int stride, int rowA, int rowB, int col0) {
    return join<T>(lds_col4<T>(X, stride, rowA, col0), lds_col4<T>(X, stride, rowB, col0));
}

// ---------------------------------------------------------------- wave scans
__device__ __forceinline__ float wave_inclusive_sum(float x) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        float y = __shfl_up(x, d, 64);
        if (lane_id() >= d) x += y;
    }
    return x;
}

// ---------------------------------------------------------------- sequences
// Token range [bos, eos) of sequence i in the flattened [B*T] token stream.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int64_t T, int64_t i,
                                           int64_t &bos, int64_t &eos) {
    if (cu == nullptr) {
        bos = i * T;
        eos = bos + T;
    } else {
        int64_t a = cu[i], b = cu[i + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        bos = a;
        eos = b;
    }
}

__device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Block-cooperative lookup of linear item `id` over sequences, where
// sequence i owns ceil(len_i * rows_per_token / chunk) consecutive items.
// Every thread of the block must call it (it uses barriers).  Returns the
// sequence (or -1 if id is past the last item), the item's index inside its
// sequence, and the number of items of all earlier sequences.
struct ChunkLoc {
    int64_t seq, c, base, bos, eos;
};

__device__ __forceinline__ ChunkLoc find_chunk(const int32_t *cu, int64_t nseq, int64_t T,
                                               int64_t rows_per_token, int64_t chunk, int64_t id) {
    ChunkLoc r;
    if (cu == nullptr) {
        const int64_t per = ceil_div64(T * rows_per_token, chunk);
        r.seq = per > 0 ? id / per : -1;
        if (r.seq >= nseq) r.seq = -1;
        r.c = per > 0 ? id % per : 0;
        r.base = r.seq >= 0 ? r.seq * per : 0;
        seq_bounds(nullptr, T, r.seq < 0 ? 0 : r.seq, r.bos, r.eos);
        return r;
    }
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_found[3];
    const int tid = threadIdx.x, nt = blockDim.x;
    if (tid == 0) { s_found[0] = -1; s_found[1] = 0; s_found[2] = 0; }
    int64_t carry = 0;
    for (int64_t i0 = 0; i0 < nseq; i0 += nt) {
        __syncthreads();
        const int64_t i = i0 + tid;
        int64_t n = 0;
        if (i < nseq) {
            int64_t b, e;
            seq_bounds(cu, T, i, b, e);
            n = ceil_div64((e - b) * rows_per_token, chunk);
        }
        s_scan[tid] = n;
        __syncthreads();
        for (int d = 1; d < nt; d <<= 1) {
            int64_t y = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += y;
            __syncthreads();
        }
        const int64_t incl = carry + s_scan[tid];
        const int64_t excl = incl - n;
        if (i < nseq && n > 0 && id >= excl && id < incl) {
            s_found[0] = i;
            s_found[1] = id - excl;
            s_found[2] = excl;
        }
        carry += s_scan[nt - 1];
    }
    __syncthreads();
    r.seq = s_found[0];
    r.c = s_found[1];
    r.base = s_found[2];
    if (r.seq >= 0) seq_bounds(cu, T, r.seq, r.bos, r.eos);
    else { r.bos = 0; r.eos = 0; }
    __syncthreads();
    return r;
}

// Number of items of sequences [0, i) (block-cooperative, barriers inside).
__device__ __forceinline__ int64_t items_before(const int32_t *cu, int64_t T, int64_t rows_per_token,
                                                int64_t chunk, int64_t i) {
    if (cu == nullptr) return i * ceil_div64(T * rows_per_token, chunk);
    __shared__ int64_t s_red[256];
    const int tid = threadIdx.x, nt = blockDim.x;
    int64_t acc = 0;
    for (int64_t j = tid; j < i; j += nt) {
        int64_t b, e;
        seq_bounds(cu, T, j, b, e);
        acc += ceil_div64((e - b) * rows_per_token, chunk);
    }
    __syncthreads();
    s_red[tid] = acc;
    __syncthreads();
    for (int d = nt / 2; d > 0; d >>= 1) {
        if (tid < d) s_red[tid] += s_red[tid + d];
        __syncthreads();
    }
    int64_t r = s_red[0];
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------- tile staging
// Copy ROWS rows of D elements (global row stride `rs` elements) into a
// row-major LDS tile with row stride LD, using 16-byte units spread over the
// whole block (NT threads).  Rows >= n are zero-filled.  If ssq is given, the
// per-row sum of squares of the stored values is written to ssq[row]; this
// needs the units of one row to sit in consecutive lanes of one wave.
template <typename T, int ROWS, int D, int LD, int NT>
__device__ __forceinline__ void stage_tile(T *dst, const T *src, int64_t rs, int n, float *ssq) {
    constexpr int E = 16 / sizeof(T);
    constexpr int UPR = D / E;
    static_assert(UPR <= 64 && (UPR & (UPR - 1)) == 0, "row must fit one wave");
    static_assert((ROWS * UPR) % NT == 0, "tile must split evenly");
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < (ROWS * UPR) / NT; ++it) {
        const int uidx = tid + NT * it;
        const int row = uidx / UPR, cu = uidx % UPR;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (row < n) val = *(const uint4 *)(src + (int64_t)row * rs + cu * E);
        *(uint4 *)(dst + row * LD + cu * E) = val;
        if (ssq) {
            const T *e = (const T *)&val;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float f = to_f32(e[i]);
                s += f * f;
            }
#pragma unroll
            for (int d = 1; d < UPR; d <<= 1) s += __shfl_xor(s, d, 64);
            if (cu == 0) ssq[row] = s;
        }
    }
}

}  // namespace gdp
