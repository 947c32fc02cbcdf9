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

#include <type_traits>

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
// Wave index inside the block, known to the compiler as wave-uniform (it
// can then live in SGPRs and feed buffer descriptors).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp16 operands (values made on chip, where fp16's 11-bit significand is
// the better fit than bf16's 8 bits): v_mfma_f32_16x16x32_f16
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// bf16 values as fp16: exact for magnitudes in fp16's normal range
// [2^-14, 65504]; smaller ones go to fp16's subnormal grid (truncated), larger
// ones saturate at 65504 (the conversion rounds toward zero, so it never
// makes an infinity from a finite value)
__device__ __forceinline__ f16x8 bf16_to_f16(bf16x8 a) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const u32x4 r = __builtin_bit_cast(u32x4, a);
    f16x8 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_bit_cast(float, r[i] << 16), hi = __builtin_bit_cast(float, r[i] & 0xffff0000u);
        const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(lo, hi));
        out[2 * i] = h[0];
        out[2 * i + 1] = h[1];
    }
    return out;
}
// an fp32 value as fp16, rounded to nearest, saturating at +-65504
__device__ __forceinline__ f16 f16_sat(float x) { return (f16)__builtin_amdgcn_fmed3f(x, -65504.0f, 65504.0f); }
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

// A float operand of a bf16 matrix-core product as a sum of two bf16 values:
// hi = from_f32(x), x rounded to bf16, and lo = split_lo(x, hi), the rounded
// remainder (x - hi is exact in float), so hi + lo carries about 16
// significant bits instead of 8.  Two products, one per part, then replace
// one product on the rounded operand.  For float storage nothing is split
// (Split<float>::on is false and lo is never used).
template <typename T> struct Split { static constexpr bool on = false; };
template <> struct Split<bf16> { static constexpr bool on = true; };
template <typename T>
__device__ __forceinline__ T split_lo(float x, T hi) {
    if constexpr (Split<T>::on) return from_f32<T>(x - to_f32(hi));
    else return T(0);
}

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
// x moved across lanes by a DPP pattern; rows outside row_mask, and lanes
// whose source lies outside their row, receive 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes of a wave, on DPP moves only (no
// LDS permutes): a Hillis-Steele scan inside each row of 16 lanes (shifts
// by 1, 2, 4, 8), then row 1 and row 3 add the last lane of the row before
// (row_bcast:15), then rows 2 and 3 add lane 31 (row_bcast:31).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_or_zero<0x111>(x);  // row_shr:1
    x += dpp_or_zero<0x112>(x);  // row_shr:2
    x += dpp_or_zero<0x114>(x);  // row_shr:4
    x += dpp_or_zero<0x118>(x);  // row_shr:8
    x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// ---------------------------------------------------------------- gates
// (core.ssm.ops.gdp.prepare: the gates of gdp_prefill_prepare; shared by the
// prepare kernels and the WY stage that fuses prepare in)
// The gates in float32, in the order and with the functions of the eager
// tensor expressions they replace (core.ssm.ops.gdp.prepare, module
// description: the gates are to match the eager path bit for bit): the
// device's float32 exp and log1p, float32 rounding after each operation,
// no contraction.
// beta = 1 / (1 + exp(-b))
__device__ __forceinline__ float gate_beta(float b) {
#pragma clang fp contract(off)
    const float e = expf(-b);
    const float d = 1.0f + e;
    return 1.0f / d;
}

// g = -exp(A_log) * softplus(a + dt_bias); softplus(s) = s for s > 20,
// else log1p(exp(s)) (core.ssm.ops.gdp.prepare, softplus).
__device__ __forceinline__ float gate_g(float a, float A_log, float dt_bias) {
#pragma clang fp contract(off)
    const float s = a + dt_bias;
    const float sp = s > 20.0f ? s : log1pf(expf(s));
    const float ea = expf(A_log);
    return -(ea * sp);
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

// Exact x / d for 0 <= x < 2^31 and d in [1, 4] (the Householder copy count)
// with one multiply-high: magic = floor((2^32 - 1) / d) + 1, 0 meaning d = 1.
__device__ __forceinline__ uint32_t small_div_magic(int d) { return d == 1 ? 0u : 0xFFFFFFFFu / (uint32_t)d + 1u; }
// x / d for x >= 0 and d in {1, 2, 3, 4}, exact over the whole range: a
// shift, or for 3 the high half of x * ceil(2^65 / 3) shifted once more
__device__ __forceinline__ int64_t div_m(int64_t x, int d) {
    return d == 3 ? (int64_t)(__umul64hi((uint64_t)x, 0xAAAAAAAAAAAAAAABull) >> 1) : x >> (d >> 1);
}
__device__ __forceinline__ uint32_t small_div(uint32_t x, uint32_t magic) { return magic ? __umulhi(x, magic) : x; }

// A value the caller knows is the same in every lane, made visibly uniform
// (scalar registers) for the compiler.
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum of a 64-bit value over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_inclusive_sum_i64(int64_t x) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t y = __shfl_up(x, d, 64);
        if (lane_id() >= d) x += y;
    }
    return x;
}
// Sum of a 64-bit value over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

// Cross-row moves on gfx950's permlane swaps (VALU, no LDS permutes).
// v_permlane16_swap exchanges the odd 16-lane rows of one operand with the
// even rows of the other, v_permlane32_swap the upper half of one with the
// lower half of the other; with both operands x the two results together
// hold x and its partner row in every lane.
__device__ __forceinline__ float xor16_sum(float x) {  // x + x[lane ^ 16], bit for bit
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {  // x + x[lane ^ 32], bit for bit
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x[16 row + lane % 16] in every lane (row wave-uniform, 0..3)
__device__ __forceinline__ float row_broadcast(float x, int row) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t b = row < 2 ? a[0] : a[1];  // rows (row & ~1, row | 1) twice
    const auto c = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return __uint_as_float((row & 1) ? c[1] : c[0]);
}

// x moved across lanes by a DPP pattern (every source lane is in range for
// the patterns used here).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over each aligned group of N consecutive lanes (N a power of two up to
// 64); every lane of the group gets the same bits.  Within 16 lanes the
// partners come from DPP: swap neighbours, swap pairs, mirror the half row,
// mirror the row -- after each step all lanes of the growing group agree;
// across rows from the permlane swaps.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group size");
    if constexpr (N >= 2) x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp_move<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp_move<0x140>(x); // row_mirror
    if constexpr (N >= 32) x = xor16_sum(x);
    if constexpr (N >= 64) x = xor32_sum(x);
    return x;
}

// Block-cooperative lookup of linear item `id` over sequences, where
// sequence i owns ceil(len_i * rows_per_token / chunk) consecutive items.
// Every thread of the block must call it (it uses barriers); wave 0 scans
// the sequences 64 at a time, so any block size works.  Returns the
// sequence (or -1 if id is past the last item), the item's index inside its
// sequence, and the number of items of all earlier sequences.
struct ChunkLoc {
    int64_t seq, c, base, bos, eos;
};

__device__ __forceinline__ ChunkLoc find_chunk(const int32_t *cu, int64_t nseq, int64_t T,
                                               int64_t rows_per_token, int64_t chunk, int64_t id) {
    ChunkLoc r;
    if (cu == nullptr) {
        // chunk counts and ids stay below 2^31 (the launch limits), so the
        // division runs in 32 bits
        const int64_t per = ceil_div64(T * rows_per_token, chunk);
        const uint32_t q = per > 0 ? (uint32_t)id / (uint32_t)per : 0u;
        r.seq = per > 0 ? (int64_t)q : -1;
        if (r.seq >= nseq) r.seq = -1;
        r.c = per > 0 ? (int64_t)((uint32_t)id - q * (uint32_t)per) : 0;
        r.base = r.seq >= 0 ? r.seq * per : 0;
        seq_bounds(nullptr, T, r.seq < 0 ? 0 : r.seq, r.bos, r.eos);
        return r;
    }
    __shared__ int64_t s_found[3];
    if (wave_id() == 0) {
        const int lane = lane_id();
        if (lane == 0) {
            s_found[0] = -1;
            s_found[1] = 0;
            s_found[2] = 0;
        }
        int64_t carry = 0;
        for (int64_t i0 = 0; i0 < nseq; i0 += 64) {
            const int64_t i = i0 + lane;
            int64_t n = 0;
            if (i < nseq) {
                int64_t b, e;
                seq_bounds(cu, T, i, b, e);
                n = ceil_div64((e - b) * rows_per_token, chunk);
            }
            const int64_t incl = carry + wave_inclusive_sum_i64(n);
            const int64_t excl = incl - n;
            if (i < nseq && n > 0 && id >= excl && id < incl) {  // at most one lane
                s_found[0] = i;
                s_found[1] = id - excl;
                s_found[2] = excl;
            }
            carry = __shfl(incl, 63, 64);
        }
    }
    __syncthreads();
    r.seq = uniform_i64(s_found[0]);
    r.c = uniform_i64(s_found[1]);
    r.base = uniform_i64(s_found[2]);
    if (r.seq >= 0) seq_bounds(cu, T, r.seq, r.bos, r.eos);
    else { r.bos = 0; r.eos = 0; }
    __syncthreads();
    return r;
}

// Number of items of sequences [0, i) (block-cooperative, barriers inside;
// any block size up to 1024 threads).
__device__ __forceinline__ int64_t items_before(const int32_t *cu, int64_t T, int64_t rows_per_token,
                                                int64_t chunk, int64_t i) {
    if (cu == nullptr) return i * ceil_div64(T * rows_per_token, chunk);
    __shared__ int64_t s_part[16];
    const int tid = threadIdx.x, nt = blockDim.x;
    int64_t acc = 0;
    for (int64_t j = tid; j < i; j += nt) {
        int64_t b, e;
        seq_bounds(cu, T, j, b, e);
        acc += ceil_div64((e - b) * rows_per_token, chunk);
    }
    acc = wave_sum_i64(acc);
    __syncthreads();
    if (lane_id() == 0) s_part[tid >> 6] = acc;
    __syncthreads();
    int64_t r = 0;
    for (int w = 0; w < (nt + 63) / 64; ++w) r += s_part[w];
    __syncthreads();
    return uniform_i64(r);
}

// Index of (head hd, expanded row e) in a head-major per-row array
// [B, NH, T*M]: e is the flattened expanded row over all batch rows, bi the
// batch row it belongs to (0 for packed sequences) and TM = T*M.
__device__ __forceinline__ int64_t hm_index(int64_t bi, int nh, int hd, int64_t TM, int64_t e) {
    return (bi * nh + hd) * TM + (e - bi * TM);
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
            s = group_sum<UPR>(s);
            if (cu == 0) ssq[row] = s;
        }
    }
}

// ---------------------------------------------------------------- buffer access
// Raw buffer resources: the hardware range check returns zeros for loads
// past `bytes` and drops stores past it, which handles ragged tails without
// per-row branches.  Offsets are 32-bit byte offsets from `base`.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, untyped access

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, uint2 v) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 v) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)off, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, then s_barrier.  Outstanding global loads stay in flight (a
// plain __syncthreads also drains them).  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- HBM -> LDS DMA
// buffer_load ... lds: each lane's 16 (or 4) bytes land at LDS address
// lds_base + 16*lane (4*lane).  Issued through inline assembly so the
// compiler does not add its conservative wait-for-everything before later
// LDS reads; the caller waits with wait_vmcnt<N>() where N counts only DMAs
// issued after the ones it needs (other vector memory operations in between
// can only make that wait stricter, never looser, as the counter retires in
// order).  lds_base must be wave-uniform.  Lanes outside the buffer range do
// not fetch memory and write zeros.  One wait state separates the M0 write
// from the DMA that reads it.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voffset, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_base), "v"(voffset), "s"(r) : "memory");
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voffset, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds_base), "v"(voffset), "s"(r) : "memory");
}
// As dma16 / dma4 with the LDS destination at lds_base + off (off a
// compile-time constant folded into the M0 write).
__device__ __forceinline__ void dma16_at(rsrc_t r, uint32_t voffset, uint32_t lds_base, int off) {
    asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_base), "v"(voffset), "s"(r), "i"(off) : "memory", "scc");
}
__device__ __forceinline__ void dma4_at(rsrc_t r, uint32_t voffset, uint32_t lds_base, int off) {
    asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds_base), "v"(voffset), "s"(r), "i"(off) : "memory", "scc");
}
// Windowed form: set_m0(base) once, then up to four dma16_m0<IMM> whose LDS
// destination is base + IMM (+ 16*lane).  The 12-bit instruction offset is
// added to both the LDS and the memory address and is part of the buffer
// range check, so the caller passes voffset - IMM.
__device__ __forceinline__ void set_m0(uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" :: "s"(lds_base) : "memory");
}
template <int IMM>
__device__ __forceinline__ void dma16_m0(rsrc_t r, uint32_t voffset) {
    static_assert(IMM >= 0 && IMM < 4096, "12-bit instruction offset");
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds" :: "v"(voffset), "s"(r), "n"(IMM) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// 32-bit LDS byte address of a __shared__ object.
template <typename P>
__device__ __forceinline__ uint32_t lds_addr(const P *p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)p);
}

}  // namespace gdp
