// scan.hip -- segment-parallel form of the inter-chunk state recurrence (the
// chunk_h stage whose outputs core.ssm.ops.gdp.chunk_o consumes, over the w
// and u of core.ssm.ops.gdp.wy_fast, recompute_w_u_fwd).
//
// Over one chunk c the state update of the chunk_h stage is affine in the
// state entering it (h is the K x V transpose of the state S):
//   h <- exp2(gl) h + K^T diag(kdecay) (u - w h)
//      = D_c h + E_c,  D_c = exp2(gl) I - K^T diag(kdecay) w,
//                      E_c = K^T diag(kdecay) u
// (the chunk transition of the WY representation of a product of
// generalised Householder factors).  Composing the maps of the chunks of a
// segment gives the segment's map h_end = D h_start + E, so the long serial
// chain splits into three stages:
//   1. gdp_seg_map_k: every segment (in parallel) runs the recurrence on the
//      augmented state X = [E | D] (K x (V + K)), started from [0 | I] and
//      fed [u | 0].  Both halves follow the update above, so at the
//      segment's end X holds its E and D.
//   2. gdp_seg_scan_k: per value head, a short serial pass over the
//      segments: h_start[s+1] = D_s h_start[s] + E_s, from the caller's
//      initial state.
//   3. the chunk_h stage, all segments at once, each from its h_start (the
//      segments are handed to it as packed sequences with initial states).
// Only the last stage writes h and v_new.
#include "gdp_common.h"
#include "gdp_internal.h"

#include <type_traits>

namespace gdp {

namespace {
constexpr int C = 64;
}  // namespace

// K index held by slot i (= 4 lg + q) of the map kernel's state tile kt.
__device__ __forceinline__ int kperm(int kt, int i) { return 32 * (kt >> 1) + 8 * (i >> 2) + 4 * (kt & 1) + (i & 3); }

// LDS ring of the map kernel, NS stages of one chunk each, grouped by tile
// so that every fragment read is one per-lane offset register plus a
// compile-time offset below 64 KiB: the w and K tiles (rows of KD
// elements, 16-byte units XOR-swizzled by a function of the row), the u tile in 16-column
// slices as in HBM, and the per-row key decays and cumulative decays.
template <int KD, int VD, int NS>
struct MapRing {
    bf16 w[NS][64 * KD];
    bf16 k[NS][64 * KD];
    bf16 u[NS][VD / 16][64 * 16];
    float kd[NS][64];
    float gc[NS][64];
};

// One block of (KD + VD) / 32 waves per (segment, value head); wave wv owns
// columns [32 wv, 32 wv + 32) of X for the whole segment, as fp32 result
// tiles in a permuted K order: xs[kt][ct][q] holds X[kperm(kt, 4 lg + q)]
// [32 wv + 16 ct + lc] with kperm(kt, i) = 32(kt/2) + 8(i/4) + 4(kt%2) +
// i%4, so that the bf16 copy of tiles 2ks and 2ks+1 holds 8 consecutive K
// indices per lane and the w operand of phase 1 is one 16-byte row read.
// Columns below VD are E (fed by u), the others D.  Each chunk streams from
// HBM straight into the three-stage LDS ring (buffer loads with the LDS as
// destination, chunk c + 2's issued late in step c and shared out over all
// waves), so a chunk's loads have more than a step to land and hold no
// registers.
template <int KD, int VD>
__global__ void __launch_bounds__((KD + VD) * 2)
gdp_seg_map_k(QKRows qk, const float *__restrict__ kdecay, const bf16 *__restrict__ w,
              const bf16 *__restrict__ u, const float *__restrict__ gcum, int64_t Ttok, int64_t seg_tok,
              int nmap, int H, int HV, int M, int64_t uv_ss, float *__restrict__ maps,
              const int32_t *__restrict__ seg_cu, const int32_t *__restrict__ seg_last) {
    constexpr int XW = KD + VD;            // columns of X
    constexpr int NW = XW / 32;            // waves
    constexpr int NKT = KD / 16;           // 16-row tiles of X
    constexpr int NKS = KD / 32;           // phase-1 contraction steps
    constexpr int RB = KD * 2;             // bytes per tile row
    constexpr int UPR = RB / 16;           // 16-byte units per tile row
    constexpr int TS = 64 * RB;            // bytes per w or K tile
    constexpr int US = 64 * VD * 2;        // bytes per u tile
    constexpr int NIT = TS / 1024;         // 1 KiB DMA instructions per w or K tile
    constexpr int NIU = US / 1024;         // per u tile
    constexpr int NS = 3;                  // ring stages: loads run two chunks ahead
    typedef MapRing<KD, VD, NS> Ring;
    constexpr int OW = (int)__builtin_offsetof(Ring, w), OK = (int)__builtin_offsetof(Ring, k);
    constexpr int OU = (int)__builtin_offsetof(Ring, u), OD = (int)__builtin_offsetof(Ring, kd);
    constexpr int OG = (int)__builtin_offsetof(Ring, gc);
    static_assert(XW % 64 == 0 && NKS >= 1 && NIT >= NW, "shape: an even number of waves");
    static_assert(2 * TS + 16 * RB * 3 < 65536 && 2 * US + US < 65536, "fragment offsets fit 16 bits");

    __shared__ __attribute__((aligned(16))) Ring ring;

    const int s = (int)(blockIdx.x / HV);
    const int hv = (int)(blockIdx.x % HV);
    if (s >= nmap) return;
    // packed requests: slot s is a segment of the plan; the last segment of
    // each request (and every unused slot) needs no map
    if (seg_cu != nullptr && seg_last[s] != 0) return;
    const int hk = hv / (HV / H);
    const int64_t TM = Ttok * M;
    // first expanded row of the segment: one sequence is cut at multiples of
    // seg_tok; packed requests start where the plan says
    const int64_t r0 = (seg_cu != nullptr ? (int64_t)seg_cu[s] : (int64_t)s * seg_tok) * M;
    const int nch = (int)(seg_tok * M / 64);      // s < nmap: a whole segment, whole chunks

    const int lane = lane_id(), wv = wave_id();
    const int lg = lane >> 4, lc = lane & 15, j = lane & 15;
    const bool is_e = 32 * wv < VD;               // wave-uniform
    const float ue = is_e ? 1.f : 0.f;            // weight of u in the wave's columns
    const uint32_t ring0 = lds_addr(&ring);
    const char *lds = (const char *)&ring;

    // ---- per-lane fragment offsets (bytes from the ring), fixed for the kernel
    // phase 1, w[16rt + lc][32ks + 8lg .. +7] (one unit): o1[ks] + st TS + rt 16 RB
    uint32_t o1[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) o1[ks] = (uint32_t)(OW + lc * RB + ((((4 * ks + lg) ^ lc) & (UPR - 1)) << 4));
    // phase 2, K read transposed: source lane j of group lg points at row
    // 4lg + j/4 (+ 32s + 16h), columns kperm(kt, 0) + 8(j%4) .. +3 (half a
    // unit), so output lane i receives column kperm(kt, i):
    // o2[kt / 2] + 8 (kt % 2) + st TS + (32s + 16h) RB (tiles 2i and 2i + 1
    // read the two halves of the same 16-byte unit)
    // The K tile's units are XOR-swizzled by xk(row mod 16), the w tile's by
    // the row.  With 256-byte rows (KD = 128) the 16 lanes of a group read
    // 4 rows x 4 units; xk's two bit fields put those 16 reads on 16
    // different units, where the row itself put them on 4 (rocprofv3
    // SQ_LDS_BANK_CONFLICT 2.4e7 -> 0.8e7 cycles per launch at the
    // benchmark shape, 6 us less; every lane still reads the same half of
    // its unit, so two groups of a 32-lane pass share the banks).
    auto xk = [](int r) { return UPR == 16 ? ((r & 3) << 2) | ((r >> 2) & 3) : r & (UPR - 1); };
    uint32_t o2[NKT / 2];
    const int ra0 = 4 * lg + (j >> 2);
#pragma unroll
    for (int kp = 0; kp < NKT / 2; ++kp)
        o2[kp] = (uint32_t)(OK + ra0 * RB + ((((4 * kp + (j & 3)) ^ xk(ra0)) & (UPR - 1)) << 4));
    // u slice 2wv + ct, rows 16rt + 4lg + j/4, columns 4(j%4): ou + st US + ct 2048 + rt 512
    const uint32_t ou = (uint32_t)(OU + (is_e ? 2 * wv : 0) * 2048 + (4 * lg + (j >> 2)) * 32 + 8 * (j & 3));
    const uint32_t okd = (uint32_t)(OD + 16 * lg);

    // ---- DMA slots of this wave: instructions wv, wv + NW, ... of the w
    // tile, of the K tile and of the u tile of a chunk.  Instruction ii of a
    // w or K tile fills LDS bytes [1024 ii, 1024 ii + 1024) of the tile: lane
    // L's 16 bytes at 1024 ii + 16 L hold unit (L mod UPR) of row (1024 ii +
    // 16 L) / RB after the swizzle, so the lane fetches the source unit that
    // the swizzle puts there.  Key rows are addressed by token and copy
    // (QKRows: the k tensor or the activations): key copy j of token t sits
    // t k_ts + j k_js elements from the key head's base.
    constexpr int NJT = (NIT + NW - 1) / NW;  // w (and K) slots per wave
    constexpr int NJU = (NIU + NW - 1) / NW;  // u slots per wave
    // loads every wave issues per chunk (some issue more): the ring waits
    // count from this, which is exact or stricter for each wave
    constexpr int MINC = 2 * (NIT / NW) + NIU / NW;
    const int64_t ldw_b = (int64_t)HV * KD * 2;  // w row stride (bytes)
    const uint32_t mdiv = small_div_magic(M);
    const char *kbase = (const char *)qk.k + (int64_t)(hk / qk.hpg) * qk.hs * 2;
    // element offset of expanded row e0 + r from the token holding row e0
    auto krel = [&](int64_t e0, int r) {
        const uint32_t e = (uint32_t)(e0 + r), tb = small_div((uint32_t)e0, mdiv);
        const uint32_t t = small_div(e, mdiv);
        return (int64_t)(t - tb) * qk.k_ts + (int64_t)(e - t * (uint32_t)M) * qk.k_js;
    };
    // when M divides the chunk every chunk starts on a token (r0 is one), so
    // the key rows' offsets are the same for every chunk: made once here
    const bool kfix = (64 % M) == 0;
    uint32_t ow[NJT], okk[NJT];
    int krow[NJT];
#pragma unroll
    for (int jj = 0; jj < NJT; ++jj) {
        const int byte = 1024 * (wv + NW * jj) + 16 * lane;
        const int r = byte / RB, us = (byte % RB) / 16;
        ow[jj] = (uint32_t)(r * ldw_b) + (uint32_t)(16 * ((us ^ r) & (UPR - 1)));
        okk[jj] = (uint32_t)(16 * ((us ^ xk(r & 15)) & (UPR - 1))) + (kfix ? (uint32_t)(krel(r0, r) * 2) : 0u);
        krow[jj] = r;
    }
    // LDS destinations of this wave's slots in stage 0 (slot jj adds
    // 1024 NW jj, stage st adds st TS or st US); u instruction iu fills bytes
    // [1024 iu, 1024 iu + 1024) of the u tile: slice iu / 2, rows 32 (iu % 2) ..
    const uint32_t mw = ring0 + (uint32_t)(OW + 1024 * wv), mk = ring0 + (uint32_t)(OK + 1024 * wv);
    const uint32_t mu = ring0 + (uint32_t)(OU + 1024 * wv);
    // sources of the next chunk to issue, advanced by each issue (NW is even,
    // so slot jj of the u tile is slice wv / 2 + jj NW / 2, same half)
    const char *pw = (const char *)(w + (r0 * HV + hv) * KD);
    const int64_t stw = 64 * ldw_b;
    const char *pkf = kbase + (int64_t)small_div((uint32_t)r0, mdiv) * qk.k_ts * 2;  // kfix: the chunk's first token
    const int64_t stk = kfix ? (int64_t)(64 / M) * qk.k_ts * 2 : 0;
    const uint32_t kspan_fix = kfix ? __builtin_amdgcn_readfirstlane((uint32_t)(krel(r0, 63) * 2)) + RB : 0u;
    int64_t e_issue = r0;  // first expanded row of the next chunk (per-chunk key offsets)
    const char *pu = (const char *)(u + ((int64_t)hv * (VD / 16) + wv / 2) * uv_ss + r0 * 16);
    const int64_t du = (int64_t)(NW / 2) * uv_ss * 2;
    const uint32_t ouu = (uint32_t)(1024 * (wv & 1) + 16 * lane);
    // waves 0 and 1 also load the per-row key decays and cumulative decays
    const char *p4 = (const char *)((wv == 0 ? kdecay : gcum) + (int64_t)hv * TM + r0);
    const uint32_t m4 = ring0 + (uint32_t)(wv == 0 ? OD : OG);
    auto issue = [&](auto stc) {
        constexpr int st = decltype(stc)::value;
        const rsrc_t rw = make_rsrc(pw, (uint32_t)(63 * ldw_b + RB));
        static_for<0, NJT>([&](auto jc) {
            constexpr int jj = decltype(jc)::value;
            if (NIT % NW == 0 || wv + NW * jj < NIT) dma16_at(rw, ow[jj], mw, st * TS + 1024 * NW * jj);
        });
        if (kfix) {
            const rsrc_t rk = make_rsrc(pkf, kspan_fix);
            static_for<0, NJT>([&](auto jc) {
                constexpr int jj = decltype(jc)::value;
                if (NIT % NW == 0 || wv + NW * jj < NIT) dma16_at(rk, okk[jj], mk, st * TS + 1024 * NW * jj);
            });
        } else {  // M does not divide the chunk, so M >= 3 and the divisor's magic is not 0
            const uint32_t e0 = (uint32_t)e_issue, tb = __umulhi(e0, mdiv);
            auto kr = [&](int r) {
                const uint32_t e = e0 + (uint32_t)r, t = __umulhi(e, mdiv);
                return (uint32_t)(((int64_t)(t - tb) * qk.k_ts + (int64_t)(e - t * (uint32_t)M) * qk.k_js) * 2);
            };
            const rsrc_t rk = make_rsrc(kbase + (int64_t)tb * qk.k_ts * 2, __builtin_amdgcn_readfirstlane(kr(63)) + RB);
            static_for<0, NJT>([&](auto jc) {
                constexpr int jj = decltype(jc)::value;
                if (NIT % NW == 0 || wv + NW * jj < NIT) dma16_at(rk, okk[jj] + kr(krow[jj]), mk, st * TS + 1024 * NW * jj);
            });
        }
        static_for<0, NJU>([&](auto jc) {
            constexpr int jj = decltype(jc)::value;
            if (NIU % NW == 0 || wv + NW * jj < NIU)
                dma16_at(make_rsrc(pu + jj * du, 2048), ouu, mu, st * US + 1024 * NW * jj);
        });
        if (wv < 2) dma4_at(make_rsrc(p4, 256), (uint32_t)(4 * lane), m4, st * 256);
        pw += stw;
        pkf += stk;
        e_issue += 64;
        pu += 2048;
        p4 += 256;
    };
    // this wave's loads of the chunk before the last issue have landed
    auto wait_ring = [&]() {
        if (wv < 2)
            wait_vmcnt<MINC + 1>();
        else
            wait_vmcnt<MINC>();
    };
    // the K blocks this wave loaded into ring stage st, bf16 -> fp16 in place
    // (phase 2 takes K^T as fp16; every wave reads the whole tile, so each
    // converts only its own share, once)
    auto convert_k = [&](auto stc) {
        constexpr int st = decltype(stc)::value;
        static_for<0, NJT>([&](auto jc) {
            constexpr int jj = decltype(jc)::value;
            const int ii = wv + NW * jj;
            if (NIT % NW == 0 || ii < NIT) {
                bf16x8 *p = (bf16x8 *)((char *)&ring + OK + st * TS + 1024 * ii + 16 * lane);
                *p = __builtin_bit_cast(bf16x8, bf16_to_f16(*p));
            }
        });
    };

    // X = [0 | I]
    f32x4 xs[NKT][2];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = kperm(kt, 4 * lg + q), col = 32 * wv + 16 * ct + lc;
                xs[kt][ct][q] = (col - VD == row) ? 1.f : 0.f;
            }
    // phase-1 operand: xb[ks][ct] holds X rows 32ks + 8lg + i (slot i) of
    // column 32wv + 16ct + lc
    bf16x8 xb[NKS][2];
    auto pack = [&]() {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xb[ks][ct][q] = (bf16)xs[2 * ks][ct][q];
                    xb[ks][ct][4 + q] = (bf16)xs[2 * ks + 1][ct][q];
                }
    };
    pack();

    // one chunk on ring stage ST (compile-time, so every LDS offset is an
    // immediate on top of the per-lane registers above)
    auto step = [&](int c, auto stc) {
        constexpr int ST = decltype(stc)::value;
        const bool more = c + 2 < nch;  // uniform

        // phase 1: P = w X (64 x 32), contraction order of xb
        f32x4 acc[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 a = *(const bf16x8 *)(lds + o1[ks] + (ST * TS + rt * 16 * RB));
                if (ks == 0) {
                    acc[rt][0] = mma(a, xb[0][0], zero4());
                    acc[rt][1] = mma(a, xb[0][1], zero4());
                } else {
                    acc[rt][0] = mma(a, xb[ks][0], acc[rt][0]);
                    acc[rt][1] = mma(a, xb[ks][1], acc[rt][1]);
                }
            }
        }
        // phase 2: X = exp2(gl) X + K^T (kd ((u | 0) - P)), one half of the
        // contraction (rows 32 s2 .. 32 s2 + 31 of the chunk) at a time, on
        // fp16 operands: K^T as converted in the ring (exact in fp16's normal
        // range) and the fp32 operand kd ((u | 0) - P) rounded to fp16 (11
        // significant bits, saturating), one product per pair where two bf16
        // parts would need two; vb[ct] holds rows 32s2 + 4lg + q (slots 0-3)
        // and 32s2 + 16 + 4lg + q (4-7).  Forming each half's operand just
        // before its products keeps fewer registers live than forming both
        // first.
        const float gl = __builtin_amdgcn_exp2f(ring.gc[ST][63]);  // the chunk's decay (<= 1)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q) xs[kt][ct][q] *= gl;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            f16x8 vb[2];
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int rt = 2 * s2 + r2;
                const f32x4 kd4 = *(const f32x4 *)(lds + okd + (ST * 256 + rt * 64));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    // every wave reads a u slice (the D waves' reads are
                    // weighted by 0), so no branch splits the step
                    const bf16x4 uu = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(lds + ou) +
                                      (ST * US + ct * 2048 + rt * 512))));
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float x = __builtin_fmaf((float)uu[q], ue, -acc[rt][ct][q]) * kd4[q];
                        vb[ct][4 * r2 + q] = f16_sat(x);
                    }
                }
            }
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                typedef __attribute__((address_space(3))) const char *lp;
                const lp pk = (lp)(lds + o2[kt >> 1] + 8 * (kt & 1));
                const bf16x4 x0 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(pk + (ST * TS + 32 * s2 * RB))));
                const bf16x4 x1 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(pk + (ST * TS + (32 * s2 + 16) * RB))));
                const f16x8 a = __builtin_bit_cast(f16x8, join<bf16>(x0, x1));
                xs[kt][0] = mma(a, vb[0], xs[kt][0]);
                xs[kt][1] = mma(a, vb[1], xs[kt][1]);
            }
        }
        // chunk c + 2's loads, issued after this step's products: at the top
        // of the step their issue, waiting on the CU's vector memory path,
        // held back phase 1 (3 us)
        if (more) issue(std::integral_constant<int, (ST + 2) % NS>{});
        // chunk c + 1: this wave's loads have landed (all but this step's
        // own), and its key blocks go to fp16 for the next step
        if (c + 1 < nch) {
            if (more)
                wait_ring();
            else
                wait_vmcnt<0>();
            convert_k(std::integral_constant<int, (ST + 1) % NS>{});
        }
        pack();
        lds_barrier();  // orders LDS only: the DMAs of chunk c + 2 stay in flight
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    issue(I0{});
    if (nch > 1) issue(I1{});
    wait_vmcnt<0>();
    convert_k(I0{});
    lds_barrier();
    for (int c = 0; c < nch; c += 3) {
        step(c, I0{});
        if (c + 1 < nch) step(c + 1, I1{});
        if (c + 2 < nch) step(c + 2, I2{});
    }

    // the segment's map: E (KD x VD fp32, below), then D as matrix-core A
    // fragments of the scan's bf16 products, a high and a low part: 1 KiB
    // block ((rt KD/32 + ks) 2 + part) holds D[16 rt + (L mod 16)][32 ks +
    // 8 (L / 16) .. +7] in lane L's 16 bytes
    float *dst = maps + ((int64_t)s * HV + hv) * KD * XW;
    if (is_e) {
        // E in the scan's accumulator layout: 1 KiB block (sl KD/16 + rt)
        // holds E[16 rt + 4 (L / 16) + q][16 sl + (L mod 16)], q = 0..3, in
        // lane L's 16 bytes; a lane's four rows here are consecutive
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int r0 = kperm(kt, 4 * lg), sl = 2 * wv + ct;  // 16-column slice of the wave's columns 32 wv + 16 ct ..
                *(f32x4 *)(dst + (((sl * (KD / 16) + (r0 >> 4)) * 64 + 16 * ((r0 & 15) >> 2) + lc) << 2)) = xs[kt][ct];
            }
    } else {
        bf16 *df = (bf16 *)(dst + KD * VD);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = kperm(kt, 4 * lg + q), c = 32 * wv - VD + 16 * ct + lc;
                    const int o = ((r >> 4) * (KD / 32) + (c >> 5)) * 1024 + (((c & 31) >> 3) * 16 + (r & 15)) * 8 + (c & 7);
                    const bf16 hi = (bf16)xs[kt][ct][q];
                    df[o] = hi;
                    df[o + 512] = split_lo<bf16>(xs[kt][ct][q], hi);
                }
    }
}

// One block of KD / 32 waves per (value head, 16 value columns): the state
// slice h[k][j0 .. j0+16), carried over the segments in fp32 registers:
// hstart[s] is the state S entering segment s ([nseg, HV, VD, KD], the
// layout of initial states), hstart[s+1] = D_s hstart[s] + E_s.  Wave w owns
// rows [32 w, 32 w + 32) of the result, as two 16x16 tiles.  The product
// runs on bf16 matrix-core tiles with each operand split into a high and a
// low bf16 part (D_s as the map kernel stored it, the state split here):
// D h = Dhi hhi + Dhi hlo + Dlo hhi, the dropped Dlo hlo term and the
// parts' rounding about 2^-16 of each product, with fp32 accumulation.
// Each wave loads its rows of D_s straight into its A fragments (one 1 KiB
// block per instruction), two segments ahead of their use, through two
// register sets; the state's parts go through LDS (two buffers, one barrier
// per segment) as the B operand.  Block 0 also writes the segment offsets
// cu[0..nseg] (tokens).  With packed requests (req_first set) the grid holds
// per_req blocks per request r, each running the same pass over r's
// segments req_first[r] .. + req_nseg[r] - 1 of the plan, from r's initial
// state; the plan kernel has written the offsets.
template <int KD, int VD>
__global__ void __launch_bounds__(KD * 2)
gdp_seg_scan_k(const float *__restrict__ maps, const float *__restrict__ h0, int nseg, int HV, int64_t seg_tok,
               int64_t Ttok, float *__restrict__ hstart, int32_t *__restrict__ cu,
               const int32_t *__restrict__ req_first, const int32_t *__restrict__ req_nseg, int per_req) {
    constexpr int XW = KD + VD;
    constexpr int CB = 16;           // value columns per block
    constexpr int NKS = KD / 32;     // contraction steps
    constexpr int LDB = 2 * KD + 8;  // LDS row stride of the state's parts (bf16)
    constexpr int SL = VD / CB;      // slices per head
    __shared__ __attribute__((aligned(16))) bf16 Hb[2][CB * LDB];  // row j: h[0..KD)[j] high, then low

    // block -> (value head, slice): the slices of one head share an XCD
    // (blocks i and i + 8 do), so each D_s comes from HBM once per head and
    // from that XCD's L2 for the other slices
    int64_t blk = blockIdx.x;
    const int tid = threadIdx.x;
    if (req_first != nullptr) {  // request r: its segments are consecutive slots of the plan
        const int64_t r = blk / per_req;
        blk %= per_req;
        const int64_t s0 = req_first[r];
        nseg = req_nseg[r];
        maps += s0 * HV * KD * XW;
        hstart += s0 * HV * VD * KD;
        if (h0) h0 += r * HV * VD * KD;
    } else if (blk == 0 && tid <= nseg) {
        const int64_t t = (int64_t)tid * seg_tok;
        cu[tid] = (int32_t)(t < Ttok ? t : Ttok);
    }
    const int slot = (int)(blk / 8), xcd = (int)(blk % 8);
    const int hv = (slot / SL) * 8 + xcd;
    const int j0 = (slot % SL) * CB;
    if (hv >= HV || nseg <= 0) return;
    const int lane = lane_id(), wv = wave_id();
    const int lg = lane >> 4, lc = lane & 15;
    // this lane's state entries: h[32 wv + 16 t + 4 lg + q][j0 + lc], in the
    // [VD, KD] layout four consecutive floats
    const int64_t so = (int64_t)(j0 + lc) * KD + 32 * wv + 4 * lg;

    // the map of segment s in flight in registers: this wave's A fragments
    // of D_s (tiles 2 wv + t) and its result tiles' entries of E_s
    struct MapRegs {
        bf16x8 a[2][NKS][2];
        f32x4 e[2];
    };
    auto load_map = [&](MapRegs &R, int s) {
        const float *m = maps + ((int64_t)s * HV + hv) * KD * XW;
        const bf16 *df = (const bf16 *)(m + KD * VD) + 8 * lane;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    R.a[t][ks][p] = *(const bf16x8 *)(df + (((2 * wv + t) * NKS + ks) * 2 + p) * 512);
#pragma unroll
        for (int t = 0; t < 2; ++t) R.e[t] = *(const f32x4 *)(m + ((((j0 >> 4) * (KD / 16) + 2 * wv + t) * 64 + lane) << 2));
    };
    auto write_state = [&](int s, const f32x4 (&h)[2]) {
        float *out = hstart + ((int64_t)s * HV + hv) * VD * KD + so;
        *(f32x4 *)out = h[0];
        *(f32x4 *)(out + 16) = h[1];
    };
    // initial state (S = h^T, V x K)
    f32x4 cur[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) cur[t] = h0 ? *(const f32x4 *)(h0 + (int64_t)hv * VD * KD + so + 16 * t) : zero4();
    const int nm = nseg - 1;  // maps to apply
    MapRegs R0, R1;
    if (nm > 0) load_map(R0, 0);
    if (nm > 1) load_map(R1, 1);
    // state entering segment s (cur) -> hstart[s], then apply map s (from
    // R) and reload R for segment s + 2.  Buffer s % 2 of Hb is rewritten
    // two segments later, after every wave has passed the next barrier and
    // so finished its reads of it.
    auto step = [&](int s, MapRegs &R) {
        bf16 *hb = Hb[s & 1];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x4 hi, lo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hi[q] = (bf16)cur[t][q];
                lo[q] = split_lo<bf16>(cur[t][q], hi[q]);
            }
            const int k0 = 32 * wv + 16 * t + 4 * lg;
            *(bf16x4 *)(&hb[lc * LDB + k0]) = hi;
            *(bf16x4 *)(&hb[lc * LDB + KD + k0]) = lo;
        }
        write_state(s, cur);
        f32x4 acc[2] = {R.e[0], R.e[1]};
        lds_barrier();  // Hb[s % 2] holds the state
        // acc[t] += D[32wv + 16t + .., 32ks + ..] h[32ks + .., ..]: lane holds
        // A[lc][8lg .. +7] = D[row][32ks + 8lg ..] and B = h[32ks + 8lg ..][lc]
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 bh = *(const bf16x8 *)(&hb[lc * LDB + 32 * ks + 8 * lg]);
            const bf16x8 bl = *(const bf16x8 *)(&hb[lc * LDB + KD + 32 * ks + 8 * lg]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                acc[t] = mma(R.a[t][ks][1], bh, acc[t]);
                acc[t] = mma(R.a[t][ks][0], bl, acc[t]);
                acc[t] = mma(R.a[t][ks][0], bh, acc[t]);
            }
        }
        if (s + 2 < nm) load_map(R, s + 2);  // in flight for two segments
        cur[0] = acc[0];
        cur[1] = acc[1];
    };
    int s = 0;
    for (; s + 1 < nm; s += 2) {
        step(s, R0);
        step(s + 1, R1);
    }
    if (s < nm) step(s, R0);
    write_state(nm, cur);  // the state entering the last segment
}

// Segment plan of packed requests (one block): request r of length L_r is
// cut into n_r = ceil(L_r / seg_tok) segments of seg_tok tokens, the last
// one possibly shorter, numbered consecutively over the requests (first
// segment req_first[r]).  Slot s of the plan gets its start seg_cu[s], and
// seg_last[s] = 1 when it is the last segment of its request or unused (no
// map needed).  Unused slots up to nslot are empty segments at the end of
// the packed stream; slots past nslot are dropped (only a non-monotone
// cu_seqlens, whose results are undefined, can ask for more).  Every
// non-last segment holds seg_tok tokens, so its rows are whole chunks and
// its chunk count is a multiple of M.
__global__ void __launch_bounds__(256)
gdp_seg_plan_k(const int32_t *__restrict__ cu_req, int64_t nreq, int64_t Ttok, int64_t seg_tok, int nslot,
               int32_t *__restrict__ seg_cu, int32_t *__restrict__ seg_last, int32_t *__restrict__ req_first,
               int32_t *__restrict__ req_nseg) {
    __shared__ int64_t s_part[4];
    __shared__ int64_t s_carry;
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < nreq; base += 256) {
        const int64_t i = base + tid;
        int64_t bos = 0, eos = 0, n = 0;
        if (i < nreq) {
            seq_bounds(cu_req, Ttok, i, bos, eos);
            n = ceil_div64(eos - bos, seg_tok);
        }
        // block-wide inclusive prefix sum of n
        const int64_t incl_w = wave_inclusive_sum_i64(n);
        if (lane == 63) s_part[wv] = incl_w;
        __syncthreads();
        int64_t before = s_carry;
        for (int w = 0; w < wv; ++w) before += s_part[w];
        const int64_t first = before + incl_w - n;
        if (i < nreq) {
            req_first[i] = (int32_t)(first < nslot ? first : nslot);
            req_nseg[i] = (int32_t)(first + n <= nslot ? n : (first < nslot ? nslot - first : 0));
            for (int64_t j = 0; j < n && first + j < nslot; ++j) {
                seg_cu[first + j] = (int32_t)(bos + j * seg_tok);
                seg_last[first + j] = j + 1 == n ? 1 : 0;
            }
        }
        __syncthreads();
        if (tid == 255) s_carry = first + n;  // inclusive total of this group
        __syncthreads();
    }
    // the end of the last segment, and the unused slots as empty segments there
    int64_t end = 0;
    if (nreq > 0) {
        int64_t b0, e0;
        seq_bounds(cu_req, Ttok, nreq - 1, b0, e0);
        end = e0;
    }
    const int64_t used = s_carry < nslot ? s_carry : nslot;
    for (int64_t s = used + tid; s <= nslot; s += 256) {
        seg_cu[s] = (int32_t)end;
        if (s < nslot) seg_last[s] = 1;
    }
}

// Final state of each packed request (grid: request x value head): the
// state after the last segment, which the chunk_h pass left in place of
// that segment's entering state; the initial state (or zero) for an empty
// request.
__global__ void __launch_bounds__(256)
gdp_seg_final_k(const float *__restrict__ hstart, const float *__restrict__ h0, const int32_t *__restrict__ req_first,
                const int32_t *__restrict__ req_nseg, int HV, int64_t state_elems, float *__restrict__ ht) {
    const int64_t r = blockIdx.x / HV;
    const int hv = (int)(blockIdx.x % HV);
    const int n = req_nseg[r];
    const float *src = n > 0 ? hstart + ((int64_t)(req_first[r] + n - 1) * HV + hv) * state_elems
                             : (h0 ? h0 + (r * HV + hv) * state_elems : nullptr);
    float *dst = ht + (r * HV + hv) * state_elems;
    for (int64_t i = threadIdx.x * 4; i < state_elems; i += 256 * 4)
        *(f32x4 *)(dst + i) = src ? *(const f32x4 *)(src + i) : zero4();
}

template <int KD, int VD>
static hipError_t launch_map_t(const ScanParams &sp, hipStream_t stream) {
    const gdp_chunk_args &a = sp.p.a;
    const bool packed = a.cu_seqlens != nullptr;
    // maps of every segment but the last (of each request): one sequence has
    // nseg - 1; packed requests launch every plan slot and skip the others
    const int64_t nmap = packed ? sp.nseg : sp.nseg - 1;
    if (nmap <= 0) return hipSuccess;
    hipLaunchKernelGGL((gdp_seg_map_k<KD, VD>), dim3((unsigned)(nmap * a.HV)), dim3((KD + VD) * 2), 0, stream,
                       sp.p.qk, a.kdecay, (const bf16 *)a.w, (const bf16 *)a.u, a.gcum, a.T, sp.seg_tok,
                       (int)nmap, a.H, a.HV, a.M, sp.p.uv_ss, sp.maps, packed ? sp.cu : nullptr, sp.seg_last);
    return hipGetLastError();
}

template <int KD, int VD>
static hipError_t launch_scan_t(const ScanParams &sp, hipStream_t stream) {
    const gdp_chunk_args &a = sp.p.a;
    const bool packed = a.cu_seqlens != nullptr;
    const int per_req = (a.HV + 7) / 8 * 8 * (VD / 16);
    const int64_t nblk = packed ? sp.p.nseq * per_req : per_req;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((gdp_seg_scan_k<KD, VD>), dim3((unsigned)nblk), dim3(KD * 2), 0, stream, sp.maps, a.h0,
                       (int)sp.nseg, a.HV, sp.seg_tok, a.T, sp.hstart, sp.cu, packed ? sp.req_first : nullptr,
                       sp.req_nseg, per_req);
    return hipGetLastError();
}

hipError_t launch_seg_plan(const ScanParams &sp, hipStream_t stream) {
    const gdp_chunk_args &a = sp.p.a;
    hipLaunchKernelGGL(gdp_seg_plan_k, dim3(1), dim3(256), 0, stream, a.cu_seqlens, sp.p.nseq, a.T, sp.seg_tok,
                       (int)sp.nseg, sp.cu, sp.seg_last, sp.req_first, sp.req_nseg);
    return hipGetLastError();
}

hipError_t launch_seg_final(const ScanParams &sp, hipStream_t stream) {
    const gdp_chunk_args &a = sp.p.a;
    if (sp.p.nseq == 0) return hipSuccess;
    hipLaunchKernelGGL(gdp_seg_final_k, dim3((unsigned)(sp.p.nseq * a.HV)), dim3(256), 0, stream, sp.hstart, a.h0,
                       sp.req_first, sp.req_nseg, a.HV, (int64_t)a.V * a.K, a.ht);
    return hipGetLastError();
}

hipError_t launch_seg_map(const ScanParams &sp, hipStream_t stream) {
    const gdp_chunk_args &a = sp.p.a;
    if (a.K == 128 && a.V == 128) return launch_map_t<128, 128>(sp, stream);
    if (a.K == 128 && a.V == 64) return launch_map_t<128, 64>(sp, stream);
    if (a.K == 64 && a.V == 128) return launch_map_t<64, 128>(sp, stream);
    if (a.K == 64 && a.V == 64) return launch_map_t<64, 64>(sp, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_seg_scan(const ScanParams &sp, hipStream_t stream) {
    const gdp_chunk_args &a = sp.p.a;
    if (a.K == 128 && a.V == 128) return launch_scan_t<128, 128>(sp, stream);
    if (a.K == 128 && a.V == 64) return launch_scan_t<128, 64>(sp, stream);
    if (a.K == 64 && a.V == 128) return launch_scan_t<64, 128>(sp, stream);
    if (a.K == 64 && a.V == 64) return launch_scan_t<64, 64>(sp, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdp
