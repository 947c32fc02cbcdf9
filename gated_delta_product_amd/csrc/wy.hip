// wy.hip -- per-chunk WY factors of the Gated Delta Product
// (core.ssm.ops.gdp.wy_fast: module description, recompute_w_u_fwd).
//
// One block (4 waves) per (64-row chunk of the expanded stream, value head),
// heads fastest in the launch order.
// Fused steps, all on chip:
//   khat = k / sqrt(sum k^2 + 1e-6)           (L2 norm left to the chunk op,
//                                               core.ssm.ops.gdp.prepare, Returns)
//   gamma_e = within-chunk cumulative log decay; a token's decay sits on its
//             first copy (also written out in log2 units for chunk_h, with
//             kdecay_e = rnorm_e exp(gamma_last - gamma_e))
//   L[a][b] = beta_a exp(gamma_a - gamma_b) khat_a . khat_b   (b < a)
//   A = (I + L)^-1                             (the solve_tril block)
//   u = A diag(beta) V                         (effective values)
//   w = A diag(beta exp(gamma)) Khat           (effective keys with decay)
// The Gram matrix K K^T and the two products run on the matrix cores (bf16 in,
// fp32 accumulate); the norms are applied as fp32 row scales so the raw bf16
// inputs are the operands.  The fp32 factors A diag(beta) and
// A diag(beta e^gamma r) enter the two products as a high and a low bf16
// part (two products each), so A is not cut to 8 significant bits.  A is
// built in fp32: the four 16x16 diagonal blocks by forward substitution (one
// lane per column), the off-diagonal blocks level by level with fp32 MFMA:
// A_ij = -A_ii sum_{j<=m<i} L_im A_mj.
// L and A share one LDS array: A's diagonal blocks replace L's (dead once
// solved) and its lower blocks are stored transposed in the upper triangle,
// which L leaves unused; the lower blocks of L stay intact until the last
// level, after which A's lower blocks move into their place.  With that array, the K tile and the gates the block takes about
// 35 KB of LDS at K = V = 128 bf16, so four blocks share a CU.
// u and w are computed transposed (u^T = V^T A1^T) so each lane ends up with
// four consecutive columns of one output row, stored as one 8-byte write.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

namespace {

constexpr int C = 64;      // chunk rows
constexpr int LDA = C + 4;  // fp32 row stride of L and A in LDS

// 16 bytes of padding per LDS row: row reads of 16 consecutive rows hit 16
// distinct bank groups
template <typename T> struct Pad { static constexpr int value = 16 / (int)sizeof(T); };

}  // namespace

// With FUSE the block also does the prefill prepare of its rows (one
// sequence, HV == H): it reads its key and value copies, query and gate
// inputs straight from the post-conv activations x and ba (layouts of
// core.ssm.ops.gdp.prepare, gdp_prefill_prepare), writes prepare's outputs
// for them (q, k, v, beta, g, exactly as the prepare kernel does; q and g of
// a token by the block holding its copy 0) and uses the same values.  v and
// beta may be NULL: no later stage reads them (the values enter u here), so
// they are then not stored.  q and k may be NULL together: the later stages
// then read their rows from x, and they are neither stored nor (q) loaded.
template <typename T>
struct WyFuse {
    const T *x;
    int64_t xts;  // x row stride (elements)
    const T *ba;
    int64_t bts;  // ba row stride (elements)
    const float *A_log, *dt_bias;
    int G;
    T *q, *k, *v;
    float *beta, *g;
};

template <typename T, int KD, int VD, bool FUSE>
__global__ void __launch_bounds__(256)
gdp_wy_k(const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ beta,
         const float *__restrict__ g, const int32_t *__restrict__ cu, int64_t nseq, int64_t Ttok,
         int H, int HV, int M, float *__restrict__ k_rnorm, float *__restrict__ gcum,
         float *__restrict__ kdecay, T *__restrict__ w,
         T *__restrict__ u, int64_t uv_ss, WyFuse<T> fz, int64_t seg_nch, int64_t seg_n) {
    typedef typename Frag<T>::type FragT;
    constexpr int LDK = KD + Pad<T>::value;
    constexpr int LDV = VD + Pad<T>::value;
    constexpr int LA_BYTES = (C * LDA * 4 > C * LDV * (int)sizeof(T)) ? C * LDA * 4 : C * LDV * (int)sizeof(T);
    constexpr int VUPR = VD * (int)sizeof(T) / 16;   // 16-byte units per V row
    constexpr int VPT = C * VUPR / 256;               // V units per thread
    __shared__ __attribute__((aligned(16))) T Ks[C * LDK];
    // L and A (fp32, row stride LDA) while A is being built, then the V
    // tile (V waits in registers until then)
    __shared__ __attribute__((aligned(16))) char LA[LA_BYTES];
    __shared__ __attribute__((aligned(16))) float s_beta[C], s_gam[C], s_rk[C], s_ws[C];
    float *Lm = (float *)LA;
    T *Vs = (T *)LA;
    // A[r][c] for r, c in the same 16-row block or r > c: the diagonal
    // blocks in place, the lower blocks transposed
    auto a_at = [&](int r, int c) -> float & {
        return (r >> 4) == (c >> 4) ? Lm[r * LDA + c] : Lm[c * LDA + r];
    };

    // block -> (chunk, value head), heads fastest: the blocks in flight
    // together cover whole rows of k, v and w (all heads of a few chunks),
    // so HBM sees long contiguous runs
    const int64_t lin = blockIdx.x;
    // launch ids and chunk counts stay below 2^31 (the launch limits): 32-bit
    // divisions
    int64_t ci = (uint32_t)lin / (uint32_t)HV;
    // With a segment plan (one sequence, seg_n segments of seg_nch chunks,
    // the last one nlast <= seg_nch), chunk j of every segment goes before
    // chunk j - 1 of any: the segment maps, which start at each segment's
    // first chunk, then meet the most recently written lines first.
    if (seg_n > 1) {
        const uint32_t F = (uint32_t)(seg_n - 1), nlast = (uint32_t)((Ttok * M + C - 1) / C - F * seg_nch);
        const uint32_t hi = ((uint32_t)seg_nch - nlast) * F;  // launch slots of the chunks j >= nlast (F each)
        const uint32_t c32 = (uint32_t)ci;
        uint32_t j, sg;
        if (c32 < hi) {
            j = (uint32_t)seg_nch - 1 - c32 / F;
            sg = c32 % F;
        } else {
            j = nlast - 1 - (c32 - hi) / (F + 1);
            sg = (c32 - hi) % (F + 1);
        }
        ci = (int64_t)sg * seg_nch + j;
    }
    const ChunkLoc loc = find_chunk(cu, nseq, Ttok, M, C, ci);
    if (loc.seq < 0) return;
    const int hv = (int)((uint32_t)lin % (uint32_t)HV);
    const int hk = hv / (HV / H);
    const int64_t r0 = loc.bos * M + C * loc.c;  // first expanded row (global)
    const int64_t rend = loc.eos * M;
    const int n = (int)((rend - r0) < C ? (rend - r0) : C);
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int lg = lane >> 4, lc = lane & 15;
    const int64_t bi = cu ? 0 : loc.seq, TM = Ttok * M;  // head-major per-row outputs

    // ---- every global load of the block goes out first: the gates (wave
    // 0), V into registers (it is needed last), then K into LDS with row
    // norms, so their latencies overlap
    const int64_t e_row = r0 + lane;
    const bool e_in = lane < n;
    float b_in = 0.f, gd_in = 0.f;
    if constexpr (FUSE) {
        // (the gates are computed below, once the tile loads are out)
    } else if (wv == 0) {
        b_in = e_in ? beta[e_row * HV + hv] : 0.f;
        gd_in = (g != nullptr && e_in && e_row - div_m(e_row, M) * M == 0) ? g[div_m(e_row, M) * HV + hv] : 0.f;  // NULL: ungated
    }
    uint4 vreg[VPT];
    if constexpr (FUSE) {
        // value copy j of token t: x[t, (j H + h) P ..]; key copy j: x[t,
        // M H P + (j G + h / (H/G)) N ..]; query: x[t, M H P + M G N +
        // (h / (H/G)) N ..] (value head h == key head)
        constexpr int E = 16 / (int)sizeof(T);
        constexpr int KUPR = KD / E;          // units per key row (one wave holds whole rows)
        constexpr int KPT = (C * KUPR) / 256;  // key units per thread
        const int grp = hv / (H / fz.G);
        const int64_t kb = (int64_t)M * H * VD, qb = kb + (int64_t)M * fz.G * KD;
        // every load first (values, keys, the queries of copy-0 rows), then
        // the stores, so the loads' latencies overlap
        uint4 kreg[KPT], qreg[KPT];
#pragma unroll
        for (int it = 0; it < VPT; ++it) {
            const int uidx = tid + 256 * it, row = uidx / VUPR, cu16 = uidx % VUPR;
            vreg[it] = make_uint4(0, 0, 0, 0);
            if (row < n) {
                const int64_t e = r0 + row, t = div_m(e, M);
                const int j = (int)(e - t * M);
                vreg[it] = *(const uint4 *)(fz.x + t * fz.xts + ((int64_t)j * H + hv) * VD + cu16 * E);
            }
        }
#pragma unroll
        for (int it = 0; it < KPT; ++it) {
            const int uidx = tid + 256 * it, row = uidx / KUPR, cu16 = uidx % KUPR;
            kreg[it] = make_uint4(0, 0, 0, 0);
            qreg[it] = make_uint4(0, 0, 0, 0);
            if (row < n) {
                const int64_t e = r0 + row, t = div_m(e, M);
                const int j = (int)(e - t * M);
                kreg[it] = *(const uint4 *)(fz.x + t * fz.xts + kb + ((int64_t)j * fz.G + grp) * KD + cu16 * E);
                if (j == 0 && fz.q != nullptr)
                    qreg[it] = *(const uint4 *)(fz.x + t * fz.xts + qb + (int64_t)grp * KD + cu16 * E);
            }
        }
        // the gates of the block's rows: beta per row, g per token (on its copy 0)
        if (wv == 0 && e_in) {
            const int64_t t = div_m(e_row, M);
            const int j = (int)(e_row - t * M);
            b_in = gate_beta(to_f32(fz.ba[t * fz.bts + j * H + hv]));
            if (j == 0) gd_in = gate_g(to_f32(fz.ba[t * fz.bts + M * H + hv]), fz.A_log[hv], fz.dt_bias[hv]);
        }
        if (fz.v != nullptr) {
#pragma unroll
            for (int it = 0; it < VPT; ++it) {
                const int uidx = tid + 256 * it, row = uidx / VUPR, cu16 = uidx % VUPR;
                if (row < n) *(uint4 *)(fz.v + ((r0 + row) * H + hv) * (int64_t)VD + cu16 * E) = vreg[it];
            }
        }
        if (wv == 0 && e_in) {
            const int64_t t = div_m(e_row, M);
            if (fz.beta != nullptr) fz.beta[e_row * H + hv] = b_in;
            if (e_row - t * M == 0) fz.g[t * H + hv] = gd_in;
        }
#pragma unroll
        for (int it = 0; it < KPT; ++it) {
            const int uidx = tid + 256 * it, row = uidx / KUPR, cu16 = uidx % KUPR;
            const int64_t e = r0 + row, t = div_m(e, M);
            const int j = (int)(e - t * M);
            if (row < n && fz.k != nullptr) {  // q and k may be NULL: the later stages then read x
                *(uint4 *)(fz.k + (e * H + hv) * (int64_t)KD + cu16 * E) = kreg[it];
                if (j == 0) *(uint4 *)(fz.q + (t * H + hv) * (int64_t)KD + cu16 * E) = qreg[it];  // once per token
            }
            *(uint4 *)(Ks + row * LDK + cu16 * E) = kreg[it];
            const T *el = (const T *)&kreg[it];
            float sq = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float f = to_f32(el[i]);
                sq += f * f;
            }
            sq = group_sum<KUPR>(sq);  // DPP within 16 lanes, bit for bit the xor butterfly
            if (cu16 == 0) s_rk[row] = sq;
        }
    } else {
        const T *vsrc = v + (r0 * HV + hv) * (int64_t)VD;
#pragma unroll
        for (int it = 0; it < VPT; ++it) {
            const int uidx = tid + 256 * it, row = uidx / VUPR, cu16 = uidx % VUPR;
            vreg[it] = row < n ? *(const uint4 *)(vsrc + (int64_t)row * HV * VD + cu16 * (16 / (int)sizeof(T)))
                               : make_uint4(0, 0, 0, 0);
        }
        stage_tile<T, C, KD, LDK, 256>(Ks, k + (r0 * H + hk) * (int64_t)KD, (int64_t)H * KD, n, s_rk);
    }
    if (wv == 0) {
        const float gam = wave_inclusive_sum(gd_in);
        s_beta[lane] = b_in;
        s_gam[lane] = gam;
        if (e_in) gcum[hm_index(bi, HV, hv, TM, e_row)] = gam * 1.4426950408889634f;  // log2 units for chunk_h
    }
    __syncthreads();

    if (wv == 0) {
        const float rk = 1.0f / sqrtf(s_rk[lane] + 1e-6f);
        s_rk[lane] = rk;
        s_ws[lane] = s_beta[lane] * __expf(s_gam[lane]) * rk;
        if (lane < n && (hv % (HV / H)) == 0) k_rnorm[hm_index(bi, H, hk, TM, r0 + lane)] = rk;
        if (lane < n) {  // decay of the row's key to the chunk end, times its norm
            const float g2 = s_gam[lane] * 1.4426950408889634f;
            const float gl2 = s_gam[n - 1] * 1.4426950408889634f;
            kdecay[hm_index(bi, HV, hv, TM, r0 + lane)] = rk * exp2f(gl2 - g2);
        }
    }
    __syncthreads();

    // ---- diagonal 16x16 block d of A by forward substitution (lane =
    // column), in place of L's: every row of the block is read before any is
    // written.  It needs only L's diagonal tile d, which the same wave has
    // just written (one wave's LDS accesses complete in order).
    auto solve_diag = [&](int d0) {
        if (lane < 16) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == lane) ? 1.f : 0.f;
                f32x4 lr[4];  // row i of the diagonal block (same address in every lane)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (4 * q < i) lr[q] = *(const f32x4 *)&Lm[(d0 + i) * LDA + d0 + 4 * q];
#pragma unroll
                for (int b = 0; b < i; ++b) s -= lr[b >> 2][b & 3] * x[b];
                x[i] = s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Lm[(d0 + i) * LDA + d0 + lane] = x[i];
        }
    };

    // ---- L = strictly lower beta_a exp(g_a - g_b) r_a r_b (K K^T)_ab: the
    // ten 16x16 tiles (rt, ct <= rt) shared out three, three, two and two
    // over the waves, each wave's first tile a diagonal one, whose block of
    // A it then solves at once, so the solves overlap the other waves' tiles
    // and need no barrier of their own.  Tile (rt, ct) is coded rt * 4 + ct,
    // one byte per tile of a wave.
    {
        const uint32_t tiles = wv == 0 ? 0x000D0C00u : (wv == 1 ? 0x000E0405u : (wv == 2 ? 0x0000080Au : 0x0000090Fu));
        const int ntile = wv < 2 ? 3 : 2;
        for (int it = 0; it < ntile; ++it) {
            const int code = (int)((tiles >> (8 * it)) & 0xffu), rt = code >> 2, ct = code & 3;
            const int ra = 16 * rt;
            // factors of this lane's four rows: beta * rnorm, and gamma
            const f32x4 b4 = *(const f32x4 *)&s_beta[ra + 4 * lg], r4 = *(const f32x4 *)&s_rk[ra + 4 * lg];
            const f32x4 gr = *(const f32x4 *)&s_gam[ra + 4 * lg];
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                FragT a = lds_row8<T>(Ks + (ra + lc) * LDK + 32 * ks + 8 * lg);
                FragT b = lds_row8<T>(Ks + (16 * ct + lc) * LDK + 32 * ks + 8 * lg);
                acc = mma(a, b, acc);
            }
            const int col = 16 * ct + lc;
            const float gc = s_gam[col], rc = s_rk[col];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = ra + 4 * lg + i;
                const float val = col < row ? b4[i] * r4[i] * rc * __expf(gr[i] - gc) * acc[i] : 0.f;
                Lm[row * LDA + col] = val;
            }
            if (it == 0) solve_diag(ra);  // the wave's diagonal tile (rt == ct == wv)
        }
    }
    __syncthreads();

    // ---- off-diagonal blocks, level by level:
    //   T_ij = sum_{j<=m<i} L_im A_mj ;  A_ij = -A_ii T_ij
    // fp32 MFMA 16x16x4; T stays in registers and feeds the second product:
    // slot s of lane (g,c) holds T[4g+s][c], so step s contracts over rows
    // {4g+s} and reads A_ii[row][4g+s].
    // Every operand of a level (up to three products L_im A_mj and A_ii) is
    // read first, then the products run, so the reads overlap.
#pragma unroll
    for (int lev = 1; lev < 4; ++lev) {
        if (wv < 4 - lev) {
            const int j = wv, i = wv + lev;
            float la[3][4], am[3][4], ai[4];
#pragma unroll
            for (int mm = 0; mm < 3; ++mm) {
                if (mm < lev) {  // m = j + mm < i
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        la[mm][k] = Lm[(16 * i + lc) * LDA + 16 * (j + mm) + 4 * k + lg];  // L_im
                        am[mm][k] = a_at(16 * (j + mm) + 4 * k + lg, 16 * j + lc);       // A_mj, m >= j
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) ai[s] = Lm[(16 * i + lc) * LDA + 16 * i + 4 * lg + s];  // A_ii
            f32x4 t = zero4();
#pragma unroll
            for (int mm = 0; mm < 3; ++mm) {
                if (mm < lev) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) t = __builtin_amdgcn_mfma_f32_16x16x4f32(la[mm][k], am[mm][k], t, 0, 0, 0);
                }
            }
            f32x4 r = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) r = __builtin_amdgcn_mfma_f32_16x16x4f32(ai[s], t[s], r, 0, 0, 0);
            // A_ij, transposed: rows 16i + 4lg .. +3 of column 16j + lc
            *(f32x4 *)&Lm[(16 * j + lc) * LDA + 16 * i + 4 * lg] = -r;
        }
        __syncthreads();
    }

    // ---- the lower blocks of A into place (row-major, over L's dead lower
    // blocks), so that each lane's 8 elements of a row of A below are two
    // 16-byte reads: read down a column of the transposed copy they put
    // 4 lanes on one bank, about 10 us of bank-conflict stalls per launch
    // at the benchmark shape
    {
        // element [r][c] of each block; this lane order keeps both the column
        // reads and the row writes of every wave on 64 different banks
        const int r = tid & 15, c = (4 * ((tid >> 4) & 3) + r + (tid >> 6)) & 15;
#pragma unroll
        for (int b = 0; b < 6; ++b) {
            const int i = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3), j = b < 3 ? 0 : (b < 5 ? 1 : 2);  // (1,0) .. (3,2)
            Lm[(16 * i + r) * LDA + 16 * j + c] = Lm[(16 * j + c) * LDA + 16 * i + r];
        }
    }
    __syncthreads();

    // ---- u^T = V^T (A diag(beta))^T and w^T = Khat^T (A diag(beta e^gamma r))^T
    //      over the four 16-row blocks of output rows.  Blocks 2 and 3
    //      contract over two 32-row steps of A, blocks 0 and 1 over one, so
    //      each wave takes one kind of product for one small and one large
    //      block: wave 0 u of blocks 0 and 2, wave 1 w of blocks 0 and 2,
    //      wave 2 u of blocks 1 and 3, wave 3 w of blocks 1 and 3.  The
    //      lanes' rows of A go to registers first (blocks past the diagonal
    //      are 0), then the V tile takes the array's space.
    {
        const bool do_u = (wv & 1) == 0;           // wave-uniform
        const int rlo = wv >> 1, rhi = rlo + 2;     // the wave's row blocks (one step, two steps)
        // A diag(beta) (u) or A diag(beta e^gamma r) (w) as bf16 operands
        // split into high and low parts (split_lo): rounding them to one
        // bf16 each was the largest single error of the bf16 path in the
        // long-memory regime
        constexpr bool SPL = Split<T>::on;
        auto a_frag = [&](int rt, int ks, FragT &hi, FragT &lo) {
            const int a_row = 16 * rt + lc;
            const int b0 = 32 * ks + 8 * lg, bb = b0 >> 4;  // A[a_row][b0 .. b0 + 7], block bb
            const float *fv = do_u ? s_beta : s_ws;
            const f32x4 f0 = *(const f32x4 *)&fv[b0], f1 = *(const f32x4 *)&fv[b0 + 4];
            // blocks on or below the diagonal are row-major; the ones past it are 0
            const f32x4 v0 = *(const f32x4 *)&Lm[a_row * LDA + b0], v1 = *(const f32x4 *)&Lm[a_row * LDA + b0 + 4];
            float av[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                av[m] = bb <= rt ? v0[m] : 0.f;
                av[4 + m] = bb <= rt ? v1[m] : 0.f;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float x0 = av[m] * f0[m], x1 = av[4 + m] * f1[m];
                hi[m] = from_f32<T>(x0);
                hi[4 + m] = from_f32<T>(x1);
                if constexpr (SPL) {
                    lo[m] = split_lo<T>(x0, hi[m]);
                    lo[4 + m] = split_lo<T>(x1, hi[4 + m]);
                }
            }
        };
        FragT bs[3], bsl[3];  // [0]: block rlo, step 0; [1], [2]: block rhi, steps 0 and 1
        a_frag(rlo, 0, bs[0], bsl[0]);
        a_frag(rhi, 0, bs[1], bsl[1]);
        a_frag(rhi, 1, bs[2], bsl[2]);
        __syncthreads();  // every row of A is in registers
#pragma unroll
        for (int it = 0; it < VPT; ++it) {
            const int uidx = tid + 256 * it, row = uidx / VUPR, cu16 = uidx % VUPR;
            *(uint4 *)(Vs + row * LDV + cu16 * (16 / (int)sizeof(T))) = vreg[it];
        }
        __syncthreads();
        // tile of the wave's kind for row block j (0: rlo, one step; 1: rhi,
        // two steps) and column tile ct: V^T or Khat^T times the split A rows
        auto prod = [&](int j, const T *X, int ldx, int ct) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks <= j) {
                    FragT a = lds_col8<T>(X, ldx, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * ct);
                    acc = mma(a, bs[j + ks], acc);
                    if constexpr (SPL) acc = mma(a, bsl[j + ks], acc);
                }
            }
            return acc;
        };
        typename Frag<T>::half wq[2][KD / 16];  // w[16 rt + lc][16kt + 4lg .. +3] of the wave's two blocks
        if (do_u) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int a_row = 16 * (j ? rhi : rlo) + lc;
                const bool row_ok = a_row < n;
                const int64_t grow = r0 + a_row;
#pragma unroll
                for (int vt = 0; vt < VD / 16; ++vt) {
                    const f32x4 acc = prod(j, Vs, LDV, vt);
                    if (row_ok) {  // u is slice-major: 4 consecutive columns of the row
                        typename Frag<T>::half o4;
#pragma unroll
                        for (int q = 0; q < 4; ++q) o4[q] = from_f32<T>(acc[q]);
                        *(typename Frag<T>::half *)(u + uv_index(bi, grow - bi * TM, hv, 16 * vt + 4 * lg, HV, VD, uv_ss)) = o4;
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int kt = 0; kt < KD / 16; ++kt) {
                    const f32x4 acc = prod(j, Ks, LDK, kt);
#pragma unroll
                    for (int q = 0; q < 4; ++q) wq[j][kt][q] = from_f32<T>(acc[q]);
                }
        }
        // w leaves through the K tile's space so that every store writes
        // whole 128-byte lines (a lane's four columns are only 8 bytes)
        __syncthreads();  // every wave is done reading K
        if (!do_u) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int kt = 0; kt < KD / 16; ++kt)
                    *(typename Frag<T>::half *)(Ks + (16 * (j ? rhi : rlo) + lc) * LDK + 16 * kt + 4 * lg) = wq[j][kt];
        }
        __syncthreads();
        constexpr int WU = KD * (int)sizeof(T) / 16;  // 16-byte units per w row
        T *wdst = w + (r0 * HV + hv) * (int64_t)KD;
#pragma unroll
        for (int it = 0; it < C * WU / 256; ++it) {
            const int uidx = tid + 256 * it, row = uidx / WU, c16 = uidx % WU;
            if (row < n)
                *(uint4 *)(wdst + (int64_t)row * HV * KD + c16 * (16 / (int)sizeof(T))) =
                    *(const uint4 *)(Ks + row * LDK + c16 * (16 / (int)sizeof(T)));
        }
    }
}

template <typename T, int KD, int VD, bool FUSE = false>
static hipError_t launch_wy_t(const ChunkParams &p, hipStream_t stream, const WyFuse<T> &fz = WyFuse<T>{}) {
    const gdp_chunk_args &a = p.a;
    if (p.max_items * a.HV > 0x7fffffff) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)(p.max_items * a.HV));
    hipLaunchKernelGGL((gdp_wy_k<T, KD, VD, FUSE>), grid, dim3(256), 0, stream,
                       (const T *)a.k, (const T *)a.v, a.beta, a.g, a.cu_seqlens, p.nseq, a.T,
                       a.H, a.HV, a.M, a.k_rnorm, a.gcum, a.kdecay, (T *)a.w, (T *)a.u, p.uv_ss, fz,
                       p.seg_nch, p.seg_n);
    return hipGetLastError();
}

// bf16: K in {64, 128} x V in {64, 128, 256}; f32 (small-case reference
// precision): K = 64, V in {64, 128}.
static hipError_t launch_wy_bf16(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_wy_t<bf16, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_wy_t<bf16, 64, 128>(p, stream);
    if (K == 64 && V == 256) return launch_wy_t<bf16, 64, 256>(p, stream);
    if (K == 128 && V == 64) return launch_wy_t<bf16, 128, 64>(p, stream);
    if (K == 128 && V == 128) return launch_wy_t<bf16, 128, 128>(p, stream);
    if (K == 128 && V == 256) return launch_wy_t<bf16, 128, 256>(p, stream);
    return hipErrorInvalidValue;
}
static hipError_t launch_wy_f32(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_wy_t<float, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_wy_t<float, 64, 128>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_wy(const ChunkParams &p, hipStream_t stream) {
    if (p.max_items == 0) return hipSuccess;
    return p.a.dtype == GDP_BF16 ? launch_wy_bf16(p, stream) : launch_wy_f32(p, stream);
}

// WY with the prefill prepare fused in (bf16, K and V in {64, 128}); the
// caller has checked both argument sets.
hipError_t launch_wy_prepare(const ChunkParams &p, const PrepareParams &pp, hipStream_t stream) {
    if (p.max_items == 0) return hipSuccess;
    const WyFuse<bf16> fz{(const bf16 *)pp.x, pp.x_t_stride, (const bf16 *)pp.ba, pp.ba_t_stride, pp.A_log,
                          pp.dt_bias, pp.G, (bf16 *)pp.q, (bf16 *)pp.k, (bf16 *)pp.v, pp.beta, pp.g};
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_wy_t<bf16, 64, 64, true>(p, stream, fz);
    if (K == 64 && V == 128) return launch_wy_t<bf16, 64, 128, true>(p, stream, fz);
    if (K == 128 && V == 64) return launch_wy_t<bf16, 128, 64, true>(p, stream, fz);
    if (K == 128 && V == 128) return launch_wy_t<bf16, 128, 128, true>(p, stream, fz);
    return hipErrorInvalidValue;
}

}  // namespace gdp
