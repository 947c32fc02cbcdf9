// chunk_o.hip -- output of the Gated Delta Product
// (core.ssm.ops.gdp.chunk_o: module description,
// chunk_gated_delta_product_fwd_o).
//
// One block (4 waves) per (64-token chunk i of a sequence, value head, slab
// of up to 128 value columns).  The queries are one per token; keys and
// corrected values live on the expanded stream, copy j of token s at row
// s*M + j.  With G the within-chunk cumulative log decay of the tokens and S
// the V x K state entering the chunk (the chunk_h snapshot at expanded chunk
// i*M):
//   o_t = scale * [ exp(G_t) S qhat_t
//                   + sum_j sum_{s <= t} exp(G_t - G_s) (qhat_t . khat_{sM+j}) v_new_{sM+j} ]
// computed transposed, O^T = S Q^T + sum_j V_j^T P_j^T, so a result lane
// holds four consecutive output columns of one token.  Wave w owns tokens
// [16w, 16w + 16) and skips the key tiles past them, so its scores never
// leave its registers: the score tile P_j^T = K_j Q^T comes out of the
// matrix cores with each lane holding four consecutive key rows of one
// query column, which is the operand layout of the P V product once V_j^T
// is read with the same row order (LDS transpose reads).
//
// Only the operands that several waves share or that need a transpose go
// through LDS: the state slab (copied in with buffer_load ... lds) and the
// copy's V_j slab.  Q and K_j fragments are plain 16-byte row reads straight
// into registers.  That keeps LDS near 50 KB so three blocks share a CU and
// one block's loads overlap another's math.  In bf16 the fp32 scores enter
// the P V product as a high and a low bf16 part (two products).  Norms enter as fp32 scales on
// the scores and on the inter term; rows past the end of a sequence read as
// zeros through the buffer range checks.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

namespace {
constexpr int C = 64;
}  // namespace

template <typename T, int KD, int VB>
__global__ void __launch_bounds__(256)
gdp_chunk_o_k(const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ k_rnorm,
              const T *__restrict__ v_new, const T *__restrict__ hst, const float *__restrict__ g,
              const int32_t *__restrict__ cu, int64_t nseq, int64_t Ttok, int H, int HV, int M, int VD,
              int64_t h_chunks, float scale, T *__restrict__ o, int64_t uv_ss) {
    typedef typename Frag<T>::type FragT;
    typedef typename Frag<T>::half HalfT;
    constexpr int ES = (int)sizeof(T);
    constexpr int NKS = KD / 32;           // contraction steps over K
    constexpr int NVT = VB / 16;           // 16-column output tiles
    constexpr int SRB = KD * ES;           // bytes per state row
    constexpr int SUPR = SRB / 16;         // 16-byte units per state row
    constexpr int VRB = VB * ES;           // bytes per V slab row (as o stores it)
    constexpr int CSB = C * 16 * ES;       // bytes of one copy in a 16-column slice of the V slab
    constexpr int NSD = VB * SRB / 1024;   // DMA instructions for the state slab
    constexpr int NVD = C * VRB / 1024;    // DMA instructions per copy of the V slab
    static_assert(NSD % 4 == 0 && NVD % 4 == 0 && SUPR >= 8 && CSB % 1024 == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) T Ss[VB * KD];   // state slab, swizzled rows
    // the V slab of all M copies: VB/16 slices of 64 M rows x 16, rows in
    // v_new's order (token r, copy j at row r M + j); M * C * VB elements of
    // dynamic LDS
    extern __shared__ __attribute__((aligned(16))) char v_dyn[];
    T *Vs = (T *)v_dyn;
    __shared__ float sG[4][C], sRk[4][C];                    // per-wave scratch

    // block -> (token chunk, value head, value slab), heads fastest: the
    // blocks in flight together cover whole rows of q, k and o (all heads of
    // a few chunks), so HBM sees long contiguous runs.  With two slabs (V =
    // 256) the slabs of one (chunk, head) are 8 launch positions apart, so
    // they run on one XCD and the second reads the query and key rows the
    // first brought into that XCD's L2: items (chunk, head) go in groups of
    // 8, each group's slab s blocks at 8 s + x.
    const int nslab = VD / VB;
    const int64_t lin = blockIdx.x;
    const int64_t grp = lin / (8 * nslab), rem = lin % (8 * nslab);
    const int64_t item = grp * 8 + rem % 8;  // (token chunk, value head), heads fastest
    const ChunkLoc loc = find_chunk(cu, nseq, Ttok, 1, C, item / HV);
    if (loc.seq < 0) return;
    const int hv = (int)(item % HV);
    const int hk = hv / (HV / H);
    const int vb0 = VB * (int)(rem / 8);
    const int64_t t0 = loc.bos + C * loc.c;  // first token (flattened)
    const int nt = (int)((loc.eos - t0) < C ? (loc.eos - t0) : C);
    const int64_t hidx = items_before(cu, Ttok, M, C, loc.seq) + loc.c * M;
    const int lane = lane_id(), wv = wave_id();
    const int lg = lane >> 4, lc = lane & 15;
    const int tt = wv;               // token tile of this wave
    const int t_loc = 16 * tt + lc;  // token whose column this lane holds
    auto span = [](int n, int stride_b, int width_b) { return (uint32_t)(n > 0 ? (n - 1) * stride_b + width_b : 0); };
    // swizzled byte offsets of the state slab: rows XOR their 16-byte unit
    // with the row.  The V slab is slice-major like v_new (row r of slice vt
    // at vt * M * CSB + (r M + j) * 16 * ES for token r, copy j): the four
    // rows of a transposed read sit M * 16 * ES bytes apart, in distinct
    // bank groups.
    auto s_off = [](int r, int unit) { return r * SRB + ((unit ^ (r & (SUPR - 1))) << 4); };
    const int vsb = M * CSB;  // bytes per slice of the slab
    auto v_at = [&](int vt, int r, int j) { return vt * vsb + (r * M + j) * 16 * ES; };

    // ---- state slab (rows vb0 .. vb0 + VB of S) -> LDS; the snapshot is
    // zero-filled past h_chunks by the range check
    {
        const rsrc_t rs = make_rsrc(hst + ((hidx * HV + hv) * (int64_t)VD + vb0) * KD,
                                    hidx < h_chunks ? (uint32_t)(VB * SRB) : 0u);
        const uint32_t base = lds_addr(Ss);
#pragma unroll
        for (int i = 0; i < NSD / 4; ++i) {
            const int blk = wv * (NSD / 4) + i;
            const int r = blk * (1024 / SRB) + lane / SUPR, u = lane % SUPR;
            dma16(rs, (uint32_t)(r * SRB + ((u ^ (r & (SUPR - 1))) << 4)), base + blk * 1024);
        }
    }
    const int64_t ldkv_k = (int64_t)M * H * KD;  // key row stride per token
    // V slab: rows t0 M .. (t0 + nt) M of the VB/16 slices of v_new from
    // column vb0, all copies at once, so every 128-byte line is read whole;
    // one DMA instruction fills RPI consecutive rows of one slice; rows past
    // the chunk are zero-filled
    const int64_t bseq = cu ? 0 : loc.seq;  // batch row of the sequence
    {
        constexpr int RPI = 1024 / (16 * ES);  // rows per instruction
        constexpr int UPRV = 16 * ES / 16;     // 16-byte units per slice row
        const int ips = M * (CSB / 1024);      // DMA instructions per slice
        const T *vbase = v_new + uv_index(bseq, (t0 - bseq * Ttok) * M, hv, vb0, HV, VD, uv_ss);
        const uint32_t base = lds_addr(Vs);
        for (int i = 0; i < M * (NVD / 4); ++i) {
            const int blk = wv * M * (NVD / 4) + i;
            const int slc = blk / ips, r = (blk % ips) * RPI + lane / UPRV, u = lane % UPRV;
            const rsrc_t rv = make_rsrc(vbase + slc * uv_ss, (uint32_t)(nt * M * 16 * ES));
            dma16(rv, (uint32_t)(r * 16 * ES + u * 16), base + blk * 1024);
        }
    }

    // ---- register operands: this lane's query row (B operand of both
    // products), its keys per copy, the decays and key norms
    const rsrc_t rq = make_rsrc(q + (t0 * H + hk) * (int64_t)KD, span(nt, H * KD * ES, SRB));
    FragT qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t off = (uint32_t)((t_loc * H * KD + 32 * ks + 8 * lg) * ES);
        if constexpr (ES == 2) {
            qf[ks] = __builtin_bit_cast(FragT, buf_load16(rq, off));
        } else {
            qf[ks] = join<T>(__builtin_bit_cast(HalfT, buf_load16(rq, off)),
                             __builtin_bit_cast(HalfT, buf_load16(rq, off + 16)));
        }
    }
    const float gl = (g != nullptr && lane < nt) ? g[(t0 + lane) * HV + hv] : 0.f;  // NULL: ungated
    FragT kf[4][NKS];
    float rkl = 0.f;
    auto load_k = [&](int j) {
        const rsrc_t rk = make_rsrc(k + ((t0 * M + j) * H + hk) * (int64_t)KD, span(nt, (int)(ldkv_k * ES), SRB));
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (st <= tt) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const uint32_t off = (uint32_t)(((16 * st + lc) * ldkv_k + 32 * ks + 8 * lg) * ES);
                    if constexpr (ES == 2) {
                        kf[st][ks] = __builtin_bit_cast(FragT, buf_load16(rk, off));
                    } else {
                        kf[st][ks] = join<T>(__builtin_bit_cast(HalfT, buf_load16(rk, off)),
                                             __builtin_bit_cast(HalfT, buf_load16(rk, off + 16)));
                    }
                }
            }
        }
        rkl = lane < nt ? k_rnorm[hm_index(cu ? 0 : loc.seq, H, hk, Ttok * M, (t0 + lane) * M + j)] : 0.f;
    };
    load_k(0);

    // ---- decays and the query norm (no LDS traffic beyond this wave's own)
    const float Gl = wave_inclusive_sum(gl);
    sG[wv][lane] = Gl;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = to_f32(qf[ks][i]);
            ss += x * x;
        }
    ss = xor32_sum(xor16_sum(ss));
    const float fq = scale / sqrtf(ss + 1e-6f);  // scale * rnorm(q_t)
    const float Gt = sG[wv][t_loc];

    wait_vmcnt<0>();
    __syncthreads();  // state slab and V slab landed

    // ---- inter-chunk term: O^T[vt] = S[16vt.., :] Q^T[:, t]
    f32x4 acc[NVT];
    {
        const float f = fq * __expf(Gt);
        const char *sb = (const char *)Ss;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            f32x4 a4 = zero4();
            const int r = 16 * vt + lc;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                FragT a;
                if constexpr (ES == 2) {
                    a = *(const FragT *)(sb + s_off(r, 4 * ks + lg));
                } else {
                    a = join<T>(*(const HalfT *)(sb + s_off(r, 8 * ks + 2 * lg)),
                                *(const HalfT *)(sb + s_off(r, 8 * ks + 2 * lg + 1)));
                }
                a4 = mma(a, qf[ks], a4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[vt][i] = a4[i] * f;
        }
    }

    // exp(G_t - G_s) of the key rows this lane holds (s = 16st + 4lg + i),
    // masked to s <= t and s < nt; shared by all copies
    f32x4 dec[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sidx = 16 * st + 4 * lg + i;
            dec[st][i] = (st <= tt && sidx <= t_loc && sidx < nt) ? fq * __expf(Gt - sG[wv][sidx]) : 0.f;
        }

    // ---- intra-chunk attention, one Householder copy at a time
    for (int j = 0; j < M; ++j) {
        sRk[wv][lane] = rkl;
        // scores P^T tiles for key tiles st <= tt, as a high and a low bf16
        // part (the P V product runs once per part): one rounded bf16 score
        // per entry was one of the larger errors of the bf16 path
        FragT pb[2], pbl[2];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 p = zero4();
            if (st <= tt) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) p = mma(kf[st][ks], qf[ks], p);
            }
            const f32x4 rk4 = *(const f32x4 *)&sRk[wv][16 * st + 4 * lg];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = p[i] * dec[st][i] * rk4[i];
                pb[st >> 1][4 * (st & 1) + i] = from_f32<T>(x);
                if constexpr (Split<T>::on) pbl[st >> 1][4 * (st & 1) + i] = split_lo<T>(x, pb[st >> 1][4 * (st & 1) + i]);
            }
        }
        if (j + 1 < M) load_k(j + 1);  // next copy's keys while this one's products run
        // O^T[vt] += V_j^T[vt, s] P^T[s, t]; contraction slot m <-> s = 32ks + 16(m/4) + 4lg + m%4
        const char *vb = (const char *)Vs;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (2 * ks <= tt) {
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    HalfT x0, x1;
                    if constexpr (ES == 2) {
                        // transposed reads: source lane jj of the 16-lane group
                        // points at row rowA + jj/4, columns 16vt + 4(jj%4) .. +3
                        const int jj = lane & 15;
                        const int ra = 32 * ks + 4 * lg + (jj >> 2), rb = ra + 16;
                        const int cb = 4 * (jj & 3) * ES;  // byte of the column inside the slice row
                        x0 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(vb + v_at(vt, ra, j) + cb))));
                        x1 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(vb + v_at(vt, rb, j) + cb))));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            x0[i] = *(const float *)(vb + v_at(vt, 32 * ks + 4 * lg + i, j) + lc * ES);
                            x1[i] = *(const float *)(vb + v_at(vt, 32 * ks + 16 + 4 * lg + i, j) + lc * ES);
                        }
                    }
                    const FragT vf = join<T>(x0, x1);
                    acc[vt] = mma(vf, pb[ks], acc[vt]);
                    if constexpr (Split<T>::on) acc[vt] = mma(vf, pbl[ks], acc[vt]);
                }
            }
        }

    }

    // ---- store: lane holds o[t_loc][vb0 + 16vt + 4lg + i]
    const rsrc_t ro = make_rsrc(o + (t0 * HV + hv) * (int64_t)VD + vb0, span(nt, HV * VD * ES, VRB));
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
        HalfT o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = from_f32<T>(acc[vt][i]);
        const uint32_t off = (uint32_t)((t_loc * HV * VD + 16 * vt + 4 * lg) * ES);
        if constexpr (ES == 2)
            buf_store8(ro, off, __builtin_bit_cast(uint2, o4));
        else
            buf_store16(ro, off, __builtin_bit_cast(uint4, o4));
    }
}

template <typename T, int KD, int VB>
static hipError_t launch_chunk_o_t(const ChunkParams &p, hipStream_t stream) {
    const gdp_chunk_args &a = p.a;
    // (token chunk, head) items padded to a multiple of 8, times the slabs
    const int64_t nblk = (p.max_tok_chunks * a.HV + 7) / 8 * 8 * (a.V / VB);
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)nblk);
    const size_t vdyn = (size_t)a.M * 64 * VB * sizeof(T);  // the V slab of all copies (<= 64 KiB)
    hipLaunchKernelGGL((gdp_chunk_o_k<T, KD, VB>), grid, dim3(256), vdyn, stream,
                       (const T *)a.q, (const T *)a.k, a.k_rnorm, (const T *)a.v_new, (const T *)a.h, a.g,
                       a.cu_seqlens, p.nseq, a.T, a.H, a.HV, a.M, a.V, a.h_chunks, a.scale, (T *)a.o, p.uv_ss);
    return hipGetLastError();
}

// bf16: K in {64, 128} x V in {64, 128, 256} (V = 256 as two 128-column
// slabs); f32 (small-case reference precision): K = 64, V in {64, 128}.
static hipError_t launch_chunk_o_bf16(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_o_t<bf16, 64, 64>(p, stream);
    if (K == 64 && (V == 128 || V == 256)) return launch_chunk_o_t<bf16, 64, 128>(p, stream);
    if (K == 128 && V == 64) return launch_chunk_o_t<bf16, 128, 64>(p, stream);
    if (K == 128 && (V == 128 || V == 256)) return launch_chunk_o_t<bf16, 128, 128>(p, stream);
    return hipErrorInvalidValue;
}
static hipError_t launch_chunk_o_f32(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_o_t<float, 64, 64>(p, stream);
    // the V slab of all M copies stays within 64 KiB of dynamic LDS
    if (K == 64 && V == 128) return p.a.M <= 2 ? launch_chunk_o_t<float, 64, 128>(p, stream)
                                               : launch_chunk_o_t<float, 64, 64>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_o(const ChunkParams &p, hipStream_t stream) {
    if (p.max_tok_chunks == 0) return hipSuccess;
    return p.a.dtype == GDP_BF16 ? launch_chunk_o_bf16(p, stream) : launch_chunk_o_f32(p, stream);
}

}  // namespace gdp
