// chunk_ho.hip -- the inter-chunk state recurrence and the output of the
// Gated Delta Product in one pass: the chunk_h stage (state at each chunk
// boundary, corrected values) and core.ssm.ops.gdp.chunk_o
// (chunk_gated_delta_product_fwd_o: the boundary state plus causal in-chunk
// attention summed over the Householder copies), for callers that need only
// the output.  Neither the corrected values nor the boundary states leave
// the chip: each is consumed where it is made.
//
// Per sequence and value head, serially over the 64-row chunks c of the
// expanded stream (token chunk i = c / M holds chunks iM .. iM + M - 1), with
// h the K x V state entering c:
//   v_new = u - w h                          (the chunk's corrected values)
//   h    <- exp2(gl) h + K^T diag(kdecay) v_new
//   o_t   = scale [ exp(G_t) qhat_t h_{iM}
//                   + sum over rows e = sM + j of chunks iM.., s <= t:
//                       exp(G_t - G_s) (qhat_t . khat_e) v_new_e ]
// with G the within-token-chunk cumulative decay (the chunk_o page's
// g_cumsum over tokens), the same quantities the two separate stages
// compute.
//
// One block of eight waves per (sequence, value head, 64 value columns):
// * Chain waves 0-3.  Wave p runs the state chain of the 16-column slice p
//   exactly as the whole-K form of the chunk_h stage does (fp32 state in
//   registers, the same operands and order, so the states agree bit for
//   bit), and publishes to LDS the chunk's v_new (fp16, one buffer per step
//   parity) and, at the end of each token chunk, the state entering the next
//   one (bf16).  They also stream each chunk into a three-stage LDS ring,
//   chunk c + 2 late in step c (buffer loads with the LDS destination; the range
//   check zero-fills rows past the end): wave p a half tile of w (p < 2) or
//   K (p >= 2), its u slice and (p < 2) one of kdecay and gcum.
// * Output waves 4-7.  Wave 4 + t owns output token tile t (tokens 16t ..
//   16t + 15 of each token chunk) over all 64 columns of the block:
//     - before the step's barrier, the scores of its tokens against the
//       chunk's keys (the K tile is in the LDS ring), scaled by the norms and
//       decays, masked to s <= t, in fp16, and in a token chunk's second
//       step its inter-chunk term O^T = S Q^T exp(G) from the exchanged
//       state;
//     - after it, O^T += V^T P^T for the previous chunk with every slice's
//       v_new from the exchange, and at a token chunk's end the store of o.
//   Their query rows and the key norms of the token chunk's rows are loaded
//   a token chunk ahead, and a step before the token chunk starts each
//   output wave writes a row table (every expanded row's decay less its
//   log2 key norm) so that a score's whole factor is one 2^x.
// One barrier per chunk orders it all: the ring stage of chunk c is read
// before it, the exchanges are written after it and read after the next.
// Requires M >= 2, so that the state exchange of one token chunk is read
// before the next is written.
//
// Precision.  The state chain keeps the chunk_h stage's operands exactly.
// The output product O^T += V^T P^T runs on fp16 operands: both are made on
// chip (v_new by the chain waves, P by the output waves), |P| <= scale, and
// fp16's 11-bit significand keeps them closer to their fp32 values than
// bf16 does, with one product per pair where bf16 needed a high and a low
// part.  v_new must stay within fp16's range (|v_new| < 65504); beyond it
// the output is not finite.
#include "gdp_common.h"
#include "gdp_internal.h"

namespace gdp {

namespace {
constexpr int C = 64;
constexpr int NP = 4;  // 16-column slices per block
}  // namespace

template <int KD>
struct HoStage {
    bf16 w[2][C * (KD / 2)];  // w half tiles [K half], swizzled rows
    bf16 k[2][C * (KD / 2)];  // K half tiles [K half], swizzled rows
    bf16 u[NP][C * 16];       // u slices, plain rows of 16 elements
    float kd[C];              // key decay factor per row (0 past the end)
    float gc[C];              // cumulative log2 decay per row
};

template <int KD, int VD>
__global__ void __launch_bounds__(2 * NP * 64)
gdp_chunk_ho_k(QKRows qk, const float *__restrict__ kdecay, const bf16 *__restrict__ w,
               const bf16 *__restrict__ u, const float *__restrict__ gcum, const float *__restrict__ k_rnorm,
               const float *__restrict__ g, const int32_t *__restrict__ cu,
               int64_t nseq, int64_t Ttok, int H, int HV, int M, const float *h0, float *ht,
               bf16 *__restrict__ o, int64_t uv_ss, float scale) {
    typedef bf16x8 FragT;
    typedef bf16x4 HalfT;
    constexpr int ES = 2;
    constexpr int KH = KD / 2;           // K rows per half tile
    constexpr int RB = KH * ES;          // bytes per half-tile row
    constexpr int UPR = RB / 16;         // 16-byte units per half-tile row
    constexpr int RPI = 64 / UPR;        // half-tile rows per DMA instruction
    constexpr int NU = C * 16 * ES / 16 / 64;  // DMA instructions per u slice
    constexpr int NS = 3;                // ring stages (loads two chunks ahead)
    constexpr int NKT = KH / 16;         // 16-row state tiles per K half
    constexpr int NKS = KH / 32;         // contraction steps per K half
    constexpr int S = VD / 16;           // column slices per head
    constexpr int SG = S / NP;           // blocks per head
    constexpr int SB = (int)sizeof(HoStage<KD>);
    // ring loads per chunk of chain wave p: a half tile of w or K, its u
    // slice and (p < 2) one per-row vector
    constexpr int NDMA = UPR + NU + 1;
    static_assert(NKS >= 1 && (UPR & (UPR - 1)) == 0 && S % NP == 0 && SB % 16 == 0, "tile shape");
    static_assert(NDMA < 64, "in-flight count must fit the vector memory counter");

    __shared__ __attribute__((aligned(16))) HoStage<KD> ring[NS];
    // v_new of the chunk, fp16, as O^T = V^T P^T operands: [parity][slice][key half s][lane]
    __shared__ __attribute__((aligned(16))) f16x8 Vx[2][NP][2][64];
    // state entering a token chunk, bf16, as O^T = S Q^T operands: [slice][K half][step][lane]
    __shared__ __attribute__((aligned(16))) FragT Sx[NP][2][NKS][64];
    // per output wave, the cumulative decay (log2 units) of the token of
    // each expanded row of its current token chunk (64 M rows, M <= 4)
    __shared__ __attribute__((aligned(16))) float Grow[NP][4 * C];

    // ---- block -> (sequence, value head, slice group); the groups of one
    // head share an XCD
    const int64_t P = nseq * HV;
    const int64_t id = blockIdx.x;
    const int64_t slot = id / 8, xcd = id % 8;
    const int64_t pair = (slot / SG) * 8 + xcd;
    const int slg = (int)(slot % SG);
    if (pair >= P) return;
    const int64_t seq = pair / HV;
    const int hv = (int)(pair % HV);
    const int hk = hv / (HV / H);
    int64_t bos, eos;
    seq_bounds(cu, Ttok, seq, bos, eos);
    const int64_t rows = (eos - bos) * M;
    const int nch = (int)ceil_div64(rows, C);

    const int lane = lane_id(), wave = wave_id();
    const int lg = lane >> 4, lc = lane & 15;
    // the fp32 state of a compute wave in the permuted K order of the chunk_h
    // stage: element (kw, kt, q) is S[16 sl + lc][kw KH + 32(kt/2) + 8 lg +
    // 4(kt%2) + q], one 16-byte unit of h0 / ht
    auto state_off = [&](int sl_, int kw_, int kt) {
        return ((seq * HV + hv) * (int64_t)VD + 16 * sl_ + lc) * KD + kw_ * KH + 32 * (kt >> 1) + 8 * lg +
               4 * (kt & 1);
    };
    if (nch == 0) {  // empty sequence: the final state is the initial one
        if (ht != nullptr && wave < NP) {
            const int sl = NP * slg + wave;
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    *(f32x4 *)(ht + state_off(sl, kw, kt)) = h0 ? *(const f32x4 *)(h0 + state_off(sl, kw, kt)) : zero4();
        }
        return;
    }
    const int ldw = HV * KD;  // w row stride (elements)
    // q and k rows by token and copy (the q and k tensors, or the activations)
    const int64_t qkh = (int64_t)(hk / qk.hpg) * qk.hs;  // the key head's element offset in a row
    const int64_t r0 = bos * M;              // first expanded row of the sequence
    const int64_t bseq = cu ? 0 : seq;       // batch row of the sequence
    const int64_t TM = Ttok * M;
    const int64_t h0r = hm_index(bseq, HV, hv, TM, r0);  // kdecay / gcum of row r0
    const int64_t k0r = hm_index(bseq, H, hk, TM, r0);   // k_rnorm of row r0

    auto clamp_rows = [](int r) { return r < 0 ? 0 : (r < C ? r : C); };
    auto span = [](int n, int stride_b, int width_b) { return (uint32_t)(n > 0 ? (n - 1) * stride_b + width_b : 0); };
    // 16-byte units of half-tile row r are XOR-swizzled by xw(r) in the w
    // tiles and by xk(r) in the K tiles.  The K tiles are read both as rows
    // (scores) and transposed (phase 2, ds_read_b64_tr_b16); with 128-byte
    // rows, r mod 8 keeps the transposed reads free of bank conflicts and
    // leaves the row reads 2-way, where (r / 2) mod 8 gave the reverse
    // (rocprofv3 SQ_LDS_BANK_CONFLICT: 2.5e7 -> 0.9e7 cycles per launch at
    // the benchmark shape, 6 us less)
    auto xw = [](int r) { return (r >> 1) & (UPR - 1); };
    auto xk = [](int r) { return UPR == 8 ? r & 7 : (r >> 1) & (UPR - 1); };
    // byte offset of element column `col` of half-tile row r, w or K tile
    auto swz_at = [&](int r, int col, int x) {
        const int b = col * ES;
        return r * RB + ((((b >> 4) ^ x)) << 4) + (b & 15);
    };
    auto swz = [&](int r, int col) { return swz_at(r, col, xw(r)); };
    auto swzk = [&](int r, int col) { return swz_at(r, col, xk(r)); };

    const int ntok = (int)(eos - bos);
    // x / M as __umulhi(x, mdiv): exact for every x < 2^31 when M is 2, 3 or 4
    const uint32_t mdiv = small_div_magic(M);
    const uint32_t ring_base = lds_addr(&ring[0]);
    const int64_t st4 = (int64_t)C * 4;  // bytes of one chunk of a per-row vector

    if (wave >= NP) {
        // ======================= output waves =======================
        // Output wave tt owns tokens 16 tt .. 16 tt + 15 of each token chunk
        // over the block's 64 columns.  Its only global memory instructions
        // are its query loads and output stores.
        const int tt = wave - NP;

        // ---- the output tile: queries (B operands of both output
        // products), their norms and decays for the current token chunk
        FragT qf[2][NKS], qn[2][NKS];  // this token chunk's queries, and the next one's in flight
        float gn = 0.f, gnn = 0.f;
        float rkn[4];  // key norms of the next token chunk's rows of token `lane` (copies 0 .. M - 1)
        auto load_q = [&](int ti, FragT (&qf)[2][NKS], float &gn) {
            const int nt = __builtin_amdgcn_readfirstlane(clamp_rows(ntok - C * ti));
            const rsrc_t rq = make_rsrc((const bf16 *)qk.q + (bos + (int64_t)C * ti) * qk.q_ts + qkh,
                                        span(nt, (int)qk.q_ts * ES, KD * ES));
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    qf[kw][ks] = __builtin_bit_cast(
                        FragT, buf_load16(rq, (uint32_t)(((16 * tt + lc) * (int)qk.q_ts + kw * KH + 32 * ks + 8 * lg) * ES)));
            gn = (g != nullptr && lane < nt) ? g[(bos + (int64_t)C * ti + lane) * HV + hv] : 0.f;
            // rows past the end read as 0 (range check)
            const rsrc_t rr = make_rsrc(k_rnorm + k0r + (int64_t)C * M * ti, (uint32_t)(nt * M * 4));
#pragma unroll
            for (int j = 0; j < 4; ++j) rkn[j] = j < M ? buf_load_f32(rr, (uint32_t)((lane * M + j) * 4)) : 0.f;
        };
        // Gq = G_t + log2(scale / ||q_t||) (log2 units) of this lane's token,
        // for the current token chunk and (made a step before it starts) the
        // next; the row table of the token chunk being set up holds
        // G_s - log2(1 / ||k_e||) for each expanded row e (token s), so one
        // 2^(Gq - table) is the whole score factor.  It is written after the
        // last read of the current one's (same wave, in order).
        float Gq = 0.f, Gqn = 0.f;
        auto token_setup = [&](const FragT (&qs)[2][NKS], float gs, const float (&rks)[4], float &Gq) {
            const float Gl = wave_inclusive_sum(gs) * 1.44269504088896341f;  // G of token `lane`
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < M) Grow[tt][lane * M + j] = Gl - __builtin_amdgcn_logf(rks[j]);
            float ss = 0.f;
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float x = (float)qs[kw][ks][i];
                        ss += x * x;
                    }
            ss = xor32_sum(xor16_sum(ss));
            Gq = row_broadcast(Gl, tt) + __builtin_amdgcn_logf(scale / sqrtf(ss + 1e-6f));
        };
        // O^T tiles: oa[ct] holds o[token 16 tt + lc][64 slg + 16 ct + 4 lg + r]
        f32x4 oa[NP];
        auto inter = [&]() {  // O^T = S Q^T exp(G_t), S from the state exchange
            const float f = __builtin_amdgcn_exp2f(Gq);  // scale / ||q_t|| 2^G_t
            FragT sx[NP][2][NKS];  // every state fragment first, then the products
#pragma unroll
            for (int ct = 0; ct < NP; ++ct)
#pragma unroll
                for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) sx[ct][kw][ks] = Sx[ct][kw][ks][lane];
            __builtin_amdgcn_sched_barrier(0);  // keep the reads together, ahead of the products
            f32x4 a4[NP];  // the slices' chains interleaved, each in (kw, ks) order
#pragma unroll
            for (int ct = 0; ct < NP; ++ct) a4[ct] = zero4();
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int ct = 0; ct < NP; ++ct) a4[ct] = mma(sx[ct][kw][ks], qf[kw][ks], a4[ct]);
#pragma unroll
            for (int ct = 0; ct < NP; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) oa[ct][r] = a4[ct][r] * f;
        };
        auto store_o = [&](int ti) {
            const int nt = __builtin_amdgcn_readfirstlane(clamp_rows(ntok - C * ti));
            const rsrc_t ro = make_rsrc(o + ((bos + (int64_t)C * ti) * HV + hv) * VD + 64 * slg,
                                        span(nt, HV * VD * ES, 64 * ES));
#pragma unroll
            for (int ct = 0; ct < NP; ++ct) {
                HalfT o4v;
#pragma unroll
                for (int r = 0; r < 4; ++r) o4v[r] = (bf16)oa[ct][r];
                buf_store8(ro, (uint32_t)(((16 * tt + lc) * HV * VD + 16 * ct + 4 * lg) * ES),
                           __builtin_bit_cast(uint2, o4v));
            }
        };

        load_q(0, qf, gn);
        token_setup(qf, gn, rkn, Gq);
        lds_barrier();  // stage 0 landed; the initial state exchange is visible
        // O^T of a token chunk starts as its inter-chunk term, made in the
        // token chunk's second step before the barrier (the state exchange
        // holds the entering state from the step before the token chunk's
        // first barrier until its M-th), then gathers each chunk's P V
        bool inter_due = true;
        int rem = (int)rows;
        const int t_me = 16 * tt + lc;  // this lane's token (within the token chunk)
        // scores of one chunk as the fp16 B operands of O^T += V^T P^T, per
        // key half: made for chunk c before step c's barrier, consumed once
        // chunk c's v_new is in the exchange (after step c + 1's barrier)
        f16x8 pb[2];
        auto pv = [&](int cprev) {  // O^T += V^T P^T over the block's column slices
            // every v_new fragment first, then the products (masked scores
            // are exact zeros, so the products of inactive key halves add
            // nothing)
            f16x8 vx[NP][2];
#pragma unroll
            for (int ct = 0; ct < NP; ++ct)
#pragma unroll
                for (int s = 0; s < 2; ++s) vx[ct][s] = Vx[cprev & 1][ct][s][lane];
            __builtin_amdgcn_sched_barrier(0);  // keep the reads together, ahead of the products
#pragma unroll
            for (int ct = 0; ct < NP; ++ct)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    oa[ct] = mma(vx[ct][s], pb[s], oa[ct]);
                }
        };
        for (int c = 0, st_ = 0; c < nch; ++c, st_ = st_ == NS - 1 ? 0 : st_ + 1) {
            const int ti = (int)__umulhi((uint32_t)c, mdiv);  // token chunk
            const int m = c - ti * M;
            if (m == 0 && c > 0) {  // token chunk ti starts: its queries arrived a token chunk ago
#pragma unroll
                for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) qf[kw][ks] = qn[kw][ks];
                Gq = Gqn;
            }
            // the next token chunk's queries, a token chunk ahead
            if (m == 0 && C * (ti + 1) < ntok) load_q(ti + 1, qn, gnn);
            const HoStage<KD> &Sg = ring[st_];
            const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem));  // valid rows of the chunk
            // ---- the chunk's key rows (A operands of the scores) and norms
            FragT kr[4][2][NKS];
            f32x4 gr4[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        kr[st][kw][ks] = *(const FragT *)((const char *)Sg.k[kw] + swzk(16 * st + lc, 32 * ks + 8 * lg));
                gr4[st] = *(const f32x4 *)(&Grow[tt][C * m + 16 * st + 4 * lg]);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the reads together, ahead of their uses
            // ---- the score factors: dec = (scale / ||q_t||) (1 / ||k_r||)
            // 2^(G_t - G_s) = 2^(Gq - table) for key row r of the chunk
            // (expanded row 64 m + r of the token chunk: token s = (64 m + r)
            // / M) when s <= t and r < n, else 2^-inf = 0.  s <= t exactly
            // when 64 m + r < (t + 1) M, so one bound per lane covers both
            // tests; branch-free
            const int lim = min((t_me + 1) * M - C * m, n) - 4 * lg;  // row 16 st + 4 lg + r is live when 16 st + r < lim
            float dec[4][4];
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = 16 * st + r < lim;
                    dec[st][r] = __builtin_amdgcn_exp2f(ok ? Gq - gr4[st][r] : -__builtin_inff());
                }
            // ---- scores of the tile's tokens against the chunk's keys,
            // P^T[key r][token t] = dec[r][t] (k_r . q_t), the four
            // sub-tiles' products interleaved (masked entries are zeroed by
            // dec)
            f32x4 p[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) p[st] = zero4();
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int st = 0; st < 4; ++st) p[st] = mma(kr[st][kw][ks], qf[kw][ks], p[st]);
            f16x8 pn[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int st = 2 * s + s2;
                        const float x = p[st][r] * dec[st][r];
                        pn[s][4 * s2 + r] = (f16)x;
                    }
            if (inter_due && m == 1) {
                inter();  // the state entering token chunk ti
                inter_due = false;
            }
            lds_barrier();  // ring stage c read; chunk c - 1's v_new is in the exchange

            if (c > 0) {
                pv(c - 1);
                if (m == 0) {  // chunk c - 1 ended token chunk ti - 1
                    store_o(ti - 1);
                    inter_due = true;
                }
            }
            // the next token chunk's norms and decays, a step before it starts
            if (m == M - 1 && C * (ti + 1) < ntok) token_setup(qn, gnn, rkn, Gqn);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                pb[s] = pn[s];
            }
            rem -= C;
        }
        lds_barrier();  // the last chunk's v_new is in the exchange
        if (inter_due) inter();  // the last token chunk has a single chunk
        pv(nch - 1);
        store_o((int)__umulhi((uint32_t)(nch - 1), mdiv));
        return;
    }

    // ======================= chain waves =======================
    // Wave pp runs the state chain of the block's 16-column slice pp, with
    // the operands and order of the chunk_h stage's whole-K form, and
    // publishes the chunk's v_new (and at token-chunk ends the state) to
    // the exchanges.  It also streams part of each chunk into the ring, two
    // chunks ahead: half pp % 2 of the w (pp < 2) or K (pp >= 2) tile, its
    // own u slice and (pp < 2) one per-row vector (pp = 0: kdecay, 1:
    // gcum), with no other global memory instruction in the loop, so its
    // counted waits are exact.  One code path for all four waves and all
    // three ring stages (the wave and the stage are runtime values), so the
    // code fits the instruction cache.
    const int pp = wave;
    // the state chain is the longer dependency path: its instructions go
    // first when both waves of a SIMD are ready
    __builtin_amdgcn_s_setprio(2);
    const int sl = NP * slg + pp;
    typedef HoStage<KD> Stage;
    constexpr int OFW = (int)__builtin_offsetof(Stage, w);
    constexpr int OFK = (int)__builtin_offsetof(Stage, k);
    constexpr int OFU = (int)__builtin_offsetof(Stage, u);
    constexpr int OFD = (int)__builtin_offsetof(Stage, kd);
    constexpr int OFG = (int)__builtin_offsetof(Stage, gc);
    constexpr int HALF = C * KH * ES;  // bytes of one half tile
    const bool rw = pp < 2;             // w (else K)
    const int hh = pp & 1;              // half of the tile's columns
    // per-lane source offsets inside a chunk, less the DMA's offset in its
    // 4 KiB M0 window; key rows are addressed by token and copy, so their
    // row part is added per chunk (krel)
    uint32_t ot[UPR];
#pragma unroll
    for (int i = 0; i < UPR; ++i) {
        const int r = i * RPI + lane / UPR;
        const int unit = (lane % UPR) ^ (rw ? xw(r) : xk(r));
        ot[i] = (uint32_t)((rw ? r * ldw * ES : 0) + hh * KH * ES + unit * 16 - 1024 * (i % 4));
    }
    // element offset of expanded row e0 + r from the token holding row e0
    auto krel = [&](int64_t e0, int r) {
        const uint32_t e = (uint32_t)(e0 + r), tb = __umulhi((uint32_t)e0, mdiv), t = __umulhi(e, mdiv);
        return (int64_t)(t - tb) * qk.k_ts + (int64_t)(e - t * (uint32_t)M) * qk.k_js;
    };
    // when M divides the chunk, every chunk starts on a token (r0 is one), so
    // the key rows' offsets are the same for every chunk: made once here
    const bool kfix = !rw && (C % M) == 0;
    if (kfix) {
#pragma unroll
        for (int i = 0; i < UPR; ++i) ot[i] += (uint32_t)(krel(r0, i * RPI + lane / UPR) * ES);
    }
    uint32_t ou[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) ou[i] = (uint32_t)((i * 64 + lane) * 16 - 1024 * (i % 4));
    const uint32_t o4 = (uint32_t)(lane * 4);
    // the tile's source: w rows of the chunk, or (fixed offsets) the key rows
    // from the chunk's first token, advanced by one chunk per issue; with
    // per-chunk offsets the key head's base
    const char *kb0 = (const char *)((const bf16 *)qk.k + qkh);
    const char *pt = rw ? (const char *)(w + (r0 * HV + hv) * KD)
                        : (kfix ? kb0 + (int64_t)__umulhi((uint32_t)r0, mdiv) * qk.k_ts * ES : kb0);
    const int64_t stt = rw ? (int64_t)C * ldw * ES : (kfix ? (int64_t)(C / M) * qk.k_ts * ES : 0);
    // bytes spanned by a chunk's first n key rows when it starts on a token
    auto kspan_fix = [&](int n) {
        const uint32_t rr = (uint32_t)(n - 1), t = __umulhi(rr, mdiv);
        return (uint32_t)(((int64_t)t * qk.k_ts + (int64_t)(rr - t * (uint32_t)M) * qk.k_js) * ES) + KD * ES;
    };
    const uint32_t kspan_full = kfix ? kspan_fix(C) : 0u;
    int64_t e_issue = r0;  // first expanded row of the next chunk to issue
    const char *pu = (const char *)(u + uv_index(bseq, r0 - bseq * TM, hv, 16 * sl, HV, VD, uv_ss));
    const int64_t stu = (int64_t)C * 16 * ES;
    const char *p4 = pp == 0 ? (const char *)(kdecay + h0r) : (const char *)(gcum + h0r);
    const int off4 = pp == 0 ? OFD : OFG;
    const int tile_off = (rw ? OFW : OFK) + hh * HALF;
    int rem_issue = (int)rows;
    auto issue = [&](int st) {  // the next chunk into ring stage st (rows past the end read as zero)
        const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem_issue));
        const uint32_t sb = ring_base + st * SB + tile_off;
        // whole rows: the half is in the offsets
        if (rw || kfix) {  // wave-uniform: fixed offsets, no per-chunk row arithmetic
            const uint32_t range = rw ? span(n, ldw * ES, KD * ES)
                                      : (n == C ? kspan_full : (n > 0 ? kspan_fix(n) : 0u));
            const rsrc_t rt = make_rsrc(pt, range);
            static_for<0, UPR>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i % 4 == 0) set_m0(sb + 1024 * i);
                dma16_m0<1024 * (i % 4)>(rt, ot[i]);
            });
        } else {
            const int64_t tb = (int64_t)__umulhi((uint32_t)e_issue, mdiv);
            const uint32_t kspan =
                n > 0 ? __builtin_amdgcn_readfirstlane((uint32_t)(krel(e_issue, n - 1) * ES)) + KD * ES : 0u;
            const rsrc_t rt = make_rsrc(pt + tb * qk.k_ts * ES, kspan);
            static_for<0, UPR>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i % 4 == 0) set_m0(sb + 1024 * i);
                dma16_m0<1024 * (i % 4)>(rt, ot[i] + (uint32_t)(krel(e_issue, i * RPI + lane / UPR) * ES));
            });
        }
        const rsrc_t ru = make_rsrc(pu, (uint32_t)(n * 16 * ES));
        const uint32_t sbu = ring_base + st * SB + OFU + pp * (C * 16 * ES);
        static_for<0, NU>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i % 4 == 0) set_m0(sbu + 1024 * i);
            dma16_m0<1024 * (i % 4)>(ru, ou[i]);
        });
        if (pp < 2) dma4(make_rsrc(p4, (uint32_t)(n * 4)), o4, ring_base + st * SB + off4);
        pt += stt;
        e_issue += C;
        pu += stu;
        p4 += st4;
        rem_issue -= C;
    };
    // the chunk before the last issue landed: everything but that issue's loads
    auto wait_ring = [&]() {
        if (pp < 2)
            wait_vmcnt<NDMA>();
        else
            wait_vmcnt<NDMA - 1>();
    };
    issue(0);
    issue(1);
    f32x4 hs[2][NKT];
#pragma unroll
    for (int kw = 0; kw < 2; ++kw)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) hs[kw][kt] = h0 ? *(const f32x4 *)(h0 + state_off(sl, kw, kt)) : zero4();
    FragT hb[2][NKS];
    auto pack = [&]() {
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    hb[kw][ks][qq] = (bf16)hs[kw][2 * ks][qq];
                    hb[kw][ks][4 + qq] = (bf16)hs[kw][2 * ks + 1][qq];
                }
    };
    auto publish_state = [&]() {
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) Sx[pp][kw][ks][lane] = hb[kw][ks];
    };
    pack();
    publish_state();
    wait_ring();    // chunk 0 landed
    lds_barrier();  // stage 0 landed; the initial state exchange is visible
    int rem = (int)rows;
    for (int c = 0, st_ = 0; c < nch; ++c, st_ = st_ == NS - 1 ? 0 : st_ + 1) {
        const HoStage<KD> &Sg = ring[st_];
        const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem));  // valid rows of the chunk
        const int ti = (int)__umulhi((uint32_t)c, mdiv);
        const int m = c - ti * M;

        // ---- phase 1: the partial products of the two K halves (w h).
        // Consecutive products go to different accumulators (each still sums
        // its own products in ks order), so none waits for the one before.
        f32x4 acc[2][4];
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[kw][rt] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const FragT a = *(const FragT *)((const char *)Sg.w[kw] + swz(16 * rt + lc, 32 * ks + 8 * lg));
                    acc[kw][rt] = mma(a, hb[kw][ks], acc[kw][rt]);
                }
        // every other read of the ring stage, before the barrier that frees
        // it: u, the key decays, the chunk's decay and K^T (read transposed,
        // ds_read_b64_tr_b16, rows in the state's permuted K order)
        HalfT uu[4];
        f32x4 kd4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            uu[rt] = lds_col4<bf16>(Sg.u[pp], 16, 16 * rt + 4 * lg, 0);
            kd4[rt] = *(const f32x4 *)(&Sg.kd[16 * rt + 4 * lg]);
        }
        const float glast = Sg.gc[n > 0 ? n - 1 : 0];
        FragT ka[2][NKT][2];
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const char *kb = (const char *)Sg.k[kw];
                    const int kbase = 32 * (kt >> 1) + 4 * (kt & 1);
                    const int j = lane & 15;
                    const int ra = 32 * s + 4 * lg + (j >> 2), rb = ra + 16;
                    const int col = kbase + 8 * (j & 3);
                    const HalfT x0 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swzk(ra, col)))));
                    const HalfT x1 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swzk(rb, col)))));
                    ka[kw][kt][s] = join<bf16>(x0, x1);
                }
        const float gl = n > 0 ? __builtin_amdgcn_exp2f(glast) : 1.0f;
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) hs[kw][kt][r] *= gl;
        // chunk c + 2 into the stage chunk c - 1 left (free since the last
        // barrier), issued after this step's products and reads: at the top
        // of the step the DMA issue, waiting on the CU's vector memory path,
        // held back phase 1 (about 7 us), and one step is time enough for
        // the loads
        issue(st_ == 0 ? 2 : st_ - 1);
        wait_ring();    // chunk c + 1 landed
        lds_barrier();  // ring stage c read; the exchanges of chunk c - 1 were read

        // ---- v_new (published to the exchange as fp16) and the phase-2
        // operands, with the arithmetic of the chunk_h stage's whole-K form
        // (v_new = u - (P0 + P1), no contraction), then phase 2, h = exp2(gl)
        // h + K^T (kd * v_new), one key half s (rows 32 s .. 32 s + 31) at a
        // time; every accumulator sees the same products in the same order as
        // there, so the states agree bit for bit
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            FragT vb, vbl;
            f16x8 v8;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int rt = 2 * s + r2;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma clang fp contract(off)
                    const float v = (float)uu[rt][r] - (acc[0][rt][r] + acc[1][rt][r]);
                    v8[4 * r2 + r] = (f16)v;
                    const float x = v * kd4[rt][r];
                    vb[4 * r2 + r] = (bf16)x;
                    vbl[4 * r2 + r] = split_lo<bf16>(x, vb[4 * r2 + r]);
                }
            }
            Vx[c & 1][pp][s][lane] = v8;
            // every accumulator's high-part product, then every low-part one:
            // each accumulator sums the same products in the same order, and
            // consecutive products are independent
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) hs[kw][kt] = mma(ka[kw][kt][s], vb, hs[kw][kt]);
#pragma unroll
            for (int kw = 0; kw < 2; ++kw)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) hs[kw][kt] = mma(ka[kw][kt][s], vbl, hs[kw][kt]);
        }
        pack();
        if (m == M - 1 && c + 1 < nch) publish_state();  // the state entering the next token chunk
        rem -= C;
    }
    lds_barrier();  // the last chunk's v_new is in the exchange (matches the output waves)
    wait_vmcnt<0>();  // no DMA may still target LDS when the block retires
    if (ht != nullptr) {
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) *(f32x4 *)(ht + state_off(sl, kw, kt)) = hs[kw][kt];
    }
}

template <int KD, int VD>
static hipError_t launch_ho_t(const ChunkParams &p, hipStream_t stream) {
    const gdp_chunk_args &a = p.a;
    const int64_t P = p.nseq * a.HV;
    const int64_t SG = VD / 16 / NP;
    const int64_t nblk = ((P + 7) / 8) * 8 * SG;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdp_chunk_ho_k<KD, VD>), dim3((unsigned)nblk), dim3(2 * NP * 64), 0, stream,
                       p.qk, a.kdecay, (const bf16 *)a.w, (const bf16 *)a.u, a.gcum, a.k_rnorm,
                       a.g, a.cu_seqlens, p.nseq, a.T, a.H, a.HV, a.M, a.h0, a.ht, (bf16 *)a.o,
                       p.uv_ss, a.scale);
    return hipGetLastError();
}

// bf16 with K in {64, 128}, V in {64, 128, 256}, M in [2, 4]
hipError_t launch_chunk_ho(const ChunkParams &p, hipStream_t stream) {
    if (p.nseq == 0 || p.a.T == 0) return hipSuccess;
    const int K = p.a.K, V = p.a.V;
    if (p.a.dtype != GDP_BF16 || p.a.M < 2) return hipErrorInvalidValue;
    if (K == 64 && V == 64) return launch_ho_t<64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_ho_t<64, 128>(p, stream);
    if (K == 64 && V == 256) return launch_ho_t<64, 256>(p, stream);
    if (K == 128 && V == 64) return launch_ho_t<128, 64>(p, stream);
    if (K == 128 && V == 128) return launch_ho_t<128, 128>(p, stream);
    if (K == 128 && V == 256) return launch_ho_t<128, 256>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdp
