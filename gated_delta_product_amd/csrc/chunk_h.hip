// chunk_h.hip -- inter-chunk state recurrence of the Gated Delta Product
// (the chunk_h stage whose outputs core.ssm.ops.gdp.chunk_o consumes: the
// state at each chunk boundary and the corrected values).
//
// For one sequence and one value head, serially over its 64-row chunks c of
// the expanded stream, with h the K x V transpose of the state S entering c:
//   snapshot  h[c] = h                     (stored as S = h^T, V x K)
//   v_new     = u - w h                    (corrected values of the chunk)
//   h         = exp2(gl) h + K^T diag(kdecay) v_new
// where gl is the chunk's total decay in log2 units (the within-chunk
// cumulative decay gcum on its last row) and kdecay = rnorm(k) exp2(gl - gcum)
// per row, both precomputed by the WY stage.
//
// hstep > 1 writes only the snapshots of chunks c with c % hstep == 0 (c
// counted from the sequence's first chunk).  With hstep = M these are the
// states the output stage reads (it takes the state entering each 64-token
// chunk, which is expanded chunk c = i*M); the other slots of h are left as
// they were.  A skipped store keeps its instruction but gets an empty buffer
// range, so the hardware drops it and nothing else in the schedule changes.
//
// One block of five waves per (sequence, value head, 16 value columns), with
// three roles (the two-slice and whole-K forms are described below):
//
// * Compute waves 0 and 1 run the serial chain and issue no global memory
//   instruction at all.  Wave k owns rows [k K/2, (k+1) K/2) of the fp32
//   state slice, in registers for the whole sequence.  Per chunk each forms
//   its partial w h over its half of K on the matrix cores; the halves meet
//   in LDS behind the step's one barrier; both form v_new, and each updates
//   its half of h.  Result tiles feed the next product directly: a result
//   tile gives a lane four consecutive rows of one column, a valid operand
//   fragment once the other operand reads its contraction index in the same
//   order (w with its K columns permuted to match h; K^T, transposed on the
//   fly by ds_read_b64_tr_b16, with its rows permuted to match v_new).  They
//   leave v_new (transposed) and the next state snapshot in LDS.
// * Prefetch wave 4 pulls the w and K lines of the chunk five ahead into L2
//   (each of a head's column blocks a share), so the memory waves hit L2.
//   The small contiguous u slice is left to the memory waves' own lead.
// * Memory waves 2 and 3 stream w, K, u, kdecay and gcum from HBM straight
//   into a three-stage LDS ring (buffer loads with the LDS destination, two
//   chunks ahead; the range check zero-fills rows past the end), and write
//   v_new and the snapshots from LDS to HBM.  They wait on their own loads
//   before each barrier, so the barrier also publishes the next stage.
//
// A compute wave's step is then bound by its own instruction stream, not by
// the memory queue.  Tile rows are XOR-swizzled in 16-byte units so the
// fragment reads of both products avoid bank conflicts.
//
// With chains to spare (many sequences, or the segments of the
// segment-parallel forward) a block runs NP = 2 column slices: compute waves
// 2p and 2p + 1 run slice p, waves 4 and 5 stream the shared w and K tiles
// and both slices' u, and wave 6 prefetches.  The tiles then cross a CU once
// per 32 columns.  To fit LDS, the compute waves store their own snapshots
// and the partial sums are exchanged through two buffers by step parity.
//
// With more chains still (bf16, V >= 128), the whole-K form runs NP = 4
// slices with one compute wave per slice: wave p holds all K rows of slice
// p's state and forms both K halves' partial products itself, in the same
// order as the split form, so the bits match and no partial-sum exchange is
// needed.  Waves 4 and 5 stream the tiles and the four u slices, wave 6
// prefetches; the tiles cross a CU once per 64 columns.
#include "gdp_common.h"
#include "gdp_internal.h"

#include <type_traits>

namespace gdp {

namespace {
constexpr int C = 64;
}  // namespace

template <typename T, int KD, int NP>
struct HStage {
    T w[2][C * (KD / 2)];  // w half tiles [K half], swizzled rows
    T k[2][C * (KD / 2)];  // K half tiles [K half], swizzled rows
    T u[NP][C * 16];       // u slices, plain rows of 16 elements
    float kd[C];           // key decay factor per row (0 past the end)
    float gc[C];           // cumulative log2 decay per row
};

// h0 and ht may be the same buffer (the segment-parallel forward hands each
// segment its entering state and takes its final state in place): every
// lane reads its own 16-byte units of h0 before the chain starts and writes
// the same units of ht after it ends, so neither is declared __restrict__.
template <typename T, int KD, int VD, int NP, bool FK>
__global__ void __launch_bounds__(((FK ? NP : 2 * NP) + 3) * 64)
gdp_chunk_h_k(const T *__restrict__ k, const float *__restrict__ kdecay, const T *__restrict__ w,
              const T *__restrict__ u, const float *__restrict__ gcum, const int32_t *__restrict__ cu,
              int64_t nseq, int64_t Ttok, int H, int HV, int M, int64_t h_chunks,
              const float *h0, float *ht, T *__restrict__ v_new,
              T *__restrict__ hout, int64_t uv_ss, int hstep) {
    typedef typename Frag<T>::type FragT;
    typedef typename Frag<T>::half HalfT;
    constexpr int ES = (int)sizeof(T);
    constexpr int KH = KD / 2;                 // state rows per compute wave
    constexpr int RB = KH * ES;                // bytes per half-tile row
    constexpr int UPR = RB / 16;               // 16-byte units per half-tile row
    constexpr int RPI = 64 / UPR;              // half-tile rows per DMA instruction
    constexpr int UUPR = 16 * ES / 16;         // 16-byte units per u row
    constexpr int NU = C * UUPR / 64;          // DMA instructions for the u slice
    constexpr int NS = 3;                      // ring stages (prefetch distance 2)
    // With one column pair the memory waves store the state snapshots from
    // an LDS staging area; with two, the compute waves store their own (a
    // 16-byte store per state tile pair), which keeps the block within LDS.
    constexpr bool SNAP_LDS = NP == 1;
    // FK: one compute wave per slice holds both K halves of its state (no
    // exchange of partial products); otherwise two waves per slice, one per
    // K half, swap their phase-1 partials through LDS
    constexpr int NC = FK ? NP : 2 * NP;       // compute waves
    static_assert(!FK || (NP > 1 && !SNAP_LDS), "the whole-K form stores its own snapshots");
    constexpr int NX = NP == 1 ? NS : 2;       // exchange buffers (by stage, or by step parity)
    constexpr int NKT = KH / 16;               // 16-row state tiles per compute wave
    constexpr int NKS = KH / 32;               // phase-1 contraction steps per wave
    constexpr int LDT = 64 + 32 / ES;          // row stride of the v_new transpose
    constexpr int LDH = KD + 16 / ES;          // row stride of the snapshot staging
    constexpr int S = VD / 16;                 // column slices per head
    constexpr int SG = S / NP;                 // blocks per head (NP slices each)
    constexpr int SB = (int)sizeof(HStage<T, KD, NP>);
    // memory wave 0 loads the w halves and kdecay, wave 1 the K halves, u and gcum
    constexpr int NDMA0 = 2 * UPR + 1, NDMA1 = 2 * UPR + NU * NP + 1;
    constexpr int HLPR = KD * ES / 16;         // lanes per snapshot row (16 B each)
    constexpr int HRPI = 64 / HLPR;            // snapshot rows per store instruction
    constexpr int NHS = 8 / HRPI > 0 ? 8 / HRPI : 1;  // snapshot stores per memory wave (8 rows)
    constexpr int NVS = 2;                     // v_new stores per memory wave (32 rows)
    static_assert(NKS >= 1 && (UPR & (UPR - 1)) == 0 && HRPI <= 8, "tile shape");
    constexpr int NHS_M = SNAP_LDS ? NHS : 0;  // snapshot stores per memory wave and slice
    static_assert(NDMA1 + (NHS_M + NVS) * NP < 64, "in-flight count must fit the vector memory counter");
    static_assert(S % NP == 0, "column pairs per block");
    static_assert(SB % 16 == 0, "stage size");

    __shared__ __attribute__((aligned(16))) HStage<T, KD, NP> ring[NS];
    __shared__ __attribute__((aligned(16))) f32x4 Xs[FK ? 1 : NX][FK ? 1 : NP][FK ? 1 : 2][FK ? 1 : 4][64];  // [buffer][pair][wave][row tile][lane]
    __shared__ __attribute__((aligned(16))) T Vt[2][NP][16 * LDT];       // [parity][pair] v_new, column-major
    __shared__ __attribute__((aligned(16))) T Hs[SNAP_LDS ? 2 : 1][NP][SNAP_LDS ? 16 * LDH : 8];  // [parity][pair] snapshot rows (V x K)
    __shared__ __attribute__((aligned(16))) char Pf[1024];            // landing area of L2 prefetches

    // ---- block -> (sequence, value head, slice group); the groups of one
    // head share an XCD.  Group slg holds the NP slices [NP slg, NP slg + NP):
    // compute waves 2p and 2p + 1 run slice NP slg + p.
    const int64_t P = nseq * HV;
    const int64_t id = blockIdx.x;
    const int64_t slot = id / 8, xcd = id % 8;
    const int64_t pair = (slot / SG) * 8 + xcd;
    const int slg = (int)(slot % SG);
    const int sl0 = NP * slg;
    if (pair >= P) return;
    const int64_t seq = pair / HV;
    const int hv = (int)(pair % HV);
    const int hk = hv / (HV / H);
    int64_t bos, eos;
    seq_bounds(cu, Ttok, seq, bos, eos);
    const int64_t rows = (eos - bos) * M;
    const int nch = (int)ceil_div64(rows, C);
    const int64_t cbase = items_before(cu, Ttok, M, C, seq);

    const int lane = lane_id(), wave = wave_id();
    const int lg = lane >> 4, lc = lane & 15;
    const int sl = sl0 + (wave < NC ? (FK ? wave : wave >> 1) : 0);  // a compute wave's slice
    // The fp32 state of compute wave kw in its permuted K order (see below):
    // element (kt, q) is S[16sl + lc][kw*KH + 32(kt/2) + 8lg + 4(kt%2) + q],
    // four consecutive K indices per (kt), i.e. one 16-byte unit of h0 / ht.
    auto state_off = [&](int kw_, int kt) {
        return ((seq * HV + hv) * (int64_t)VD + 16 * sl + lc) * KD + kw_ * KH + 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1);
    };
    if (nch == 0) {  // empty sequence: the final state is the initial one
        if (ht != nullptr && wave < NC) {
#pragma unroll
            for (int h2 = 0; h2 < (FK ? 2 : 1); ++h2) {
                const int kwe = FK ? h2 : (wave & 1);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    *(f32x4 *)(ht + state_off(kwe, kt)) = h0 ? *(const f32x4 *)(h0 + state_off(kwe, kt)) : zero4();
            }
        }
        return;
    }
    const int ldk = H * KD, ldw = HV * KD;  // global row strides (elements)
    const int64_t r0 = bos * M;  // first expanded row of the sequence
    const int64_t h0r = hm_index(cu ? 0 : seq, HV, hv, Ttok * M, r0);  // kdecay / gcum of row r0

    auto clamp_rows = [](int r) { return r < 0 ? 0 : (r < C ? r : C); };
    // bytes a buffer resource must cover for n rows of `width_b` bytes
    auto span = [](int n, int stride_b, int width_b) { return (uint32_t)(n > 0 ? (n - 1) * stride_b + width_b : 0); };
    // 16-byte units of half-tile row r are XOR-swizzled by xw(r) in the w
    // tiles and by xk(r) in the K tiles, which are only read transposed:
    // for bf16 128-byte rows r mod 8 keeps those reads at the 2-way bank
    // floor of same-half 8-byte reads, where (r / 2) mod 8 made them 4-way
    auto xw = [](int r) { return (r >> 1) & (UPR - 1); };
    auto xk = [](int r) { return (UPR == 8 && ES == 2) ? r & 7 : (r >> 1) & (UPR - 1); };
    // byte offset of element column `col` of half-tile row r, w or K tile
    auto swz_at = [&](int r, int col, int x) {
        const int b = col * ES;
        return r * RB + ((((b >> 4) ^ x)) << 4) + (b & 15);
    };
    auto swz = [&](int r, int col) { return swz_at(r, col, xw(r)); };
    auto swzk = [&](int r, int col) { return swz_at(r, col, xk(r)); };

    if (wave == NC + 2) {
        // ======================= prefetch wave =======================
        // Pulls the lines of chunk c + PF into L2 while the memory waves
        // stream chunk c + 2 into LDS, so their loads hit L2 instead of
        // waiting on HBM.  The SG blocks of a head share an XCD (and its L2);
        // block slg prefetches rows [RPB slg, RPB slg + RPB) of each chunk.
        // The data lands in a scratch LDS area that nothing reads.
        // prefetch distance in chunks; the whole-K form's two blocks per head
        // need their lines within a step of each other (3 ahead: 1.34x the
        // algorithmic bytes; 2 ahead is faster)
        constexpr int PF = NP == 1 ? 5 : (FK ? 2 : 3);
        constexpr int RPB = C / SG;              // rows per block per chunk
        static_assert(RPB * KD * ES / 128 <= 64 && KD * ES >= 128,
                      "one 4-byte load per line must cover a block's rows");
        const uint32_t pf = lds_addr(&Pf[0]);
        const int rbw = KD * ES;  // row bytes of w / k
        const char *pw = (const char *)(w + ((r0 + RPB * slg) * HV + hv) * KD);
        const char *pk = (const char *)(k + ((r0 + RPB * slg) * H + hk) * KD);
        const char *pd = (const char *)(kdecay + h0r);
        const char *pg = (const char *)(gcum + h0r);
        const int64_t stw = (int64_t)C * ldw * ES, stk = (int64_t)C * ldk * ES, st4 = (int64_t)C * 4;
        // rows [0, nr) of a tile with `rb`-byte rows `ld` bytes apart: one
        // 4-byte load per 128-byte line is enough to bring it into L2
        auto rows_to_l2 = [&](const char *base, int nr, int ld, int rb) {
            const int lpr = rb / 128;  // lines per row
            const rsrc_t r = make_rsrc(base, span(nr, ld, rb));
            dma4(r, (uint32_t)((lane / lpr) * ld + (lane % lpr) * 128), pf);  // rows >= nr: out of range
        };
        int rem_pf = (int)rows;
        auto prefetch = [&](int c) {
            const int nr = __builtin_amdgcn_readfirstlane(clamp_rows(rem_pf - C * c - RPB * slg));
            const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem_pf - C * c));
            const int64_t oc = c;
            rows_to_l2(pw + oc * stw, nr < RPB ? nr : RPB, ldw * ES, rbw);
            rows_to_l2(pk + oc * stk, nr < RPB ? nr : RPB, ldk * ES, rbw);
            if (slg == 0) {  // 256 contiguous bytes each: one block of the head is enough
                dma4(make_rsrc(pd + oc * st4, (uint32_t)(n * 4)), (uint32_t)(lane * 4), pf);
                dma4(make_rsrc(pg + oc * st4, (uint32_t)(n * 4)), (uint32_t)(lane * 4), pf);
            }
        };
        for (int c = 2; c < PF; ++c) prefetch(c);
        lds_barrier();
        for (int c = 0; c < nch; ++c) {
            prefetch(c + PF);
            wait_vmcnt<24>();  // bound the number of prefetches in flight
            lds_barrier();
        }
        lds_barrier();
        wait_vmcnt<0>();
        return;
    }

    if (wave >= NC) {
        // ======================= memory waves =======================
        const int mw = wave - NC;
        const int64_t hroom = h_chunks - cbase;  // chunks whose snapshot fits below h_chunks
        const int hlim = hroom < 0 ? 0 : (hroom > nch ? nch : (int)hroom);
        const uint32_t ring_base = lds_addr(&ring[0]);
        typedef HStage<T, KD, NP> Stage;
        constexpr int OFW = (int)__builtin_offsetof(Stage, w);
        constexpr int OFK = (int)__builtin_offsetof(Stage, k);
        constexpr int OFU = (int)__builtin_offsetof(Stage, u);
        constexpr int OFD = (int)__builtin_offsetof(Stage, kd);
        constexpr int OFG = (int)__builtin_offsetof(Stage, gc);
        constexpr int HALF = C * KH * ES;  // bytes of one half tile
        // per-lane source offsets inside a chunk, less the DMA's offset in
        // its 4 KiB M0 window; tile t (0: w, 1: K) half hh
        uint32_t ot[2][UPR];
#pragma unroll
        for (int i = 0; i < UPR; ++i) {
            const int r = i * RPI + lane / UPR;
            const int unit = (lane % UPR) ^ (mw == 0 ? xw(r) : xk(r));
            const int ld = mw == 0 ? ldw : ldk;
            ot[0][i] = (uint32_t)((r * ld) * ES + unit * 16 - 1024 * (i % 4));
            ot[1][i] = ot[0][i] + KH * ES;  // second K half of the same rows
        }
        uint32_t ou[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i)
            ou[i] = (uint32_t)((i * 64 + lane) * 16 - 1024 * (i % 4));  // the slice's rows are contiguous
        const uint32_t o4 = (uint32_t)(lane * 4);

        const char *pt = mw == 0 ? (const char *)(w + (r0 * HV + hv) * KD) : (const char *)(k + (r0 * H + hk) * KD);
        const int ldt = mw == 0 ? ldw : ldk;
        const int64_t stt = (int64_t)C * ldt * ES;
        const int64_t bseq = cu ? 0 : seq;  // batch row of the sequence
        const char *pu = (const char *)(u + uv_index(bseq, r0 - bseq * Ttok * M, hv, 16 * sl0, HV, VD, uv_ss));
        const int64_t ssb = uv_ss * ES;  // bytes between consecutive slices of u / v_new
        const char *p4 = mw == 0 ? (const char *)(kdecay + h0r) : (const char *)(gcum + h0r);
        const int64_t stu = (int64_t)C * 16 * ES, st4 = (int64_t)C * 4;  // slice bytes per chunk
        const int tile_off = mw == 0 ? OFW : OFK;
        const int off4 = mw == 0 ? OFD : OFG;
        int rem_issue = (int)rows;

        // stream the next chunk into stage st (NDMA0 or NDMA1 instructions)
        auto issue = [&](int st) {
            const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem_issue));
            const uint32_t sb = ring_base + st * SB + tile_off;
            const rsrc_t rt = make_rsrc(pt, span(n, ldt * ES, KD * ES));
            static_for<0, 2>([&](auto hc) {
                constexpr int hh = decltype(hc)::value;
                static_for<0, UPR>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if constexpr (i % 4 == 0) set_m0(sb + (hh * HALF + 1024 * i));
                    dma16_m0<1024 * (i % 4)>(rt, ot[hh][i]);
                });
            });
            if (mw == 1) {
                static_for<0, NP>([&](auto pc) {
                    constexpr int pp = decltype(pc)::value;
                    const rsrc_t ru = make_rsrc(pu + pp * ssb, (uint32_t)(n * 16 * ES));
                    const uint32_t sbu = ring_base + st * SB + OFU + pp * (C * 16 * ES);
                    static_for<0, NU>([&](auto ic) {
                        constexpr int i = decltype(ic)::value;
                        if constexpr (i % 4 == 0) set_m0(sbu + 1024 * i);
                        dma16_m0<1024 * (i % 4)>(ru, ou[i]);
                    });
                });
            }
            dma4(make_rsrc(p4, (uint32_t)(n * 4)), o4, ring_base + st * SB + off4);
            pt += stt;
            pu += stu;
            p4 += st4;
            rem_issue -= C;
        };

        // snapshot of the state entering chunk c: rows [8mw, 8mw + 8) of each
        // of the block's V slices, from Hs[c & 1]
        char *ph = (char *)(hout + (cbase * HV + hv) * (int64_t)VD * KD + (int64_t)(16 * sl0) * KD);
        const int64_t sth = (int64_t)HV * VD * KD * ES;
        auto store_h = [&](int c) {
            const rsrc_t rh = make_rsrc(ph, c < hlim && c % hstep == 0 ? (uint32_t)(NP * 16 * KD * ES) : 0u);
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) {
                const T *src = Hs[SNAP_LDS ? (c & 1) : 0][pp];
#pragma unroll
                for (int i = 0; i < NHS; ++i) {
                    const int r = 8 * mw + i * HRPI + lane / HLPR;
                    const int e = (lane % HLPR) * (16 / ES);
                    const uint4 val = *(const uint4 *)(src + r * LDH + e);
                    buf_store16(rh, (uint32_t)(((pp * 16 + r) * KD + e) * ES), val);
                }
            }
            ph += sth;
        };
        // v_new rows [32mw, 32mw + 32) of chunk c, from Vt[c & 1]
        char *pv = (char *)(v_new + uv_index(bseq, r0 - bseq * Ttok * M, hv, 16 * sl0, HV, VD, uv_ss));
        int rem_v = (int)rows;
        auto store_v = [&](int c) {
            const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem_v));
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) {
                const rsrc_t rv = make_rsrc(pv + pp * ssb, (uint32_t)(n * 16 * ES));
#pragma unroll
                for (int r2 = 0; r2 < NVS; ++r2) {
                    const HalfT o4v = lds_col4<T>(Vt[c & 1][pp], LDT, 4 * lg, 32 * mw + 16 * r2);
                    const uint32_t off = (uint32_t)(((32 * mw + 16 * r2 + lc) * 16 + 4 * lg) * ES);
                    if constexpr (ES == 2)
                        buf_store8(rv, off, __builtin_bit_cast(uint2, o4v));
                    else
                        buf_store16(rv, off, __builtin_bit_cast(uint4, o4v));
                }
            }
            pv += stu;
            rem_v -= C;
        };

        auto loop = [&](auto ndc) {
            constexpr int ND = decltype(ndc)::value;
            issue(0);
            issue(1);
            wait_vmcnt<ND>();  // chunk 0 landed
            lds_barrier();     // publishes stage 0 and the zero snapshot
            for (int c = 0; c < nch; ++c) {
                // chunk c + 2 into the stage that chunk c - 1 left (its tiles
                // went to registers before the last barrier)
                issue((c + 2) % NS);
                // chunk c + 1 landed: count what was issued after its DMAs
                if (c == 0)
                    wait_vmcnt<ND>();
                else if (c == 1)
                    wait_vmcnt<ND + NHS_M * NP>();
                else
                    wait_vmcnt<ND + (NHS_M + NVS) * NP>();
                lds_barrier();  // compute step c's exchange; publishes stage c + 1
                if constexpr (SNAP_LDS) store_h(c);
                if (c >= 1) store_v(c - 1);
            }
            lds_barrier();  // v_new of the last chunk is in Vt
            store_v(nch - 1);
            wait_vmcnt<0>();  // no DMA may still target LDS when the block retires
        };
        if (mw == 0)
            loop(std::integral_constant<int, NDMA0>{});
        else
            loop(std::integral_constant<int, NDMA1>{});
        return;
    }

    // ======================= compute waves =======================
    // (instantiated per wave so every wave-dependent offset is a constant)
    auto compute = [&](auto wc) {
    constexpr int kw = decltype(wc)::value & 1;   // K half of the slice
    constexpr int pp = decltype(wc)::value >> 1;  // column pair of the block
    // State slice of this wave, in a permuted K order: hs[kt][q] holds h at
    // K index kw*KH + kperm(kt, 4lg + q), column 16sl + lc, with
    //   kperm(kt, i) = 32(kt/2) + 8(i/4) + 4(kt%2) + i%4,
    // so that hb[ks] (tiles 2ks, 2ks+1 in storage precision) holds 8
    // consecutive K indices 32ks + 8lg .. +7: the phase-1 operand matches a
    // plain 16-byte row read of w and the snapshot is a 16-byte write.  K^T
    // is read with the same permutation.
    f32x4 hs[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) hs[kt] = h0 ? *(const f32x4 *)(h0 + state_off(kw, kt)) : zero4();
    FragT hb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hb[ks][q] = from_f32<T>(hs[2 * ks][q]);
            hb[ks][4 + q] = from_f32<T>(hs[2 * ks + 1][q]);
        }
    // the state entering chunk cc: staged in LDS for the memory waves, or
    // stored straight to h (16 bytes per lane and tile pair; none at or past
    // h_chunks, nor where cc % hstep != 0)
    const int64_t hroom_c = h_chunks - cbase;
    const int hlim_c = hroom_c < 0 ? 0 : (hroom_c > nch ? nch : (int)hroom_c);
    auto put_snapshot = [&](int cc) {
        if constexpr (!SNAP_LDS) {
            const T *base = hout + ((cbase + cc) * HV + hv) * (int64_t)VD * KD + (int64_t)(16 * sl) * KD;
            const rsrc_t rh = make_rsrc(base, cc < hlim_c && cc % hstep == 0 ? (uint32_t)(16 * KD * ES) : 0u);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                buf_store16(rh, (uint32_t)((lc * KD + kw * KH + 32 * ks + 8 * lg) * ES),
                            __builtin_bit_cast(uint4, hb[ks]));
            return;
        }
        T *dst = Hs[SNAP_LDS ? (cc & 1) : 0][pp];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            T *p = dst + lc * LDH + kw * KH + 32 * ks + 8 * lg;
            if constexpr (ES == 2) {
                *(FragT *)p = hb[ks];
            } else {
                HalfT lo, hi;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    lo[q] = hb[ks][q];
                    hi[q] = hb[ks][4 + q];
                }
                *(HalfT *)p = lo;
                *(HalfT *)(p + 4) = hi;
            }
        }
    };
    put_snapshot(0);  // h[0]: the initial state
    lds_barrier();        // stage 0 landed
    int rem = (int)rows;  // rows left from the current chunk

    // One chunk on ring stage ST (a compile-time constant, so every LDS
    // address below is a fixed offset from a per-lane base).
    auto step = [&](int c, auto stc) {
        constexpr int ST = decltype(stc)::value;
        const HStage<T, KD, NP> &Sg = ring[ST];
        const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem));  // uniform

        // phase 1: partial w h over this wave's half of K (w columns
        // 32ks + 8lg .. +7, the order of hb)
        f32x4 acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            acc[rt] = zero4();
            const int r = 16 * rt + lc;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const char *wb = (const char *)Sg.w[kw];
                FragT a;
                if constexpr (ES == 2) {
                    a = *(const FragT *)(wb + swz(r, 32 * ks + 8 * lg));
                } else {
                    a = join<T>(*(const HalfT *)(wb + swz(r, 32 * ks + 8 * lg)),
                                *(const HalfT *)(wb + swz(r, 32 * ks + 8 * lg + 4)));
                }
                acc[rt] = mma(a, hb[ks], acc[rt]);
            }
        }

        // reads that need no barrier: u, key decays, the chunk decay, K^T
        HalfT uu[4];
        f32x4 kd4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            uu[rt] = lds_col4<T>(Sg.u[pp], 16, 16 * rt + 4 * lg, 0);
            kd4[rt] = *(const f32x4 *)(&Sg.kd[16 * rt + 4 * lg]);
        }
        const float glast = Sg.gc[n > 0 ? n - 1 : 0];
        FragT ka[NKT][2];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                HalfT x0, x1;
                const char *kb = (const char *)Sg.k[kw];
                const int kbase = 32 * (kt >> 1) + 4 * (kt & 1);  // kperm(kt, 0)
                if constexpr (ES == 2) {
                    // transposed read: source lane j of the 16-lane group
                    // points at row rowA + j/4 and the 4 K indices
                    // kperm(kt, 4(j%4) .. +3); output lane i then holds
                    // K index kperm(kt, i) of rows rowA .. rowA+3
                    const int j = lane & 15;
                    const int ra = 32 * s + 4 * lg + (j >> 2), rb = ra + 16;
                    const int col = kbase + 8 * (j & 3);
                    x0 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swzk(ra, col)))));
                    x1 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swzk(rb, col)))));
                } else {
                    const int col = kbase + 8 * (lc >> 2) + (lc & 3);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x0[i] = *(const float *)(kb + swzk(32 * s + 4 * lg + i, col));
                        x1[i] = *(const float *)(kb + swzk(32 * s + 16 + 4 * lg + i, col));
                    }
                }
                ka[kt][s] = join<T>(x0, x1);
            }
        // gl <= 0; rows past the end carry key decay 0
        const float gl = n > 0 ? __builtin_amdgcn_exp2f(glast) : 1.0f;
        // the decayed state, before the barrier
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q) hs[kt][q] *= gl;

        // exchange partials (one buffer per ring stage, or by step parity
        // with two column pairs: the partner reads a buffer before the next
        // barrier, and it is written again two barriers later)
        const int xb = NP == 1 ? ST : (c & 1);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Xs[xb][pp][kw][rt][lane] = acc[rt];
        lds_barrier();

        // v_new = u - (P0 + P1), the two halves' partials summed (the sum
        // is the same in both waves, addition being commutative), and the
        // phase-2 operand kd * v_new, in bf16 as a high and a low part
        // (split_lo), one product each; no contraction, so every form of
        // the stage rounds the same operations
        FragT vb[2], vbl[2];
        T *vt = Vt[c & 1][pp];
        static_for<0, 4>([&](auto rtc) {
            constexpr int rt = decltype(rtc)::value;
            const f32x4 other = Xs[xb][pp][kw ^ 1][rt][lane];
            HalfT v4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma clang fp contract(off)
                const float v = to_f32(uu[rt][q]) - (acc[rt][q] + other[q]);
                v4[q] = from_f32<T>(v);
                const float x = v * kd4[rt][q];
                vb[rt >> 1][4 * (rt & 1) + q] = from_f32<T>(x);
                if constexpr (Split<T>::on) vbl[rt >> 1][4 * (rt & 1) + q] = split_lo<T>(x, vb[rt >> 1][4 * (rt & 1) + q]);
            }
            // compute wave kw publishes rows [32kw, 32kw + 32)
            if constexpr ((rt >> 1) == kw) *(HalfT *)(&vt[lc * LDT + 16 * rt + 4 * lg]) = v4;
        });

        // phase 2: h = exp2(gl) h + K^T (kd * v_new), this wave's K half
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                hs[kt] = mma(ka[kt][s], vb[s], hs[kt]);
                if constexpr (Split<T>::on) hs[kt] = mma(ka[kt][s], vbl[s], hs[kt]);
            }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hb[ks][q] = from_f32<T>(hs[2 * ks][q]);
                hb[ks][4 + q] = from_f32<T>(hs[2 * ks + 1][q]);
            }
        if (SNAP_LDS || c + 1 < nch) put_snapshot(c + 1);  // the state entering chunk c + 1
        rem -= C;
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    static_assert(NS == 3, "the loop below is unrolled over three ring stages");
    for (int c = 0; c < nch; c += 3) {
        step(c, I0{});
        if (c + 1 < nch) step(c + 1, I1{});
        if (c + 2 < nch) step(c + 2, I2{});
    }
    lds_barrier();  // publishes the last chunk's v_new
    if (ht != nullptr) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) *(f32x4 *)(ht + state_off(kw, kt)) = hs[kt];
    }
    };

    if constexpr (FK) {
    // ============ compute waves, whole-K form (one wave per slice) ============
    // The same arithmetic as the split form above, in the same order, so the
    // bits match: the two K halves' phase-1 partials P0, P1 are formed apart
    // and v_new = u - (P0 + P1).  No exchange buffer and no partner: the one
    // barrier per chunk stays where the split form has it.
    auto compute_fk = [&](auto wc) {
    constexpr int pp = decltype(wc)::value;  // slice of the block
    f32x4 hs[2][NKT];
#pragma unroll
    for (int kw = 0; kw < 2; ++kw)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) hs[kw][kt] = h0 ? *(const f32x4 *)(h0 + state_off(kw, kt)) : zero4();
    FragT hb[2][NKS];
    auto pack = [&]() {
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    hb[kw][ks][q] = from_f32<T>(hs[kw][2 * ks][q]);
                    hb[kw][ks][4 + q] = from_f32<T>(hs[kw][2 * ks + 1][q]);
                }
    };
    pack();
    const int64_t hroom_c = h_chunks - cbase;
    const int hlim_c = hroom_c < 0 ? 0 : (hroom_c > nch ? nch : (int)hroom_c);
    auto put_snapshot = [&](int cc) {
        const T *base = hout + ((cbase + cc) * HV + hv) * (int64_t)VD * KD + (int64_t)(16 * sl) * KD;
        const rsrc_t rh = make_rsrc(base, cc < hlim_c && cc % hstep == 0 ? (uint32_t)(16 * KD * ES) : 0u);
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                buf_store16(rh, (uint32_t)((lc * KD + kw * KH + 32 * ks + 8 * lg) * ES),
                            __builtin_bit_cast(uint4, hb[kw][ks]));
    };
    put_snapshot(0);      // h[0]: the initial state
    lds_barrier();        // stage 0 landed
    int rem = (int)rows;  // rows left from the current chunk

    auto step = [&](int c, auto stc) {
        constexpr int ST = decltype(stc)::value;
        const HStage<T, KD, NP> &Sg = ring[ST];
        const int n = __builtin_amdgcn_readfirstlane(clamp_rows(rem));  // uniform

        // phase 1: the partial products of the two K halves
        f32x4 acc[2][4];
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                acc[kw][rt] = zero4();
                const int r = 16 * rt + lc;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const FragT a = *(const FragT *)((const char *)Sg.w[kw] + swz(r, 32 * ks + 8 * lg));
                    acc[kw][rt] = mma(a, hb[kw][ks], acc[kw][rt]);
                }
            }
        // every other read of the stage, before the barrier that frees it
        HalfT uu[4];
        f32x4 kd4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            uu[rt] = lds_col4<T>(Sg.u[pp], 16, 16 * rt + 4 * lg, 0);
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
                    const int kbase = 32 * (kt >> 1) + 4 * (kt & 1);  // kperm(kt, 0)
                    const int j = lane & 15;
                    const int ra = 32 * s + 4 * lg + (j >> 2), rb = ra + 16;
                    const int col = kbase + 8 * (j & 3);
                    const HalfT x0 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swzk(ra, col)))));
                    const HalfT x1 = __builtin_bit_cast(HalfT, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) const char *)(kb + swzk(rb, col)))));
                    ka[kw][kt][s] = join<T>(x0, x1);
                }
        const float gl = n > 0 ? __builtin_amdgcn_exp2f(glast) : 1.0f;
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int q = 0; q < 4; ++q) hs[kw][kt][q] *= gl;
        lds_barrier();  // publishes the next stage; Vt[c & 1] is free again

        FragT vb[2], vbl[2];  // phase-2 operands: high and low bf16 parts
        T *vt = Vt[c & 1][pp];
        static_for<0, 4>([&](auto rtc) {
            constexpr int rt = decltype(rtc)::value;
            HalfT v4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma clang fp contract(off)
                const float v = to_f32(uu[rt][q]) - (acc[0][rt][q] + acc[1][rt][q]);
                v4[q] = from_f32<T>(v);
                const float x = v * kd4[rt][q];
                vb[rt >> 1][4 * (rt & 1) + q] = from_f32<T>(x);
                if constexpr (Split<T>::on) vbl[rt >> 1][4 * (rt & 1) + q] = split_lo<T>(x, vb[rt >> 1][4 * (rt & 1) + q]);
            }
            *(HalfT *)(&vt[lc * LDT + 16 * rt + 4 * lg]) = v4;
        });

        // phase 2, both halves: h = exp2(gl) h + K^T (kd * v_new)
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    hs[kw][kt] = mma(ka[kw][kt][s], vb[s], hs[kw][kt]);
                    if constexpr (Split<T>::on) hs[kw][kt] = mma(ka[kw][kt][s], vbl[s], hs[kw][kt]);
                }
        pack();
        if (c + 1 < nch) put_snapshot(c + 1);  // the state entering chunk c + 1
        rem -= C;
    };

    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    for (int c = 0; c < nch; c += 3) {
        step(c, J0{});
        if (c + 1 < nch) step(c + 1, J1{});
        if (c + 2 < nch) step(c + 2, J2{});
    }
    lds_barrier();  // publishes the last chunk's v_new
    if (ht != nullptr) {
#pragma unroll
        for (int kw = 0; kw < 2; ++kw)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) *(f32x4 *)(ht + state_off(kw, kt)) = hs[kw][kt];
    }
    };

        static_for<0, NP>([&](auto wc) {
            if (wave == decltype(wc)::value) compute_fk(wc);
        });
    } else {
        if (wave == 0)
            compute(std::integral_constant<int, 0>{});
        else if (wave == 1 || NP == 1)
            compute(std::integral_constant<int, 1>{});
        else if constexpr (NP == 2) {
            if (wave == 2)
                compute(std::integral_constant<int, 2>{});
            else
                compute(std::integral_constant<int, 3>{});
        }
    }
}

template <typename T, int KD, int VD, int NP, bool FK = false>
static hipError_t launch_chunk_h_np(const ChunkParams &p, hipStream_t stream) {
    const gdp_chunk_args &a = p.a;
    const int64_t P = p.nseq * a.HV;
    const int64_t SG = VD / 16 / NP;
    const int64_t nblk = ((P + 7) / 8) * 8 * SG;
    constexpr int NC = FK ? NP : 2 * NP;
    hipLaunchKernelGGL((gdp_chunk_h_k<T, KD, VD, NP, FK>), dim3((unsigned)nblk), dim3((NC + 3) * 64), 0, stream,
                       (const T *)a.k, a.kdecay, (const T *)a.w, (const T *)a.u, a.gcum, a.cu_seqlens,
                       p.nseq, a.T, a.H, a.HV, a.M, a.h_chunks, a.h0, a.ht, (T *)a.v_new, (T *)a.h, p.uv_ss,
                       p.hstep);
    return hipGetLastError();
}

// One 16-column slice per block gives the most chains; two slices per block
// halve the w and K tiles each CU streams per column, and the whole-K form's
// four slices halve them again.  More slices per block pay once there are
// chains enough to fill every CU twice over: the whole-K form is taken for
// bf16 with V >= 128 when sequences x value heads x V / 64 >= 512 blocks,
// else the two-slice form when sequences x value heads x V / 32 >= 512,
// else one slice.  All three give the same bits: every slice runs the same
// arithmetic.
template <typename T, int KD, int VD>
static hipError_t launch_chunk_h_t(const ChunkParams &p, hipStream_t stream) {
    if constexpr (std::is_same<T, bf16>::value && VD >= 128) {
        if (p.nseq * p.a.HV * (VD / 64) >= 512) return launch_chunk_h_np<T, KD, VD, 4, true>(p, stream);
    }
    if constexpr (std::is_same<T, bf16>::value && VD >= 32) {
        if (p.nseq * p.a.HV * (VD / 32) >= 512) return launch_chunk_h_np<T, KD, VD, 2>(p, stream);
    }
    return launch_chunk_h_np<T, KD, VD, 1>(p, stream);
}

// bf16: K in {64, 128} x V in {64, 128, 256}; f32 (small-case reference
// precision): K = 64, V in {64, 128}.
static hipError_t launch_chunk_h_bf16(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_h_t<bf16, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_chunk_h_t<bf16, 64, 128>(p, stream);
    if (K == 64 && V == 256) return launch_chunk_h_t<bf16, 64, 256>(p, stream);
    if (K == 128 && V == 64) return launch_chunk_h_t<bf16, 128, 64>(p, stream);
    if (K == 128 && V == 128) return launch_chunk_h_t<bf16, 128, 128>(p, stream);
    if (K == 128 && V == 256) return launch_chunk_h_t<bf16, 128, 256>(p, stream);
    return hipErrorInvalidValue;
}
static hipError_t launch_chunk_h_f32(const ChunkParams &p, hipStream_t stream) {
    const int K = p.a.K, V = p.a.V;
    if (K == 64 && V == 64) return launch_chunk_h_t<float, 64, 64>(p, stream);
    if (K == 64 && V == 128) return launch_chunk_h_t<float, 64, 128>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_h(const ChunkParams &p, hipStream_t stream) {
    if (p.nseq == 0 || p.a.T == 0) return hipSuccess;
    return p.a.dtype == GDP_BF16 ? launch_chunk_h_bf16(p, stream) : launch_chunk_h_f32(p, stream);
}

}  // namespace gdp
