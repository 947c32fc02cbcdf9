// gdp_internal.h -- launcher interface between the C ABI (api.cpp) and the
// kernel translation units.  Host-only declarations; no device code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdp.h"

namespace gdp {

struct PrepareParams {
    const void *x;
    int64_t x_n_stride, x_t_stride;
    const void *ba;
    int64_t ba_n_stride, ba_t_stride;
    const float *A_log, *dt_bias;
    int64_t n, T;
    int M, H, G, P, N;
    gdp_dtype dtype;
    bool decode;  // query and g interleaved onto the copies
    bool vec16;  // every row start and segment is 16-byte aligned
    void *q, *k, *v;
    float *beta, *g;
};

hipError_t launch_prepare(const PrepareParams &p, hipStream_t stream);
hipError_t launch_decode(const gdp_decode_args &a, hipStream_t stream);

// Where the stages that read q and k by row (the segment maps and the fused
// chunk_h + chunk_o pass) find them.  Key copy j of global token t for key
// head hk starts at element  k_ts t + k_js j + (hk / hpg) hs  of k, and the
// query of token t at  q_ts t + (hk / hpg) hs  of q.  By default these
// describe the q [B, T, H, K] and k [B, T*M, H, K] tensors of the call; the
// fused prefill with q and k not stored points them into the activations x
// (query/key groups: hpg heads per group, segments of hs elements).
struct QKRows {
    const void *k = nullptr, *q = nullptr;
    int64_t k_ts = 0, k_js = 0, q_ts = 0, hs = 0;
    int hpg = 1;
};

// Validated chunk-stage arguments (scale resolved, nseq resolved).
struct ChunkParams {
    gdp_chunk_args a;
    int64_t nseq;       // sequences: num_seqs with cu_seqlens, else B
    int64_t max_items;  // upper bound on 64-row chunks over all sequences
    int64_t max_tok_chunks;  // upper bound on 64-token chunks
    // u and v_new are stored as 16-column slices [B, HV, V/16, T*M, 16]:
    // elements between consecutive slices (T*M*16 for a plain call; the
    // whole sequence's for one segment of the pipelined forward)
    int64_t uv_ss;
    // chunk_h writes the state snapshot of chunk c (counted per sequence)
    // only when c % hstep == 0; 1 writes them all
    int hstep = 1;
    QKRows qk;  // q and k rows for the segment maps and the fused pass
    // WY launch order for one sequence cut into seg_n segments of seg_nch
    // chunks (the last may be shorter): 0 keeps the plain order
    int64_t seg_nch = 0, seg_n = 0;
};

// Element offset of (batch row b, expanded row e relative to the batch row,
// value head hv, column col) in a slice-major u / v_new tensor.
__host__ __device__ inline int64_t uv_index(int64_t b, int64_t e, int hv, int col, int HV, int VD, int64_t ss) {
    return (b * HV * (VD / 16) + (int64_t)hv * (VD / 16) + col / 16) * ss + e * 16 + col % 16;
}

// Segment-parallel state recurrence.  One long sequence (B == 1, no
// cu_seqlens): nseg segments of seg_tok tokens (the last one may be
// shorter), the maps of segments [0, nseg - 1) in `maps`
// ([nseg - 1, HV, K, V + K] fp32), the state entering every segment in
// `hstart` ([nseg, HV, V, K] fp32) and the segment offsets in `cu`
// ([nseg + 1] int32), all in caller-owned device memory.  Packed requests
// (cu_seqlens, B == 1): nseg is the number of plan slots, ceil(T / seg_tok)
// + num_seqs, each request cut into segments of seg_tok tokens by
// launch_seg_plan on the device; maps and hstart hold one entry per slot,
// seg_last[slot] marks segments that need no map, and req_first / req_nseg
// give each request's slots.
struct ScanParams {
    ChunkParams p;
    int64_t nseg, seg_tok;
    float *maps, *hstart;
    int32_t *cu;
    int32_t *seg_last, *req_first, *req_nseg;  // packed requests only
};

// Packed requests: the segment plan (one block), before launch_seg_scan.
hipError_t launch_seg_plan(const ScanParams &sp, hipStream_t stream);
// Packed requests: each request's final state into ht, after chunk_h.
hipError_t launch_seg_final(const ScanParams &sp, hipStream_t stream);
// The segment maps (every segment that needs one), then the scan over the
// segments (not the chunk_h pass).
hipError_t launch_seg_map(const ScanParams &sp, hipStream_t stream);
hipError_t launch_seg_scan(const ScanParams &sp, hipStream_t stream);

hipError_t launch_wy(const ChunkParams &p, hipStream_t stream);
// launch_wy with the prefill prepare of its rows fused in (B == n == 1, one
// sequence or packed requests, HV == H, bf16, K and V in {64, 128}): reads
// pp.x / pp.ba, writes pp's outputs and uses them as the chunk inputs
hipError_t launch_wy_prepare(const ChunkParams &p, const PrepareParams &pp, hipStream_t stream);
hipError_t launch_chunk_h(const ChunkParams &p, hipStream_t stream);
hipError_t launch_chunk_o(const ChunkParams &p, hipStream_t stream);
// chunk_h and chunk_o as one pass that stores neither v_new nor h (bf16, K
// in {64, 128}, V in {64, 128, 256}, M in [2, 4]); h0 / ht as for chunk_h
hipError_t launch_chunk_ho(const ChunkParams &p, hipStream_t stream);

}  // namespace gdp
