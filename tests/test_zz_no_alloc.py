"""gdp_chunk_fwd_scan_noalloc (the allocation-free form of the
segment-parallel forward) against gdp_chunk_fwd_scan on the GPU, through the
C ABI: two calls in a row, the second on a smaller problem, each bit-identical
to the workspace form (same kernels, deterministic)."""
import pytest
import torch

from gated_delta_product_amd import binding as G
from gated_delta_product_amd import synth
from helpers import gates, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

FIELDS = ("o", "v_new", "w", "u", "k_rnorm", "gcum", "kdecay", "ht")


def _buffers(T, H, HV, K, V, M, seed, h0):
    d = synth.chunk_draws(1, T, H, HV, K, V, M, "bf16", seed)
    beta, g = gates(d)
    beta = beta.reshape(1, T * M, HV)
    init = synth.initial_state_draws(1, HV, V, K, seed + 1).to(DEV) if h0 else None
    ins = [t.to(DEV) for t in (d["q"], d["k"], d["v"], beta, g)]
    return [G.ChunkBuffers(*ins, initial_state=init, output_final_state=True) for _ in range(2)]


def _compare(T, H, HV, K, V, M, nseg, seed, h0):
    log("noalloc: T=%d H=%d HV=%d K=%d V=%d M=%d segments=%d seed=%d" % (T, H, HV, K, V, M, nseg, seed))
    ref, na = _buffers(T, H, HV, K, V, M, seed, h0)
    ref.h.fill_(7.0)
    na.h.fill_(7.0)
    ref.forward_scan(nseg)
    na.forward_scan_noalloc(nseg)
    torch.cuda.synchronize()
    for nm in FIELDS:
        assert torch.equal(getattr(ref, nm), getattr(na, nm)), nm
    assert torch.equal(ref.h, na.h), "h"
    assert torch.isfinite(na.o.float()).all()
    return ref.o.float().abs().max().item()


def test_noalloc_matches_workspace_form_two_calls():
    """Two calls in a row, the second smaller (fewer heads, tokens and
    segments, other head dims and M), so stale scratch from the first call
    must not leak into the second."""
    big = (4096, 2, 4, 128, 128, 2, 16, 51, True)
    small = (700, 1, 2, 64, 128, 3, 4, 52, False)
    need_big = G.lib().gdp_scan_workspace_bytes(big[0], big[2], big[3], big[4], big[6])
    need_small = G.lib().gdp_scan_workspace_bytes(small[0], small[2], small[3], small[4], small[6])
    assert need_small < need_big <= G.NOALLOC_SCRATCH_BYTES
    _compare(*big)
    _compare(*small)
