"""Seeded synthetic inputs for the chunked GDP forward.

This module only draws random numbers.  It holds none of the method's
arithmetic: gates (beta, g) are computed from these draws by the code under
test or by the oracle, never here.  Query and key directions are sampled
uniformly on the unit sphere (a Gaussian draw divided by its norm), which is
the input distribution of the workloads, not a step of the method.

Every workload is defined by a config dict and a seed; the draw order within
a seed is fixed, so the same call always yields the same bytes.
"""
import numpy as np
import torch

# Workloads: the small oracle-sized case, the Householder-copy case, the GVA
# varlen prefill case (with prepare), the long single-sequence prefill (the
# timed workload) and the wide-head stress case with extreme gates.
CONFIGS = {
    1: dict(name="tiny_f32", B=1, T=128, H=2, HV=2, K=64, V=64, M=1,
            dtype="f32", a_sigma=1.0),
    2: dict(name="householder_m2", B=2, T=1024, H=8, HV=8, K=128, V=128, M=2,
            dtype="bf16", a_sigma=1.0),
    3: dict(name="gva_varlen_prepare", n_req=8, len_lo=64, len_hi=4096,
            H=4, HV=16, K=128, V=128, M=2, dtype="bf16", a_sigma=1.0,
            prep=dict(H=16, G=4, P=128, N=128)),
    4: dict(name="long_prefill_32k", B=1, T=32768, H=16, HV=16, K=128, V=128,
            M=2, dtype="bf16", a_sigma=1.0),
    5: dict(name="wide_head_stress", B=4, T=8192, H=32, HV=32, K=128, V=256,
            M=3, dtype="bf16", a_sigma=3.0, plant_edges=True),
}

# Values of a + dt_bias planted to reach both softplus branches and the
# exp under/overflow edges of the gates.
EDGE_S = np.array([20.0, np.nextafter(np.float32(20.0), np.float32(np.inf)),
                   25.0, 88.0, -16.0, -30.0, -90.0, -104.0], dtype=np.float32)


def seed_of(cfg_id):
    return 1000 + int(cfg_id)


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(rng, shape, sigma=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _sphere(rng, shape):
    """Gaussian draw divided by its norm over the last dimension."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32))
    x /= n[..., None]
    return x


def _cast(x, dtype):
    return torch.from_numpy(x).to(torch_dtype(dtype))


def chunk_draws(B, T, H, HV, K, V, M, dtype, seed, a_sigma=1.0,
                plant_edges=False, sphere_qk=True):
    """Inputs of the chunk forward for B equal-length sequences of T tokens.

    Draw order: q, k, v, b, a, A_log, dt_bias.
    Returns CPU tensors: q [B,T,H,K], k [B,T*M,H,K], v [B,T*M,HV,V] in
    ``dtype``; b [B,T*M,HV], a [B,T,HV], A_log [HV], dt_bias [HV] in float32.
    b and a are the raw gate pre-activations: beta = sigmoid(b) and
    g = -exp(A_log) * softplus(a + dt_bias) are formed downstream.
    With plant_edges, batch 0 / head 0 gets a + dt_bias equal to EDGE_S on
    its first tokens (dt_bias[0] set to 0 so the sum is exact).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    draw_qk = _sphere if sphere_qk else _normal
    q = draw_qk(rng, (B, T, H, K))
    k = draw_qk(rng, (B, T * M, H, K))
    v = _normal(rng, (B, T * M, HV, V))
    b = _normal(rng, (B, T * M, HV))
    a = _normal(rng, (B, T, HV), a_sigma)
    A_log = np.log(rng.uniform(1.0, 16.0, size=HV)).astype(np.float32)
    dt_bias = rng.uniform(-1.0, 1.0, size=HV).astype(np.float32)
    if plant_edges:
        n = min(T, EDGE_S.size)
        dt_bias[0] = 0.0
        a[0, :n, 0] = EDGE_S[:n]
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                b=torch.from_numpy(b), a=torch.from_numpy(a),
                A_log=torch.from_numpy(A_log), dt_bias=torch.from_numpy(dt_bias))


def initial_state_draws(nseq, HV, V, K, seed, sigma=0.1):
    """A float32 initial state S [nseq, HV, V, K] ~ N(0, sigma^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy(_normal(rng, (nseq, HV, V, K), sigma))


def varlen_lengths(n_req, lo, hi, seed):
    """Request lengths uniform in [lo, hi] (inclusive) and their cu_seqlens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lo, hi + 1, size=n_req).astype(np.int64)
    cu = np.zeros(n_req + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    return lens, cu


def prepare_draws(n, T, M, H, G, P, N, dtype, seed):
    """Post-conv x [n,T,M*H*P+M*G*N+G*N] and ba [n,T,M*H+H] ~ N(0,1) in
    ``dtype``; A_log = log U[1,16] and dt_bias ~ U[-1,1] per head (float32).
    Draw order: x, ba, A_log, dt_bias."""
    rng = np.random.Generator(np.random.PCG64(seed))
    width = M * H * P + M * G * N + G * N
    x = _normal(rng, (n, T, width))
    ba = _normal(rng, (n, T, M * H + H))
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
    return dict(x=_cast(x, dtype), ba=_cast(ba, dtype),
                A_log=torch.from_numpy(A_log), dt_bias=torch.from_numpy(dt_bias))


def varlen_prepare_draws(cfg_id=3):
    """The GVA varlen prefill workload: lengths first (own seed stream), then
    the prepare inputs for the packed n == 1 stream."""
    c = CONFIGS[cfg_id]
    seed = seed_of(cfg_id)
    lens, cu = varlen_lengths(c["n_req"], c["len_lo"], c["len_hi"], seed)
    p = c["prep"]
    d = prepare_draws(1, int(cu[-1]), c["M"], p["H"], p["G"], p["P"], p["N"],
                      c["dtype"], seed + 100)
    d["lens"] = lens
    d["cu_seqlens"] = cu
    return d


def config_chunk_draws(cfg_id):
    """chunk_draws for one of the equal-length configs (1, 2, 4, 5)."""
    c = CONFIGS[cfg_id]
    return chunk_draws(c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], c["M"],
                       c["dtype"], seed_of(cfg_id), a_sigma=c.get("a_sigma", 1.0),
                       plant_edges=c.get("plant_edges", False))
