"""TEST INFRASTRUCTURE ONLY -- CPU oracle of the fused prefill prepare step.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never does.

Follows core.ssm.ops.gdp.prepare (module description; gdp_prefill_prepare,
Parameters and Returns; softplus):

* x is the post-conv activation [n, T, M*H*P + M*G*N + G*N] holding value,
  key and query one after the other along the last dimension; ba is
  [n, T, M*H + H].
* value and key come out on the Householder-expanded stream (copies folded
  into the sequence dimension, row t*M + j for copy j); query stays one per
  token.  Query and key are GQA-expanded from G groups to H heads.
* beta = sigmoid(b) per (token, copy, head); g = -exp(A_log) * softplus(a +
  dt_bias) per (token, head), both float32.
* softplus saturates to the identity above 20 and otherwise uses log1p(exp(x)).

Readings where the page leaves a step open (each listed in the design notes):
* segment layout: the value segment is laid out (M, H, P), the key segment
  (M, G, N), the query segment (G, N); ba is b laid out (M, H), then a (H).
* head h reads group h // (H // G).
* gate rounding: float32 inputs, every operation rounded once to float32 in the
  order written, each transcendental evaluated in float64 and then rounded.
  softplus uses a strict "> 20" test.
"""
import numpy as np

_F32 = np.float32
_F64 = np.float64


def _rn32(x):
    """Round a float64 array once to float32 (round to nearest even)."""
    return np.asarray(x, dtype=_F64).astype(_F32)


def sigmoid_rn32(b):
    """beta = 1 / (1 + exp(-b)), each step rounded to float32."""
    b = np.asarray(b, dtype=_F32)
    with np.errstate(over="ignore"):
        e = _rn32(np.exp(-b.astype(_F64)))
    d = (_F32(1.0) + e).astype(_F32)
    with np.errstate(divide="ignore"):
        return (_F32(1.0) / d).astype(_F32)


def softplus_rn32(s):
    """softplus(s) = s if s > 20 else log1p(exp(s)), float32 result."""
    s = np.asarray(s, dtype=_F32)
    with np.errstate(over="ignore"):
        e = _rn32(np.exp(s.astype(_F64)))
        lp = _rn32(np.log1p(e.astype(_F64)))
    return np.where(s > _F32(20.0), s, lp).astype(_F32)


def decay_rn32(a, A_log, dt_bias):
    """g = -(exp(A_log) * softplus(a + dt_bias)), float32, per op rounding.

    a: [..., H]; A_log, dt_bias: [H] (float32).
    """
    a = np.asarray(a, dtype=_F32)
    s = (a + np.asarray(dt_bias, dtype=_F32)).astype(_F32)
    sp = softplus_rn32(s)
    ea = _rn32(np.exp(np.asarray(A_log, dtype=_F32).astype(_F64)))
    return (-(ea * sp).astype(_F32)).astype(_F32)


def prefill_prepare(x, ba, A_log, dt_bias, M, H, G, P, N):
    """Split, expand and gate a prefill step.

    x: float32 [n, T, M*H*P + M*G*N + G*N]; ba: float32 [n, T, M*H + H];
    A_log, dt_bias: float32 [H].
    Returns (q [n,T,H,N], k [n,T*M,H,N], v [n,T*M,H,P], beta [n,T*M,H],
    g [n,T,H]) as float32 arrays.
    """
    x = np.asarray(x, dtype=_F32)
    ba = np.asarray(ba, dtype=_F32)
    n, T, width = x.shape
    if width != M * H * P + M * G * N + G * N:
        raise ValueError("x last dimension does not match M*H*P + M*G*N + G*N")
    if ba.shape != (n, T, M * H + H):
        raise ValueError("ba must be [n, T, M*H + H]")
    if H % G:
        raise ValueError("H must be a multiple of G")
    hpg = H // G
    kb = M * H * P
    qb = kb + M * G * N

    v = x[:, :, :kb].reshape(n, T, M, H, P).reshape(n, T * M, H, P)
    kg = x[:, :, kb:qb].reshape(n, T, M, G, N)
    k = np.repeat(kg, hpg, axis=3).reshape(n, T * M, H, N)
    qg = x[:, :, qb:].reshape(n, T, G, N)
    q = np.repeat(qg, hpg, axis=2)

    b = ba[:, :, : M * H].reshape(n, T, M, H).reshape(n, T * M, H)
    a = ba[:, :, M * H:]
    beta = sigmoid_rn32(b)
    g = decay_rn32(a, A_log, dt_bias)
    return (np.ascontiguousarray(q), np.ascontiguousarray(k),
            np.ascontiguousarray(v), beta, g)


def decode_prepare(x, ba, A_log, dt_bias, M, H, G, P, N):
    """Split, expand and gate a decode step whose S tokens walk the
    Householder copies as one sequence of S*M rows (core.ssm.ops.gdp.prepare,
    module description, the decode bullet; gdp_decode_prepare, Returns): the
    query sits on the last copy of each token and the decay on the first,
    zeros elsewhere.  Key, value and beta are as in prefill.

    Returns (q [n,S*M,H,N], k [n,S*M,H,N], v [n,S*M,H,P], beta [n,S*M,H],
    g [n,S*M,H]) as float32 arrays.
    """
    q, k, v, beta, g = prefill_prepare(x, ba, A_log, dt_bias, M, H, G, P, N)
    n, S = q.shape[0], q.shape[1]
    qi = np.zeros((n, S, M, H, N), dtype=_F32)
    qi[:, :, M - 1] = q
    gi = np.zeros((n, S, M, H), dtype=_F32)
    gi[:, :, 0] = g
    return qi.reshape(n, S * M, H, N), k, v, beta, gi.reshape(n, S * M, H)
