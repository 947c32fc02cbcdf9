"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names the fact it checks and the mistake it would catch.  The
oracle computes the recurrence in the corrected-value form; the tests use the
literal matrix form of the gated delta rule, closed forms (pure decay, exact
write, reflection), the Householder-product identity of the WY
representation, an independently written chunked form, and the decode
interleave equivalence of the prepare page.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import prepare as P

RTOL = 1e-11


def _case(L, M, K, V, seed, beta_lo=0.05, beta_hi=0.95, g_scale=1.0, zero_g=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, K)).astype(np.float32)
    k = rng.standard_normal((L * M, K)).astype(np.float32)
    v = rng.standard_normal((L * M, V)).astype(np.float32)
    beta = rng.uniform(beta_lo, beta_hi, L * M).astype(np.float32)
    g = None if zero_g else (-g_scale * rng.uniform(0.0, 1.5, L)).astype(np.float32)
    return q, k, v, beta, g


def _nrm(x, eps):
    x = x.astype(np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def _literal(q, k, v, beta, g, M, scale, chunk, eps=1e-6, h0=None):
    """The gated delta rule written as matrices: S <- a*S*(I - b k k^T) + b v k^T,
    decay on the first copy of a token, query read after its last copy.
    Returns o, delta (recovered from the state change), h snapshots, final S."""
    L, K = q.shape
    V = v.shape[1]
    S = np.zeros((V, K)) if h0 is None else h0.copy()
    kh = _nrm(k, eps)
    qh = _nrm(q, eps)
    nc = -(-(L * M) // chunk)
    o = np.zeros((L, V))
    dl = np.zeros((L * M, V))
    hs = np.zeros((nc, V, K))
    I = np.eye(K)
    for t in range(L):
        for j in range(M):
            e = t * M + j
            if e % chunk == 0:
                hs[e // chunk] = S
            a = np.exp(float(g[t])) if (j == 0 and g is not None) else 1.0
            b = float(beta[e])
            kk = kh[e][:, None]
            Snew = a * S @ (I - b * kk @ kk.T) + b * v[e].astype(np.float64)[:, None] @ kk.T
            dl[e] = (Snew - a * S) @ kh[e] / (kh[e] @ kh[e])
            S = Snew
        o[t] = scale * S @ qh[t]
    return o, dl, hs, S


def _close(a, b, tol=RTOL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(1.0, float(np.abs(b).max()))
    assert float(np.abs(a - b).max()) <= tol * den, float(np.abs(a - b).max())


@pytest.mark.parametrize("M,chunk", [(1, 8), (2, 8), (3, 8), (2, 5), (3, 16)])
def test_matches_literal_matrix_form(M, chunk):
    """C0: the corrected-value form equals the literal product form.  Catches a
    transposed state, a decay on the wrong copy, the query read on the wrong
    copy, a missing beta, a wrong snapshot position."""
    L, K, V = 13, 8, 6
    q, k, v, beta, g = _case(L, M, K, V, seed=10 + M)
    scale = 0.37
    r = oracle.recurrence(q, k, v, beta, g, M, scale=scale, chunk=chunk)
    o, dl, hs, S = _literal(q, k, v, beta, g, M, scale, chunk)
    _close(r["o"], o)
    _close(r["v_new"], dl)
    _close(r["h"], hs)
    _close(r["h_final"], S)


def test_delta_rule_when_m1_g0():
    """C1: M = 1 and no decay reduce to the plain delta rule, written in its
    error-correction form S += beta (v - S k) k^T (DeltaNet)."""
    L, K, V = 20, 7, 5
    q, k, v, beta, _ = _case(L, 1, K, V, seed=3, zero_g=True)
    r = oracle.recurrence(q, k, v, beta, None, 1, scale=1.0, chunk=64)
    S = np.zeros((V, K))
    kh, qh = _nrm(k, 1e-6), _nrm(q, 1e-6)
    for t in range(L):
        err = v[t].astype(np.float64) - S @ kh[t]
        S = S + float(beta[t]) * np.outer(err, kh[t])
        _close(r["o"][t], S @ qh[t])


@pytest.mark.parametrize("M", [1, 2, 3])
def test_pure_decay_when_beta0(M):
    """C2: beta = 0 leaves only the decay of the initial state.  Closed form:
    h[c] = exp(sum of g over tokens whose first copy precedes row c*C) h0 and
    o_t = scale exp(sum_{s<=t} g_s) h0 qhat_t.  Catches decay on the wrong copy,
    decay applied per copy, a wrong sign, a missing scale."""
    L, K, V, C = 17, 6, 4, 8
    q, k, v, beta, g = _case(L, M, K, V, seed=5)
    beta[:] = 0.0
    rng = np.random.default_rng(9)
    h0 = rng.standard_normal((V, K))
    scale = 0.5
    r = oracle.recurrence(q, k, v, beta, g, M, scale=scale, chunk=C, h0=h0)
    gd = g.astype(np.float64)
    qh = _nrm(q, 1e-6)
    for t in range(L):
        _close(r["o"][t], scale * np.exp(gd[: t + 1].sum()) * h0 @ qh[t])
    for c in range(r["h"].shape[0]):
        first_rows = [t for t in range(L) if t * M < c * C]
        _close(r["h"][c], np.exp(gd[first_rows].sum()) * h0)
    assert np.all(r["v_new"] == 0.0)


@pytest.mark.parametrize("M", [1, 2, 3])
def test_exact_write_when_beta1(M):
    """C5: with beta = 1 on the last copy of token t, S khat = v on that row for
    any history and decay (eps = 0 makes khat unit-norm exactly), so with
    q_t = k of that row, o_t = scale * v of that row."""
    L, K, V = 15, 8, 5
    q, k, v, beta, g = _case(L, M, K, V, seed=21)
    for t in range(L):
        e = t * M + M - 1
        beta[e] = 1.0
        q[t] = k[e]
    r = oracle.recurrence(q, k, v, beta, g, M, scale=0.25, chunk=64, eps=0.0)
    for t in range(L):
        _close(r["o"][t], 0.25 * v[t * M + M - 1].astype(np.float64), 1e-12)


def test_inert_copies_equal_single_copy():
    """C6: copies j >= 1 with beta = 0 change nothing; the result equals an
    M = 1 run on copy 0.  Catches wrong strides between copies."""
    L, K, V, M = 14, 8, 6, 3
    q, k, v, beta, g = _case(L, M, K, V, seed=31)
    beta_m = beta.copy()
    for t in range(L):
        beta_m[t * M + 1: t * M + M] = 0.0
    r = oracle.recurrence(q, k, v, beta_m, g, M, scale=1.0, chunk=64)
    r1 = oracle.recurrence(q, np.ascontiguousarray(k[0::M]), np.ascontiguousarray(v[0::M]),
                           np.ascontiguousarray(beta_m[0::M]), g, 1, scale=1.0, chunk=64)
    _close(r["o"], r1["o"])
    _close(r["v_new"][0::M], r1["v_new"])


@pytest.mark.parametrize("M", [2, 3])
def test_decode_interleave_equivalence(M):
    """C7: GDP over T tokens with M copies equals the gated delta rule over the
    T*M-row stream with the decay placed on the first copy, zero decay on the
    others and the query placed on the last copy (prepare page, decode
    layout); outputs are read at rows t*M + M - 1."""
    L, K, V = 11, 8, 5
    q, k, v, beta, g = _case(L, M, K, V, seed=41)
    r = oracle.recurrence(q, k, v, beta, g, M, scale=0.7, chunk=64)
    gi = np.zeros(L * M, np.float32)
    gi[0::M] = g
    qi = np.zeros((L * M, K), np.float32)
    qi[M - 1::M] = q
    ri = oracle.recurrence(qi, k, v, beta, gi, 1, scale=0.7, chunk=64)
    _close(r["o"], ri["o"][M - 1::M])
    _close(r["v_new"], ri["v_new"])


def test_reflection_preserves_norm():
    """C9: beta = 2, no decay, v = 0 makes each step a Householder reflection
    S <- S (I - 2 khat khat^T), which preserves the Frobenius norm."""
    L, K, V, M = 25, 8, 6, 2
    q, k, v, beta, _ = _case(L, M, K, V, seed=51, zero_g=True)
    beta[:] = 2.0
    v[:] = 0.0
    rng = np.random.default_rng(2)
    h0 = rng.standard_normal((V, K))
    r = oracle.recurrence(q, k, v, beta, None, M, scale=1.0, chunk=4, h0=h0, eps=0.0)
    n0 = np.linalg.norm(h0)
    for c in range(r["h"].shape[0]):
        assert abs(np.linalg.norm(r["h"][c]) - n0) <= 1e-12 * n0
    assert abs(np.linalg.norm(r["h_final"]) - n0) <= 1e-12 * n0


def _gam(g, M, c0, n):
    run, out = 0.0, []
    for a in range(n):
        e = c0 + a
        if e % M == 0 and g is not None:
            run += float(g[e // M])
        out.append(run)
    return np.array(out)


@pytest.mark.parametrize("M,chunk", [(1, 8), (2, 8), (3, 8), (2, 6)])
def test_householder_product_equals_wy(M, chunk):
    """C4: over one chunk, the product of the gated Householder factors
    prod_{e=last..first} alpha_e (I - beta_e khat_e khat_e^T) equals
    exp(gamma_last) I - Khat^T diag(exp(gamma_last - gamma)) W, with W the
    oracle's w.  Pins w without the recurrence."""
    L, K, V = 12, 8, 5
    q, k, v, beta, g = _case(L, M, K, V, seed=61 + M)
    w, _ = oracle.wy(k, v, beta, g, M, chunk=chunk)
    kh = _nrm(k, 1e-6)
    rows = L * M
    for c0 in range(0, rows, chunk):
        n = min(chunk, rows - c0)
        Pm = np.eye(K)
        for a in range(n):
            e = c0 + a
            al = np.exp(float(g[e // M])) if e % M == 0 else 1.0
            Pm = al * (np.eye(K) - float(beta[e]) * np.outer(kh[e], kh[e])) @ Pm
        gm = _gam(g, M, c0, n)
        Kc = kh[c0:c0 + n]
        rhs = np.exp(gm[-1]) * np.eye(K) - Kc.T @ np.diag(np.exp(gm[-1] - gm)) @ w[c0:c0 + n]
        _close(Pm, rhs)


@pytest.mark.parametrize("M,chunk", [(1, 8), (2, 8), (3, 8)])
def test_u_is_vnew_of_a_zero_state_chunk(M, chunk):
    """With a zero incoming state the corrected values of a chunk are u.
    Pins u against the literal matrix form (first chunk of the sequence)."""
    L, K, V = 9, 8, 5
    q, k, v, beta, g = _case(L, M, K, V, seed=71 + M)
    _, u = oracle.wy(k, v, beta, g, M, chunk=chunk)
    _, dl, _, _ = _literal(q, k, v, beta, g, M, 1.0, chunk)
    n = min(chunk, L * M)
    _close(u[:n], dl[:n])


@pytest.mark.parametrize("M,Ct", [(1, 8), (2, 4), (2, 8), (3, 4)])
def test_chunked_form_equals_serial(M, Ct):
    """C3: an independently written chunked form (v_new = u - w h per state
    chunk; state update h' = e^{gamma_last} h + sum e^{gamma_last-gamma} delta khat^T;
    output per token chunk of Ct tokens = M state chunks from the boundary
    state plus causal in-chunk attention summed over the copies) reproduces
    the serial oracle's o, v_new and h."""
    L, K, V = 16, 8, 6
    C = Ct  # state chunk: Ct rows; token chunk: Ct tokens = M state chunks
    q, k, v, beta, g = _case(L, M, K, V, seed=81 + M)
    scale = 0.6
    r = oracle.recurrence(q, k, v, beta, g, M, scale=scale, chunk=C)
    w, u = oracle.wy(k, v, beta, g, M, chunk=C)
    kh, qh = _nrm(k, 1e-6), _nrm(q, 1e-6)
    rows = L * M
    S = np.zeros((V, K))
    hs, dl = [], np.zeros((rows, V))
    for c0 in range(0, rows, C):
        n = min(C, rows - c0)
        hs.append(S.copy())
        d = u[c0:c0 + n] - w[c0:c0 + n] @ S.T
        dl[c0:c0 + n] = d
        gm = _gam(g, M, c0, n)
        S = np.exp(gm[-1]) * S + (d * np.exp(gm[-1] - gm)[:, None]).T @ kh[c0:c0 + n]
    _close(np.array(hs), r["h"], 1e-10)
    _close(dl, r["v_new"], 1e-10)
    # output per token chunk of Ct tokens, boundary state h[i*M]
    o = np.zeros((L, V))
    gd = g.astype(np.float64)
    for i0 in range(0, L, Ct):
        Sb = hs[(i0 * M) // C]
        G = np.cumsum(gd[i0:min(i0 + Ct, L)])
        for t in range(i0, min(i0 + Ct, L)):
            acc = np.exp(G[t - i0]) * Sb @ qh[t]
            for s in range(i0, t + 1):
                for j in range(M):
                    e = s * M + j
                    acc = acc + np.exp(G[t - i0] - G[s - i0]) * (qh[t] @ kh[e]) * dl[e]
            o[t] = scale * acc
    _close(o, r["o"], 1e-10)


def test_zero_rows_stay_finite():
    """Padding rows of zeros normalise to zero (eps > 0), never NaN."""
    L, K, V, M = 6, 8, 4, 2
    q, k, v, beta, g = _case(L, M, K, V, seed=91)
    q[2] = 0.0
    k[3] = 0.0
    r = oracle.recurrence(q, k, v, beta, g, M, chunk=4)
    assert np.all(np.isfinite(r["o"])) and np.all(r["o"][2] == 0.0)


# ---------------------------------------------------------------- prepare

def _golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "gate_edges.txt")
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, xin, xout = line.split()[:3]
            rows.append((kind, int(xin, 16), int(xout, 16)))
    return rows


def _f32(bits):
    return np.array([bits], np.uint32).view(np.float32)


def test_gate_golden_edges():
    """C10: closed-form gate values at the branch edges (tests/golden)."""
    rows = _golden()
    assert len(rows) >= 8
    for kind, xin, xout in rows:
        x = _f32(xin)
        if kind == "softplus":
            y = P.softplus_rn32(x)
        else:
            y = P.sigmoid_rn32(x)
        assert y.view(np.uint32)[0] == xout, (kind, hex(xin), hex(int(y.view(np.uint32)[0])))


def _ulp_diff(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def test_gates_within_one_ulp_of_exact():
    """beta and softplus stay close to the exact functions (float64, rounded
    once).  sigmoid rounds three times (exp, the add, the divide), each at most
    half an ulp relative, so it may sit up to 2 ulp away (for b < 0, where
    1 + exp(-b) carries the rounding of exp), and within 1 ulp for b >= 0
    where exp(-b) <= 1; softplus rounds twice on the log1p branch.  A wrong
    formula (log instead of log1p, a sign, a missing branch) misses by far
    more."""
    x = np.linspace(-30, 30, 20001, dtype=np.float32)
    xd = x.astype(np.float64)
    sig = (1.0 / (1.0 + np.exp(-xd))).astype(np.float32)
    d = _ulp_diff(P.sigmoid_rn32(x), sig)
    assert d.max() <= 2
    assert d[x >= 0].max() <= 1
    sp = np.where(xd > 20, xd, np.log1p(np.exp(xd))).astype(np.float32)
    assert _ulp_diff(P.softplus_rn32(x), sp).max() <= 1


def test_decay_closed_forms():
    """g = -exp(A_log) softplus(a + dt_bias): A_log = 0 gives -softplus;
    A_log = ln 2 gives -2 softplus exactly (exp(ln 2) rounds to 2)."""
    a = np.array([[0.5, -1.0, 3.0]], np.float32)
    dt = np.array([0.25, 0.5, -2.0], np.float32)
    s = (a + dt).astype(np.float32)
    g0 = P.decay_rn32(a, np.zeros(3, np.float32), dt)
    assert np.array_equal(g0, -P.softplus_rn32(s))
    g2 = P.decay_rn32(a, np.full(3, np.log(2.0), np.float32), dt)
    assert np.array_equal(g2, (-2.0 * P.softplus_rn32(s)).astype(np.float32))
    assert np.all(g0 <= 0)


def test_prepare_index_maps_by_construction():
    """Build x by appending, per token, the value heads copy by copy, then the
    key groups copy by copy, then the query groups (the concatenation the
    prepare page describes), and check that prepare recovers value/key on
    the expanded stream and GQA-expands query/key (head h reads group
    h // (H // G))."""
    n, T, M, H, G, Pd, N = 2, 5, 3, 6, 2, 4, 3
    rng = np.random.default_rng(7)
    vv = rng.standard_normal((n, T, M, H, Pd)).astype(np.float32)
    kg = rng.standard_normal((n, T, M, G, N)).astype(np.float32)
    qg = rng.standard_normal((n, T, G, N)).astype(np.float32)
    x = np.zeros((n, T, M * H * Pd + M * G * N + G * N), np.float32)
    for b in range(n):
        for t in range(T):
            row = []
            for j in range(M):
                for h in range(H):
                    row.extend(vv[b, t, j, h])
            for j in range(M):
                for gg in range(G):
                    row.extend(kg[b, t, j, gg])
            for gg in range(G):
                row.extend(qg[b, t, gg])
            x[b, t] = row
    ba = rng.standard_normal((n, T, M * H + H)).astype(np.float32)
    A_log = np.log(rng.uniform(1, 16, H)).astype(np.float32)
    dt = rng.uniform(-1, 1, H).astype(np.float32)
    q, k, v, beta, g = P.prefill_prepare(x, ba, A_log, dt, M, H, G, Pd, N)
    assert q.shape == (n, T, H, N) and k.shape == (n, T * M, H, N)
    assert v.shape == (n, T * M, H, Pd) and beta.shape == (n, T * M, H) and g.shape == (n, T, H)
    for b in range(n):
        for t in range(T):
            for h in range(H):
                assert np.array_equal(q[b, t, h], qg[b, t, h // (H // G)])
                assert g[b, t, h] == P.decay_rn32(ba[b, t, M * H + h], A_log[h], dt[h])
                for j in range(M):
                    assert np.array_equal(v[b, t * M + j, h], vv[b, t, j, h])
                    assert np.array_equal(k[b, t * M + j, h], kg[b, t, j, h // (H // G)])
                    assert beta[b, t * M + j, h] == P.sigmoid_rn32(ba[b, t, j * H + h])
    # decode form: the same inputs walk the copies as one sequence of T*M
    # rows, the query on each token's last copy and the decay on its first
    dq, dk, dv, dbeta, dg = P.decode_prepare(x, ba, A_log, dt, M, H, G, Pd, N)
    assert dq.shape == (n, T * M, H, N) and dg.shape == (n, T * M, H)
    assert np.array_equal(dk, k) and np.array_equal(dv, v) and np.array_equal(dbeta, beta)
    for b in range(n):
        for t in range(T):
            for h in range(H):
                for j in range(M):
                    e = t * M + j
                    want_q = qg[b, t, h // (H // G)] if j == M - 1 else np.zeros(N, np.float32)
                    assert np.array_equal(dq[b, e, h], want_q)
                    want_g = P.decay_rn32(ba[b, t, M * H + h], A_log[h], dt[h]) if j == 0 else 0.0
                    assert dg[b, e, h] == want_g
