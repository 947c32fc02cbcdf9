"""Shared test helpers: oracle runs over (sequence, head) pairs and error
metrics.  Only tests import this."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from oracle import prepare as OP

# Tolerances for bf16 inputs with fp32 accumulation: max-abs and relative L2
# over the compared tensor.  The f32 path keeps fp32 operands throughout.
TOL = {
    torch.bfloat16: dict(max_abs=2e-2, rel_l2=5e-3),
    torch.float32: dict(max_abs=1e-3, rel_l2=1e-4),
}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32(t):
    """Exact float32 numpy copy of a CPU/GPU tensor (bf16 widens exactly)."""
    return t.detach().to("cpu", torch.float32).numpy()


def gates(d):
    """beta and g from the raw draws, by the oracle's float32 gate functions."""
    beta = OP.sigmoid_rn32(d["b"].numpy())
    g = OP.decay_rn32(d["a"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    return torch.from_numpy(beta), torch.from_numpy(g)


def metrics(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = x - ref
    max_abs = float(np.abs(err).max()) if err.size else 0.0
    den = float(np.sqrt((ref * ref).sum()))
    rel = float(np.sqrt((err * err).sum()) / den) if den > 0 else float(np.sqrt((err * err).sum()))
    return max_abs, rel, bool(np.all(np.isfinite(x)))


class Acc:
    """Accumulates squared errors over slices so rel-L2 covers the whole
    compared set.

    Two max-abs figures are kept: the raw one, and the one left after each
    element's own storage quantum (half a bf16 ulp of the reference value),
    which no bf16-stored result can avoid.  For o the raw figure is checked;
    for the bf16 intermediates (w, u, v_new, h), whose values reach ~10 where
    half an ulp is 0.03, the arithmetic error beyond storage rounding is."""

    def __init__(self, name, raw_max_abs=False):
        self.name, self.e2, self.r2, self.max_abs, self.finite, self.n = name, 0.0, 0.0, 0.0, True, 0
        self.beyond, self.ref_max, self.raw = 0.0, 0.0, raw_max_abs
        self.bf16 = True

    def add(self, x, ref, bf16=True):
        x = np.asarray(x, np.float64)
        ref = np.asarray(ref, np.float64)
        e = x - ref
        self.e2 += float((e * e).sum())
        self.r2 += float((ref * ref).sum())
        if e.size:
            ae = np.abs(e)
            self.max_abs = max(self.max_abs, float(ae.max()))
            self.ref_max = max(self.ref_max, float(np.abs(ref).max()))
            if bf16:
                mag = np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
                half_ulp = np.exp2(np.floor(np.log2(mag)) - 8.0)
                self.beyond = max(self.beyond, float(np.maximum(ae - half_ulp, 0.0).max()))
            else:
                self.beyond = max(self.beyond, float(ae.max()))
        self.finite &= bool(np.all(np.isfinite(x)))
        self.n += x.size

    def rel(self):
        return np.sqrt(self.e2 / self.r2) if self.r2 > 0 else np.sqrt(self.e2)

    def check(self, tol):
        log("  %-6s n=%-10d max|ref|=%.2e max_abs=%.3e beyond_storage=%.3e rel_l2=%.3e"
            % (self.name, self.n, self.ref_max, self.max_abs, self.beyond, self.rel()))
        assert self.finite, self.name + ": non-finite values"
        m = self.max_abs if self.raw else self.beyond
        assert m <= tol["max_abs"], (self.name, m)
        assert self.rel() <= tol["rel_l2"], (self.name, self.rel())


def oracle_pair(qn, kn, vn, bn, gn, M, scale, want_wu=True, h0=None):
    """Run the oracle for one (sequence, value head) given float32 numpy
    slices q [L,K], k [L*M,K], v [L*M,V], beta [L*M], g [L] (or None: ungated)
    and an optional initial state h0 [V,K]."""
    r = oracle.recurrence(qn, kn, vn, bn, gn, M, scale=scale, chunk=64, h0=h0)
    if want_wu:
        w, u = oracle.wy(kn, vn, bn, gn, M, chunk=64)
        r["w"], r["u"] = w, u
    return r


def run_pairs(fn, items, workers=16):
    with ThreadPoolExecutor(min(workers, max(1, len(items)))) as ex:
        return list(ex.map(fn, items))
