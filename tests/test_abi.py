"""CPU checks of the C ABI: the header compiles as C99, libgdp.so exports
every function the header declares, the ctypes mirror of gdp_chunk_args has
the C layout, and argument validation rejects bad calls before any launch (so
no GPU is touched)."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_product_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdp.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdp_[a-z_0-9]+)\s*\(", src)))


def test_header_compiles_as_c99(tmp_path):
    c = tmp_path / "t.c"
    c.write_text('#include "gdp.h"\nint main(void){ gdp_chunk_args a; (void)a; return 0; }\n')
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                           "-I", os.path.join(ROOT, "include"), str(c)])


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"gdp_prefill_prepare", "gdp_decode_prepare", "gdp_recompute_w_u", "gdp_chunk_h", "gdp_chunk_o",
            "gdp_chunk_fwd", "gdp_chunk_fwd_pipelined", "gdp_pipeline_segments", "gdp_pipeline_plan", "gdp_decode_update",
            "gdp_chunk_fwd_scan", "gdp_scan_segments", "gdp_scan_workspace_bytes",
            "gdp_num_state_chunks", "gdp_last_error", "gdp_version"} <= set(names)
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.check_output(["nm", "-D", "--defined-only", B.LIB_PATH], text=True)
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert set(names) <= exported


def test_every_entry_point_has_ctypes_signature():
    """Each declared function has argtypes in the binding, so no pointer or
    64-bit argument is passed as a default 32-bit int."""
    L = B.lib()
    for n in _declared():
        assert getattr(L, n).argtypes is not None, n


@pytest.mark.parametrize("cls,cname", [(B.ChunkArgs, "gdp_chunk_args"), (B.DecodeArgs, "gdp_decode_args"),
                                      (B.PrepareArgs, "gdp_prepare_args")])
def test_struct_layout_matches_c(tmp_path, cls, cname):
    fields = [f for f, _ in cls._fields_]
    prog = '#include <stdio.h>\n#include <stddef.h>\n#include "gdp.h"\nint main(void){\n'
    prog += 'printf("%%zu\\n", sizeof(%s));\n' % cname
    for f in fields:
        prog += 'printf("%%zu\\n", offsetof(%s, %s));\n' % (cname, f)
    prog += "return 0;}\n"
    c = tmp_path / "layout.c"
    c.write_text(prog)
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)])
    vals = [int(x) for x in subprocess.check_output([str(exe)], text=True).split()]
    assert vals[0] == ctypes.sizeof(cls)
    for f, off in zip(fields, vals[1:]):
        assert getattr(cls, f).offset == off, f


def test_version_string():
    assert "gfx950" in B.version()


def _args(**kw):
    base = dict(B=1, T=128, H=2, HV=2, K=64, V=64, M=1, chunk_size=64, scale=0.0, dtype=B.GDP_BF16,
                cu_seqlens=None, num_seqs=0, h_chunks=2,
                q=0x10000, k=0x20000, v=0x30000, beta=0x40000, g=0x50000, k_rnorm=0x60000,
                gcum=0x68000, kdecay=0x6C000, w=0x70000, u=0x80000, v_new=0x90000, h=0xA0000, o=0xB0000)
    base.update(kw)
    return B.ChunkArgs(**base)


# Every case fails validation, so nothing reaches the HIP runtime.
BAD_CHUNK = [
    ("M=5", dict(M=5), B.GDP_ERR_UNSUPPORTED),
    ("M=0", dict(M=0), B.GDP_ERR_UNSUPPORTED),
    ("chunk 32", dict(chunk_size=32), B.GDP_ERR_UNSUPPORTED),
    ("K=96", dict(K=96), B.GDP_ERR_UNSUPPORTED),
    ("V=512", dict(V=512), B.GDP_ERR_UNSUPPORTED),
    ("f32 K=128", dict(dtype=B.GDP_F32, K=128), B.GDP_ERR_UNSUPPORTED),
    ("HV % H", dict(H=2, HV=3), B.GDP_ERR_INVALID),
    ("H=0", dict(H=0), B.GDP_ERR_INVALID),
    ("dtype", dict(dtype=7), B.GDP_ERR_INVALID),
    ("B<0", dict(B=-1), B.GDP_ERR_INVALID),
    ("varlen B=2", dict(B=2, cu_seqlens=0x1000, num_seqs=2), B.GDP_ERR_INVALID),
    ("h too small", dict(h_chunks=1), B.GDP_ERR_INVALID),
    ("null k", dict(k=None), B.GDP_ERR_INVALID),
    ("misaligned v", dict(v=0x30008), B.GDP_ERR_INVALID),
    ("nan scale", dict(scale=float("nan")), B.GDP_ERR_INVALID),
    ("misaligned g", dict(g=0x50008), B.GDP_ERR_INVALID),
    ("misaligned h0", dict(h0=0xC0008), B.GDP_ERR_INVALID),
    ("misaligned ht", dict(ht=0xD0004), B.GDP_ERR_INVALID),
]


@pytest.mark.parametrize("name,kw,status", BAD_CHUNK, ids=[c[0] for c in BAD_CHUNK])
def test_chunk_fwd_rejects(name, kw, status):
    a = _args(**kw)
    st = B.lib().gdp_chunk_fwd(ctypes.byref(a), None)
    assert st == status, (st, B.lib().gdp_last_error())
    assert B.lib().gdp_last_error()


def test_stage_specific_requirements():
    # chunk_o needs q and o but not v/beta/w/u; recompute_w_u needs v and beta
    L = B.lib()
    assert L.gdp_chunk_o(ctypes.byref(_args(q=None)), None) == B.GDP_ERR_INVALID
    assert L.gdp_recompute_w_u(ctypes.byref(_args(beta=None)), None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_h(ctypes.byref(_args(u=None)), None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_h(ctypes.byref(_args(kdecay=None)), None) == B.GDP_ERR_INVALID


def test_pipelined_rejects_and_segments():
    L = B.lib()
    ws = ctypes.c_void_p(0x100000)
    assert L.gdp_chunk_fwd_pipelined(ctypes.byref(_args(B=2, h_chunks=4)), 4, ws, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_pipelined(ctypes.byref(_args(cu_seqlens=0x1000, num_seqs=1)), 4, ws, None,
                                     None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_pipelined(ctypes.byref(_args()), 0, ws, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_pipelined(ctypes.byref(_args()), 2, None, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_pipelined(ctypes.byref(_args(q=None)), 2, ws, None, None) == B.GDP_ERR_INVALID
    # segments of whole 64-token chunks, at most the number asked for
    assert B.pipeline_segments(32768, 8) == 8
    assert B.pipeline_segments(1000, 3) == 3      # 16 chunks -> 5, 6, 5
    assert B.pipeline_segments(100, 8) == 2       # 2 chunks
    assert B.pipeline_segments(0, 8) == 0
    assert L.gdp_pipeline_segments(10, 0) == -1
    assert L.gdp_pipeline_plan(10, 2, None) == -1
    # the plan: equal shares of whole chunks, T covered once
    assert B.pipeline_plan(32768, 3) == [0, 10944, 21824, 32768]  # 512 chunks: 171, 170, 171
    assert B.pipeline_plan(1000, 3) == [0, 320, 704, 1000]        # 16 chunks: 5, 6, 5
    assert B.pipeline_plan(0, 4) == [0]
    for T in list(range(1, 700, 7)) + [4096, 32767, 32768, 100000]:
        for ns in range(1, 10):
            st = B.pipeline_plan(T, ns)
            assert len(st) - 1 == B.pipeline_segments(T, ns) == min(ns, (T + 63) // 64)
            assert st[0] == 0 and st[-1] == T
            assert all(b > a for a, b in zip(st, st[1:]))
            assert all(x % 64 == 0 for x in st[:-1])
            n_ch = [(b - a + 63) // 64 for a, b in zip(st, st[1:])]
            assert max(n_ch) - min(n_ch) <= 1, (T, ns, n_ch)


def test_prefill_pipelined_rejects():
    L = B.lib()
    ws = ctypes.c_void_p(0x100000)
    pa = B.PrepareArgs(x=0x200000, x_n_stride=0, x_t_stride=2 * 64 * 2 + 2 * 1 * 64 + 1 * 64, ba=0x300000,
                       ba_n_stride=0, ba_t_stride=3 * 2, A_log=0x400000, dt_bias=0x500000, G=1)
    # prepare makes H value heads: HV != H is refused before anything runs
    assert L.gdp_prefill_fwd_pipelined(ctypes.byref(pa), ctypes.byref(_args(H=2, HV=4)), 2, ws, None,
                                       None) == B.GDP_ERR_INVALID
    # g is written by prepare, so it must be given
    assert L.gdp_prefill_fwd_pipelined(ctypes.byref(pa), ctypes.byref(_args(g=None)), 2, ws, None,
                                       None) == B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_pipelined(None, ctypes.byref(_args()), 2, ws, None, None) == B.GDP_ERR_INVALID
    # prepare's own checks: H % G
    bad = B.PrepareArgs(x=0x200000, x_n_stride=0, x_t_stride=4096, ba=0x300000, ba_n_stride=0, ba_t_stride=64,
                        A_log=0x400000, dt_bias=0x500000, G=3)
    assert L.gdp_prefill_fwd_pipelined(ctypes.byref(bad), ctypes.byref(_args()), 2, ws, None,
                                       None) == B.GDP_ERR_INVALID
    assert b"G=3" in L.gdp_last_error()


def test_null_args_rejected():
    assert B.lib().gdp_chunk_fwd(None, None) == B.GDP_ERR_INVALID


def test_empty_problem_launches_nothing():
    # T == 0: valid, returns OK without touching the GPU
    a = _args(T=0, q=None, k=None, v=None, beta=None, g=None, k_rnorm=None, gcum=None, kdecay=None, w=None, u=None,
              v_new=None, h=None, o=None, h_chunks=0)
    assert B.lib().gdp_chunk_fwd(ctypes.byref(a), None) == B.GDP_OK


def test_fused_pass_requirements():
    """v_new and h both NULL select chunk_h and chunk_o as one pass: it needs
    q, k_rnorm and o, bf16 and M >= 2; one of the two NULL is an error.
    Every case is refused before any launch."""
    L = B.lib()
    fz = dict(v_new=None, h=None, M=2, T=128, h_chunks=4)
    assert L.gdp_chunk_fwd(ctypes.byref(_args(**dict(fz, M=1))), None) == B.GDP_ERR_UNSUPPORTED
    assert L.gdp_chunk_fwd(ctypes.byref(_args(**dict(fz, dtype=B.GDP_F32))), None) == B.GDP_ERR_UNSUPPORTED
    for nm in ("q", "k_rnorm", "o", "w", "u", "kdecay", "gcum"):
        assert L.gdp_chunk_fwd(ctypes.byref(_args(**dict(fz, **{nm: None}))), None) == B.GDP_ERR_INVALID, nm
    assert L.gdp_chunk_fwd(ctypes.byref(_args(M=2, T=128, h_chunks=4, v_new=None)), None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd(ctypes.byref(_args(M=2, T=128, h_chunks=4, h=None)), None) == B.GDP_ERR_INVALID
    ws = ctypes.c_void_p(0x100000)
    a = _args(**dict(fz, M=1, K=128, V=128))
    assert L.gdp_chunk_fwd_scan(ctypes.byref(a), 2, ws, 1 << 40, None, None) == B.GDP_ERR_UNSUPPORTED


def _prep_call(fn, **kw):
    base = dict(x=0x10000, xn=0, xt=5632, ba=0x20000, bn=0, bt=48, A_log=0x30000, dt_bias=0x40000,
                n=1, T=16, M=2, H=16, G=4, P=128, N=128, dtype=B.GDP_BF16,
                q=0x50000, k=0x60000, v=0x70000, beta=0x80000, g=0x90000)
    base.update(kw)
    b = base
    return fn(b["x"], b["xn"], b["xt"], b["ba"], b["bn"], b["bt"], b["A_log"], b["dt_bias"], b["n"], b["T"],
              b["M"], b["H"], b["G"], b["P"], b["N"], b["dtype"], b["q"], b["k"], b["v"], b["beta"], b["g"], None)


def _prep_prefill(**kw):
    return _prep_call(B.lib().gdp_prefill_prepare, **kw)


def _prep_decode(**kw):
    return _prep_call(B.lib().gdp_decode_prepare, **kw)


@pytest.mark.parametrize("decode", [False, True])
def test_prepare_rejects(decode):
    _prep = _prep_decode if decode else _prep_prefill
    assert _prep(G=3) == B.GDP_ERR_INVALID          # H % G
    assert _prep(M=0) == B.GDP_ERR_INVALID
    assert _prep(dtype=5) == B.GDP_ERR_INVALID
    assert _prep(q=None) == B.GDP_ERR_INVALID
    assert _prep(xt=100) == B.GDP_ERR_INVALID       # rows would overlap
    assert _prep(T=-1) == B.GDP_ERR_INVALID
    assert _prep(T=0, x=None) == B.GDP_OK           # empty: nothing launched


def test_num_state_chunks():
    assert B.num_state_chunks(1000, 2, B=3) == 3 * 32
    cu = [0, 1, 64, 64, 200]   # lengths 1, 63, 0, 136
    M = 3
    expect = sum(-(-(l * M) // 64) for l in (1, 63, 0, 136))
    assert B.num_state_chunks(200, M, cu_seqlens_host=cu) == expect
    # offsets are clamped into [0, T]
    assert B.num_state_chunks(100, 1, cu_seqlens_host=[0, 500]) == 2
    assert B.lib().gdp_num_state_chunks(None, 0, 1, -1, 1, 64) == -1


def _dec(**kw):
    base = dict(n=4, S=1, H=2, HV=4, K=128, V=128, M=2, scale=0.0, dtype=B.GDP_BF16, pool=8,
                q=0x10000, k=0x20000, v=0x30000, beta=0x40000, g=0x50000, state=0x60000, slots=None, o=0x70000)
    base.update(kw)
    return B.lib().gdp_decode_update(ctypes.byref(B.DecodeArgs(**base)), None)


BAD_DECODE = [
    ("K=96", dict(K=96), B.GDP_ERR_UNSUPPORTED),
    ("V=32", dict(V=32), B.GDP_ERR_UNSUPPORTED),
    ("M=5", dict(M=5), B.GDP_ERR_UNSUPPORTED),
    ("S*M too long", dict(S=2049), B.GDP_ERR_UNSUPPORTED),
    ("HV % H", dict(HV=3), B.GDP_ERR_INVALID),
    ("dtype", dict(dtype=4), B.GDP_ERR_INVALID),
    ("n<0", dict(n=-1), B.GDP_ERR_INVALID),
    ("pool < n without slots", dict(pool=3), B.GDP_ERR_INVALID),
    ("null state", dict(state=None), B.GDP_ERR_INVALID),
    ("null beta", dict(beta=None), B.GDP_ERR_INVALID),
    ("misaligned k", dict(k=0x20008), B.GDP_ERR_INVALID),
    ("misaligned state", dict(state=0x60004), B.GDP_ERR_INVALID),
    ("inf scale", dict(scale=float("inf")), B.GDP_ERR_INVALID),
]


@pytest.mark.parametrize("name,kw,status", BAD_DECODE, ids=[c[0] for c in BAD_DECODE])
def test_decode_update_rejects(name, kw, status):
    st = _dec(**kw)
    assert st == status, (st, B.lib().gdp_last_error())
    assert B.lib().gdp_last_error()


def test_decode_update_empty_and_null():
    assert B.lib().gdp_decode_update(None, None) == B.GDP_ERR_INVALID
    # nothing to do: valid without buffers, nothing launched
    assert _dec(n=0, q=None, k=None, v=None, beta=None, g=None, state=None, o=None) == B.GDP_OK
    assert _dec(S=0, q=None, k=None, v=None, beta=None, g=None, state=None, o=None) == B.GDP_OK
    # with slots the pool may be smaller than n (slots name the rows used)
    assert _dec(n=0, pool=0, slots=0x80000, q=None, k=None, v=None, beta=None, state=None, o=None) == B.GDP_OK


def test_scan_rejects_and_plan():
    """gdp_chunk_fwd_scan refuses what it does not run before launching
    anything; the segment plan and workspace size follow the header."""
    L = B.lib()
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 40
    a = lambda **kw: ctypes.byref(_args(**dict(dict(K=128, V=128), **kw)))
    assert L.gdp_chunk_fwd_scan(a(B=2, h_chunks=4), 4, ws, big, None, None) == B.GDP_ERR_INVALID
    # packed requests go through cu_seqlens with B == 1
    assert L.gdp_chunk_fwd_scan(a(B=2, cu_seqlens=0x1000, num_seqs=1), 4, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(cu_seqlens=0x1000, num_seqs=-1), 4, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(), 0, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(), 65, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(), 2, None, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(), 2, ctypes.c_void_p(0x100010), big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(), 2, ws, 1024, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(q=None), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan(a(dtype=B.GDP_F32, K=64, V=64), 2, ws, big, None, None) == B.GDP_ERR_UNSUPPORTED
    assert L.gdp_chunk_fwd_scan(ctypes.byref(_args(K=128, V=256)), 2, ws, big, None, None) == B.GDP_ERR_UNSUPPORTED
    assert B.lib().gdp_last_error()
    # T == 0 launches nothing and needs no workspace
    assert L.gdp_chunk_fwd_scan(a(T=0), 2, None, 0, None, None) == B.GDP_OK
    # segments of ceil(ceil(T/64) / n) chunks; the last may be shorter
    assert B.scan_segments(32768, 16) == 16
    assert B.scan_segments(1000, 3) == 3     # 16 chunks -> 6, 6, 4
    assert B.scan_segments(1000, 7) == 6     # 16 chunks -> 3 each, 6 segments
    assert B.scan_segments(100, 64) == 2
    assert B.scan_segments(0, 4) == 0
    assert L.gdp_scan_segments(10, 0) == -1 and L.gdp_scan_segments(10, 65) == -1
    # maps of all segments but the last, one state per segment, the offsets
    up = lambda x: (x + 255) // 256 * 256
    HV, K, V = 16, 128, 128
    want = up(15 * HV * K * (K + V) * 4) + up(16 * HV * V * K * 4) + up(17 * 4)
    assert L.gdp_scan_workspace_bytes(32768, HV, K, V, 16) == want
    assert L.gdp_scan_workspace_bytes(32768, HV, K, V, 0) == -1
    # packed requests: a map and a state for each of ceil(T / seg_tok) + N
    # slots, the offsets and last flags per slot, first slot and count per
    # request (seg_tok = 17 chunks for 16600 tokens in 16 segments)
    T, N = 16600, 8
    slots = -(-T // (17 * 64)) + N
    want = up(slots * HV * K * (K + V) * 4) + up(slots * HV * V * K * 4) + up((slots + 1) * 4) + up(slots * 4) \
        + 2 * up(N * 4)
    assert L.gdp_scan_workspace_bytes_varlen(T, N, HV, K, V, 16) == want
    assert L.gdp_scan_workspace_bytes_varlen(T, -1, HV, K, V, 16) == -1
    # a packed call checks its workspace against the varlen size
    assert L.gdp_chunk_fwd_scan(a(T=T, H=HV, HV=HV, cu_seqlens=0x1000, num_seqs=N, h_chunks=600), 16, ws,
                                want - 256, None, None) == B.GDP_ERR_INVALID
    assert b"workspace" in L.gdp_last_error()


def test_prefill_scan_rejects():
    """gdp_prefill_fwd_scan refuses before launching anything: value heads
    other than prepare's, a missing g, bad prepare arguments, and whatever
    gdp_chunk_fwd_scan refuses."""
    L = B.lib()
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 40
    pa = B.PrepareArgs(x=0x200000, x_n_stride=0, x_t_stride=2 * 2 * 128 + 2 * 1 * 128 + 1 * 128, ba=0x300000,
                       ba_n_stride=0, ba_t_stride=2 * 2 + 2, A_log=0x400000, dt_bias=0x500000, G=1)
    a = lambda **kw: ctypes.byref(_args(**dict(dict(K=128, V=128, M=2, H=2, HV=2, h_chunks=8), **kw)))
    assert L.gdp_prefill_fwd_scan(None, a(), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(HV=4), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(g=None), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    bad = B.PrepareArgs(**dict((f, getattr(pa, f)) for f, _ in B.PrepareArgs._fields_))
    bad.G = 3  # H % G != 0
    assert L.gdp_prefill_fwd_scan(ctypes.byref(bad), a(), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(B=2, h_chunks=16), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(), 0, ws, big, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(), 2, ws, 64, None, None) == B.GDP_ERR_INVALID
    assert B.lib().gdp_last_error()
    # v and beta may be NULL here (not stored): the call gets as far as the
    # workspace check; the plain scan form still needs them
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(v=None, beta=None), 2, ws, 64, None, None) == B.GDP_ERR_INVALID
    assert b"workspace" in B.lib().gdp_last_error()
    assert L.gdp_chunk_fwd_scan(a(v=None), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert b"v is NULL" in B.lib().gdp_last_error()
    assert L.gdp_chunk_fwd_scan(a(beta=None), 2, ws, big, None, None) == B.GDP_ERR_INVALID
    assert b"beta is NULL" in B.lib().gdp_last_error()
    # q and k: both NULL only with v_new and h NULL (then read from x; the
    # call gets as far as the workspace check), never one of them alone
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(q=None, k=None, v_new=None, h=None), 2, ws, 64, None,
                                  None) == B.GDP_ERR_INVALID
    assert b"workspace" in B.lib().gdp_last_error()
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(q=None, k=None), 2, ws, big, None, None) == \
        B.GDP_ERR_UNSUPPORTED
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(q=None, v_new=None, h=None), 2, ws, big, None, None) == \
        B.GDP_ERR_INVALID
    assert L.gdp_prefill_fwd_scan(ctypes.byref(pa), a(k=None, v_new=None, h=None), 2, ws, big, None, None) == \
        B.GDP_ERR_INVALID
    # the plain scan form has no activations to read them from
    assert L.gdp_chunk_fwd_scan(a(q=None, k=None, v_new=None, h=None), 2, ws, big, None, None) == \
        B.GDP_ERR_INVALID


def test_scan_noalloc_rejects_before_any_hip_call():
    """gdp_chunk_fwd_scan_noalloc refuses, with no HIP call (this runs without
    a GPU), a call whose workspace would pass its scratch array, with a
    message naming the limit, and everything gdp_chunk_fwd_scan refuses."""
    L = B.lib()
    T, HV, K, V, nseg = 32768, 32, 128, 128, 16
    need = L.gdp_scan_workspace_bytes(T, HV, K, V, nseg)
    m = re.search(r"#define GDP_NOALLOC_SCRATCH_BYTES \((\d+)LL \* 1024 \* 1024\)", open(HEADER).read())
    assert m and int(m.group(1)) << 20 == B.NOALLOC_SCRATCH_BYTES
    assert need > B.NOALLOC_SCRATCH_BYTES
    a = lambda **kw: ctypes.byref(_args(**dict(dict(K=K, V=V, T=T, H=HV, HV=HV, M=2, h_chunks=1024), **kw)))
    assert L.gdp_chunk_fwd_scan_noalloc(a(), nseg, None, None) == B.GDP_ERR_UNSUPPORTED
    msg = L.gdp_last_error()
    assert b"scratch" in msg and str(need).encode() in msg and b"GDP_NOALLOC_SCRATCH_BYTES" in msg
    # the 32768-token, 16-head workload of the benchmark fits
    assert L.gdp_scan_workspace_bytes(T, 16, K, V, nseg) <= B.NOALLOC_SCRATCH_BYTES
    # the checks of gdp_chunk_fwd_scan come first
    assert L.gdp_chunk_fwd_scan_noalloc(None, 4, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan_noalloc(a(B=2, h_chunks=2048), 4, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan_noalloc(a(), 0, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan_noalloc(a(q=None), 4, None, None) == B.GDP_ERR_INVALID
    assert L.gdp_chunk_fwd_scan_noalloc(a(dtype=B.GDP_F32, K=64, V=64), 4, None, None) == B.GDP_ERR_UNSUPPORTED
    # nothing to do: no scratch, no HIP call
    assert L.gdp_chunk_fwd_scan_noalloc(a(T=0), 4, None, None) == B.GDP_OK
