"""Thin ctypes binding of libgdp.so (include/gdp.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch provides device memory (outputs are allocated
with torch.empty on the inputs' device) and the current stream.  If the
library is not built this module raises; there is no fallback path.

Names follow the Megatron-Core GDP op pages: prefill_prepare
(core.ssm.ops.gdp.prepare), recompute_w_u (core.ssm.ops.gdp.wy_fast),
chunk_h and chunk_o (core.ssm.ops.gdp.chunk_o) and chunk_fwd for the three
chunk stages in order.
"""
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdp.so")

GDP_OK, GDP_ERR_INVALID, GDP_ERR_UNSUPPORTED, GDP_ERR_HIP = 0, 1, 2, 3
GDP_F32, GDP_BF16 = 0, 1
CHUNK = 64
# size of the library's own scratch array used by gdp_chunk_fwd_scan_noalloc (GDP_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_i64, _i32, _f32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class ChunkArgs(ctypes.Structure):
    """Mirror of gdp_chunk_args (include/gdp.h)."""
    _fields_ = [
        ("B", _i64), ("T", _i64), ("H", _i32), ("HV", _i32), ("K", _i32), ("V", _i32),
        ("M", _i32), ("chunk_size", _i32), ("scale", _f32), ("dtype", ctypes.c_int),
        ("cu_seqlens", _vp), ("num_seqs", _i64), ("h_chunks", _i64),
        ("q", _vp), ("k", _vp), ("v", _vp), ("beta", _vp), ("g", _vp), ("k_rnorm", _vp),
        ("gcum", _vp), ("kdecay", _vp), ("w", _vp), ("u", _vp), ("v_new", _vp), ("h", _vp), ("o", _vp),
        ("h0", _vp), ("ht", _vp),
    ]


class DecodeArgs(ctypes.Structure):
    """Mirror of gdp_decode_args (include/gdp.h)."""
    _fields_ = [
        ("n", _i64), ("S", _i64), ("H", _i32), ("HV", _i32), ("K", _i32), ("V", _i32), ("M", _i32),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int), ("pool", _i64),
        ("q", _vp), ("k", _vp), ("v", _vp), ("beta", _vp), ("g", _vp), ("state", _vp), ("slots", _vp), ("o", _vp),
    ]


class PrepareArgs(ctypes.Structure):
    """Mirror of gdp_prepare_args (include/gdp.h)."""
    _fields_ = [
        ("x", _vp), ("x_n_stride", _i64), ("x_t_stride", _i64), ("ba", _vp), ("ba_n_stride", _i64),
        ("ba_t_stride", _i64), ("A_log", _vp), ("dt_bias", _vp), ("G", _i32),
    ]


class GdpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("gdp status %d: %s" % (status, msg))
        self.status = status


_lib = None


def lib():
    """Load libgdp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdp.so is not built; run gated_delta_product_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.gdp_prefill_prepare.restype = ctypes.c_int
        L.gdp_prefill_prepare.argtypes = [
            _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp,
            _i64, _i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
            _vp, _vp, _vp, _vp, _vp, _vp]
        for name in ("gdp_recompute_w_u", "gdp_chunk_h", "gdp_chunk_o", "gdp_chunk_fwd"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.POINTER(ChunkArgs), _vp]
        L.gdp_decode_prepare.restype = ctypes.c_int
        L.gdp_decode_prepare.argtypes = L.gdp_prefill_prepare.argtypes
        L.gdp_decode_update.restype = ctypes.c_int
        L.gdp_decode_update.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        L.gdp_chunk_fwd_pipelined.restype = ctypes.c_int
        L.gdp_chunk_fwd_pipelined.argtypes = [ctypes.POINTER(ChunkArgs), _i32, _vp, _vp, _vp]
        L.gdp_prefill_fwd_pipelined.restype = ctypes.c_int
        L.gdp_prefill_fwd_pipelined.argtypes = [ctypes.POINTER(PrepareArgs), ctypes.POINTER(ChunkArgs), _i32, _vp,
                                                _vp, _vp]
        L.gdp_chunk_fwd_scan.restype = ctypes.c_int
        L.gdp_chunk_fwd_scan.argtypes = [ctypes.POINTER(ChunkArgs), _i32, _vp, _i64, _vp, _vp]
        L.gdp_chunk_fwd_scan_noalloc.restype = ctypes.c_int
        L.gdp_chunk_fwd_scan_noalloc.argtypes = [ctypes.POINTER(ChunkArgs), _i32, _vp, _vp]
        L.gdp_prefill_fwd_scan.restype = ctypes.c_int
        L.gdp_prefill_fwd_scan.argtypes = [ctypes.POINTER(PrepareArgs), ctypes.POINTER(ChunkArgs), _i32, _vp, _i64,
                                           _vp, _vp]
        L.gdp_scan_segments.restype = _i32
        L.gdp_scan_segments.argtypes = [_i64, _i32]
        L.gdp_scan_workspace_bytes.restype = _i64
        L.gdp_scan_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32]
        L.gdp_scan_workspace_bytes_varlen.restype = _i64
        L.gdp_scan_workspace_bytes_varlen.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32]
        L.gdp_pipeline_segments.restype = _i32
        L.gdp_pipeline_segments.argtypes = [_i64, _i32]
        L.gdp_pipeline_plan.restype = _i32
        L.gdp_pipeline_plan.argtypes = [_i64, _i32, ctypes.POINTER(_i64)]
        L.gdp_num_state_chunks.restype = _i64
        L.gdp_num_state_chunks.argtypes = [ctypes.POINTER(_i32), _i64, _i64, _i64, _i32, _i32]
        L.gdp_last_error.restype = ctypes.c_char_p
        L.gdp_last_error.argtypes = []
        L.gdp_version.restype = ctypes.c_char_p
        L.gdp_version.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != GDP_OK:
        raise GdpError(status, lib().gdp_last_error().decode())


def _dtype_code(t):
    if t == torch.bfloat16:
        return GDP_BF16
    if t == torch.float32:
        return GDP_F32
    raise TypeError("unsupported dtype %s (bf16 or f32)" % t)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices")
    return dev


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# ------------------------------------------------------------------ prepare

def prefill_prepare(x, ba, A_log, dt_bias, num_householder, num_heads, num_groups, head_dim, state_dim,
                    out=None):
    """Split, GQA-expand, Householder-fold and gate a prefill step.

    x [n, T, M*H*P + M*G*N + G*N] and ba [n, T, M*H + H] (bf16 or f32, last
    dim contiguous, rows may be strided); A_log, dt_bias [H] float32.
    Returns (q [n,T,H,N], k [n,T*M,H,N], v [n,T*M,H,P], beta [n,T*M,H] f32,
    g [n,T,H] f32).  ``out`` may hold preallocated (q, k, v, beta, g).
    """
    M, H, G, P, N = num_householder, num_heads, num_groups, head_dim, state_dim
    dev = _need_cuda(x, ba, A_log, dt_bias)
    if x.dim() != 3 or ba.dim() != 3:
        raise ValueError("x and ba must be 3-D [n, T, ...]")
    if x.stride(-1) != 1 or ba.stride(-1) != 1:
        raise ValueError("the last dimension of x and ba must be contiguous")
    if ba.dtype != x.dtype:
        raise ValueError("x and ba must share a dtype")
    if A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise ValueError("A_log and dt_bias must be float32")
    _contig(A_log, "A_log")
    _contig(dt_bias, "dt_bias")
    n, T = x.shape[0], x.shape[1]
    shapes = [((n, T, H, N), x.dtype), ((n, T * M, H, N), x.dtype), ((n, T * M, H, P), x.dtype),
              ((n, T * M, H), torch.float32), ((n, T, H), torch.float32)]
    if out is None:
        out = [torch.empty(s, dtype=d, device=dev) for s, d in shapes]
    for t, (s, d) in zip(out, shapes):
        if tuple(t.shape) != s or t.dtype != d or not t.is_contiguous() or t.device != dev:
            raise ValueError("out tensor mismatch: want %s %s" % (s, d))
    q, k, v, beta, g = out
    if x.shape[2] != M * H * P + M * G * N + G * N:
        raise ValueError("x last dim %d != M*H*P + M*G*N + G*N" % x.shape[2])
    if tuple(ba.shape) != (n, T, M * H + H):
        raise ValueError("ba must be [n, T, M*H + H]")
    _check(lib().gdp_prefill_prepare(
        _ptr(x), x.stride(0), x.stride(1), _ptr(ba), ba.stride(0), ba.stride(1),
        _ptr(A_log), _ptr(dt_bias), n, T, M, H, G, P, N, _dtype_code(x.dtype),
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _stream(dev)))
    return q, k, v, beta, g


# ------------------------------------------------------------------ chunk stages

def pipeline_segments(T, num_segments):
    """Segments gdp_chunk_fwd_pipelined runs for T tokens."""
    return int(lib().gdp_pipeline_segments(int(T), int(num_segments)))


def pipeline_plan(T, num_segments):
    """Token offsets where those segments start, then T (a list of n + 1)."""
    buf = (_i64 * (max(int(num_segments), 0) + 1))()
    n = lib().gdp_pipeline_plan(int(T), int(num_segments), buf)
    if n < 0:
        raise GdpError(GDP_ERR_INVALID, "bad arguments to gdp_pipeline_plan")
    return [int(buf[i]) for i in range(n + 1)]


def scan_segments(T, num_segments):
    """Segments gdp_chunk_fwd_scan runs for T tokens."""
    n = lib().gdp_scan_segments(int(T), int(num_segments))
    if n < 0:
        raise ValueError("bad arguments")
    return n


def num_state_chunks(T, M, B=1, cu_seqlens_host=None):
    """Chunks h must hold (sum over sequences of ceil(len*M/64))."""
    if cu_seqlens_host is None:
        return B * math.ceil(T * M / CHUNK)
    cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    n = cu.numel() - 1
    arr = (_i32 * (n + 1))(*cu.tolist())
    return int(lib().gdp_num_state_chunks(arr, n, 1, T, M, CHUNK))


class ChunkBuffers:
    """All tensors of one chunk forward (inputs, scratch and outputs)."""

    def __init__(self, q, k, v, beta, g, cu_seqlens=None, scale=None, h_chunks=None,
                 cu_seqlens_host=None, num_householder=None, initial_state=None, output_final_state=False):
        dev = _need_cuda(q, k, v, beta, g, cu_seqlens, initial_state)
        for t, nm in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (g, "g"), (initial_state, "initial_state")):
            if t is not None:
                _contig(t, nm)
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
            raise ValueError("q, k, v must be 4-D")
        B, T, H, K = q.shape
        M = num_householder if num_householder is not None else k.shape[1] // max(T, 1)
        HV, V = v.shape[2], v.shape[3]
        if tuple(k.shape) != (B, T * M, H, K):
            raise ValueError("k must be [B, T*M, H, K] = %s, got %s" % ((B, T * M, H, K), tuple(k.shape)))
        if tuple(v.shape[:2]) != (B, T * M):
            raise ValueError("v must be [B, T*M, HV, V]")
        if tuple(beta.shape) != (B, T * M, HV) or beta.dtype != torch.float32:
            raise ValueError("beta must be float32 [B, T*M, HV]")
        if g is not None and (tuple(g.shape) != (B, T, HV) or g.dtype != torch.float32):
            raise ValueError("g must be float32 [B, T, HV] (or None: ungated)")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("q, k, v must share a dtype")
        nseq = B
        if cu_seqlens is not None:
            if cu_seqlens.dtype != torch.int32:
                raise ValueError("cu_seqlens must be int32")
            _contig(cu_seqlens, "cu_seqlens")
            nseq = cu_seqlens.numel() - 1
        if h_chunks is None:
            if cu_seqlens is None:
                h_chunks = num_state_chunks(T, M, B)
            elif cu_seqlens_host is not None:
                h_chunks = num_state_chunks(T, M, 1, cu_seqlens_host)
            else:
                h_chunks = math.ceil(T * M / CHUNK) + nseq
        if initial_state is not None and (tuple(initial_state.shape) != (nseq, HV, V, K)
                                          or initial_state.dtype != torch.float32):
            raise ValueError("initial_state must be float32 [nseq, HV, V, K] = %s" % ((nseq, HV, V, K),))
        dt = q.dtype
        self.dims = dict(B=B, T=T, H=H, HV=HV, K=K, V=V, M=M, nseq=nseq)
        self.h0 = initial_state
        self.ht = torch.empty((nseq, HV, V, K), dtype=torch.float32, device=dev) if output_final_state else None
        self.q, self.k, self.v, self.beta, self.g = q, k, v, beta, g
        self.cu_seqlens = cu_seqlens
        self.k_rnorm = torch.empty((B, H, T * M), dtype=torch.float32, device=dev)
        self.gcum = torch.empty((B, HV, T * M), dtype=torch.float32, device=dev)
        self.kdecay = torch.empty((B, HV, T * M), dtype=torch.float32, device=dev)
        self.w = torch.empty((B, T * M, HV, K), dtype=dt, device=dev)
        # u and v_new are stored as 16-column slices [B, HV, V/16, T*M, 16]
        # (slices_to_rows gives the [B, T*M, HV, V] view)
        self.u = torch.empty((B, HV, V // 16, T * M, 16), dtype=dt, device=dev)
        self.v_new = torch.empty((B, HV, V // 16, T * M, 16), dtype=dt, device=dev)
        self.h = torch.empty((h_chunks, HV, V, K), dtype=dt, device=dev)
        self.o = torch.empty((B, T, HV, V), dtype=dt, device=dev)
        self.device = dev
        self.args = ChunkArgs(
            B=B, T=T, H=H, HV=HV, K=K, V=V, M=M, chunk_size=CHUNK,
            scale=float(scale) if scale is not None else 0.0, dtype=_dtype_code(dt),
            cu_seqlens=None if cu_seqlens is None else cu_seqlens.data_ptr(),
            num_seqs=nseq, h_chunks=h_chunks,
            q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), beta=beta.data_ptr(),
            g=None if g is None else g.data_ptr(),
            k_rnorm=self.k_rnorm.data_ptr(), gcum=self.gcum.data_ptr(), kdecay=self.kdecay.data_ptr(), w=self.w.data_ptr(), u=self.u.data_ptr(),
            v_new=self.v_new.data_ptr(), h=self.h.data_ptr(), o=self.o.data_ptr(),
            h0=None if initial_state is None else initial_state.data_ptr(),
            ht=None if self.ht is None else self.ht.data_ptr())

    def set(self, **tensors):
        """Point a slot (e.g. h, v_new) at another tensor of the same shape."""
        for name, t in tensors.items():
            cur = getattr(self, name)
            if tuple(t.shape) != tuple(cur.shape) or t.dtype != cur.dtype or not t.is_contiguous():
                raise ValueError("%s: shape/dtype mismatch" % name)
            setattr(self, name, t)
            setattr(self.args, name, t.data_ptr())

    def _call(self, fn, stream=None):
        s = stream if stream is not None else _stream(self.device)
        _check(fn(ctypes.byref(self.args), s))

    def recompute_w_u(self, stream=None):
        self._call(lib().gdp_recompute_w_u, stream)

    def chunk_h(self, stream=None):
        self._call(lib().gdp_chunk_h, stream)

    def chunk_o(self, stream=None):
        self._call(lib().gdp_chunk_o, stream)

    def forward(self, stream=None, store_vnew_h=True):
        """gdp_chunk_fwd.  store_vnew_h=False passes v_new and h as NULL:
        chunk_h and chunk_o then run as one pass that stores neither (bf16,
        M >= 2)."""
        if store_vnew_h:
            self._call(lib().gdp_chunk_fwd, stream)
        else:
            s = stream if stream is not None else _stream(self.device)
            _check(lib().gdp_chunk_fwd(ctypes.byref(self._args_without("v_new", "h")), s))
        return self.o

    def prefill_pipelined(self, x, ba, A_log, dt_bias, num_groups, num_segments, stream=None, chunk_h_events=None):
        """gdp_prefill_fwd_pipelined: prepare x / ba into this buffer's q, k,
        v, beta, g (allocated with the prepare shapes) and run the pipelined
        chunk forward, each segment's prepare overlapped with the serial
        stage.  Arguments as prefill_prepare and forward_pipelined."""
        _need_cuda(x, ba, A_log, dt_bias)
        d = self.dims
        if x.dim() != 3 or x.stride(2) != 1 or ba.dim() != 3 or ba.stride(2) != 1:
            raise ValueError("x and ba must be 3-D with a contiguous last dimension")
        if x.shape[:2] != (d["B"], d["T"]) or ba.shape[:2] != (d["B"], d["T"]) or x.dtype != self.q.dtype:
            raise ValueError("x / ba do not match the buffers")
        pa = PrepareArgs(x=x.data_ptr(), x_n_stride=x.stride(0), x_t_stride=x.stride(1), ba=ba.data_ptr(),
                         ba_n_stride=ba.stride(0), ba_t_stride=ba.stride(1), A_log=A_log.data_ptr(),
                         dt_bias=dt_bias.data_ptr(), G=int(num_groups))
        return self._pipelined(lambda ws, ev, s: lib().gdp_prefill_fwd_pipelined(
            ctypes.byref(pa), ctypes.byref(self.args), int(num_segments), ws, ev, s), num_segments, stream,
            chunk_h_events)

    def forward_pipelined(self, num_segments, stream=None, chunk_h_events=None):
        """gdp_chunk_fwd_pipelined: the same results for B == 1 without
        cu_seqlens, with the parallel stages of neighbouring segments
        overlapping the serial one.  chunk_h_events: optional list of
        2 * pipeline_segments(T, num_segments) torch.cuda.Event (timing
        enabled, recorded at least once) marking each segment's chunk_h."""
        return self._pipelined(lambda ws, ev, s: lib().gdp_chunk_fwd_pipelined(
            ctypes.byref(self.args), int(num_segments), ws, ev, s), num_segments, stream, chunk_h_events)

    def _args_without(self, *names):
        """A copy of the argument struct with the named tensors set to NULL."""
        args = type(self.args).from_buffer_copy(self.args)
        for nm in names:
            setattr(args, nm, None)
        return args

    def prefill_scan(self, x, ba, A_log, dt_bias, num_groups, num_segments, stream=None, stage_events=None,
                     store_v_beta=True, store_vnew_h=True, store_qk=True):
        """gdp_prefill_fwd_scan: prepare x / ba into this buffer's q, k, v,
        beta, g (allocated with the prepare shapes) inside the WY stage of the
        segment-parallel forward.  Arguments as prefill_prepare and
        forward_scan.  store_v_beta=False passes v and beta as NULL: nothing
        after the WY stage reads them, and they are left untouched.
        store_vnew_h=False as for forward_scan.  store_qk=False (with
        store_vnew_h=False) passes q and k as NULL: the later stages read their
        rows from x, and q and k are left untouched."""
        _need_cuda(x, ba, A_log, dt_bias)
        d = self.dims
        if x.dim() != 3 or x.stride(2) != 1 or ba.dim() != 3 or ba.stride(2) != 1:
            raise ValueError("x and ba must be 3-D with a contiguous last dimension")
        if x.shape[:2] != (d["B"], d["T"]) or ba.shape[:2] != (d["B"], d["T"]) or x.dtype != self.q.dtype:
            raise ValueError("x / ba do not match the buffers")
        pa = PrepareArgs(x=x.data_ptr(), x_n_stride=x.stride(0), x_t_stride=x.stride(1), ba=ba.data_ptr(),
                         ba_n_stride=ba.stride(0), ba_t_stride=ba.stride(1), A_log=A_log.data_ptr(),
                         dt_bias=dt_bias.data_ptr(), G=int(num_groups))
        args = self._args_without(*((() if store_v_beta else ("v", "beta")) +
                                    (() if store_vnew_h else ("v_new", "h")) +
                                    (() if store_qk else ("q", "k"))))
        return self._scan(lambda ws, nb, ev, s: lib().gdp_prefill_fwd_scan(
            ctypes.byref(pa), ctypes.byref(args), int(num_segments), ws, nb, ev, s), num_segments, stream,
            stage_events)

    def forward_scan(self, num_segments, stream=None, stage_events=None, store_vnew_h=True):
        """gdp_chunk_fwd_scan: the results of forward() for B == 1, one
        sequence or packed requests (cu_seqlens), to rounding past the first
        segment of each sequence, with every long serial chunk_h chain cut
        into segments run in parallel from the states a scan over the
        segments' composed maps gives.  Of h only the states entering chunks
        i*M (the ones chunk_o reads) are written; the other slots keep what
        they held.
        stage_events: optional 5 events with a cuda_event handle (timing
        enabled, recorded at least once), recorded after the WY stage, the
        segment maps, the scan, chunk_h and chunk_o.
        store_vnew_h=False passes v_new and h as NULL: chunk_h and chunk_o
        then run as one pass that stores neither (M >= 2), and they keep
        what they held."""
        args = self.args if store_vnew_h else self._args_without("v_new", "h")
        return self._scan(lambda ws, nb, ev, s: lib().gdp_chunk_fwd_scan(
            ctypes.byref(args), int(num_segments), ws, nb, ev, s), num_segments, stream, stage_events)

    def forward_scan_noalloc(self, num_segments, stream=None, stage_events=None, store_vnew_h=True):
        """gdp_chunk_fwd_scan_noalloc: forward_scan with the workspace taken
        from the library's own device scratch array (GDP_NOALLOC_SCRATCH_BYTES)
        instead of a tensor; nothing is allocated by the call.  Calls that
        overlap on one GPU share that array."""
        ev = _stage_events(stage_events)
        s = stream if stream is not None else _stream(self.device)
        args = self.args if store_vnew_h else self._args_without("v_new", "h")
        _check(lib().gdp_chunk_fwd_scan_noalloc(ctypes.byref(args), int(num_segments), ev, s))
        return self.o

    def scan_workspace_bytes(self, num_segments):
        """Workspace bytes gdp_chunk_fwd_scan needs for these buffers."""
        d = self.dims
        if self.cu_seqlens is not None:
            return lib().gdp_scan_workspace_bytes_varlen(d["T"], d["nseq"], d["HV"], d["K"], d["V"],
                                                         int(num_segments))
        return lib().gdp_scan_workspace_bytes(d["T"], d["HV"], d["K"], d["V"], int(num_segments))

    def _scan(self, call, num_segments, stream, stage_events):
        need = self.scan_workspace_bytes(num_segments)
        if need < 0:
            raise ValueError("num_segments %r out of range" % (num_segments,))
        ws = getattr(self, "_scan_ws", None)
        if ws is None or ws.numel() < need:
            # torch's caching allocator returns 512-byte aligned blocks
            self._scan_ws = ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        ev = _stage_events(stage_events)
        s = stream if stream is not None else _stream(self.device)
        _check(call(ws.data_ptr(), ws.numel(), ev, s))
        return self.o

    def _pipelined(self, call, num_segments, stream, chunk_h_events):
        d = self.dims
        if getattr(self, "_ws", None) is None:
            self._ws = torch.empty((2, d["HV"], d["V"], d["K"]), dtype=torch.float32, device=self.device)
        ev = None
        if chunk_h_events is not None:
            n = pipeline_segments(d["T"], num_segments)
            if len(chunk_h_events) != 2 * n:
                raise ValueError("need %d events" % (2 * n))
            ev = (_vp * (2 * n))(*[e.cuda_event for e in chunk_h_events])
        s = stream if stream is not None else _stream(self.device)
        _check(call(self._ws.data_ptr(), ev, s))
        return self.o


def _stage_events(events):
    """The 5 stage events of the segment-parallel forward as a C array."""
    if events is None:
        return None
    if len(events) != 5:
        raise ValueError("need 5 events")
    return (_vp * 5)(*[e.cuda_event for e in events])


def slices_to_rows(t):
    """A slice-major u / v_new [B, HV, V/16, T*M, 16] as [B, T*M, HV, V] (a copy)."""
    B, HV, S, TM, _ = t.shape
    return t.permute(0, 3, 1, 2, 4).reshape(B, TM, HV, S * 16)


def rows_to_slices(t):
    """[B, T*M, HV, V] -> the slice-major [B, HV, V/16, T*M, 16] layout of u / v_new."""
    B, TM, HV, V = t.shape
    return t.reshape(B, TM, HV, V // 16, 16).permute(0, 2, 3, 1, 4).contiguous()


def chunk_fwd(q, k, v, beta, g, scale=None, cu_seqlens=None, cu_seqlens_host=None, initial_state=None,
              output_final_state=False):
    """Chunked GDP forward.  q [B,T,H,K]; k [B,T*M,H,K]; v [B,T*M,HV,V];
    beta [B,T*M,HV] f32; g [B,T,HV] f32 natural-log decay per token, or None
    (ungated); initial_state [nseq,HV,V,K] f32 or None.
    Returns the ChunkBuffers holding o, the intermediates (w, u, v_new, h) and,
    if output_final_state, ht [nseq,HV,V,K] f32."""
    buf = ChunkBuffers(q, k, v, beta, g, cu_seqlens=cu_seqlens, scale=scale, cu_seqlens_host=cu_seqlens_host,
                       initial_state=initial_state, output_final_state=output_final_state)
    buf.forward()
    return buf


def version():
    return lib().gdp_version().decode()


# ------------------------------------------------------------------ decode

def decode_prepare(x, ba, A_log, dt_bias, M, H, G, P, N, out=None):
    """gdp_decode_prepare: x [n, S, M*H*P + M*G*N + G*N], ba [n, S, M*H + H]
    (last dimensions contiguous).  Returns (q [n,S*M,H,N] with the query on
    each token's last copy, k [n,S*M,H,N], v [n,S*M,H,P], beta [n,S*M,H]
    f32, g [n,S*M,H] f32 with the decay on each token's first copy)."""
    dev = _need_cuda(x, ba, A_log, dt_bias)
    n, S, width = x.shape
    if width != M * H * P + M * G * N + G * N or x.stride(2) != 1:
        raise ValueError("x must be [n, S, M*H*P + M*G*N + G*N] with a contiguous last dimension")
    if tuple(ba.shape) != (n, S, M * H + H) or ba.stride(2) != 1:
        raise ValueError("ba must be [n, S, M*H + H]")
    if out is None:
        dt = x.dtype
        out = (torch.empty((n, S * M, H, N), dtype=dt, device=dev), torch.empty((n, S * M, H, N), dtype=dt, device=dev),
               torch.empty((n, S * M, H, P), dtype=dt, device=dev),
               torch.empty((n, S * M, H), dtype=torch.float32, device=dev),
               torch.empty((n, S * M, H), dtype=torch.float32, device=dev))
    q, k, v, beta, g = out
    _check(lib().gdp_decode_prepare(
        _ptr(x), x.stride(0), x.stride(1), _ptr(ba), ba.stride(0), ba.stride(1),
        _ptr(A_log), _ptr(dt_bias), n, S, M, H, G, P, N, _dtype_code(x.dtype),
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _stream(dev)))
    return out


def decode_update(q, k, v, beta, g, state, M, slots=None, scale=None, o=None):
    """gdp_decode_update: one decode step over rows from decode_prepare.
    q, k [n, S*M, H, K]; v [n, S*M, HV, V]; beta, g [n, S*M, HV] f32 (g may
    be None); state [pool, HV, V, K] f32 updated in place; slots int32 [n]
    or None.  Returns o [n, S*M, HV, V]."""
    dev = _need_cuda(q, k, v, beta, g, state, slots)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (g, "g"), (state, "state"), (slots, "slots")):
        if t is not None:
            _contig(t, nm)
    n, L, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if L % M:
        raise ValueError("rows per request must be a multiple of M")
    if tuple(k.shape) != (n, L, H, K) or tuple(v.shape[:2]) != (n, L) or tuple(beta.shape) != (n, L, HV):
        raise ValueError("q, k, v, beta shapes disagree")
    if g is not None and tuple(g.shape) != (n, L, HV):
        raise ValueError("g must be [n, S*M, HV]")
    if state.dtype != torch.float32 or tuple(state.shape[1:]) != (HV, V, K):
        raise ValueError("state must be float32 [pool, HV, V, K]")
    if slots is not None and (slots.dtype != torch.int32 or tuple(slots.shape) != (n,)):
        raise ValueError("slots must be int32 [n]")
    if o is None:
        o = torch.empty((n, L, HV, V), dtype=q.dtype, device=dev)
    a = DecodeArgs(n=n, S=L // M, H=H, HV=HV, K=K, V=V, M=M, scale=float(scale) if scale is not None else 0.0,
                   dtype=_dtype_code(q.dtype), pool=state.shape[0], q=_ptr(q), k=_ptr(k), v=_ptr(v),
                   beta=_ptr(beta), g=None if g is None else _ptr(g), state=_ptr(state),
                   slots=None if slots is None else _ptr(slots), o=_ptr(o))
    _check(lib().gdp_decode_update(ctypes.byref(a), _stream(dev)))
    return o
