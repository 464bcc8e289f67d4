"""moeq: NF4 / row-wise int8 quantization of fused MoE expert tensors and the
routed experts forward straight from the packed storage, on MI355X (gfx950).

This module is a thin ctypes binding over ``libmoeq.so`` (declared in
``include/moeq.h``): it marshals torch tensors into device pointers and the
current HIP stream, allocates outputs with torch, and raises on any non-zero
status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  A missing library is an error, never a silent switch
to another path.
"""

import ctypes
import os

import torch

__all__ = [
    "MoeqError", "QWeight", "FMT_NF4", "FMT_INT8_ROWWISE", "NF4_BLOCKSIZE",
    "moeq_abi_version", "moeq_status_string", "moeq_nf4_codebook",
    "moeq_quantize_nf4", "moeq_quantize_int8_rowwise", "moeq_dequantize",
    "moeq_experts_forward_workspace_bytes", "moeq_experts_forward",
    "moeq_route_workspace_bytes", "moeq_route_buckets", "library_path",
    "moeq_experts_backward_workspace_bytes", "moeq_experts_backward", "moeq_router_topk",
    "moeq_router_route_workspace_bytes",
    "moeq_qweight_copy_async", "FMT_NF4_DQ", "DQ_GROUP", "moeq_compress_absmax",
    "moeq_stream_reference", "moeq_router_route", "moeq_experts_forward_routed", "Routing",
    "moeq_experts_forward_noalloc", "NOALLOC_SCRATCH_BYTES",
]

FMT_NF4 = 1
FMT_INT8_ROWWISE = 2
FMT_NF4_DQ = 3
NF4_BLOCKSIZE = 64
DQ_GROUP = 256
ABI_VERSION = 3
NOALLOC_SCRATCH_BYTES = 64 << 20

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libmoeq.so")
_lib = None


class MoeqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {moeq_status_string(status)} (status {status})")


class _QW(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("blocksize", ctypes.c_int32), ("qdata", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("scale_codes", ctypes.c_void_p)]


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libmoeq.so is not built ({_LIB_PATH}); run "
                           "`python -m bit_weight_quantization_moeq_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    QP = ctypes.POINTER(_QW)
    sig = {
        "moeq_abi_version": (I32, []),
        "moeq_status_string": (ctypes.c_char_p, [I32]),
        "moeq_nf4_codebook": (I32, [ctypes.POINTER(ctypes.c_float)]),
        "moeq_quantize_nf4": (I32, [P, QP, P]),
        "moeq_quantize_int8_rowwise": (I32, [P, QP, P]),
        "moeq_stream_reference": (I32, [P, QP, P]),
        "moeq_compress_absmax": (I32, [QP, QP, P]),
        "moeq_dequantize": (I32, [QP, P, P]),
        "moeq_experts_forward_workspace_bytes": (SZ, [I32, I32, QP, QP]),
        "moeq_experts_forward": (I32, [P, P, P, I32, I32, QP, QP, P, P, SZ, P]),
        "moeq_experts_forward_timed": (I32, [P, P, P, I32, I32, QP, QP, P, P, SZ, P, P]),
        "moeq_route_workspace_bytes": (SZ, [I32, I32, I32]),
        "moeq_experts_backward_workspace_bytes": (SZ, [I32, I32, QP, QP]),
        "moeq_experts_backward": (I32, [P, P, P, I32, I32, QP, QP, P, P, P, P, SZ, P]),
        "moeq_router_topk": (I32, [P, P, I32, I32, I32, I32, I32, P, P, P]),
        "moeq_qweight_copy_async": (I32, [QP, QP, P]),
        "moeq_route_buckets": (I32, [P, I32, I32, I32, P, P, P, P, P, SZ, P]),
        "moeq_router_route_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "moeq_router_route": (I32, [P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, SZ, P]),
        "moeq_experts_forward_routed": (I32, [P, P, P, I32, I32, QP, QP, P, P, P, P, P, SZ, P]),
        "moeq_experts_forward_noalloc": (I32, [P, P, P, I32, I32, QP, QP, P, P]),
        "moeq_experts_forward_save": (I32, [P, P, P, I32, I32, QP, QP, P, P, P, SZ, P]),
        "moeq_experts_backward_saved_workspace_bytes": (SZ, [I32, I32, QP, QP]),
        "moeq_experts_backward_saved": (I32, [P, P, I32, I32, QP, QP, P, P, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if lib.moeq_abi_version() != ABI_VERSION:
        raise RuntimeError("libmoeq ABI version mismatch")
    _lib = lib
    return lib


def _check(status, where):
    if status != 0:
        raise MoeqError(status, where)


# The current stream's raw handle without building a Stream object (the
# public current_stream() costs a few microseconds of host time per call).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device=None):
    """Raw hipStream_t: ``stream``'s, else the current stream of ``device``
    (a CUDA device of the call's tensors), else of the current device."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None and device is not None and device.index is not None:
        return ctypes.c_void_p(_raw_stream(device.index))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    """A tensor's device address for a c_void_p argument (None: NULL)."""
    return t.data_ptr() if t is not None else None


def _dev(t, dtype, name, shape=None):
    """Structural check of a caller tensor before its pointer reaches the
    library: exact shape (when given), dtype and contiguity.  The C side sees
    only raw pointers and trusts the sizes it is given, so a wrong-sized
    buffer must be refused here, loudly, rather than read or written out of
    bounds.  Where the tensors live is checked once per call, after every
    structural check (:func:`_on_device`)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if shape is not None and t.shape != shape:
        want = tuple(int(d) for d in shape)
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(where, *tensors):
    """Every tensor is a CUDA (HIP) tensor, all on one device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{where}: every tensor must be a CUDA (HIP) tensor")
        d = t.device
        if dev is None:
            dev = d
        elif d != dev:
            ds = sorted({str(u.device) for u in tensors if u is not None})
            raise ValueError(f"{where}: tensors on different devices {ds}")
    return dev


def _match_qweight(q, shape, formats, name):
    """q is a QWeight of one of ``formats`` describing ``shape`` [E, rows, cols]."""
    if not isinstance(q, QWeight):
        raise TypeError(f"{name} must be a QWeight")
    if q.format not in formats:
        raise ValueError(f"{name} has format {q.format}, expected one of {formats}")
    if tuple(q.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} describes {tuple(q.shape)}, expected {tuple(shape)}")


def _forward_weights(gate_up, down, H):
    """gate_up [E, 2I, H] and down [E, H, I]: each checked against its own
    layout and the hidden width H (the library derives H from gate_up; whether
    the two tensors fit each other is the library's own check)."""
    for name, q in (("gate_up", gate_up), ("down", down)):
        if not isinstance(q, QWeight):
            raise TypeError(f"{name} must be a QWeight")
        q.validate_layout()
    if gate_up.cols != H:
        raise ValueError(f"hidden width {H} must equal gate_up cols ({gate_up.cols})")
    return gate_up._tensors() + down._tensors()


def _routed_inputs(hidden, top_k_index, top_k_weights):
    """(T, H, K) of hidden [T, H] bf16, top_k_index [T, K] int32 and
    top_k_weights [T, K] fp32, structurally checked."""
    for name, t in (("hidden", hidden), ("top_k_index", top_k_index), ("top_k_weights", top_k_weights)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    T, H = hidden.shape
    K = top_k_index.shape[1]
    _dev(hidden, torch.bfloat16, "hidden")
    _dev(top_k_index, torch.int32, "top_k_index", (T, K))
    _dev(top_k_weights, torch.float32, "top_k_weights", (T, K))
    return int(T), int(H), int(K)


def _workspace(workspace, need, device):
    """The caller's workspace (a uint8 device tensor, size checked by the
    library) or a new one of ``need`` bytes."""
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor")
    _on_device("workspace", workspace)
    if workspace.device != device:
        raise ValueError("workspace must be on the device of the activations")
    return workspace


class QWeight:
    """A quantized expert tensor ``[E, rows, cols]``: packed codes plus scales.

    NF4: ``qdata`` uint8 ``[E, rows, cols/2]``, ``scales`` fp32 absmax
    ``[E, rows*cols/64]``.  int8: ``qdata`` int8 ``[E, rows, cols]``,
    ``scales`` fp32 ``[E, rows]``.  NF4 with double-quantized absmax: NF4
    ``qdata``, ``scale_codes`` uint8 ``[E, rows*cols/64]`` and ``scales``
    fp32 group scales ``[E, ceil(rows*cols/64 / 256)]``.  Plain tensors, so
    they serialise with ``torch.save``.
    """

    def __init__(self, fmt, num_experts, rows, cols, qdata, scales, scale_codes=None):
        self.format = fmt
        self.num_experts, self.rows, self.cols = int(num_experts), int(rows), int(cols)
        self.blocksize = NF4_BLOCKSIZE if fmt in (FMT_NF4, FMT_NF4_DQ) else self.cols
        self.qdata, self.scales, self.scale_codes = qdata, scales, scale_codes

    @classmethod
    def empty(cls, fmt, num_experts, rows, cols, device):
        E, R, C = int(num_experts), int(rows), int(cols)
        codes = None
        if fmt in (FMT_NF4, FMT_NF4_DQ):
            nb = R * (C // NF4_BLOCKSIZE)
            q = torch.empty((E, R, C // 2), dtype=torch.uint8, device=device)
            if fmt == FMT_NF4:
                s = torch.empty((E, nb), dtype=torch.float32, device=device)
            else:
                s = torch.empty((E, (nb + DQ_GROUP - 1) // DQ_GROUP), dtype=torch.float32, device=device)
                codes = torch.empty((E, nb), dtype=torch.uint8, device=device)
        elif fmt == FMT_INT8_ROWWISE:
            q = torch.empty((E, R, C), dtype=torch.int8, device=device)
            s = torch.empty((E, R), dtype=torch.float32, device=device)
        else:
            raise ValueError(f"unknown format {fmt}")
        return cls(fmt, E, R, C, q, s, codes)

    @property
    def shape(self):
        return (self.num_experts, self.rows, self.cols)

    def _tensors(self):
        return [t for t in (self.qdata, self.scales, self.scale_codes) if t is not None]

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in self._tensors())

    def expert(self, e):
        """Expert ``e`` alone (E = 1), sharing storage."""
        codes = self.scale_codes[e:e + 1] if self.scale_codes is not None else None
        return QWeight(self.format, 1, self.rows, self.cols, self.qdata[e:e + 1], self.scales[e:e + 1], codes)

    def like(self, device, pin_memory=False):
        """An empty QWeight of the same format and shape on ``device`` (host
        tensors pinned when ``pin_memory``)."""
        new = [torch.empty(t.shape, dtype=t.dtype, device=device, pin_memory=pin_memory) for t in self._tensors()]
        codes = new[2] if len(new) == 3 else None
        return QWeight(self.format, self.num_experts, self.rows, self.cols, new[0], new[1], codes)

    def layout(self):
        """``[(name, shape, dtype)]`` of the tensors this format and shape need."""
        E, R, C = self.num_experts, self.rows, self.cols
        if self.format in (FMT_NF4, FMT_NF4_DQ):
            nb = R * (C // NF4_BLOCKSIZE)
            lay = [("qdata", (E, R, C // 2), torch.uint8)]
            if self.format == FMT_NF4:
                return lay + [("scales", (E, nb), torch.float32)]
            return lay + [("scales", (E, (nb + DQ_GROUP - 1) // DQ_GROUP), torch.float32),
                          ("scale_codes", (E, nb), torch.uint8)]
        if self.format == FMT_INT8_ROWWISE:
            return [("qdata", (E, R, C), torch.int8), ("scales", (E, R), torch.float32)]
        raise ValueError(f"unknown format {self.format}")

    def validate_layout(self):
        """Every tensor has exactly the size and dtype that the format and
        shape need and is contiguous.  Raises ValueError / TypeError."""
        if self.format in (FMT_NF4, FMT_NF4_DQ) and self.cols % NF4_BLOCKSIZE != 0:
            raise ValueError(f"NF4 needs cols % {NF4_BLOCKSIZE} == 0, got cols={self.cols}")
        lay = self.layout()
        if self.format != FMT_NF4_DQ and self.scale_codes is not None:
            raise ValueError("scale_codes is only used by the double-quantized NF4 format")
        for name, shape, dtype in lay:
            t = getattr(self, name)
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"QWeight.{name} must be a torch tensor")
            n = shape[0] * shape[1] * (shape[2] if len(shape) == 3 else 1)
            if t.numel() != n:
                raise ValueError(f"QWeight.{name} must hold {shape} ({n} elements), got {tuple(t.shape)}")
            if t.dtype != dtype:
                raise TypeError(f"QWeight.{name} must be {dtype}, got {t.dtype}")
            if not t.is_contiguous():
                raise ValueError(f"QWeight.{name} must be contiguous")
        return self

    def validate(self, allow_host=False):
        """validate_layout(), and every tensor on one device: a CUDA device,
        or pinned host memory when ``allow_host``."""
        self.validate_layout()
        ts = self._tensors()
        for t in ts:
            if not t.is_cuda and not (allow_host and t.device.type == "cpu" and t.is_pinned()):
                raise TypeError("QWeight tensors must be CUDA (HIP) tensors"
                                + (" or pinned host memory" if allow_host else ""))
        if len({t.device for t in ts}) > 1:
            raise ValueError("QWeight tensors on different devices")
        return self

    def _c(self, allow_host=False):
        self.validate(allow_host)
        return self._desc()

    def _desc(self):
        """The C descriptor, for a caller that has validated this QWeight."""
        codes = self.scale_codes.data_ptr() if self.scale_codes is not None else None
        return _QW(self.format, self.num_experts, self.rows, self.cols, self.blocksize,
                   self.qdata.data_ptr(), self.scales.data_ptr(), codes)


def moeq_abi_version():
    return _load().moeq_abi_version()


def moeq_status_string(status):
    return _load().moeq_status_string(int(status)).decode()


def moeq_nf4_codebook():
    buf = (ctypes.c_float * 16)()
    _check(_load().moeq_nf4_codebook(buf), "moeq_nf4_codebook")
    return [float(v) for v in buf]


def moeq_quantize_nf4(w, out=None, stream=None, double_quant=False):
    """bf16 ``[E, rows, cols]`` -> NF4 :class:`QWeight` (blocksize 64), with
    the absmax double-quantized when ``double_quant`` (or ``out`` has that
    format)."""
    if not isinstance(w, torch.Tensor) or w.dim() != 3:
        raise ValueError("w must be a [E, rows, cols] tensor")
    _dev(w, torch.bfloat16, "w")
    fmt = FMT_NF4_DQ if double_quant else FMT_NF4
    if out is not None:
        _match_qweight(out, tuple(w.shape), (FMT_NF4, FMT_NF4_DQ), "out")
        out.validate_layout()
    _on_device("moeq_quantize_nf4", w, *(out._tensors() if out is not None else []))
    q = out if out is not None else QWeight.empty(fmt, *w.shape, device=w.device)
    qc = q._c()
    _check(_load().moeq_quantize_nf4(_ptr(w), ctypes.byref(qc), _stream(stream)), "moeq_quantize_nf4")
    return q


def moeq_stream_reference(w, out):
    """Measurement reference (not part of the method): the bytes and launch
    of :func:`moeq_quantize_nf4` into the plain NF4 ``out`` with no NF4
    arithmetic; what it writes is meaningless.  Its rate is the attainable
    bandwidth for the quantize kernel's byte mix and access pattern."""
    if not isinstance(w, torch.Tensor) or w.dim() != 3:
        raise ValueError("w must be a [E, rows, cols] tensor")
    _dev(w, torch.bfloat16, "w")
    _match_qweight(out, tuple(w.shape), (FMT_NF4,), "out")
    out.validate_layout()
    _on_device("moeq_stream_reference", w, *out._tensors())
    qc = out._c()
    _check(_load().moeq_stream_reference(_ptr(w), ctypes.byref(qc), _stream(None)), "moeq_stream_reference")
    return out


def moeq_compress_absmax(src, out=None, share_codes=True, stream=None):
    """NF4 :class:`QWeight` -> the same weights with double-quantized absmax.
    With ``share_codes`` the result uses ``src.qdata`` itself; otherwise the
    packed codes are copied into ``out`` (or a new buffer)."""
    _match_qweight(src, src.shape, (FMT_NF4,), "src")
    src.validate_layout()
    if out is not None:
        _match_qweight(out, src.shape, (FMT_NF4_DQ,), "out")
        out.validate_layout()
    _on_device("moeq_compress_absmax", *src._tensors(), *(out._tensors() if out is not None else []))
    if out is None:
        out = QWeight.empty(FMT_NF4_DQ, *src.shape, device=src.qdata.device)
        if share_codes:
            out.qdata = src.qdata
    sc, oc = src._c(), out._c()
    _check(_load().moeq_compress_absmax(ctypes.byref(sc), ctypes.byref(oc), _stream(stream)),
           "moeq_compress_absmax")
    return out


def moeq_quantize_int8_rowwise(w, out=None, stream=None):
    """bf16 ``[E, rows, cols]`` -> row-wise int8 :class:`QWeight`."""
    if not isinstance(w, torch.Tensor) or w.dim() != 3:
        raise ValueError("w must be a [E, rows, cols] tensor")
    _dev(w, torch.bfloat16, "w")
    if out is not None:
        _match_qweight(out, tuple(w.shape), (FMT_INT8_ROWWISE,), "out")
        out.validate_layout()
    _on_device("moeq_quantize_int8_rowwise", w, *(out._tensors() if out is not None else []))
    q = out if out is not None else QWeight.empty(FMT_INT8_ROWWISE, *w.shape, device=w.device)
    qc = q._c()
    _check(_load().moeq_quantize_int8_rowwise(_ptr(w), ctypes.byref(qc), _stream(stream)),
           "moeq_quantize_int8_rowwise")
    return q


def moeq_dequantize(q, out=None, stream=None):
    """:class:`QWeight` -> bf16 ``[E, rows, cols]``."""
    if not isinstance(q, QWeight):
        raise TypeError("q must be a QWeight")
    q.validate_layout()
    if out is not None:
        _dev(out, torch.bfloat16, "out", q.shape)
    _on_device("moeq_dequantize", *q._tensors(), out)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.qdata.device)
    qc = q._c()
    _check(_load().moeq_dequantize(ctypes.byref(qc), _ptr(out), _stream(stream)), "moeq_dequantize")
    return out


def moeq_experts_forward_workspace_bytes(T, K, gate_up, down):
    gu, dn = gate_up._c(allow_host=True), down._c(allow_host=True)
    return int(_load().moeq_experts_forward_workspace_bytes(int(T), int(K), ctypes.byref(gu), ctypes.byref(dn)))


def moeq_experts_forward(hidden, top_k_index, top_k_weights, gate_up, down, out=None,
                         workspace=None, stream=None, stage_events=None):
    """Routed experts forward from packed storage; returns bf16 ``[T, H]``.

    ``stage_events``: optional sequence of 5 raw hipEvent_t handles (ints),
    recorded at the stage boundaries (``moeq_experts_forward_timed``).
    """
    T, H, K = _routed_inputs(hidden, top_k_index, top_k_weights)
    if out is not None:
        _dev(out, torch.bfloat16, "out", (T, H))
    wt = _forward_weights(gate_up, down, H)
    dev = _on_device("moeq_experts_forward", hidden, top_k_index, top_k_weights, out, *wt)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    gu, dn = gate_up._desc(), down._desc()  # validated by the two checks above
    lib = _load()
    need = int(lib.moeq_experts_forward_workspace_bytes(T, K, ctypes.byref(gu), ctypes.byref(dn)))
    workspace = _workspace(workspace, need, dev)
    args = (_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), T, K, ctypes.byref(gu),
            ctypes.byref(dn), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream, dev))
    if stage_events is None:
        _check(lib.moeq_experts_forward(*args), "moeq_experts_forward")
    else:
        if len(stage_events) != 5:
            raise ValueError("stage_events must hold 5 hipEvent_t handles")
        arr = (ctypes.c_void_p * 5)(*[int(e) for e in stage_events])
        _check(lib.moeq_experts_forward_timed(*args, arr), "moeq_experts_forward_timed")
    return out


def moeq_experts_forward_noalloc(hidden, top_k_index, top_k_weights, gate_up, down, out, stream=None):
    """:func:`moeq_experts_forward` into the caller's ``out`` (bf16 ``[T, H]``)
    with the library's own device scratch as workspace: the library call
    allocates nothing (for callers that cannot allocate, e.g. under graph
    capture).  Raises :class:`MoeqError` (workspace status) when the batch
    needs more than ``NOALLOC_SCRATCH_BYTES``.  Calls overlapping in time on
    one GPU share that scratch and must be serialised by the caller."""
    T, H, K = _routed_inputs(hidden, top_k_index, top_k_weights)
    _dev(out, torch.bfloat16, "out", (T, H))
    wt = _forward_weights(gate_up, down, H)
    dev = _on_device("moeq_experts_forward_noalloc", hidden, top_k_index, top_k_weights, out, *wt)
    gu, dn = gate_up._desc(), down._desc()  # validated by the two checks above
    _check(_load().moeq_experts_forward_noalloc(_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), T,
                                                K, ctypes.byref(gu), ctypes.byref(dn), _ptr(out),
                                                _stream(stream, dev)), "moeq_experts_forward_noalloc")
    return out


def moeq_experts_backward_workspace_bytes(T, K, gate_up, down):
    gu, dn = gate_up._c(allow_host=True), down._c(allow_host=True)
    return int(_load().moeq_experts_backward_workspace_bytes(int(T), int(K), ctypes.byref(gu), ctypes.byref(dn)))


def moeq_experts_backward(hidden, top_k_index, top_k_weights, gate_up, down, grad_out, grad_hidden=None,
                          grad_weights=None, workspace=None, stream=None):
    """Gradients of the experts block with respect to ``hidden`` and
    ``top_k_weights`` (packed weights frozen) for the incoming gradient
    ``grad_out`` (bf16 ``[T, H]``); returns ``(grad_hidden bf16 [T, H],
    grad_weights fp32 [T, K])``."""
    T, H, K = _routed_inputs(hidden, top_k_index, top_k_weights)
    _dev(grad_out, torch.bfloat16, "grad_out", (T, H))
    if grad_hidden is not None:
        _dev(grad_hidden, torch.bfloat16, "grad_hidden", (T, H))
    if grad_weights is not None:
        _dev(grad_weights, torch.float32, "grad_weights", (T, K))
    wt = _forward_weights(gate_up, down, H)
    dev = _on_device("moeq_experts_backward", hidden, top_k_index, top_k_weights, grad_out, grad_hidden,
                     grad_weights, *wt)
    if grad_hidden is None:
        grad_hidden = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if grad_weights is None:
        grad_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
    gu, dn = gate_up._desc(), down._desc()  # validated by the two checks above
    lib = _load()
    need = int(lib.moeq_experts_backward_workspace_bytes(T, K, ctypes.byref(gu), ctypes.byref(dn)))
    workspace = _workspace(workspace, need, dev)
    _check(lib.moeq_experts_backward(_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), T, K,
                                     ctypes.byref(gu), ctypes.byref(dn), _ptr(grad_out), _ptr(grad_hidden),
                                     _ptr(grad_weights), _ptr(workspace), workspace.numel(), _stream(stream, dev)),
           "moeq_experts_backward")
    return grad_hidden, grad_weights


def moeq_experts_forward_save(hidden, top_k_index, top_k_weights, gate_up, down, out=None, gu_saved=None,
                              workspace=None, stream=None):
    """:func:`moeq_experts_forward` that also keeps the fp32 gate and up
    pre-activations of every routed assignment for
    :func:`moeq_experts_backward_saved`; returns ``(out bf16 [T, H],
    gu_saved fp32 [T*K, 2I])`` (rows in the expert-major order of the
    routing; rows past the routed count are not written)."""
    T, H, K = _routed_inputs(hidden, top_k_index, top_k_weights)
    if out is not None:
        _dev(out, torch.bfloat16, "out", (T, H))
    wt = _forward_weights(gate_up, down, H)
    I2 = gate_up.rows
    if gu_saved is not None:
        _dev(gu_saved, torch.float32, "gu_saved", (T * K, I2))
    dev = _on_device("moeq_experts_forward_save", hidden, top_k_index, top_k_weights, out, gu_saved, *wt)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if gu_saved is None:
        gu_saved = torch.empty((T * K, I2), dtype=torch.float32, device=dev)
    gu, dn = gate_up._desc(), down._desc()  # validated by the two checks above
    lib = _load()
    need = int(lib.moeq_experts_forward_workspace_bytes(T, K, ctypes.byref(gu), ctypes.byref(dn)))
    workspace = _workspace(workspace, need, dev)
    _check(lib.moeq_experts_forward_save(_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), T, K,
                                         ctypes.byref(gu), ctypes.byref(dn), _ptr(out), _ptr(gu_saved),
                                         _ptr(workspace), workspace.numel(), _stream(stream, dev)),
           "moeq_experts_forward_save")
    return out, gu_saved


def moeq_experts_backward_saved_workspace_bytes(T, K, gate_up, down):
    gu, dn = gate_up._c(allow_host=True), down._c(allow_host=True)
    return int(_load().moeq_experts_backward_saved_workspace_bytes(int(T), int(K), ctypes.byref(gu),
                                                                   ctypes.byref(dn)))


def moeq_experts_backward_saved(top_k_index, top_k_weights, gate_up, down, gu_saved, grad_out, grad_hidden=None,
                                grad_weights=None, workspace=None, stream=None):
    """:func:`moeq_experts_backward` from the pre-activations that
    :func:`moeq_experts_forward_save` kept (``gu_saved`` fp32 ``[T*K, 2I]``),
    with no recompute of the gate_up GEMM; the same gradients bit for bit.
    Returns ``(grad_hidden bf16 [T, H], grad_weights fp32 [T, K])``."""
    if not isinstance(grad_out, torch.Tensor) or grad_out.dim() != 2:
        raise ValueError("grad_out must be a 2-D tensor")
    T, H = grad_out.shape
    _dev(grad_out, torch.bfloat16, "grad_out", (T, H))
    _dev(top_k_index, torch.int32, "top_k_index")
    if top_k_index.dim() != 2 or top_k_index.shape[0] != T:
        raise ValueError(f"top_k_index must have shape ({T}, K), got {tuple(top_k_index.shape)}")
    K = top_k_index.shape[1]
    _dev(top_k_weights, torch.float32, "top_k_weights", (T, K))
    wt = _forward_weights(gate_up, down, H)
    _dev(gu_saved, torch.float32, "gu_saved", (T * K, gate_up.rows))
    if grad_hidden is not None:
        _dev(grad_hidden, torch.bfloat16, "grad_hidden", (T, H))
    if grad_weights is not None:
        _dev(grad_weights, torch.float32, "grad_weights", (T, K))
    dev = _on_device("moeq_experts_backward_saved", top_k_index, top_k_weights, gu_saved, grad_out, grad_hidden,
                     grad_weights, *wt)
    if grad_hidden is None:
        grad_hidden = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if grad_weights is None:
        grad_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
    gu, dn = gate_up._desc(), down._desc()  # validated by the two checks above
    lib = _load()
    need = int(lib.moeq_experts_backward_saved_workspace_bytes(T, K, ctypes.byref(gu), ctypes.byref(dn)))
    workspace = _workspace(workspace, need, dev)
    _check(lib.moeq_experts_backward_saved(_ptr(top_k_index), _ptr(top_k_weights), T, K, ctypes.byref(gu),
                                           ctypes.byref(dn), _ptr(gu_saved), _ptr(grad_out), _ptr(grad_hidden),
                                           _ptr(grad_weights), _ptr(workspace), workspace.numel(),
                                           _stream(stream, dev)),
           "moeq_experts_backward_saved")
    return grad_hidden, grad_weights


def moeq_router_topk(hidden, gate, K, renormalize=False, top_k_index=None, top_k_weights=None, stream=None):
    """Router front-end: ``hidden`` bf16 ``[T, H]``, ``gate`` bf16 ``[E, H]`` ->
    ``(top_k_index int32 [T, K], top_k_weights fp32 [T, K])``."""
    if not isinstance(hidden, torch.Tensor) or hidden.dim() != 2:
        raise ValueError("hidden must be a [T, H] tensor")
    T, H = hidden.shape
    _dev(hidden, torch.bfloat16, "hidden")
    if not isinstance(gate, torch.Tensor) or gate.dim() != 2 or gate.shape[1] != H:
        raise ValueError("gate must be [E, H]")
    _dev(gate, torch.bfloat16, "gate")
    E = gate.shape[0]
    K = int(K)
    if K < 1:
        raise ValueError("K must be >= 1")
    if top_k_index is not None:
        _dev(top_k_index, torch.int32, "top_k_index", (T, K))
    if top_k_weights is not None:
        _dev(top_k_weights, torch.float32, "top_k_weights", (T, K))
    _on_device("moeq_router_topk", hidden, gate, top_k_index, top_k_weights)
    if top_k_index is None:
        top_k_index = torch.empty((T, K), dtype=torch.int32, device=hidden.device)
    if top_k_weights is None:
        top_k_weights = torch.empty((T, K), dtype=torch.float32, device=hidden.device)
    _check(_load().moeq_router_topk(_ptr(hidden), _ptr(gate), int(T), int(H), int(E), int(K),
                                    1 if renormalize else 0, _ptr(top_k_index), _ptr(top_k_weights),
                                    _stream(stream)), "moeq_router_topk")
    return top_k_index, top_k_weights


class Routing:
    """The grouping of T*K assignments by expert: ``counts`` [E],
    ``offsets`` [E+1], ``perm`` [T*K] and ``slot`` [T*K] int32 device tensors
    (as :func:`moeq_route_buckets` returns them)."""

    def __init__(self, counts, offsets, perm, slot):
        self.counts, self.offsets, self.perm, self.slot = counts, offsets, perm, slot

    def __iter__(self):
        return iter((self.counts, self.offsets, self.perm, self.slot))


def moeq_router_route_workspace_bytes(T, H, E, K):
    """Workspace bytes :func:`moeq_router_route` needs for T tokens, hidden
    size H, E experts and top-K."""
    return int(_load().moeq_router_route_workspace_bytes(int(T), int(H), int(E), int(K)))


def moeq_router_route(hidden, gate, K, renormalize=False, workspace=None, stream=None):
    """Router front-end fused with the routing stage: ``hidden`` bf16
    ``[T, H]``, ``gate`` bf16 ``[E, H]`` -> ``(top_k_index int32 [T, K],
    top_k_weights fp32 [T, K], Routing)``; the same as
    :func:`moeq_router_topk` then :func:`moeq_route_buckets`."""
    if not isinstance(hidden, torch.Tensor) or hidden.dim() != 2:
        raise ValueError("hidden must be a [T, H] tensor")
    T, H = hidden.shape
    _dev(hidden, torch.bfloat16, "hidden")
    if not isinstance(gate, torch.Tensor) or gate.dim() != 2 or gate.shape[1] != H:
        raise ValueError("gate must be [E, H]")
    _dev(gate, torch.bfloat16, "gate")
    _on_device("moeq_router_route", hidden, gate)
    E, K = int(gate.shape[0]), int(K)
    if K < 1:
        raise ValueError("K must be >= 1")
    dev = hidden.device
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    wts = torch.empty((T, K), dtype=torch.float32, device=dev)
    r = Routing(torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
                torch.empty(T * K, dtype=torch.int32, device=dev), torch.empty(T * K, dtype=torch.int32, device=dev))
    lib = _load()
    need = int(lib.moeq_router_route_workspace_bytes(int(T), int(H), E, K))
    workspace = _workspace(workspace, need, dev)
    _check(lib.moeq_router_route(_ptr(hidden), _ptr(gate), int(T), int(H), E, K, 1 if renormalize else 0,
                                 _ptr(idx), _ptr(wts), _ptr(r.counts), _ptr(r.offsets), _ptr(r.perm),
                                 _ptr(r.slot), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moeq_router_route")
    return idx, wts, r


def moeq_experts_forward_routed(hidden, top_k_index, top_k_weights, gate_up, down, routing, out=None,
                                workspace=None, stream=None):
    """:func:`moeq_experts_forward` with ``routing`` (a :class:`Routing` of
    this top_k_index) supplied, so the routing stage is skipped."""
    T, H, K = _routed_inputs(hidden, top_k_index, top_k_weights)
    if not isinstance(routing, Routing):
        raise TypeError("routing must be a Routing")
    E = gate_up.num_experts if isinstance(gate_up, QWeight) else 0
    _dev(routing.offsets, torch.int32, "routing.offsets", (E + 1,))
    _dev(routing.perm, torch.int32, "routing.perm", (T * K,))
    _dev(routing.slot, torch.int32, "routing.slot", (T * K,))
    if out is not None:
        _dev(out, torch.bfloat16, "out", (T, H))
    wt = _forward_weights(gate_up, down, H)
    dev = _on_device("moeq_experts_forward_routed", hidden, top_k_index, top_k_weights, out, routing.offsets,
                     routing.perm, routing.slot, *wt)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    gu, dn = gate_up._desc(), down._desc()  # validated by the two checks above
    lib = _load()
    need = int(lib.moeq_experts_forward_workspace_bytes(T, K, ctypes.byref(gu), ctypes.byref(dn)))
    workspace = _workspace(workspace, need, dev)
    _check(lib.moeq_experts_forward_routed(_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), T, K,
                                           ctypes.byref(gu), ctypes.byref(dn), _ptr(routing.offsets),
                                           _ptr(routing.perm), _ptr(routing.slot), _ptr(out), _ptr(workspace),
                                           workspace.numel(), _stream(stream, dev)), "moeq_experts_forward_routed")
    return out


def moeq_qweight_copy_async(src, dst, stream=None):
    """Asynchronous copy of a packed tensor between pinned host and device
    memory (either direction) on ``stream`` (default: torch's current)."""
    for name, q in (("source", src), ("destination", dst)):
        if not isinstance(q, QWeight):
            raise TypeError(f"{name} must be a QWeight")
        for t in q._tensors():
            if t.device.type == "cpu" and not t.is_pinned():
                raise ValueError(f"host {name} must be pinned")
    s, d = src._c(allow_host=True), dst._c(allow_host=True)
    _check(_load().moeq_qweight_copy_async(ctypes.byref(s), ctypes.byref(d), _stream(stream)),
           "moeq_qweight_copy_async")
    return dst


def moeq_route_workspace_bytes(T, K, E):
    return int(_load().moeq_route_workspace_bytes(int(T), int(K), int(E)))


def moeq_route_buckets(top_k_index, num_experts, workspace=None, stream=None):
    """-> ``(counts [E], offsets [E+1], perm [T*K], slot [T*K])`` int32 device tensors.

    ``perm`` entries past ``offsets[E]`` (unrouted assignments) are -1 here.
    """
    if not isinstance(top_k_index, torch.Tensor) or top_k_index.dim() != 2:
        raise ValueError("top_k_index must be a [T, K] tensor")
    _dev(top_k_index, torch.int32, "top_k_index")
    _on_device("moeq_route_buckets", top_k_index)
    T, K = top_k_index.shape
    E = int(num_experts)
    dev = top_k_index.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.full((T * K,), -1, dtype=torch.int32, device=dev)
    slot = torch.empty(T * K, dtype=torch.int32, device=dev)
    lib = _load()
    need = int(lib.moeq_route_workspace_bytes(int(T), int(K), E))
    workspace = _workspace(workspace, need, dev)
    _check(lib.moeq_route_buckets(_ptr(top_k_index), int(T), int(K), E, _ptr(counts), _ptr(offsets),
                                  _ptr(perm), _ptr(slot), _ptr(workspace), workspace.numel(),
                                  _stream(stream)), "moeq_route_buckets")
    return counts, offsets, perm, slot
