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
    "moeq_qweight_copy_async", "FMT_NF4_DQ", "DQ_GROUP", "moeq_compress_absmax",
]

FMT_NF4 = 1
FMT_INT8_ROWWISE = 2
FMT_NF4_DQ = 3
NF4_BLOCKSIZE = 64
DQ_GROUP = 256
ABI_VERSION = 2

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


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


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

    def _c(self):
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
    _dev(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [E, rows, cols]")
    fmt = FMT_NF4_DQ if double_quant else FMT_NF4
    q = out if out is not None else QWeight.empty(fmt, *w.shape, device=w.device)
    qc = q._c()
    _check(_load().moeq_quantize_nf4(_ptr(w), ctypes.byref(qc), _stream(stream)), "moeq_quantize_nf4")
    return q


def moeq_compress_absmax(src, out=None, share_codes=True, stream=None):
    """NF4 :class:`QWeight` -> the same weights with double-quantized absmax.
    With ``share_codes`` the result uses ``src.qdata`` itself; otherwise the
    packed codes are copied into ``out`` (or a new buffer)."""
    if src.format != FMT_NF4:
        raise ValueError("moeq_compress_absmax takes an NF4 QWeight")
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
    _dev(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [E, rows, cols]")
    q = out if out is not None else QWeight.empty(FMT_INT8_ROWWISE, *w.shape, device=w.device)
    qc = q._c()
    _check(_load().moeq_quantize_int8_rowwise(_ptr(w), ctypes.byref(qc), _stream(stream)),
           "moeq_quantize_int8_rowwise")
    return q


def moeq_dequantize(q, out=None, stream=None):
    """:class:`QWeight` -> bf16 ``[E, rows, cols]``."""
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.qdata.device)
    _dev(out, torch.bfloat16, "out")
    qc = q._c()
    _check(_load().moeq_dequantize(ctypes.byref(qc), _ptr(out), _stream(stream)), "moeq_dequantize")
    return out


def moeq_experts_forward_workspace_bytes(T, K, gate_up, down):
    gu, dn = gate_up._c(), down._c()
    return int(_load().moeq_experts_forward_workspace_bytes(int(T), int(K), ctypes.byref(gu), ctypes.byref(dn)))


def moeq_experts_forward(hidden, top_k_index, top_k_weights, gate_up, down, out=None,
                         workspace=None, stream=None, stage_events=None):
    """Routed experts forward from packed storage; returns bf16 ``[T, H]``.

    ``stage_events``: optional sequence of 5 raw hipEvent_t handles (ints),
    recorded at the stage boundaries (``moeq_experts_forward_timed``).
    """
    _dev(hidden, torch.bfloat16, "hidden")
    _dev(top_k_index, torch.int32, "top_k_index")
    _dev(top_k_weights, torch.float32, "top_k_weights")
    T, H = hidden.shape
    K = top_k_index.shape[1]
    if tuple(top_k_index.shape) != (T, K) or tuple(top_k_weights.shape) != (T, K):
        raise ValueError("top_k_index and top_k_weights must both be [T, K]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    _dev(out, torch.bfloat16, "out")
    if out.shape[0] != T or out.shape[1] != gate_up.cols or H != gate_up.cols:
        raise ValueError("hidden / out width must equal gate_up cols (H)")
    gu, dn = gate_up._c(), down._c()
    lib = _load()
    need = int(lib.moeq_experts_forward_workspace_bytes(int(T), int(K), ctypes.byref(gu), ctypes.byref(dn)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    args = (_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), int(T), int(K), ctypes.byref(gu),
            ctypes.byref(dn), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    if stage_events is None:
        _check(lib.moeq_experts_forward(*args), "moeq_experts_forward")
    else:
        if len(stage_events) != 5:
            raise ValueError("stage_events must hold 5 hipEvent_t handles")
        arr = (ctypes.c_void_p * 5)(*[int(e) for e in stage_events])
        _check(lib.moeq_experts_forward_timed(*args, arr), "moeq_experts_forward_timed")
    return out


def moeq_experts_backward_workspace_bytes(T, K, gate_up, down):
    gu, dn = gate_up._c(), down._c()
    return int(_load().moeq_experts_backward_workspace_bytes(int(T), int(K), ctypes.byref(gu), ctypes.byref(dn)))


def moeq_experts_backward(hidden, top_k_index, top_k_weights, gate_up, down, grad_out, grad_hidden=None,
                          grad_weights=None, workspace=None, stream=None):
    """Gradients of the experts block with respect to ``hidden`` and
    ``top_k_weights`` (packed weights frozen) for the incoming gradient
    ``grad_out`` (bf16 ``[T, H]``); returns ``(grad_hidden bf16 [T, H],
    grad_weights fp32 [T, K])``."""
    _dev(hidden, torch.bfloat16, "hidden")
    _dev(top_k_index, torch.int32, "top_k_index")
    _dev(top_k_weights, torch.float32, "top_k_weights")
    _dev(grad_out, torch.bfloat16, "grad_out")
    T, H = hidden.shape
    K = top_k_index.shape[1]
    if tuple(top_k_index.shape) != (T, K) or tuple(top_k_weights.shape) != (T, K):
        raise ValueError("top_k_index and top_k_weights must both be [T, K]")
    if tuple(grad_out.shape) != (T, H) or H != gate_up.cols:
        raise ValueError("grad_out must be [T, H] with H = gate_up cols")
    if grad_hidden is None:
        grad_hidden = torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    if grad_weights is None:
        grad_weights = torch.empty((T, K), dtype=torch.float32, device=hidden.device)
    _dev(grad_hidden, torch.bfloat16, "grad_hidden")
    _dev(grad_weights, torch.float32, "grad_weights")
    gu, dn = gate_up._c(), down._c()
    lib = _load()
    need = int(lib.moeq_experts_backward_workspace_bytes(int(T), int(K), ctypes.byref(gu), ctypes.byref(dn)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    _check(lib.moeq_experts_backward(_ptr(hidden), _ptr(top_k_index), _ptr(top_k_weights), int(T), int(K),
                                     ctypes.byref(gu), ctypes.byref(dn), _ptr(grad_out), _ptr(grad_hidden),
                                     _ptr(grad_weights), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moeq_experts_backward")
    return grad_hidden, grad_weights


def moeq_router_topk(hidden, gate, K, renormalize=False, top_k_index=None, top_k_weights=None, stream=None):
    """Router front-end: ``hidden`` bf16 ``[T, H]``, ``gate`` bf16 ``[E, H]`` ->
    ``(top_k_index int32 [T, K], top_k_weights fp32 [T, K])``."""
    _dev(hidden, torch.bfloat16, "hidden")
    _dev(gate, torch.bfloat16, "gate")
    T, H = hidden.shape
    E = gate.shape[0]
    if gate.dim() != 2 or gate.shape[1] != H:
        raise ValueError("gate must be [E, H]")
    if top_k_index is None:
        top_k_index = torch.empty((T, int(K)), dtype=torch.int32, device=hidden.device)
    if top_k_weights is None:
        top_k_weights = torch.empty((T, int(K)), dtype=torch.float32, device=hidden.device)
    _dev(top_k_index, torch.int32, "top_k_index")
    _dev(top_k_weights, torch.float32, "top_k_weights")
    _check(_load().moeq_router_topk(_ptr(hidden), _ptr(gate), int(T), int(H), int(E), int(K),
                                    1 if renormalize else 0, _ptr(top_k_index), _ptr(top_k_weights),
                                    _stream(stream)), "moeq_router_topk")
    return top_k_index, top_k_weights


def moeq_qweight_copy_async(src, dst, stream=None):
    """Asynchronous copy of a packed tensor between pinned host and device
    memory (either direction) on ``stream`` (default: torch's current)."""
    for name, q in (("source", src), ("destination", dst)):
        for t in q._tensors():
            if t.device.type == "cpu" and not t.is_pinned():
                raise ValueError(f"host {name} must be pinned")
    s, d = src._c(), dst._c()
    _check(_load().moeq_qweight_copy_async(ctypes.byref(s), ctypes.byref(d), _stream(stream)),
           "moeq_qweight_copy_async")
    return dst


def moeq_route_workspace_bytes(T, K, E):
    return int(_load().moeq_route_workspace_bytes(int(T), int(K), int(E)))


def moeq_route_buckets(top_k_index, num_experts, workspace=None, stream=None):
    """-> ``(counts [E], offsets [E+1], perm [T*K], slot [T*K])`` int32 device tensors.

    ``perm`` entries past ``offsets[E]`` (unrouted assignments) are -1 here.
    """
    _dev(top_k_index, torch.int32, "top_k_index")
    T, K = top_k_index.shape
    E = int(num_experts)
    dev = top_k_index.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.full((T * K,), -1, dtype=torch.int32, device=dev)
    slot = torch.empty(T * K, dtype=torch.int32, device=dev)
    lib = _load()
    need = int(lib.moeq_route_workspace_bytes(int(T), int(K), E))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.moeq_route_buckets(_ptr(top_k_index), int(T), int(K), E, _ptr(counts), _ptr(offsets),
                                  _ptr(perm), _ptr(slot), _ptr(workspace), workspace.numel(),
                                  _stream(stream)), "moeq_route_buckets")
    return counts, offsets, perm, slot
