"""MI355X (gfx950) factorized linear layer: Y = (X . A) . B.

Thin ctypes binding over the C-ABI library ``liblr_linear.so`` (declared in
include/lr_linear.h).  PyTorch provides device memory and the stream; every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing, or no gfx950 GPU is present, the calls
raise.

    lin = LowRankLinear(A, B, max_M=16)     # A [K x r], B [r x N] bf16 cuda
    Y = lin(X)                               # X [M x K] bf16 cuda -> Y [M x N]
    Yg, Yu = mlp_packed(gate, up, X)         # gate/up pair sharing X
    Yq, Yk, Yv = group_run([q, k, v], X)     # up to four projections sharing X
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblr_linear.so")

LR_OK = 0
LR_ERR_INVALID_ARG = 1
LR_ERR_UNSUPPORTED = 2
LR_ERR_OUT_OF_MEMORY = 3
LR_ERR_HIP = 4

LR_FLAG_NONE = 0
LR_FLAG_FORCE_DECODE = 1
LR_FLAG_FORCE_PREFILL = 2
LR_FLAG_DECODE_STREAMING = 4
LR_FLAG_PREFILL_TWO_WAVE = 8
LR_FLAG_PREFILL_ONE_WAVE = 16
LR_FLAG_DENSE = 32
LR_FLAG_FACTORED = 64
LR_FLAG_DECODE_SPLIT = 128
LR_FLAG_DECODE_RESIDENT = 256
LR_FLAG_DECODE_XCD = 512
LR_FLAG_TEST_STALL = 1 << 30
LR_DECODE_MAX_M = 16
LR_GROUP_MAX = 4

EXPORTED_SYMBOLS = (
    "lr_linear_create",
    "lr_linear_run",
    "lr_mlp_packed_run",
    "lr_group_run",
    "lr_linear_destroy",
    "lr_status_str",
    "lr_last_error",
    "lr_linear_describe",
    "lr_linear_workspace_bytes",
    "lr_linear_status",
    "lr_decode_noalloc",
    "lr_gac_select",
)


class LRError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _STATUS_NAMES.get(status, status), detail))


_STATUS_NAMES = {0: "LR_OK", 1: "LR_ERR_INVALID_ARG", 2: "LR_ERR_UNSUPPORTED",
                 3: "LR_ERR_OUT_OF_MEMORY", 4: "LR_ERR_HIP"}

_lib = None
_lib_lock = threading.Lock()


def load_library(path: str | None = None):
    """Load liblr_linear.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = path or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError("HIP library %s is missing: build it with "
                               "`python -m rank_linear_layer_amd.build` (needs hipcc, gfx950)" % path)
        lib = ctypes.CDLL(path)
        vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        lib.lr_linear_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, vp, vp, i64, u32]
        lib.lr_linear_create.restype = ctypes.c_int
        lib.lr_linear_run.argtypes = [vp, vp, vp, i64, vp]
        lib.lr_linear_run.restype = ctypes.c_int
        lib.lr_mlp_packed_run.argtypes = [vp, vp, vp, vp, vp, i64, vp]
        lib.lr_mlp_packed_run.restype = ctypes.c_int
        lib.lr_group_run.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.POINTER(vp), i64, vp]
        lib.lr_group_run.restype = ctypes.c_int
        lib.lr_linear_destroy.argtypes = [vp]
        lib.lr_linear_destroy.restype = None
        lib.lr_status_str.argtypes = [ctypes.c_int]
        lib.lr_status_str.restype = ctypes.c_char_p
        lib.lr_last_error.argtypes = []
        lib.lr_last_error.restype = ctypes.c_char_p
        lib.lr_linear_describe.argtypes = [vp, ctypes.c_char_p, i64]
        lib.lr_linear_describe.restype = ctypes.c_int
        lib.lr_linear_workspace_bytes.argtypes = [vp]
        lib.lr_linear_workspace_bytes.restype = i64
        lib.lr_linear_status.argtypes = [vp]
        lib.lr_linear_status.restype = ctypes.c_int
        lib.lr_decode_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]
        lib.lr_decode_noalloc.restype = ctypes.c_int
        P = ctypes.POINTER
        lib.lr_gac_select.argtypes = [ctypes.c_int, P(ctypes.c_double), P(i64), P(ctypes.c_double),
                                      P(ctypes.c_int), P(i64), i64, i64, P(i64), P(ctypes.c_double)]
        lib.lr_gac_select.restype = ctypes.c_int
        _lib = lib
        return lib


def _check(status: int, where: str):
    if status != LR_OK:
        detail = load_library().lr_last_error().decode(errors="replace")
        raise LRError(status, where, detail)


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _require_bf16_cuda(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 2-D tensor" % name)


class LowRankLinear:
    """One factorized projection: Y = (X . A) . B with A [K x r], B [r x N].

    A and B are borrowed (the object keeps references); the library owns a
    workspace sized for ``max_M`` rows of X.  Calls are asynchronous on the
    current torch stream; do not use one object from two streams at once.
    """

    def __init__(self, A, B, max_M: int, flags: int = LR_FLAG_NONE):
        _require_bf16_cuda(A, "A")
        _require_bf16_cuda(B, "B")
        if A.shape[1] != B.shape[0]:
            raise ValueError("A is %s but B is %s: inner ranks differ" % (tuple(A.shape), tuple(B.shape)))
        if A.device != B.device:
            raise ValueError("A and B live on different devices")
        self._lib = load_library()
        self.A, self.B = A, B
        self.K, self.r = A.shape
        self.N = B.shape[1]
        self.max_M = int(max_M)
        self.flags = int(flags)
        self.device = A.device
        h = ctypes.c_void_p()
        import torch
        with torch.cuda.device(self.device):
            st = self._lib.lr_linear_create(ctypes.byref(h), self.K, self.r, self.N,
                                            ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                            self.max_M, self.flags)
        _check(st, "lr_linear_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        _check(self._lib.lr_linear_describe(self._h, buf, 512), "lr_linear_describe")
        return buf.value.decode()

    def workspace_bytes(self) -> int:
        return int(self._lib.lr_linear_workspace_bytes(self._h))

    def status(self) -> int:
        """lr_linear_status: LR_ERR_HIP (reported once) if a decode launch of
        this handle gave up waiting for another of its workgroups, else
        LR_OK.  Synchronize the stream first to include launches in flight."""
        return int(self._lib.lr_linear_status(self._h))

    def __call__(self, X, out=None, stream=None):
        import torch
        _require_bf16_cuda(X, "X")
        if X.shape[1] != self.K:
            raise ValueError("X has %d columns, expected K=%d" % (X.shape[1], self.K))
        if X.device != self.device:
            raise ValueError("X is on %s, factors on %s" % (X.device, self.device))
        M = X.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.bfloat16, device=self.device)
        else:
            _require_bf16_cuda(out, "out")
            if tuple(out.shape) != (M, self.N):
                raise ValueError("out must be [%d x %d]" % (M, self.N))
        st = self._lib.lr_linear_run(self._h, ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                     M, _stream_ptr(stream))
        _check(st, "lr_linear_run")
        return out

    def close(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.lr_linear_destroy(h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _outputs(projs, X, outs):
    import torch
    M = X.shape[0]
    if outs is None:
        outs = [None] * len(projs)
    if len(outs) != len(projs):
        raise ValueError("%d outputs for %d projections" % (len(outs), len(projs)))
    res = []
    for p, o in zip(projs, outs):
        if o is None:
            o = torch.empty((M, p.N), dtype=torch.bfloat16, device=X.device)
        else:
            _require_bf16_cuda(o, "out")
            if tuple(o.shape) != (M, p.N):
                raise ValueError("out must be [%d x %d]" % (M, p.N))
        res.append(o)
    return res


def mlp_packed(gate: LowRankLinear, up: LowRankLinear, X, out_gate=None, out_up=None, stream=None):
    """Y_gate = (X.A_g).B_g and Y_up = (X.A_u).B_u in one pass over X."""
    _require_bf16_cuda(X, "X")
    out_gate, out_up = _outputs([gate, up], X, [out_gate, out_up])
    st = load_library().lr_mlp_packed_run(gate.handle, up.handle, ctypes.c_void_p(X.data_ptr()),
                                          ctypes.c_void_p(out_gate.data_ptr()), ctypes.c_void_p(out_up.data_ptr()),
                                          X.shape[0], _stream_ptr(stream))
    _check(st, "lr_mlp_packed_run")
    return out_gate, out_up


def group_run(projs, X, outs=None, stream=None):
    """Ys[i] = (X.A_i).B_i for up to LR_GROUP_MAX projections sharing X,
    in shared launches (lr_group_run)."""
    _require_bf16_cuda(X, "X")
    projs = list(projs)
    outs = _outputs(projs, X, outs)
    n = len(projs)
    hs = (ctypes.c_void_p * max(n, 1))(*[p.handle.value for p in projs])
    ys = (ctypes.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    st = load_library().lr_group_run(hs, n, ctypes.c_void_p(X.data_ptr()), ys, X.shape[0], _stream_ptr(stream))
    _check(st, "lr_group_run")
    return outs


def decode_noalloc(X, A, B, out, status=None, stream=None):
    """Y = (X.A).B for M <= 16 through lr_decode_noalloc: no handle and no
    allocation inside the library (the caller passes every buffer).
    `status`: optional int32 GPU tensor of one element that a wait which
    gave up sets to 1."""
    for t, name in ((X, "X"), (A, "A"), (B, "B"), (out, "out")):
        _require_bf16_cuda(t, name)
    M, K = X.shape
    if A.shape[0] != K or B.shape[0] != A.shape[1] or tuple(out.shape) != (M, B.shape[1]):
        raise ValueError("shapes X %s, A %s, B %s, out %s do not chain" % (tuple(X.shape), tuple(A.shape),
                                                                            tuple(B.shape), tuple(out.shape)))
    st_ptr = None
    if status is not None:
        if not status.is_cuda or status.element_size() != 4 or status.numel() < 1:
            raise ValueError("status must be a GPU tensor of 32-bit words")
        st_ptr = ctypes.c_void_p(status.data_ptr())
    st = load_library().lr_decode_noalloc(ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(A.data_ptr()),
                                          ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                          M, K, A.shape[1], B.shape[1], st_ptr, _stream_ptr(stream))
    _check(st, "lr_decode_noalloc")
    return out


def status_name(status: int) -> str:
    return load_library().lr_status_str(status).decode()
