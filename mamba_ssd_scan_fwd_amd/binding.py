"""ctypes binding of libssd.so: argument marshalling only.

PyTorch provides device memory and the current stream; every step of the
computation runs in the library's HIP kernels. If the library has not been
built, every call raises -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "SSDError",
    "SSDDesc",
    "lib_path",
    "load_library",
    "make_desc",
    "status_string",
    "effective_chunk_size",
    "workspace_bytes",
    "workspace_bytes_varlen",
    "workspace_status",
    "workspace_status_varlen",
    "forward",
    "forward_noalloc",
    "chunk_cumsum",
    "chunk_state",
    "cumsum_chunk_state",
    "state_passing",
    "chunk_scan",
    "decode_step",
    "forward_varlen",
    "conv1d_split",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))

# Every symbol include/ssd.h declares.
EXPORTED_SYMBOLS = (
    "ssd_status_string",
    "ssd_effective_chunk_size",
    "ssd_workspace_bytes",
    "ssd_forward",
    "ssd_forward_fused",
    "ssd_forward_split",
    "ssd_workspace_status",
    "ssd_forward_noalloc",
    "ssd_chunk_cumsum",
    "ssd_chunk_state",
    "ssd_cumsum_chunk_state",
    "ssd_state_passing",
    "ssd_chunk_scan",
    "ssd_decode_step",
    "ssd_workspace_bytes_varlen",
    "ssd_forward_varlen",
    "ssd_workspace_status_varlen",
    "ssd_conv1d_split",
)

SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class SSDDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("ngroups", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("dt_bias", ctypes.c_void_p),
        ("dt_softplus", ctypes.c_int32),
        ("dt_clamp", ctypes.c_int32),
        ("dt_min", ctypes.c_float),
        ("dt_max", ctypes.c_float),
    ]


def lib_path() -> str:
    return os.environ.get("SSD_LIB", os.path.join(_HERE, "libssd.so"))


_lib = None
_lock = threading.Lock()


def load_library():
    """Load libssd.so once. Raises if it is missing: build it first with
    ``python -m mamba_ssd_scan_fwd_amd.build``."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"libssd.so not found at {path}; build it with `python -m mamba_ssd_scan_fwd_amd.build`"
            )
        lib = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(SSDDesc)
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_effective_chunk_size.argtypes = [dp, ctypes.POINTER(i32)]
        lib.ssd_effective_chunk_size.restype = ctypes.c_int
        lib.ssd_workspace_bytes.argtypes = [dp, ctypes.POINTER(sz)]
        lib.ssd_workspace_bytes.restype = ctypes.c_int
        lib.ssd_forward.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ssd_forward.restype = ctypes.c_int
        lib.ssd_forward_fused.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ssd_forward_fused.restype = ctypes.c_int
        lib.ssd_forward_split.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ssd_forward_split.restype = ctypes.c_int
        lib.ssd_workspace_status.argtypes = [dp, vp, sz, vp, ctypes.POINTER(ctypes.c_uint32),
                                             ctypes.POINTER(ctypes.c_uint32)]
        lib.ssd_workspace_status.restype = ctypes.c_int
        lib.ssd_workspace_status_varlen.argtypes = [dp, ctypes.c_int64, vp, sz, vp, ctypes.POINTER(ctypes.c_uint32),
                                                    ctypes.POINTER(ctypes.c_uint32)]
        lib.ssd_workspace_status_varlen.restype = ctypes.c_int
        lib.ssd_forward_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.ssd_forward_noalloc.restype = ctypes.c_int
        lib.ssd_chunk_cumsum.argtypes = [dp, vp, vp, vp, vp, vp]
        lib.ssd_chunk_cumsum.restype = ctypes.c_int
        lib.ssd_chunk_state.argtypes = [dp, vp, vp, vp, vp, vp, vp]
        lib.ssd_chunk_state.restype = ctypes.c_int
        lib.ssd_cumsum_chunk_state.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.ssd_cumsum_chunk_state.restype = ctypes.c_int
        lib.ssd_state_passing.argtypes = [dp, vp, vp, vp, vp, vp]
        lib.ssd_state_passing.restype = ctypes.c_int
        lib.ssd_chunk_scan.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.ssd_chunk_scan.restype = ctypes.c_int
        lib.ssd_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.ssd_decode_step.restype = ctypes.c_int
        lib.ssd_workspace_bytes_varlen.argtypes = [dp, ctypes.c_int64, ctypes.POINTER(sz)]
        lib.ssd_workspace_bytes_varlen.restype = ctypes.c_int
        lib.ssd_forward_varlen.argtypes = [dp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ssd_forward_varlen.restype = ctypes.c_int
        lib.ssd_conv1d_split.argtypes = [dp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        lib.ssd_conv1d_split.restype = ctypes.c_int
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise SSDError(status, where)


def make_desc(batch, seqlen, nheads, headdim, dstate, ngroups, io_dtype, chunk_size=0, *,
              dt_bias=None, dt_softplus=False, dt_limit=None) -> SSDDesc:
    """The C descriptor. dt preprocessing: ``dt_bias`` (fp32 [H] device
    tensor) is added to dt, ``dt_softplus`` applies log(1 + e^z), and
    ``dt_limit = (lo, hi)`` clamps the result."""
    if isinstance(io_dtype, torch.dtype):
        io = {torch.float32: SSD_DTYPE_F32, torch.bfloat16: SSD_DTYPE_BF16}.get(io_dtype)
        if io is None:
            raise TypeError(f"unsupported io dtype {io_dtype}")
    elif io_dtype in ("fp32", "f32", "float32"):
        io = SSD_DTYPE_F32
    elif io_dtype in ("bf16", "bfloat16"):
        io = SSD_DTYPE_BF16
    else:
        io = int(io_dtype)
    d = SSDDesc(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(ngroups), io,
                int(chunk_size))
    if dt_bias is not None:
        d.dt_bias = dt_bias.data_ptr()
    d.dt_softplus = 1 if dt_softplus else 0
    if dt_limit is not None:
        d.dt_clamp = 1
        d.dt_min, d.dt_max = float(dt_limit[0]), float(dt_limit[1])
    return d


def effective_chunk_size(desc: SSDDesc) -> int:
    q = ctypes.c_int32(0)
    _check(load_library().ssd_effective_chunk_size(ctypes.byref(desc), ctypes.byref(q)),
           "ssd_effective_chunk_size")
    return int(q.value)


def workspace_bytes(desc: SSDDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "ssd_workspace_bytes")
    return int(n.value)


def workspace_bytes_varlen(desc: SSDDesc, num_seqs: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_workspace_bytes_varlen(ctypes.byref(desc), ctypes.c_int64(num_seqs), ctypes.byref(n)),
           "ssd_workspace_bytes_varlen")
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, device=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _desc_from(x, B, chunk_size, dt_pre=None):
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return make_desc(bsz, L, H, P, N, G, x.dtype, chunk_size, **_dt_kw(dt_pre, H, x.device))


def _dt_kw(dt_pre, H, dev):
    """dt_pre: None or dict(bias=tensor|None, softplus=bool, limit=(lo, hi)|None)."""
    if not dt_pre:
        return {}
    bias = dt_pre.get("bias")
    if bias is not None:
        _need(bias, "dt bias", torch.float32, dev, (H,))
    return dict(dt_bias=bias, dt_softplus=bool(dt_pre.get("softplus", False)), dt_limit=dt_pre.get("limit"))


def forward(x, dt, A, B, C, D=None, init_state=None, *, chunk_size: int = 0,
            return_final_state: bool = True, y=None, final_state=None, workspace=None,
            library_workspace: bool = False, dt_pre=None, fused: bool = False, split: bool = False,
            stream=None):
    """SSD forward pass on the GPU. Returns (y, final_state or None).

    x [b, L, H, P] and B, C [b, L, G, N] in fp32 or bf16 (all the same);
    dt [b, L, H], A [H], D [H] (optional) and init_state [b, H, P, N]
    (optional) in fp32. ``final_state`` may be passed as ``init_state`` for an
    in-place state update. With ``library_workspace=True`` the library
    allocates its workspace itself, in stream order. ``dt_pre`` asks for the
    dt preprocessing: dict(bias=[H] fp32 tensor, softplus=True, limit=(lo, hi)).
    ``fused=True`` calls ssd_forward_fused (the one-pass kernel; raises where
    the shape is not supported by it) and ``split=True`` ssd_forward_split
    (always the separate steps) instead of ssd_forward, which picks one of
    the two paths by shape.
    """
    if fused and split:
        raise ValueError("fused and split exclude each other")
    dev = x.device
    _need(x, "x", device=dev)
    io = x.dtype
    bsz, L, H, P = x.shape
    _need(B, "B", io, dev)
    G, N = B.shape[2], B.shape[3]
    _need(C, "C", io, dev, B.shape)
    _need(dt, "dt", torch.float32, dev, (bsz, L, H))
    _need(A, "A", torch.float32, dev, (H,))
    if D is not None:
        _need(D, "D", torch.float32, dev, (H,))
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, dev, (bsz, H, P, N))
    desc = _desc_from(x, B, chunk_size, dt_pre)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", io, dev, x.shape)
    if final_state is None and return_final_state:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, dev, (bsz, H, P, N))
    nws = workspace_bytes(desc)
    if library_workspace:
        workspace, wsize = None, 0
    elif workspace is None:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
        wsize = nws
    else:
        wsize = workspace.numel() * workspace.element_size()
        if wsize < nws:
            raise ValueError(f"workspace needs {nws} bytes")
    name = "ssd_forward_fused" if fused else "ssd_forward_split" if split else "ssd_forward"
    st = getattr(load_library(), name)(
        ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
        _ptr(y), _ptr(final_state), _ptr(workspace), ctypes.c_size_t(wsize), _stream(stream, dev))
    _check(st, name)
    return y, final_state


def forward_noalloc(x, dt, A, B, C, D=None, init_state=None, *, chunk_size: int = 0,
                    return_final_state: bool = True, y=None, final_state=None, dt_pre=None, stream=None):
    """ssd_forward_noalloc: the forward pass of ``forward`` with the
    workspace taken from the library's fixed per-GPU scratch (256 MiB); the
    library allocates nothing. ``y`` and ``final_state`` are allocated here
    when not given (pass them to keep the call allocation-free end to end).
    Returns (y, final_state or None)."""
    dev = x.device
    _need(x, "x", device=dev)
    io = x.dtype
    bsz, L, H, P = x.shape
    _need(B, "B", io, dev)
    G, N = B.shape[2], B.shape[3]
    _need(C, "C", io, dev, B.shape)
    _need(dt, "dt", torch.float32, dev, (bsz, L, H))
    _need(A, "A", torch.float32, dev, (H,))
    if D is not None:
        _need(D, "D", torch.float32, dev, (H,))
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, dev, (bsz, H, P, N))
    desc = _desc_from(x, B, chunk_size, dt_pre)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", io, dev, x.shape)
    if final_state is None and return_final_state:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, dev, (bsz, H, P, N))
    st = load_library().ssd_forward_noalloc(
        ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
        _ptr(y), _ptr(final_state), _stream(stream, dev))
    _check(st, "ssd_forward_noalloc")
    return y, final_state


PATH_NAMES = {0: "none", 1: "split", 2: "split-segmented", 3: "one-pass"}
STATUS_WAIT_CUT_OFF_ONE_PASS = 1
STATUS_WAIT_CUT_OFF_SEGMENTED = 2
STATUS_CHAIN_INCOMPLETE = 4
STATUS_NO_RECORD = 8


def workspace_status(desc: SSDDesc, workspace, stream=None):
    """(path name, status bits) of the last whole-forward call that used
    ``workspace`` (a uint8 device tensor) with ``desc``; synchronises the
    stream. Status 0 means the call completed as designed."""
    path = ctypes.c_uint32(0)
    bits = ctypes.c_uint32(0)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().ssd_workspace_status(ctypes.byref(desc), _ptr(workspace), ctypes.c_size_t(nbytes),
                                               _stream(stream, workspace.device), ctypes.byref(path),
                                               ctypes.byref(bits)), "ssd_workspace_status")
    return PATH_NAMES.get(int(path.value), str(path.value)), int(bits.value)


def workspace_status_varlen(desc: SSDDesc, num_seqs: int, workspace, stream=None):
    """workspace_status for the workspace of a forward_varlen call with
    ``desc`` and ``num_seqs`` sequences."""
    path = ctypes.c_uint32(0)
    bits = ctypes.c_uint32(0)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().ssd_workspace_status_varlen(
        ctypes.byref(desc), ctypes.c_int64(num_seqs), _ptr(workspace), ctypes.c_size_t(nbytes),
        _stream(stream, workspace.device), ctypes.byref(path), ctypes.byref(bits)), "ssd_workspace_status_varlen")
    return PATH_NAMES.get(int(path.value), str(path.value)), int(bits.value)


def _chunk_shape(desc):
    q = effective_chunk_size(desc)
    nc = -(-desc.seqlen // q)
    return q, nc


def chunk_cumsum(dt, A, *, headdim, dstate, ngroups=1, io_dtype=torch.bfloat16, chunk_size=0, dt_pre=None,
                 stream=None):
    """Step 1 alone. Returns (dA_cumsum, dt_chunked), each [b, H, nc, Q] fp32."""
    dev = dt.device
    _need(dt, "dt", torch.float32, dev)
    bsz, L, H = dt.shape
    _need(A, "A", torch.float32, dev, (H,))
    desc = make_desc(bsz, L, H, headdim, dstate, ngroups, io_dtype, chunk_size, **_dt_kw(dt_pre, H, dev))
    q, nc = _chunk_shape(desc)
    cs = torch.empty((bsz, H, nc, q), dtype=torch.float32, device=dev)
    dtc = torch.empty_like(cs)
    _check(load_library().ssd_chunk_cumsum(ctypes.byref(desc), _ptr(dt), _ptr(A), _ptr(cs), _ptr(dtc),
                                           _stream(stream, dev)), "ssd_chunk_cumsum")
    return cs, dtc


def chunk_state(x, B, dA_cumsum, dt_chunked, *, chunk_size=0, stream=None):
    """Step 2 alone. Returns states [b, H, nc, P, N] in the io dtype."""
    dev = x.device
    _need(x, "x", device=dev)
    _need(B, "B", x.dtype, dev)
    desc = _desc_from(x, B, chunk_size)
    q, nc = _chunk_shape(desc)
    bsz, L, H, P = x.shape
    _need(dA_cumsum, "dA_cumsum", torch.float32, dev, (bsz, H, nc, q))
    _need(dt_chunked, "dt_chunked", torch.float32, dev, (bsz, H, nc, q))
    states = torch.empty((bsz, H, nc, P, B.shape[3]), dtype=x.dtype, device=dev)
    _check(load_library().ssd_chunk_state(ctypes.byref(desc), _ptr(x), _ptr(B), _ptr(dA_cumsum),
                                          _ptr(dt_chunked), _ptr(states), _stream(stream, dev)),
           "ssd_chunk_state")
    return states


def cumsum_chunk_state(x, B, dt, A, *, chunk_size=0, dt_pre=None, stream=None):
    """Steps 1 and 2 in one call. Returns (dA_cumsum, dt_chunked, states)."""
    dev = x.device
    _need(x, "x", device=dev)
    _need(B, "B", x.dtype, dev)
    desc = _desc_from(x, B, chunk_size, dt_pre)
    q, nc = _chunk_shape(desc)
    bsz, L, H, P = x.shape
    _need(dt, "dt", torch.float32, dev, (bsz, L, H))
    _need(A, "A", torch.float32, dev, (H,))
    cs = torch.empty((bsz, H, nc, q), dtype=torch.float32, device=dev)
    dtc = torch.empty_like(cs)
    states = torch.empty((bsz, H, nc, P, B.shape[3]), dtype=x.dtype, device=dev)
    _check(load_library().ssd_cumsum_chunk_state(ctypes.byref(desc), _ptr(x), _ptr(B), _ptr(dt), _ptr(A),
                                                 _ptr(cs), _ptr(dtc), _ptr(states), _stream(stream, dev)),
           "ssd_cumsum_chunk_state")
    return cs, dtc, states


def state_passing(states, dA_cumsum, init_state=None, *, seqlen, ngroups=1, chunk_size=0,
                  return_final_state=True, final_state=None, stream=None):
    """Step 3 alone, in place over ``states``. Returns (states, final_state)."""
    dev = states.device
    _need(states, "states", device=dev)
    bsz, H, nc, P, N = states.shape
    desc = make_desc(bsz, seqlen, H, P, N, ngroups, states.dtype, chunk_size)
    q, nc2 = _chunk_shape(desc)
    if nc2 != nc:
        raise ValueError("states does not match seqlen / chunk size")
    _need(dA_cumsum, "dA_cumsum", torch.float32, dev, (bsz, H, nc, q))
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, dev, (bsz, H, P, N))
    if final_state is None and return_final_state:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=dev)
    _check(load_library().ssd_state_passing(ctypes.byref(desc), _ptr(states), _ptr(dA_cumsum),
                                            _ptr(init_state), _ptr(final_state), _stream(stream, dev)),
           "ssd_state_passing")
    return states, final_state


def chunk_scan(x, B, C, D, dA_cumsum, dt_chunked, states, *, chunk_size=0, y=None, stream=None):
    """Steps 4+5 alone. ``states`` holds the entering states. Returns y."""
    dev = x.device
    _need(x, "x", device=dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev, B.shape)
    desc = _desc_from(x, B, chunk_size)
    q, nc = _chunk_shape(desc)
    bsz, L, H, P = x.shape
    _need(dA_cumsum, "dA_cumsum", torch.float32, dev, (bsz, H, nc, q))
    _need(dt_chunked, "dt_chunked", torch.float32, dev, (bsz, H, nc, q))
    _need(states, "states", x.dtype, dev, (bsz, H, nc, P, B.shape[3]))
    if D is not None:
        _need(D, "D", torch.float32, dev, (H,))
    if y is None:
        y = torch.empty_like(x)
    _check(load_library().ssd_chunk_scan(ctypes.byref(desc), _ptr(x), _ptr(B), _ptr(C), _ptr(D),
                                         _ptr(dA_cumsum), _ptr(dt_chunked), _ptr(states), _ptr(y),
                                         _stream(stream, dev)), "ssd_chunk_scan")
    return y


def decode_step(x, dt, A, B, C, D, state, *, y=None, dt_pre=None, stream=None):
    """One recurrent step: x [b, H, P], dt [b, H], B/C [b, G, N], state
    [b, H, P, N] fp32 updated in place. Returns y [b, H, P] (io dtype)."""
    dev = x.device
    _need(x, "x", device=dev)
    bsz, H, P = x.shape
    _need(dt, "dt", torch.float32, dev, (bsz, H))
    _need(A, "A", torch.float32, dev, (H,))
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev, tuple(B.shape))
    if D is not None:
        _need(D, "D", torch.float32, dev, (H,))
    G, N = B.shape[1], B.shape[2]
    _need(state, "state", torch.float32, dev, (bsz, H, P, N))
    io = "bf16" if x.dtype == torch.bfloat16 else "fp32"
    desc = make_desc(bsz, 1, H, P, N, G, io, 0, **_dt_kw(dt_pre, H, dev))
    if y is None:
        y = torch.empty_like(x)
    _check(load_library().ssd_decode_step(ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                          _ptr(D), _ptr(state), _ptr(y), _stream(stream, dev)),
           "ssd_decode_step")
    return y


def forward_varlen(x, dt, A, B, C, D=None, *, cu_seqlens, init_states=None, chunk_size: int = 0,
                   return_final_states: bool = True, y=None, final_states=None, workspace=None,
                   dt_pre=None, stream=None):
    """Packed variable-length sequences: x [1, T, H, P], dt [1, T, H],
    B/C [1, T, G, N]; sequence s is tokens [cu_seqlens[s], cu_seqlens[s+1])
    (cu_seqlens: int32 device tensor [S+1]). Without init_states the packed
    stream is cut into fixed chunks (sequences may share a chunk); with them,
    into chunks per sequence. Returns (y, final_states [S, H, P, N] or None)."""
    dev = x.device
    _need(x, "x", device=dev)
    io = x.dtype
    one, T, H, P = x.shape
    if one != 1:
        raise ValueError("packed sequences: x must be [1, T, H, P]")
    _need(B, "B", io, dev)
    G, N = B.shape[2], B.shape[3]
    _need(C, "C", io, dev, B.shape)
    _need(dt, "dt", torch.float32, dev, (1, T, H))
    _need(A, "A", torch.float32, dev, (H,))
    if D is not None:
        _need(D, "D", torch.float32, dev, (H,))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    S = cu_seqlens.numel() - 1
    if init_states is not None:
        _need(init_states, "init_states", torch.float32, dev, (S, H, P, N))
    desc = _desc_from(x, B, chunk_size, dt_pre)
    if y is None:
        y = torch.empty_like(x)
    if final_states is None and return_final_states:
        final_states = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    lib = load_library()
    if workspace is None:
        workspace = torch.empty(workspace_bytes_varlen(desc, S), dtype=torch.uint8, device=dev)
    _check(lib.ssd_forward_varlen(ctypes.byref(desc), _ptr(cu_seqlens), ctypes.c_int64(S), _ptr(x), _ptr(dt),
                                  _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_states), _ptr(y),
                                  _ptr(final_states), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                  _stream(stream, dev)), "ssd_forward_varlen")
    return y, final_states


def conv1d_split(xbc, weight, bias=None, *, nheads, headdim, ngroups, dstate, silu=True, conv_state_in=None,
                 conv_state_out=None, stream=None):
    """Short causal depthwise convolution of the packed [x | B | C] channels,
    split into x [b, L, H, P], B and C [b, L, G, N]. weight [CH, K] fp32."""
    dev = xbc.device
    _need(xbc, "xbc", device=dev)
    bsz, L, CH = xbc.shape
    if CH != nheads * headdim + 2 * ngroups * dstate:
        raise ValueError("xbc channels must be H*P + 2*G*N")
    _need(weight, "weight", torch.float32, dev)
    K = weight.shape[1]
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (CH,))
    desc = make_desc(bsz, L, nheads, headdim, dstate, ngroups, xbc.dtype, 0)
    x = torch.empty((bsz, L, nheads, headdim), dtype=xbc.dtype, device=dev)
    B = torch.empty((bsz, L, ngroups, dstate), dtype=xbc.dtype, device=dev)
    C = torch.empty_like(B)
    _check(load_library().ssd_conv1d_split(ctypes.byref(desc), ctypes.c_int32(K), _ptr(xbc), _ptr(weight),
                                           _ptr(bias), ctypes.c_int32(1 if silu else 0), _ptr(conv_state_in),
                                           _ptr(conv_state_out), _ptr(x), _ptr(B), _ptr(C), _stream(stream, dev)),
           "ssd_conv1d_split")
    return x, B, C
