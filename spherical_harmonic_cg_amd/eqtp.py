"""Python binding of the C ABI in include/eqtp.h (argument marshalling only).

Every function has the name of the C entry point it calls.  Tensors are
PyTorch tensors on the current HIP device; work is enqueued on
``torch.cuda.current_stream()`` and nothing is synchronised.  All arithmetic
runs in the HIP library: if ``libeqtp.so`` has not been built, the first call
raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeqtp.so")

EQTP_OK, EQTP_EINVAL, EQTP_EUNSUPPORTED, EQTP_EHIP, EQTP_ETOOLARGE, EQTP_EGRAPH = 0, 1, 2, 3, 4, 5
EQTP_CHECK_WORDS = 8
EQTP_PATHS_PARITY, EQTP_PATHS_SO3 = 0, 1
EQTP_W_FIXED, EQTP_W_RADIAL = 0, 1
EQTP_EDGES_DST_SORTED, EQTP_EDGES_UNSORTED = 0, 1
EQTP_ALGO_AUTO, EQTP_ALGO_NODE_MFMA, EQTP_ALGO_EDGE_VALU, EQTP_ALGO_EDGE_SO2 = 0, 1, 2, 3
EQTP_F32, EQTP_BF16, EQTP_F32_BF16 = 0, 1, 2

EXPORTED = ("eqtp_num_paths", "eqtp_path_table", "eqtp_sh", "eqtp_conv_fused", "eqtp_conv_workspace_bytes",
            "eqtp_conv_fused_ws", "eqtp_conv_fused_noalloc", "eqtp_conv_messages",
            "eqtp_conv_backward", "eqtp_conv_backward_by_source", "eqtp_edge_rows", "eqtp_sort_edges",
            "eqtp_sort_workspace_bytes", "eqtp_sort_edges_stable",
            "eqtp_linear", "eqtp_interaction_workspace_bytes", "eqtp_interaction",
            "eqtp_status_string", "eqtp_check_graph", "eqtp_set_debug", "eqtp_test_segment_probe")


class EqtpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, eqtp_status_string(status)))


class _ConvDesc(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("lmax", ctypes.c_int32), ("C", ctypes.c_int32),
                ("path_set", ctypes.c_int32), ("weight_mode", ctypes.c_int32), ("edge_order", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("r_cut", ctypes.c_float), ("n_basis", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class _InteractionDesc(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("lmax", ctypes.c_int32), ("C", ctypes.c_int32),
                ("path_set", ctypes.c_int32), ("r_cut", ctypes.c_float), ("n_basis", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("norm", ctypes.c_float)]


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libeqtp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("HIP library %s not built; run `python -m spherical_harmonic_cg_amd.build`" % path)
            lib = ctypes.CDLL(path)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
            lib.eqtp_num_paths.argtypes = [i32, i32]
            lib.eqtp_num_paths.restype = i32
            lib.eqtp_path_table.argtypes = [i32, i32, vp]
            lib.eqtp_path_table.restype = i32
            lib.eqtp_sh.argtypes = [vp, i64, i32, vp, vp]
            lib.eqtp_sh.restype = i32
            lib.eqtp_conv_fused.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.eqtp_conv_fused.restype = i32
            lib.eqtp_conv_workspace_bytes.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64]
            lib.eqtp_conv_workspace_bytes.restype = i64
            lib.eqtp_conv_fused_ws.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64] + [vp] * 8 + [i64, vp]
            lib.eqtp_conv_fused_ws.restype = i32
            lib.eqtp_conv_fused_noalloc.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64] + [vp] * 8
            lib.eqtp_conv_fused_noalloc.restype = i32
            lib.eqtp_conv_messages.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64] + [vp] * 6
            lib.eqtp_conv_messages.restype = i32
            lib.eqtp_conv_backward.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64] + [vp] * 11
            lib.eqtp_conv_backward.restype = i32
            lib.eqtp_conv_backward_by_source.argtypes = [ctypes.POINTER(_ConvDesc), i64, i64] + [vp] * 11
            lib.eqtp_conv_backward_by_source.restype = i32
            lib.eqtp_edge_rows.argtypes = [i64, i64, vp, vp, vp]
            lib.eqtp_edge_rows.restype = i32
            lib.eqtp_sort_edges.argtypes = [i64, i64] + [vp] * 8
            lib.eqtp_sort_edges.restype = i32
            lib.eqtp_sort_workspace_bytes.argtypes = [i64, i64]
            lib.eqtp_sort_workspace_bytes.restype = i64
            lib.eqtp_sort_edges_stable.argtypes = [i64, i64] + [vp] * 8 + [i64, vp]
            lib.eqtp_sort_edges_stable.restype = i32
            lib.eqtp_linear.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp]
            lib.eqtp_linear.restype = i32
            lib.eqtp_interaction_workspace_bytes.argtypes = [ctypes.POINTER(_InteractionDesc), i64, i64]
            lib.eqtp_interaction_workspace_bytes.restype = i64
            lib.eqtp_interaction.argtypes = [ctypes.POINTER(_InteractionDesc), i64, i64] + [vp] * 11 + [i64, vp]
            lib.eqtp_interaction.restype = i32
            lib.eqtp_status_string.argtypes = [i32]
            lib.eqtp_status_string.restype = ctypes.c_char_p
            lib.eqtp_check_graph.argtypes = [i64, i64] + [vp] * 6
            lib.eqtp_check_graph.restype = i32
            lib.eqtp_set_debug.argtypes = [i32]
            lib.eqtp_set_debug.restype = i32
            lib.eqtp_test_segment_probe.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp]
            lib.eqtp_test_segment_probe.restype = i32
            _lib = lib
    return _lib


# The per-call marshalling is on the host's critical path for small graphs (a launch takes a few µs), so
# the helpers below take the cheap route first: the raw current stream of the current device, pointers as
# plain ints (ctypes converts them for c_void_p arguments), and one combined test per tensor before the
# detailed checks that name what is wrong.
_raw_stream = None


def _stream():
    global _raw_stream
    if _raw_stream is None:
        import torch

        get_raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        get_dev = getattr(torch._C, "_cuda_getDevice", None)
        if get_raw is not None and get_dev is not None:
            _raw_stream = lambda: get_raw(get_dev())
        else:
            _raw_stream = lambda: torch.cuda.current_stream().cuda_stream
    return _raw_stream()


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _check(t, name, dtype, shape=None):
    try:
        if t.is_cuda and t.dtype is dtype and t.is_contiguous() and (shape is None or t.shape == tuple(shape)):
            return
    except AttributeError:
        pass
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _raise(rc, where):
    if rc != EQTP_OK:
        raise EqtpError(rc, where)


def eqtp_status_string(status: int) -> str:
    return load_library().eqtp_status_string(int(status)).decode()


@functools.lru_cache(maxsize=None)
def _num_paths(lmax: int, path_set: int) -> int:
    return load_library().eqtp_num_paths(lmax, path_set)


def eqtp_num_paths(lmax: int, path_set: int = EQTP_PATHS_PARITY) -> int:
    P = _num_paths(int(lmax), int(path_set))
    if P < 0:
        raise EqtpError(-P, "eqtp_num_paths")
    return P


@functools.lru_cache(maxsize=256)
def _conv_desc(lmax, C, path_set, weight_mode, order, algo, r_cut, n_basis, x_dtype, out_dtype):
    # read by the library during a call only, so one instance per distinct descriptor is shared
    return _ConvDesc(ctypes.sizeof(_ConvDesc), lmax, C, path_set, weight_mode, order, algo, r_cut, n_basis, x_dtype,
                     out_dtype)


def eqtp_path_table(lmax: int, path_set: int = EQTP_PATHS_PARITY) -> np.ndarray:
    P = eqtp_num_paths(lmax, path_set)
    out = np.zeros((P, 3), dtype=np.int32)
    rc = load_library().eqtp_path_table(lmax, path_set, out.ctypes.data_as(ctypes.c_void_p))
    if rc < 0:
        raise EqtpError(-rc, "eqtp_path_table")
    return out


def eqtp_sh(vec, lmax: int, Y=None):
    """Y [E, (lmax+1)^2] fp32 = real spherical harmonics of vec [E, 3] fp32."""
    import torch

    _check(vec, "vec", torch.float32)
    E = vec.shape[0]
    if vec.dim() != 2 or vec.shape[1] != 3:
        raise ValueError("vec must be [E, 3]")
    K = (lmax + 1) ** 2
    if Y is None:
        Y = torch.empty((E, K), dtype=torch.float32, device=vec.device)
    _check(Y, "Y", torch.float32, (E, K))
    _raise(load_library().eqtp_sh(_ptr(vec), E, lmax, _ptr(Y), _stream()), "eqtp_sh")
    return Y


def _conv_args(vec, src, x, weights, lmax, row_ptr, dst, path_set, weight_mode, r_cut, n_basis, algo, out,
               out_dtype=EQTP_F32):
    """Checks the fused convolution's tensors; returns (descriptor, N, E, out)."""
    import torch

    x_dtype = EQTP_BF16 if x.dtype == torch.bfloat16 else EQTP_F32
    _check(x, "x", torch.bfloat16 if x_dtype == EQTP_BF16 else torch.float32)
    if x.dim() != 3:
        raise ValueError("x must be [N, C, K]")
    N, C, K = x.shape
    if K != (lmax + 1) ** 2:
        raise ValueError("x has %d components, lmax %d needs %d" % (K, lmax, (lmax + 1) ** 2))
    _check(vec, "vec", torch.float32)
    E = vec.shape[0]
    _check(src, "src", torch.int32, (E,))
    _check(weights, "weights", torch.float32)
    if (row_ptr is None) == (dst is None):
        raise ValueError("give exactly one of row_ptr (dst-sorted edges) or dst (any order)")
    if row_ptr is not None:
        _check(row_ptr, "row_ptr", torch.int32, (N + 1,))
        order = EQTP_EDGES_DST_SORTED
    else:
        _check(dst, "dst", torch.int32, (E,))
        order = EQTP_EDGES_UNSORTED
    P = eqtp_num_paths(lmax, path_set)
    wshape = (P, C) if weight_mode == EQTP_W_FIXED else (n_basis, P * C)
    if tuple(weights.shape) != wshape:
        raise ValueError("weights has shape %s, expected %s" % (tuple(weights.shape), wshape))
    odt = torch.bfloat16 if out_dtype == EQTP_BF16 else torch.float32
    if out is None:
        out = torch.empty((N, C, K), dtype=odt, device=x.device)
    _check(out, "out", odt, (N, C, K))
    d = _conv_desc(lmax, C, path_set, weight_mode, order, algo, float(r_cut), n_basis, x_dtype, out_dtype)
    return d, N, E, out


def eqtp_conv_fused(vec, src, x, weights, lmax: int, row_ptr=None, dst=None, path_set: int = EQTP_PATHS_PARITY,
                    weight_mode: int = EQTP_W_FIXED, r_cut: float = 0.0, n_basis: int = 8,
                    algo: int = EQTP_ALGO_AUTO, out=None, out_dtype: int = EQTP_F32):
    """out [N, C, K] = fused harmonics -> coupling -> sum into dst.

    Give ``row_ptr`` [N+1] for dst-sorted edges, or ``dst`` [E] for any order
    (atomic accumulation).  ``weights`` is [P, C] (fixed) or [8, P*C] (radial).
    ``x`` is float32, or bfloat16 (lmax <= 3, any edge order or weights); ``out``
    is float32, or bfloat16 with ``out_dtype=EQTP_BF16`` (edges in any order:
    packed bf16 atomics).
    """
    d, N, E, out = _conv_args(vec, src, x, weights, lmax, row_ptr, dst, path_set, weight_mode, r_cut, n_basis, algo,
                              out, out_dtype)
    rc = load_library().eqtp_conv_fused(ctypes.byref(d), N, E, _ptr(vec), _ptr(src), _ptr(dst), _ptr(row_ptr),
                                        _ptr(x), _ptr(weights), _ptr(out), _stream())
    _raise(rc, "eqtp_conv_fused")
    return out


def eqtp_conv_workspace_bytes(N: int, E: int, lmax: int, C: int, edge_order: int = EQTP_EDGES_UNSORTED,
                              weight_mode: int = EQTP_W_FIXED, path_set: int = EQTP_PATHS_PARITY) -> int:
    """Device workspace eqtp_conv_fused_ws needs (bytes)."""
    d = _ConvDesc(ctypes.sizeof(_ConvDesc), lmax, C, path_set, weight_mode, edge_order, EQTP_ALGO_AUTO, 1.0, 8,
                  EQTP_F32)
    n = load_library().eqtp_conv_workspace_bytes(ctypes.byref(d), N, E)
    if n < 0:
        raise EqtpError(-n, "eqtp_conv_workspace_bytes")
    return int(n)


def eqtp_conv_fused_ws(vec, src, x, weights, lmax: int, row_ptr=None, dst=None, path_set: int = EQTP_PATHS_PARITY,
                       weight_mode: int = EQTP_W_FIXED, r_cut: float = 0.0, n_basis: int = 8,
                       algo: int = EQTP_ALGO_AUTO, out=None, workspace=None):
    """eqtp_conv_fused with a workspace: edges in any order (``dst``) are grouped by destination on the GPU
    (rows in input order) and summed without atomics.  ``workspace`` is a uint8 CUDA tensor of at least
    eqtp_conv_workspace_bytes bytes (allocated here if None)."""
    import torch

    d, N, E, out = _conv_args(vec, src, x, weights, lmax, row_ptr, dst, path_set, weight_mode, r_cut, n_basis, algo,
                              out)
    need = load_library().eqtp_conv_workspace_bytes(ctypes.byref(d), N, E)
    if need < 0:
        _raise(-need, "eqtp_conv_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace", torch.uint8)
    rc = load_library().eqtp_conv_fused_ws(ctypes.byref(d), N, E, _ptr(vec), _ptr(src), _ptr(dst), _ptr(row_ptr),
                                           _ptr(x), _ptr(weights), _ptr(out), _ptr(workspace), workspace.numel(),
                                           _stream())
    _raise(rc, "eqtp_conv_fused_ws")
    return out


def eqtp_conv_fused_noalloc(vec, src, x, weights, lmax: int, row_ptr=None, dst=None,
                            path_set: int = EQTP_PATHS_PARITY, weight_mode: int = EQTP_W_FIXED, r_cut: float = 0.0,
                            n_basis: int = 8, algo: int = EQTP_ALGO_AUTO, out=None):
    """eqtp_conv_fused_ws with the library's static scratch as the workspace (no device allocation by
    the library; ``out`` must be given for a call that allocates nothing at all)."""
    d, N, E, out = _conv_args(vec, src, x, weights, lmax, row_ptr, dst, path_set, weight_mode, r_cut, n_basis, algo,
                              out)
    rc = load_library().eqtp_conv_fused_noalloc(ctypes.byref(d), N, E, _ptr(vec), _ptr(src), _ptr(dst),
                                                _ptr(row_ptr), _ptr(x), _ptr(weights), _ptr(out), _stream())
    _raise(rc, "eqtp_conv_fused_noalloc")
    return out


def eqtp_conv_messages(vec, src, x, weights, lmax: int, path_set: int = EQTP_PATHS_PARITY,
                       weight_mode: int = EQTP_W_FIXED, r_cut: float = 0.0, n_basis: int = 8, out=None,
                       algo: int = EQTP_ALGO_AUTO):
    """messages [E, C, K]: one message per edge, no destination sum (lmax 4..6 or
    algo=EQTP_ALGO_EDGE_SO2: the edge-aligned form)."""
    import torch

    _check(x, "x", torch.float32)
    if x.dim() != 3:
        raise ValueError("x must be [N, C, K]")
    N, C, K = x.shape
    if K != (lmax + 1) ** 2:
        raise ValueError("x has %d components, lmax %d needs %d" % (K, lmax, (lmax + 1) ** 2))
    _check(vec, "vec", torch.float32)
    E = vec.shape[0]
    _check(src, "src", torch.int32, (E,))
    P = eqtp_num_paths(lmax, path_set)
    wshape = (P, C) if weight_mode == EQTP_W_FIXED else (n_basis, P * C)
    _check(weights, "weights", torch.float32, wshape)
    if out is None:
        out = torch.empty((E, C, K), dtype=torch.float32, device=x.device)
    _check(out, "out", torch.float32, (E, C, K))
    d = _ConvDesc(ctypes.sizeof(_ConvDesc), lmax, C, path_set, weight_mode, EQTP_EDGES_UNSORTED, algo,
                  float(r_cut), n_basis, EQTP_F32)
    rc = load_library().eqtp_conv_messages(ctypes.byref(d), N, E, _ptr(vec), _ptr(src), _ptr(x), _ptr(weights),
                                           _ptr(out), _stream())
    _raise(rc, "eqtp_conv_messages")
    return out


def eqtp_conv_backward(vec, src, x, weights, grad_out, lmax: int, row_ptr=None, dst=None,
                       path_set: int = EQTP_PATHS_PARITY, need_x: bool = True, need_w: bool = True,
                       need_vec: bool = True, algo: int = EQTP_ALGO_AUTO, weight_mode: int = EQTP_W_FIXED,
                       r_cut: float = 0.0, n_basis: int = 8):
    """(grad_x [N,C,K] | None, grad_w | None, grad_vec [E,3] | None) of
    sum(grad_out * eqtp_conv_fused(...)) for fixed weights [P, C] (grad_w
    [P, C]) or, with weight_mode=EQTP_W_RADIAL, radial weights
    [n_basis, P*C] (grad_w of the same shape)."""
    import torch

    _check(x, "x", torch.float32)
    if x.dim() != 3:
        raise ValueError("x must be [N, C, K]")
    N, C, K = x.shape
    if K != (lmax + 1) ** 2:
        raise ValueError("x has %d components, lmax %d needs %d" % (K, lmax, (lmax + 1) ** 2))
    _check(grad_out, "grad_out", torch.float32, (N, C, K))
    _check(vec, "vec", torch.float32)
    E = vec.shape[0]
    _check(src, "src", torch.int32, (E,))
    if (row_ptr is None) == (dst is None):
        raise ValueError("give exactly one of row_ptr (dst-sorted edges) or dst (any order)")
    if row_ptr is not None:
        _check(row_ptr, "row_ptr", torch.int32, (N + 1,))
        order = EQTP_EDGES_DST_SORTED
    else:
        _check(dst, "dst", torch.int32, (E,))
        order = EQTP_EDGES_UNSORTED
    P = eqtp_num_paths(lmax, path_set)
    _check(weights, "weights", torch.float32, (P, C) if weight_mode == EQTP_W_FIXED else (n_basis, P * C))
    if not (need_x or need_w or need_vec):
        raise ValueError("request at least one gradient")
    gx = torch.empty_like(x) if need_x else None
    gw = torch.empty_like(weights) if need_w else None
    gv = torch.empty((E, 3), dtype=torch.float32, device=x.device) if need_vec else None
    d = _ConvDesc(ctypes.sizeof(_ConvDesc), lmax, C, path_set, weight_mode, order, algo, float(r_cut), n_basis,
                  EQTP_F32)
    rc = load_library().eqtp_conv_backward(ctypes.byref(d), N, E, _ptr(vec), _ptr(src), _ptr(dst), _ptr(row_ptr),
                                           _ptr(x), _ptr(weights), _ptr(grad_out), _ptr(gx), _ptr(gw), _ptr(gv),
                                           _stream())
    _raise(rc, "eqtp_conv_backward")
    return gx, gw, gv


def eqtp_conv_backward_by_source(vec_s, dst_s, src_ptr, x, weights, grad_out, lmax: int,
                                 path_set: int = EQTP_PATHS_PARITY, need_x: bool = True, need_w: bool = True,
                                 need_vec: bool = False, perm=None, weight_mode: int = EQTP_W_FIXED,
                                 r_cut: float = 0.0, n_basis: int = 8, algo: int = EQTP_ALGO_AUTO):
    """(grad_x [N,C,K] | None, grad_w | None, grad_vec [E,3] | None) from the
    edges grouped by source node: src_ptr [N+1] CSR over sources, vec_s [E,3] /
    dst_s [E] in that order, perm [E] (needed for grad_vec) the caller's index of
    each grouped edge (see eqtp_sort_edges).  grad_vec is in the caller's edge
    order.  Fixed weights [P, C] or, with weight_mode=EQTP_W_RADIAL, radial
    weights [n_basis, P*C] (grad_w of the same shape)."""
    import torch

    _check(grad_out, "grad_out", torch.float32)
    if grad_out.dim() != 3:
        raise ValueError("grad_out must be [N, C, K]")
    N, C, K = grad_out.shape
    if K != (lmax + 1) ** 2:
        raise ValueError("grad_out has %d components, lmax %d needs %d" % (K, lmax, (lmax + 1) ** 2))
    _check(vec_s, "vec_s", torch.float32)
    E = vec_s.shape[0]
    _check(dst_s, "dst_s", torch.int32, (E,))
    _check(src_ptr, "src_ptr", torch.int32, (N + 1,))
    _check(x, "x", torch.float32, (N, C, K))
    P = eqtp_num_paths(lmax, path_set)
    _check(weights, "weights", torch.float32, (P, C) if weight_mode == EQTP_W_FIXED else (n_basis, P * C))
    if not (need_x or need_w or need_vec):
        raise ValueError("request at least one gradient")
    if need_vec:
        if perm is None:
            raise ValueError("grad_vec needs perm (the caller's index of each grouped edge)")
        _check(perm, "perm", torch.int32, (E,))
    gx = torch.empty_like(grad_out) if need_x else None
    gw = torch.empty_like(weights) if need_w else None
    gv = torch.empty((E, 3), dtype=torch.float32, device=grad_out.device) if need_vec else None
    d = _ConvDesc(ctypes.sizeof(_ConvDesc), lmax, C, path_set, weight_mode, EQTP_EDGES_DST_SORTED, algo,
                  float(r_cut), n_basis, EQTP_F32)
    rc = load_library().eqtp_conv_backward_by_source(ctypes.byref(d), N, E, _ptr(vec_s), _ptr(dst_s), _ptr(src_ptr),
                                                     _ptr(x), _ptr(weights), _ptr(grad_out), _ptr(gx), _ptr(gw),
                                                     _ptr(perm if need_vec else None), _ptr(gv), _stream())
    _raise(rc, "eqtp_conv_backward_by_source")
    return gx, gw, gv


def eqtp_check_graph(N: int, E: int, row_ptr=None, src=None, dst=None, vec=None, report=None):
    """Graph checks on the GPU: report [EQTP_CHECK_WORDS] int32 (counts of out-of-range src / dst,
    decreasing row_ptr steps, row_ptr endpoint faults, edges outside their dst's row, non-finite
    vectors; then the first offending edge and row, -1 if none).  Any array may be None."""
    import torch

    for t, name, dt, shape in ((row_ptr, "row_ptr", torch.int32, (N + 1,)), (src, "src", torch.int32, (E,)),
                               (dst, "dst", torch.int32, (E,)), (vec, "vec", torch.float32, (E, 3))):
        if t is not None:
            _check(t, name, dt, shape)
    dev = next((t.device for t in (row_ptr, src, dst, vec) if t is not None), torch.device("cuda"))
    rep = report if report is not None else torch.empty(EQTP_CHECK_WORDS, dtype=torch.int32, device=dev)
    _check(rep, "report", torch.int32, (EQTP_CHECK_WORDS,))
    rc = load_library().eqtp_check_graph(N, E, _ptr(row_ptr), _ptr(src), _ptr(dst), _ptr(vec), _ptr(rep), _stream())
    _raise(rc, "eqtp_check_graph")
    return rep


def eqtp_set_debug(on: bool) -> bool:
    """Switch the library's debug mode (graph checks before every launch); returns the previous setting."""
    return bool(load_library().eqtp_set_debug(1 if on else 0))


def eqtp_edge_rows(row_ptr, E: int, out=None):
    """rows [E] int32: the destination row of every edge of a dst-sorted CSR."""
    import torch

    _check(row_ptr, "row_ptr", torch.int32)
    N = row_ptr.shape[0] - 1
    rows = out if out is not None else torch.empty(E, dtype=torch.int32, device=row_ptr.device)
    _check(rows, "rows", torch.int32, (E,))
    rc = load_library().eqtp_edge_rows(N, E, _ptr(row_ptr), _ptr(rows), _stream())
    _raise(rc, "eqtp_edge_rows")
    return rows


def eqtp_sort_edges(dst, N: int, vec=None, src=None, out=None):
    """(row_ptr [N+1], perm [E], vec[perm] | None, src[perm] | None): edges grouped
    by destination (order inside a row unspecified).  ``out`` may give the four
    output tensors (the last two None when vec / src are not given)."""
    import torch

    _check(dst, "dst", torch.int32)
    E = dst.shape[0]
    dev = dst.device
    if out is None:
        out = (torch.empty(N + 1, dtype=torch.int32, device=dev), torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty_like(vec) if vec is not None else None, torch.empty_like(src) if src is not None else None)
    row_ptr, perm, vs, ss = out
    _check(row_ptr, "row_ptr", torch.int32, (N + 1,))
    _check(perm, "perm", torch.int32, (E,))
    if vec is not None:
        _check(vec, "vec", torch.float32, (E, 3))
        _check(vs, "vec_sorted", torch.float32, (E, 3))
    if src is not None:
        _check(src, "src", torch.int32, (E,))
        _check(ss, "src_sorted", torch.int32, (E,))
    rc = load_library().eqtp_sort_edges(N, E, _ptr(dst), _ptr(vec), _ptr(src), _ptr(row_ptr), _ptr(perm),
                                        _ptr(vs if vec is not None else None), _ptr(ss if src is not None else None),
                                        _stream())
    _raise(rc, "eqtp_sort_edges")
    return row_ptr, perm, (vs if vec is not None else None), (ss if src is not None else None)


def eqtp_sort_workspace_bytes(N: int, E: int) -> int:
    """Device workspace eqtp_sort_edges_stable needs (bytes)."""
    n = load_library().eqtp_sort_workspace_bytes(N, E)
    if n < 0:
        raise EqtpError(-n, "eqtp_sort_workspace_bytes")
    return int(n)


def eqtp_sort_edges_stable(dst, N: int, vec=None, src=None, out=None, workspace=None):
    """eqtp_sort_edges with every row in input order (stable radix sort): the same four outputs, unique
    and identical from call to call.  ``workspace`` is a uint8 CUDA tensor of at least
    eqtp_sort_workspace_bytes bytes (allocated here if None)."""
    import torch

    _check(dst, "dst", torch.int32)
    E = dst.shape[0]
    dev = dst.device
    if out is None:
        out = (torch.empty(N + 1, dtype=torch.int32, device=dev), torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty_like(vec) if vec is not None else None, torch.empty_like(src) if src is not None else None)
    row_ptr, perm, vs, ss = out
    _check(row_ptr, "row_ptr", torch.int32, (N + 1,))
    _check(perm, "perm", torch.int32, (E,))
    if vec is not None:
        _check(vec, "vec", torch.float32, (E, 3))
        _check(vs, "vec_sorted", torch.float32, (E, 3))
    if src is not None:
        _check(src, "src", torch.int32, (E,))
        _check(ss, "src_sorted", torch.int32, (E,))
    need = eqtp_sort_workspace_bytes(N, E)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8)
    rc = load_library().eqtp_sort_edges_stable(N, E, _ptr(dst), _ptr(vec), _ptr(src), _ptr(row_ptr), _ptr(perm),
                                               _ptr(vs if vec is not None else None),
                                               _ptr(ss if src is not None else None), _ptr(workspace),
                                               workspace.numel(), _stream())
    _raise(rc, "eqtp_sort_edges_stable")
    return row_ptr, perm, (vs if vec is not None else None), (ss if src is not None else None)


def eqtp_linear(h, W, lmax: int, dtype: int = EQTP_F32, out=None):
    """out[n, c', l m] = sum_c W[l, c', c] h[n, c, l m] (fp32 out).

    float32 h and W: dtype EQTP_F32 (fp32 products) or EQTP_BF16 / EQTP_F32_BF16 (each value rounded to
    bf16 for the products; passed to the library as EQTP_F32_BF16).  bfloat16 h and W: bf16 storage and
    products (EQTP_BF16)."""
    import torch

    if h.dtype == torch.bfloat16:
        if dtype not in (EQTP_BF16, EQTP_F32_BF16):
            raise ValueError("bfloat16 h needs dtype EQTP_BF16")
        st, cdt = torch.bfloat16, EQTP_BF16
    else:
        st = torch.float32
        cdt = EQTP_F32 if dtype == EQTP_F32 else EQTP_F32_BF16
    _check(h, "h", st)
    N, C, K = h.shape
    _check(W, "W", st, (lmax + 1, C, C))
    if out is None:
        out = torch.empty((N, C, K), dtype=torch.float32, device=h.device)
    _check(out, "out", torch.float32, (N, C, K))
    _raise(load_library().eqtp_linear(N, C, lmax, cdt, _ptr(h), _ptr(W), _ptr(out), _stream()), "eqtp_linear")
    return out


def _ix_desc(lmax, C, path_set, r_cut, norm):
    return _InteractionDesc(ctypes.sizeof(_InteractionDesc), lmax, C, path_set, float(r_cut), 8, 64, float(norm))


def eqtp_interaction_workspace_bytes(N: int, E: int, lmax: int, C: int, r_cut: float = 1.0, norm: float = 1.0,
                                     path_set: int = EQTP_PATHS_PARITY) -> int:
    d = _ix_desc(lmax, C, path_set, r_cut, norm)
    n = load_library().eqtp_interaction_workspace_bytes(ctypes.byref(d), N, E)
    if n < 0:
        _raise(int(-n), "eqtp_interaction_workspace_bytes")
    return int(n)


def eqtp_interaction(vec, src, row_ptr, h, W_up, W1, W2, W3, W_out, lmax: int, r_cut: float, norm: float = 1.0,
                     path_set: int = EQTP_PATHS_PARITY, workspace=None, out=None):
    """One interaction layer (see include/eqtp.h): out [N, C, K] fp32 from node features h [N, C, K],
    dst-sorted edges (vec, src, row_ptr) and the weights W_up, W_out [lmax+1, C, C], W1 [8, 64],
    W2 [64, 64], W3 [64, P*C].  ``workspace``: a uint8 tensor of at least
    eqtp_interaction_workspace_bytes bytes, or None to allocate one here."""
    import torch

    _check(h, "h", torch.float32)
    if h.dim() != 3:
        raise ValueError("h must be [N, C, K]")
    N, C, K = h.shape
    if K != (lmax + 1) ** 2:
        raise ValueError("h has %d components, lmax %d needs %d" % (K, lmax, (lmax + 1) ** 2))
    _check(vec, "vec", torch.float32)
    E = vec.shape[0]
    _check(src, "src", torch.int32, (E,))
    _check(row_ptr, "row_ptr", torch.int32, (N + 1,))
    P = eqtp_num_paths(lmax, path_set)
    _check(W_up, "W_up", torch.float32, (lmax + 1, C, C))
    _check(W_out, "W_out", torch.float32, (lmax + 1, C, C))
    _check(W1, "W1", torch.float32, (8, 64))
    _check(W2, "W2", torch.float32, (64, 64))
    _check(W3, "W3", torch.float32, (64, P * C))
    d = _ix_desc(lmax, C, path_set, r_cut, norm)
    need = eqtp_interaction_workspace_bytes(N, E, lmax, C, r_cut, norm, path_set)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _check(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((N, C, K), dtype=torch.float32, device=h.device)
    _check(out, "out", torch.float32, (N, C, K))
    rc = load_library().eqtp_interaction(ctypes.byref(d), N, E, _ptr(vec), _ptr(src), _ptr(row_ptr), _ptr(h),
                                         _ptr(W_up), _ptr(W1), _ptr(W2), _ptr(W3), _ptr(W_out), _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream())
    _raise(rc, "eqtp_interaction")
    return out


def eqtp_test_segment_probe(row_ptr, src, C: int, lmax: int, algo: int = EQTP_ALGO_NODE_MFMA):
    """(count [N] int32, src_sum [N] int64) walked with the conv kernel's schedule."""
    import torch

    _check(row_ptr, "row_ptr", torch.int32)
    _check(src, "src", torch.int32)
    N = row_ptr.shape[0] - 1
    E = src.shape[0]
    count = torch.empty(N, dtype=torch.int32, device=row_ptr.device)
    src_sum = torch.empty(N, dtype=torch.int64, device=row_ptr.device)
    rc = load_library().eqtp_test_segment_probe(_ptr(row_ptr), _ptr(src), N, E, C, lmax, algo, _ptr(count),
                                                _ptr(src_sum), _stream())
    _raise(rc, "eqtp_test_segment_probe")
    return count, src_sum
