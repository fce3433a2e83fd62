"""fp64 CPU oracle for the equivariant convolution (test infrastructure).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product library never does, and shares no code
with it.  The arithmetic lives in ``eqtp_oracle.c`` (plain C, double
precision); this module only builds it with gcc and marshals numpy arrays.

What each function computes, and the page passage it follows, is stated in the
C source next to the function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eqtp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

PATHS_PARITY = 0
PATHS_SO3 = 1


def build(force: bool = False) -> str:
    """Compile eqtp_oracle.c into liboracle.so (gcc -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
            vp = ctypes.c_void_p
            lib.oracle_sh.argtypes = [i64, vp, i32, vp]
            lib.oracle_sh.restype = i32
            lib.oracle_sh_f64.argtypes = [i64, vp, i32, vp]
            lib.oracle_sh_f64.restype = i32
            lib.oracle_cg_complex.argtypes = [i32] * 6
            lib.oracle_cg_complex.restype = f64
            lib.oracle_cg_real.argtypes = [i32, i32, i32, vp, vp]
            lib.oracle_cg_real.restype = i32
            lib.oracle_paths.argtypes = [i32, i32, vp]
            lib.oracle_paths.restype = i32
            lib.oracle_envelope.argtypes = [f64]
            lib.oracle_envelope.restype = f64
            lib.oracle_radial_basis.argtypes = [f64, f64, i32, vp]
            lib.oracle_radial_basis.restype = None
            lib.oracle_conv.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, vp, vp]
            lib.oracle_conv.restype = i32
            lib.oracle_conv_f64.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, vp, vp]
            lib.oracle_conv_f64.restype = i32
            lib.oracle_linear_f64.argtypes = [i64, i32, i32, vp, vp, vp]
            lib.oracle_linear_f64.restype = i32
            lib.oracle_round_bf16.argtypes = [ctypes.c_float]
            lib.oracle_round_bf16.restype = ctypes.c_float
            lib.oracle_linear.argtypes = [i64, i32, i32, i32, vp, vp, vp]
            lib.oracle_linear.restype = i32
            lib.oracle_messages.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, vp]
            lib.oracle_messages.restype = i32
            lib.oracle_messages_f64.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, vp]
            lib.oracle_messages_f64.restype = i32
            lib.oracle_sh_grad_f64.argtypes = [i64, vp, i32, vp, vp]
            lib.oracle_sh_grad_f64.restype = i32
            lib.oracle_conv_backward.argtypes = [i64, i64, i32, i32, i32] + [vp] * 9
            lib.oracle_conv_backward.restype = i32
            lib.oracle_conv_backward_f64.argtypes = [i64, i64, i32, i32, i32] + [vp] * 9
            lib.oracle_conv_backward_f64.restype = i32
            for fn in (lib.oracle_conv_backward_radial, lib.oracle_conv_backward_radial_f64):
                fn.argtypes = [i64, i64, i32, i32, i32, f64, i32] + [vp] * 9
                fn.restype = i32
            lib.oracle_envelope_deriv.argtypes = [f64]
            lib.oracle_envelope_deriv.restype = f64
            lib.oracle_radial_basis_deriv.argtypes = [f64, f64, i32, vp]
            lib.oracle_radial_basis_deriv.restype = None
            lib.oracle_silu.argtypes = [f64]
            lib.oracle_silu.restype = f64
            lib.oracle_radial_mlp_f64.argtypes = [i64, vp, f64, i32, i32, vp, vp, vp]
            lib.oracle_radial_mlp_f64.restype = i32
            lib.oracle_conv_basis_f64.argtypes = [i64, i64, i32, i32, i32, i32] + [vp] * 7
            lib.oracle_conv_basis_f64.restype = i32
            for fn in (lib.oracle_interaction_f64, lib.oracle_interaction):
                fn.argtypes = [i64, i64, i32, i32, i32, f64, i32, i32] + [vp] * 9 + [f64, vp]
                fn.restype = i32
            lib.oracle_set_threads.argtypes = [i32]
            lib.oracle_set_threads.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = i32
            _lib = lib
    return _lib


def set_threads(n: int = 0) -> None:
    """Threads for the loops over destination rows, nodes and edges (0 = the
    OpenMP default: OMP_NUM_THREADS, else every core).  Results do not depend
    on it."""
    _load().oracle_set_threads(int(n))


def num_threads() -> int:
    """Threads the parallel loops will use."""
    return int(_load().oracle_num_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def sh(vec, lmax: int) -> np.ndarray:
    """Real spherical harmonics [E, (lmax+1)^2] (fp64) of vectors [E, 3].

    float32 input goes through the float32 entry point; float64 input through
    the double one (used where identities are checked to 1e-10)."""
    lib = _load()
    is64 = np.asarray(vec).dtype == np.float64
    v = (_f64 if is64 else _f32)(vec).reshape(-1, 3)
    K = (lmax + 1) ** 2
    Y = np.empty((v.shape[0], K), dtype=np.float64)
    fn = lib.oracle_sh_f64 if is64 else lib.oracle_sh
    if fn(v.shape[0], _p(v), lmax, _p(Y)) != 0:
        raise ValueError("oracle_sh: bad arguments")
    return Y


def cg_complex(l1, m1, l2, m2, l3, m3) -> float:
    """<l1 m1 l2 m2 | l3 m3> (Racah formula)."""
    return _load().oracle_cg_complex(l1, m1, l2, m2, l3, m3)


def cg_real(l1: int, l2: int, l3: int, return_discard: bool = False):
    """Real-basis coupling block [2l1+1, 2l2+1, 2l3+1] in page component order.

    Odd l1+l2+l3 blocks are purely imaginary; their imaginary part is returned.
    """
    lib = _load()
    out = np.empty((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1), dtype=np.float64)
    disc = ctypes.c_double(0.0)
    rc = lib.oracle_cg_real(l1, l2, l3, _p(out), ctypes.byref(disc))
    if rc < 0:
        raise ValueError("triple (%d,%d,%d) not allowed" % (l1, l2, l3))
    if return_discard:
        return out, disc.value
    return out


def paths(lmax: int, path_set: int = PATHS_PARITY) -> np.ndarray:
    """Path list [P, 3] of (l1, l2, l3) in canonical lexicographic order."""
    lib = _load()
    P = lib.oracle_paths(lmax, path_set, None)
    if P < 0:
        raise ValueError("bad lmax/path_set")
    out = np.empty((P, 3), dtype=np.int32)
    lib.oracle_paths(lmax, path_set, _p(out))
    return out


def envelope(d: float) -> float:
    return _load().oracle_envelope(float(d))


def radial_basis(r: float, r_cut: float, n_basis: int = 8) -> np.ndarray:
    R = np.empty(n_basis, dtype=np.float64)
    _load().oracle_radial_basis(float(r), float(r_cut), n_basis, _p(R))
    return R


def conv(N, vec, src, dst, x, w, lmax, path_set=PATHS_PARITY, weight_mode=0, r_cut=0.0,
         n_basis=8) -> np.ndarray:
    """fp64 convolution output [N, C, (lmax+1)^2] (see oracle_conv in the C source).

    ``x`` is [N, C, K] float32 (or float64: then vec and w are taken as float64
    too); ``w`` is [P, C] (weight_mode 0) or
    [n_basis, P*C] (weight_mode 1).  ``dst`` is one destination per edge; any
    edge order is accepted.
    """
    lib = _load()
    is64 = np.asarray(x).dtype == np.float64
    cast = _f64 if is64 else _f32
    v = cast(vec).reshape(-1, 3)
    s = _i32(src)
    d = _i32(dst)
    xx = cast(x)
    ww = cast(w)
    E = v.shape[0]
    C = xx.shape[1]
    K = (lmax + 1) ** 2
    if xx.shape != (N, C, K) or s.shape != (E,) or d.shape != (E,):
        raise ValueError("shape mismatch")
    out = np.empty((N, C, K), dtype=np.float64)
    fn = lib.oracle_conv_f64 if is64 else lib.oracle_conv
    rc = fn(N, E, lmax, C, path_set, weight_mode, float(r_cut), n_basis, _p(v), _p(s), _p(d), _p(xx), _p(ww),
            _p(out))
    if rc != 0:
        raise ValueError("oracle_conv failed (rc=%d)" % rc)
    return out


def round_bf16(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even), returned as float32."""
    lib = _load()
    flat = _f32(a).ravel()
    return np.array([lib.oracle_round_bf16(float(v)) for v in flat], dtype=np.float32).reshape(np.shape(a))


def linear(h, W, lmax: int, bf16: bool = False) -> np.ndarray:
    """fp64 per-l channel linear out[n,c',mu] = sum_c W[l(mu),c',c] h[n,c,mu].

    float64 ``h`` selects the double entry point (no bf16 option there)."""
    lib = _load()
    if np.asarray(h).dtype == np.float64:
        if bf16:
            raise ValueError("bf16 rounding applies to float32 inputs")
        hh, WW = _f64(h), _f64(W)
        N, C, K = hh.shape
        out = np.empty((N, C, K), dtype=np.float64)
        if lib.oracle_linear_f64(N, C, lmax, _p(hh), _p(WW), _p(out)) != 0:
            raise ValueError("oracle_linear_f64 failed")
        return out
    hh = _f32(h)
    WW = _f32(W)
    N, C, K = hh.shape
    if K != (lmax + 1) ** 2 or WW.shape != (lmax + 1, C, C):
        raise ValueError("shape mismatch")
    out = np.empty((N, C, K), dtype=np.float64)
    if lib.oracle_linear(N, C, lmax, 1 if bf16 else 0, _p(hh), _p(WW), _p(out)) != 0:
        raise ValueError("oracle_linear failed")
    return out


def sh_grad(vec, lmax: int):
    """(Y [E, K], G [E, K, 3]) from the polynomial route of oracle_sh_grad_f64:
    the harmonics again and their gradient with respect to the edge vector."""
    lib = _load()
    v = _f64(vec).reshape(-1, 3)
    K = (lmax + 1) ** 2
    Y = np.empty((v.shape[0], K), dtype=np.float64)
    G = np.empty((v.shape[0], K, 3), dtype=np.float64)
    if lib.oracle_sh_grad_f64(v.shape[0], _p(v), lmax, _p(Y), _p(G)) != 0:
        raise ValueError("oracle_sh_grad_f64: bad arguments")
    return Y, G


def conv_backward(N, vec, src, dst, x, w, gout, lmax, path_set=PATHS_PARITY):
    """(gx [N,C,K], gw [P,C], gvec [E,3]) fp64: gradients of sum(gout * out)
    for the fixed-weight convolution (see oracle_conv_backward in the C source).

    float64 ``x`` selects the double entry point (vec, w, gout taken as float64)."""
    lib = _load()
    is64 = np.asarray(x).dtype == np.float64
    cast = _f64 if is64 else _f32
    v = cast(vec).reshape(-1, 3)
    s = _i32(src)
    d = _i32(dst)
    xx, ww, gg = cast(x), cast(w), cast(gout)
    E = v.shape[0]
    C = xx.shape[1]
    K = (lmax + 1) ** 2
    P = paths(lmax, path_set).shape[0]
    if xx.shape != (N, C, K) or gg.shape != (N, C, K) or ww.shape != (P, C) or s.shape != (E,) or d.shape != (E,):
        raise ValueError("shape mismatch")
    gx = np.empty((N, C, K), dtype=np.float64)
    gw = np.empty((P, C), dtype=np.float64)
    gv = np.empty((E, 3), dtype=np.float64)
    fn = lib.oracle_conv_backward_f64 if is64 else lib.oracle_conv_backward
    rc = fn(N, E, lmax, C, path_set, _p(v), _p(s), _p(d), _p(xx), _p(ww), _p(gg), _p(gx), _p(gw), _p(gv))
    if rc != 0:
        raise ValueError("oracle_conv_backward failed (rc=%d)" % rc)
    return gx, gw, gv


def envelope_deriv(d: float) -> float:
    return _load().oracle_envelope_deriv(float(d))


def radial_basis_deriv(r: float, r_cut: float, n_basis: int = 8) -> np.ndarray:
    dR = np.empty(n_basis, dtype=np.float64)
    _load().oracle_radial_basis_deriv(float(r), float(r_cut), n_basis, _p(dR))
    return dR


def conv_backward_radial(N, vec, src, dst, x, W, gout, lmax, r_cut, path_set=PATHS_PARITY, n_basis=8,
                         need=(True, True, True)):
    """(gx [N,C,K], gW [n_basis, P*C], gvec [E,3]) fp64: gradients of
    sum(gout * out) for the radial-weight convolution (see
    oracle_conv_backward_radial in the C source); an output not in ``need``
    (x, W, vec) is None.  float64 ``x`` selects the double entry point."""
    lib = _load()
    is64 = np.asarray(x).dtype == np.float64
    cast = _f64 if is64 else _f32
    v = cast(vec).reshape(-1, 3)
    s = _i32(src)
    d = _i32(dst)
    xx, ww, gg = cast(x), cast(W), cast(gout)
    E = v.shape[0]
    C = xx.shape[1]
    K = (lmax + 1) ** 2
    P = paths(lmax, path_set).shape[0]
    if (xx.shape != (N, C, K) or gg.shape != (N, C, K) or ww.shape != (n_basis, P * C) or s.shape != (E,)
            or d.shape != (E,)):
        raise ValueError("shape mismatch")
    gx = np.empty((N, C, K), dtype=np.float64) if need[0] else None
    gW = np.empty((n_basis, P * C), dtype=np.float64) if need[1] else None
    gv = np.empty((E, 3), dtype=np.float64) if need[2] else None
    fn = lib.oracle_conv_backward_radial_f64 if is64 else lib.oracle_conv_backward_radial
    rc = fn(N, E, lmax, C, path_set, float(r_cut), n_basis, _p(v), _p(s), _p(d), _p(xx), _p(ww), _p(gg),
            _p(gx) if gx is not None else None, _p(gW) if gW is not None else None,
            _p(gv) if gv is not None else None)
    if rc != 0:
        raise ValueError("oracle_conv_backward_radial failed (rc=%d)" % rc)
    return gx, gW, gv


def messages(N, vec, src, x, w, lmax, path_set=PATHS_PARITY, weight_mode=0, r_cut=0.0, n_basis=8) -> np.ndarray:
    """fp64 per-edge messages [E, C, (lmax+1)^2] (see oracle_messages in the C source); float64 ``x``
    selects the double entry point."""
    lib = _load()
    is64 = np.asarray(x).dtype == np.float64
    cast = _f64 if is64 else _f32
    v = cast(vec).reshape(-1, 3)
    s = _i32(src)
    xx = cast(x)
    ww = cast(w)
    E = v.shape[0]
    C = xx.shape[1]
    K = (lmax + 1) ** 2
    if xx.shape != (N, C, K) or s.shape != (E,):
        raise ValueError("shape mismatch")
    out = np.empty((E, C, K), dtype=np.float64)
    fn = lib.oracle_messages_f64 if is64 else lib.oracle_messages
    rc = fn(N, E, lmax, C, path_set, weight_mode, float(r_cut), n_basis, _p(v), _p(s), _p(xx), _p(ww), _p(out))
    if rc != 0:
        raise ValueError("oracle_messages failed (rc=%d)" % rc)
    return out


def silu(t: float) -> float:
    return _load().oracle_silu(float(t))


def radial_mlp(vec, r_cut: float, W1, W2, n_basis: int = 8) -> np.ndarray:
    """phi [E, H] fp64: the radial network of every edge (see oracle_radial_mlp_f64)."""
    v = _f64(vec).reshape(-1, 3)
    w1, w2 = _f64(W1), _f64(W2)
    H = w2.shape[0]
    if w1.shape != (n_basis, H) or w2.shape != (H, H):
        raise ValueError("shape mismatch")
    phi = np.empty((v.shape[0], H), dtype=np.float64)
    if _load().oracle_radial_mlp_f64(v.shape[0], _p(v), float(r_cut), n_basis, H, _p(w1), _p(w2), _p(phi)) != 0:
        raise ValueError("oracle_radial_mlp_f64: bad arguments")
    return phi


def conv_basis(N, vec, src, dst, x, phi, W3, lmax, path_set=PATHS_PARITY) -> np.ndarray:
    """fp64 convolution [N, C, K] with per-edge weights w_e = phi_e W3 (see oracle_conv_basis_f64)."""
    v = _f64(vec).reshape(-1, 3)
    s, d = _i32(src), _i32(dst)
    xx, ph, w3 = _f64(x), _f64(phi), _f64(W3)
    E = v.shape[0]
    C = xx.shape[1]
    K = (lmax + 1) ** 2
    H = ph.shape[1] if ph.ndim == 2 else 0
    P = paths(lmax, path_set).shape[0]
    if xx.shape != (N, C, K) or ph.shape != (E, H) or w3.shape != (H, P * C):
        raise ValueError("shape mismatch")
    out = np.empty((N, C, K), dtype=np.float64)
    rc = _load().oracle_conv_basis_f64(N, E, lmax, C, path_set, H, _p(v), _p(s), _p(d), _p(xx), _p(ph), _p(w3),
                                       _p(out))
    if rc != 0:
        raise ValueError("oracle_conv_basis_f64 failed (rc=%d)" % rc)
    return out


def interaction(N, vec, src, dst, h, W_up, W1, W2, W3, W_out, lmax, r_cut, norm=1.0, path_set=PATHS_PARITY,
                n_basis=8) -> np.ndarray:
    """fp64 interaction layer output [N, C, K] (see oracle_interaction_f64); float64 ``h`` selects the
    double entry point (all weights taken as float64)."""
    lib = _load()
    is64 = np.asarray(h).dtype == np.float64
    cast = _f64 if is64 else _f32
    v = cast(vec).reshape(-1, 3)
    s, d = _i32(src), _i32(dst)
    hh, wu, w1, w2, w3, wo = cast(h), cast(W_up), cast(W1), cast(W2), cast(W3), cast(W_out)
    E = v.shape[0]
    C = hh.shape[1]
    K = (lmax + 1) ** 2
    H = w2.shape[0]
    P = paths(lmax, path_set).shape[0]
    if (hh.shape != (N, C, K) or wu.shape != (lmax + 1, C, C) or wo.shape != (lmax + 1, C, C)
            or w1.shape != (n_basis, H) or w2.shape != (H, H) or w3.shape != (H, P * C)):
        raise ValueError("shape mismatch")
    out = np.empty((N, C, K), dtype=np.float64)
    fn = lib.oracle_interaction_f64 if is64 else lib.oracle_interaction
    rc = fn(N, E, lmax, C, path_set, float(r_cut), n_basis, H, _p(v), _p(s), _p(d), _p(hh), _p(wu), _p(w1),
            _p(w2), _p(w3), _p(wo), float(norm), _p(out))
    if rc != 0:
        raise ValueError("oracle_interaction failed (rc=%d)" % rc)
    return out
