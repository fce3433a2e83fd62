"""The C-ABI library loads and exports every function include/eqtp.h
declares; host-only entry points and argument validation (no kernel
launches: every call here is rejected or answered before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eqtp.h")


def _lib():
    from spherical_harmonic_cg_amd import eqtp

    if not os.path.exists(eqtp.LIB_PATH):
        pytest.skip("libeqtp.so not built")
    return eqtp


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int|int64_t)\s+(eqtp_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_binding_names():
    from spherical_harmonic_cg_amd import eqtp

    assert _declared() == sorted(eqtp.EXPORTED)


def test_every_declared_symbol_is_exported():
    e = _lib()
    lib = ctypes.CDLL(e.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_num_paths_and_table_match_oracle():
    e = _lib()
    for L in range(7):
        for ps in (0, 1):
            assert e.eqtp_num_paths(L, ps) == len(oracle.paths(L, ps))
            np.testing.assert_array_equal(e.eqtp_path_table(L, ps), oracle.paths(L, ps))
    lib = e.load_library()
    assert lib.eqtp_num_paths(7, 0) == -e.EQTP_EUNSUPPORTED
    assert lib.eqtp_num_paths(3, 7) == -e.EQTP_EINVAL


def test_status_strings():
    e = _lib()
    for s in range(6):
        assert isinstance(e.eqtp_status_string(s), str)
    assert e.eqtp_status_string(1).startswith("EQTP_EINVAL")
    assert e.eqtp_status_string(e.EQTP_EGRAPH).startswith("EQTP_EGRAPH")


def test_check_graph_rejects_bad_arguments():
    e = _lib()
    lib = e.load_library()
    rep = FAKE
    assert lib.eqtp_check_graph(-1, 0, NULL, NULL, NULL, NULL, rep, NULL) == e.EQTP_EINVAL
    assert lib.eqtp_check_graph(4, -2, NULL, NULL, NULL, NULL, rep, NULL) == e.EQTP_EINVAL
    assert lib.eqtp_check_graph(1 << 31, 4, NULL, NULL, NULL, NULL, rep, NULL) == e.EQTP_EINVAL
    assert lib.eqtp_check_graph(4, 4, NULL, NULL, NULL, NULL, NULL, NULL) == e.EQTP_EINVAL
    assert lib.eqtp_check_graph(4, 4, NULL, NULL, NULL, NULL, ctypes.c_void_p(0x10002), NULL) == e.EQTP_EINVAL
    odd = ctypes.c_void_p(0x10001)
    for k in range(4):
        arrs = [NULL] * 4
        arrs[k] = odd
        assert lib.eqtp_check_graph(4, 4, *arrs, rep, NULL) == e.EQTP_EINVAL


def test_debug_switch_and_environment():
    import subprocess
    import sys

    e = _lib()
    was = e.eqtp_set_debug(True)
    try:
        assert e.eqtp_set_debug(True) is True
        lib = e.load_library()
        assert lib.eqtp_set_debug(7) == 1      # not 0 or 1: unchanged
        assert e.eqtp_set_debug(False) is True
        assert lib.eqtp_set_debug(-1) == 0
    finally:
        e.eqtp_set_debug(was)
    # the initial setting comes from EQTP_DEBUG when the library is loaded
    code = "import ctypes,sys; l=ctypes.CDLL(sys.argv[1]); print(l.eqtp_set_debug(0))"
    for val, want in (("1", "1"), ("yes", "1"), ("0", "0"), ("", "0"), (None, "0")):
        env = dict(os.environ)
        env.pop("EQTP_DEBUG", None)
        if val is not None:
            env["EQTP_DEBUG"] = val
        out = subprocess.run([sys.executable, "-c", code, e.LIB_PATH], env=env, capture_output=True, text=True,
                             timeout=120)
        assert out.returncode == 0, out.stderr
        assert out.stdout.strip() == want, (val, out.stdout)


def _desc(e, **kw):
    d = dict(lmax=3, C=64, path_set=0, weight_mode=0, edge_order=0, algo=0, r_cut=0.0, n_basis=8, x_dtype=0,
             out_dtype=0)
    d.update(kw)
    return e._ConvDesc(ctypes.sizeof(e._ConvDesc), d["lmax"], d["C"], d["path_set"], d["weight_mode"],
                       d["edge_order"], d["algo"], d["r_cut"], d["n_basis"], d["x_dtype"], d["out_dtype"])


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below is rejected first
NULL = ctypes.c_void_p(0)


@pytest.mark.parametrize("kw,want", [
    (dict(lmax=7), 2), (dict(lmax=-1), 1), (dict(lmax=4, algo=1), 2), (dict(lmax=4, algo=2), 2),
    (dict(lmax=4, weight_mode=1, r_cut=5.0), 2), (dict(lmax=4, x_dtype=1), 2), (dict(lmax=5, C=128, x_dtype=1), 2),
    (dict(lmax=6, C=128, algo=3, weight_mode=1, r_cut=5.0), 2), (dict(algo=3, weight_mode=1, r_cut=5.0, edge_order=1), 2), (dict(algo=3, weight_mode=1, r_cut=5.0, C=8), 2),
    (dict(lmax=4, algo=3, weight_mode=1, r_cut=5.0), 2), (dict(algo=3, x_dtype=1), 2), (dict(C=48), 2), (dict(C=0), 1), (dict(path_set=3), 1),
    (dict(weight_mode=2), 1), (dict(edge_order=5), 1), (dict(algo=9), 1),
    (dict(weight_mode=1, r_cut=0.0), 1), (dict(weight_mode=1, r_cut=5.0, n_basis=6), 2),
    (dict(weight_mode=1, r_cut=5.0, algo=1), 2), (dict(edge_order=1, algo=1), 2),
    # bf16 output: edges in any order on the per-edge walk only
    (dict(out_dtype=1), 2), (dict(out_dtype=1, edge_order=1, lmax=4), 2), (dict(out_dtype=1, edge_order=1, algo=3), 2),
    (dict(out_dtype=1, edge_order=1, algo=1), 2), (dict(out_dtype=1, weight_mode=1, r_cut=5.0), 2),
    (dict(out_dtype=2, edge_order=1), 1), (dict(out_dtype=-1), 1),
])
def test_conv_descriptor_validation(kw, want):
    e = _lib()
    lib = e.load_library()
    d = _desc(e, **kw)
    rc = lib.eqtp_conv_fused(ctypes.byref(d), 10, 20, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL)
    assert rc == want


def test_conv_pointer_and_size_validation():
    e = _lib()
    lib = e.load_library()
    d = _desc(e)
    call = lambda N, E, vec, src, dst, rp, x, w, out: lib.eqtp_conv_fused(ctypes.byref(d), N, E, vec, src, dst, rp,
                                                                          x, w, out, NULL)
    assert call(10, 20, FAKE, FAKE, NULL, FAKE, NULL, FAKE, FAKE) == 1      # x missing
    d5 = _desc(e, lmax=5, C=128)  # C = 128 above lmax 4 (two 64-channel halves) gets past the descriptor checks
    assert lib.eqtp_conv_fused(ctypes.byref(d5), 10, 20, FAKE, FAKE, NULL, FAKE, NULL, FAKE, FAKE, NULL) == 1
    assert call(10, 20, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE) == 1      # row_ptr missing (sorted)
    assert call(10, 20, NULL, FAKE, NULL, FAKE, FAKE, FAKE, FAKE) == 1      # vec missing
    assert call(-1, 20, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE) == 1      # negative N
    assert call(0, 20, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE) == 1       # edges without nodes
    assert call(1 << 31, 0, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE) == 1  # too many nodes
    mis = ctypes.c_void_p(0x10004)
    assert call(10, 20, FAKE, FAKE, NULL, FAKE, mis, FAKE, FAKE) == 1       # x not 16-byte aligned
    assert call(0, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 0        # empty problem: nothing to do
    du = _desc(e, edge_order=1)
    assert lib.eqtp_conv_fused(ctypes.byref(du), 10, 20, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, NULL) == 1
    bad = _desc(e)
    bad.struct_size = 4
    assert lib.eqtp_conv_fused(ctypes.byref(bad), 10, 20, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, NULL) == 1


def test_sh_and_linear_validation():
    e = _lib()
    lib = e.load_library()
    assert lib.eqtp_sh(FAKE, 10, 7, FAKE, NULL) == 2
    assert lib.eqtp_sh(FAKE, -1, 3, FAKE, NULL) == 1
    assert lib.eqtp_sh(NULL, 10, 3, FAKE, NULL) == 1
    assert lib.eqtp_sh(FAKE, 10, 3, ctypes.c_void_p(0x10008), NULL) == 1
    assert lib.eqtp_sh(NULL, 0, 3, NULL, NULL) == 0
    assert lib.eqtp_linear(10, 64, 3, 3, FAKE, FAKE, FAKE, NULL) == 1      # unknown dtype
    assert lib.eqtp_linear(10, 64, 3, 2, FAKE, FAKE, ctypes.c_void_p(0x10008), NULL) == 1  # out misaligned
    assert lib.eqtp_linear(10, 48, 3, 0, FAKE, FAKE, FAKE, NULL) == 2
    assert lib.eqtp_linear(10, 64, 3, 0, NULL, FAKE, FAKE, NULL) == 1
    assert lib.eqtp_linear(0, 64, 3, 0, NULL, NULL, NULL, NULL) == 0
    assert lib.eqtp_linear(10, 64, 7, 0, FAKE, FAKE, FAKE, NULL) == 2
    assert lib.eqtp_test_segment_probe(FAKE, FAKE, 10, 20, 64, 3, 0, FAKE, FAKE, NULL) == 1


def test_conv_backward_validation():
    e = _lib()
    lib = e.load_library()

    def call(d, N=10, E=20, vec=FAKE, src=FAKE, dst=NULL, rp=FAKE, x=FAKE, w=FAKE, g=FAKE, gx=FAKE, gw=FAKE,
             gv=FAKE):
        return lib.eqtp_conv_backward(ctypes.byref(d), N, E, vec, src, dst, rp, x, w, g, gx, gw, gv, NULL)

    assert call(_desc(e, weight_mode=1, r_cut=0.0)) == 1                 # radial weights need r_cut > 0
    assert call(_desc(e, weight_mode=1, r_cut=5.0, n_basis=6)) == 2      # radial: 8 basis functions only
    assert call(_desc(e, weight_mode=1, r_cut=5.0, C=8)) == 2            # radial: C a multiple of 16
    assert call(_desc(e, weight_mode=1, r_cut=5.0), x=NULL) == 1
    assert call(_desc(e, weight_mode=1, r_cut=5.0, edge_order=1), rp=NULL) == 1
    assert call(_desc(e, weight_mode=2)) == 1
    assert call(_desc(e, lmax=7)) == 2                                   # above lmax 6
    assert call(_desc(e, lmax=4, weight_mode=1, r_cut=5.0)) == 2         # radial weights: lmax 0..3
    assert call(_desc(e, lmax=5, C=128), x=NULL) == 1                    # C = 128 at lmax 5 (two halves) passes
    assert call(_desc(e, algo=7)) == 1                                   # unknown algorithm
    assert call(_desc(e, C=48)) == 2
    assert call(_desc(e, path_set=2)) == 1
    assert call(_desc(e), gx=NULL, gw=NULL, gv=NULL) == 1                 # nothing requested
    assert call(_desc(e), x=NULL) == 1
    assert call(_desc(e), g=NULL) == 1
    assert call(_desc(e), vec=NULL) == 1
    assert call(_desc(e), rp=NULL) == 1                                   # sorted without row_ptr
    assert call(_desc(e, edge_order=1), rp=NULL) == 1                     # unsorted without dst
    assert call(_desc(e), gx=ctypes.c_void_p(0x10004)) == 1               # grad_x not 16-byte aligned
    assert call(_desc(e), N=0) == 1                                       # edges without nodes
    bad = _desc(e)
    bad.struct_size = 8
    assert call(bad) == 1


def test_conv_messages_validation():
    e = _lib()
    lib = e.load_library()

    def call(d, N=10, E=20, vec=FAKE, src=FAKE, x=FAKE, w=FAKE, m=FAKE):
        return lib.eqtp_conv_messages(ctypes.byref(d), N, E, vec, src, x, w, m, NULL)

    assert call(_desc(e, lmax=7)) == 2
    assert call(_desc(e, lmax=4, weight_mode=1, r_cut=4.0)) == 2          # edge-aligned form: fixed weights
    assert call(_desc(e, algo=3, weight_mode=1, r_cut=4.0)) == 2
    assert call(_desc(e, lmax=5, C=128), m=NULL) == 1                     # C = 128 at lmax 5 is supported
    assert call(_desc(e, lmax=5), m=NULL) == 1
    assert call(_desc(e, C=24)) == 2
    assert call(_desc(e, weight_mode=1, r_cut=0.0)) == 1
    assert call(_desc(e, weight_mode=1, r_cut=4.0, n_basis=4)) == 2
    assert call(_desc(e), m=NULL) == 1
    assert call(_desc(e), x=NULL) == 1
    assert call(_desc(e), m=ctypes.c_void_p(0x10008)) == 1               # messages not 16-byte aligned
    assert call(_desc(e), N=0) == 1                                       # edges without nodes
    assert call(_desc(e), E=0, vec=NULL, src=NULL, m=NULL) == 0           # no edges: nothing to do


def test_descriptor_versions_and_feature_dtype():
    e = _lib()
    lib = e.load_library()
    assert ctypes.sizeof(e._ConvDesc) == 44
    conv = lambda d, **kw: lib.eqtp_conv_fused(ctypes.byref(d), 10, 20, FAKE, FAKE, kw.get("dst", NULL),
                                               kw.get("rp", FAKE), FAKE, FAKE, FAKE, NULL)
    v1 = _desc(e, lmax=7)
    v1.struct_size = 36  # a descriptor from before the x_dtype field: accepted, read as fp32 features
    assert conv(v1) == 2
    v1b = _desc(e, lmax=7, x_dtype=1)
    v1b.struct_size = 36  # x_dtype lies past struct_size, so it is not read
    assert conv(v1b) == 2
    assert conv(_desc(e, x_dtype=7)) == 1
    assert conv(_desc(e, x_dtype=1, algo=3)) == 2                               # bf16: not the edge-aligned form
    assert conv(_desc(e, x_dtype=1, lmax=4)) == 2                               # bf16: lmax <= 3 only
    assert conv(_desc(e, x_dtype=1, weight_mode=1, r_cut=4.0, algo=3)) == 2
    bf = _desc(e, x_dtype=1)
    assert lib.eqtp_conv_messages(ctypes.byref(bf), 10, 20, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == 2
    assert lib.eqtp_conv_backward(ctypes.byref(bf), 10, 20, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, NULL) == 2
    # size 40: a descriptor from before out_dtype -- x_dtype is read, out_dtype is not
    v2 = _desc(e, lmax=7, out_dtype=9)
    v2.struct_size = 40
    assert conv(v2) == 2
    v2.x_dtype = 7
    assert conv(v2) == 1
    assert conv(_desc(e, lmax=7, out_dtype=9)) == 1                             # current size: out_dtype read
    # bf16 output: the fused convolution with edges in any order only
    ob = _desc(e, out_dtype=1)
    assert lib.eqtp_conv_messages(ctypes.byref(ob), 10, 20, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == 2
    assert lib.eqtp_conv_backward(ctypes.byref(ob), 10, 20, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, NULL) == 2
    assert lib.eqtp_conv_backward_by_source(ctypes.byref(ob), 10, 20, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, NULL) == 2
    ob5 = _desc(e, out_dtype=5)
    assert lib.eqtp_conv_messages(ctypes.byref(ob5), 10, 20, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == 1
    ws = _desc(e, out_dtype=1, edge_order=1)  # the workspace call groups the edges: dst-sorted, so fp32 only
    assert lib.eqtp_conv_fused_ws(ctypes.byref(ws), 10, 20, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE,
                                  1 << 20, NULL) == 2


def test_stable_sort_validation():
    e = _lib()
    lib = e.load_library()
    assert lib.eqtp_sort_workspace_bytes(-1, 5) == -e.EQTP_EINVAL
    assert lib.eqtp_sort_workspace_bytes(5, -1) == -e.EQTP_EINVAL
    need = lib.eqtp_sort_workspace_bytes(1000, 20000)
    assert need >= 3 * 20000 * 4 and need % 256 == 0
    call = lambda N, E, dst=FAKE, vec=NULL, src=NULL, rp=FAKE, perm=FAKE, vs=NULL, ss=NULL, ws=FAKE, nb=need: \
        lib.eqtp_sort_edges_stable(N, E, dst, vec, src, rp, perm, vs, ss, ws, nb, NULL)
    assert call(1000, 20000, nb=need - 1) == 1                  # short workspace
    assert call(1000, 20000, ws=NULL) == 1                      # no workspace
    assert call(1000, 20000, ws=ctypes.c_void_p(0x10004)) == 1  # workspace not 16-byte aligned
    assert call(1000, 20000, perm=NULL) == 1
    assert call(1000, 20000, dst=NULL) == 1
    assert call(1000, 20000, rp=NULL) == 1
    assert call(1000, 20000, vs=FAKE) == 1                      # vec_sorted without vec
    assert call(1000, 20000, ss=FAKE) == 1                      # src_sorted without src
    assert call(0, 5) == 1                                      # edges without nodes
    assert call(-1, 0) == 1


def test_sort_edges_validation():
    e = _lib()
    lib = e.load_library()
    call = lambda N, E, dst=FAKE, vec=NULL, src=NULL, rp=FAKE, perm=FAKE, vs=NULL, ss=NULL: lib.eqtp_sort_edges(
        N, E, dst, vec, src, rp, perm, vs, ss, NULL)
    assert call(-1, 5) == 1
    assert call(0, 5) == 1                 # edges without nodes
    assert call(10, 5, rp=NULL) == 1
    assert call(10, 5, dst=NULL) == 1
    assert call(10, 5, perm=NULL) == 1
    assert call(10, 5, vs=FAKE) == 1       # sorted vectors requested without input vectors
    assert call(10, 5, ss=FAKE) == 1
    assert call(0, 0, dst=NULL, rp=NULL, perm=NULL) == 1  # row_ptr has N + 1 >= 1 entries
    assert call((1 << 31) - 1, 0) == 1


def test_conv_backward_by_source_validation():
    e = _lib()
    lib = e.load_library()

    def call(d, N=10, E=20, vec=FAKE, dst=FAKE, sp=FAKE, x=FAKE, w=FAKE, g=FAKE, gx=FAKE, gw=FAKE, perm=NULL,
             gv=NULL):
        return lib.eqtp_conv_backward_by_source(ctypes.byref(d), N, E, vec, dst, sp, x, w, g, gx, gw, perm, gv,
                                                NULL)

    assert call(_desc(e, weight_mode=1, r_cut=0.0)) == 1                 # radial weights need r_cut > 0
    assert call(_desc(e, weight_mode=1, r_cut=5.0, n_basis=6)) == 2      # radial: 8 basis functions only
    assert call(_desc(e, weight_mode=1, r_cut=5.0, C=8)) == 2            # radial: C a multiple of 16
    assert call(_desc(e, weight_mode=1, r_cut=5.0, lmax=4)) == 2         # radial: lmax 0..3
    assert call(_desc(e, weight_mode=1, r_cut=5.0), x=NULL, gw=NULL) == 1  # the walk reads x
    assert call(_desc(e, lmax=7)) == 2                                   # above lmax 6
    assert call(_desc(e, lmax=5, C=128), x=NULL) == 1                    # C = 128 at lmax 5 (two halves) passes
    assert call(_desc(e, algo=7)) == 1                                   # unknown algorithm
    assert call(_desc(e, C=48)) == 2
    assert call(_desc(e, x_dtype=1)) == 2                                  # bf16 features
    assert call(_desc(e, path_set=2)) == 1
    assert call(_desc(e), gx=NULL, gw=NULL) == 1                          # nothing requested
    assert call(_desc(e), gx=NULL, gw=NULL, gv=FAKE) == 1                 # grad_vec needs perm
    assert call(_desc(e), gx=NULL, gw=NULL, gv=FAKE, perm=FAKE, x=NULL) == 1  # grad_vec needs x
    assert call(_desc(e), gv=ctypes.c_void_p(0x10002), perm=FAKE) == 1    # grad_vec not 4-byte aligned
    assert call(_desc(e), x=NULL) == 1                                    # grad_w needs x
    assert call(_desc(e), g=NULL) == 1
    assert call(_desc(e), sp=NULL) == 1
    assert call(_desc(e), vec=NULL) == 1
    assert call(_desc(e), dst=NULL) == 1
    assert call(_desc(e), w=NULL) == 1
    assert call(_desc(e), gx=ctypes.c_void_p(0x10004)) == 1               # grad_x not 16-byte aligned
    assert call(_desc(e), g=ctypes.c_void_p(0x10004)) == 1                # grad_out not 16-byte aligned
    assert call(_desc(e), N=0) == 1                                       # edges without nodes
    assert call(_desc(e), N=-1) == 1


def test_edge_rows_validation():
    e = _lib()
    lib = e.load_library()
    assert lib.eqtp_edge_rows(-1, 5, FAKE, FAKE, NULL) == 1
    assert lib.eqtp_edge_rows(0, 5, FAKE, FAKE, NULL) == 1
    assert lib.eqtp_edge_rows(10, 5, NULL, FAKE, NULL) == 1
    assert lib.eqtp_edge_rows(10, 5, FAKE, NULL, NULL) == 1
    assert lib.eqtp_edge_rows(10, 5, ctypes.c_void_p(0x10002), FAKE, NULL) == 1
    assert lib.eqtp_edge_rows(10, 0, NULL, NULL, NULL) == 0                # nothing to do, nothing launched


def test_conv_ws_validation():
    e = _lib()
    lib = e.load_library()
    d = _desc(e, edge_order=1)
    need = lib.eqtp_conv_workspace_bytes(ctypes.byref(d), 100, 1000)
    al = lambda b: (b + 255) // 256 * 256
    # row pointers, five E-int regions of the radix sort, its digit counts (512 bins x (tiles + 1) + 1;
    # tiles of 256 x rounds edges, rounds = E / (256 * 512) clamped to 1..16)
    assert need == al(101 * 4) + 5 * al(1000 * 4) + al((512 * (4 + 1) + 1) * 4)
    big = lib.eqtp_conv_workspace_bytes(ctypes.byref(d), 100000, 5239100)
    assert big == al(100001 * 4) + 5 * al(5239100 * 4) + al((512 * ((5239100 + 4095) // 4096 + 1) + 1) * 4)
    assert big < (128 << 20)     # the large workload in random order fits the no-allocation scratch
    assert lib.eqtp_conv_workspace_bytes(ctypes.byref(_desc(e)), 100, 1000) == 0   # dst-sorted: none
    assert lib.eqtp_conv_workspace_bytes(ctypes.byref(d), -1, 10) == -1
    assert lib.eqtp_conv_workspace_bytes(ctypes.byref(d), 0, 0) == 0
    call = lambda ws, nb, dd=d: lib.eqtp_conv_fused_ws(ctypes.byref(dd), 100, 1000, FAKE, FAKE, FAKE, NULL, FAKE,
                                                        FAKE, FAKE, ws, nb, NULL)
    assert call(NULL, need) == 1                                  # no workspace
    assert call(FAKE, need - 1) == 1                              # short workspace
    assert call(ctypes.c_void_p(0x10008), need) == 1              # misaligned workspace
    assert lib.eqtp_conv_fused_ws(ctypes.byref(d), 100, 1000, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, need,
                                  NULL) == 1                      # no dst


def test_noalloc_refuses_beyond_its_scratch():
    e = _lib()
    lib = e.load_library()
    d = _desc(e, edge_order=1)
    assert lib.eqtp_conv_workspace_bytes(ctypes.byref(d), 100000, 10000000) > (128 << 20)
    assert lib.eqtp_conv_fused_noalloc(ctypes.byref(d), 100000, 10000000, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE,
                                       NULL) == e.EQTP_ETOOLARGE
    assert lib.eqtp_conv_fused_noalloc(ctypes.byref(d), -1, 10, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE,
                                       NULL) == 1
    assert b"scratch" in lib.eqtp_status_string(e.EQTP_ETOOLARGE)


def test_interaction_validation():
    e = _lib()
    lib = e.load_library()

    def desc(**kw):
        d = dict(lmax=3, C=64, path_set=0, r_cut=5.0, n_basis=8, hidden=64, norm=1.0)
        d.update(kw)
        return e._InteractionDesc(ctypes.sizeof(e._InteractionDesc), d["lmax"], d["C"], d["path_set"], d["r_cut"],
                                  d["n_basis"], d["hidden"], d["norm"])

    def call(d, N=10, E=20, vec=FAKE, src=FAKE, rp=FAKE, h=FAKE, ws=FAKE, wsb=1 << 40, out=FAKE):
        return lib.eqtp_interaction(ctypes.byref(d), N, E, vec, src, rp, h, FAKE, FAKE, FAKE, FAKE, FAKE, out, ws,
                                    wsb, NULL)

    assert call(desc(lmax=4)) == 2
    assert call(desc(C=48)) == 2
    assert call(desc(C=8)) == 2               # C a multiple of 16
    assert call(desc(hidden=32)) == 2
    assert call(desc(n_basis=6)) == 2
    assert call(desc(norm=0.0)) == 1
    assert call(desc(r_cut=0.0)) == 1
    assert call(desc(path_set=2)) == 1
    assert call(desc(), ws=NULL) == 1
    assert call(desc(), wsb=100) == 1         # workspace too small
    assert call(desc(), h=NULL) == 1
    assert call(desc(), rp=NULL) == 1
    assert call(desc(), vec=NULL) == 1
    assert call(desc(), out=ctypes.c_void_p(0x10004)) == 1
    assert call(desc(), N=0) == 1             # edges without nodes
    assert call(desc(), N=0, E=0) == 0        # nothing to do
    bad = desc()
    bad.struct_size = 8
    assert call(bad) == 1
    assert lib.eqtp_interaction_workspace_bytes(ctypes.byref(desc(lmax=4)), 10, 20) == -2
    n = lib.eqtp_interaction_workspace_bytes(ctypes.byref(desc()), 10, 20)
    assert n >= 2 * 10 * 64 * 16 * 4 + 20 * 64 * 4 and n % 256 == 0
