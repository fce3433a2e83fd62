"""MI355X (gfx950) equivariant convolution: fused real spherical harmonics ->
Clebsch-Gordan tensor product -> destination sum, a per-l channel linear, and
the standalone harmonics, as hand-written HIP kernels behind a C ABI
(include/eqtp.h).  ``eqtp`` is the Python binding, ``autograd`` wraps the
convolution and its gradients as a torch.autograd.Function; ``synth`` builds
seeded synthetic workloads."""
from .eqtp import (EQTP_ALGO_AUTO, EQTP_ALGO_EDGE_SO2, EQTP_ALGO_EDGE_VALU, EQTP_ALGO_NODE_MFMA, EQTP_BF16, EQTP_EDGES_DST_SORTED,
                   EQTP_CHECK_WORDS, EQTP_EDGES_UNSORTED, EQTP_EGRAPH, EQTP_EHIP, EQTP_EINVAL, EQTP_ETOOLARGE, EQTP_EUNSUPPORTED, EQTP_F32, EQTP_F32_BF16, EQTP_OK,
                   EQTP_PATHS_PARITY, EQTP_PATHS_SO3, EQTP_W_FIXED, EQTP_W_RADIAL, EqtpError, eqtp_conv_backward,
                   eqtp_check_graph, eqtp_conv_backward_by_source, eqtp_conv_fused, eqtp_conv_fused_noalloc, eqtp_conv_fused_ws,
                   eqtp_conv_messages,
                   eqtp_conv_workspace_bytes, eqtp_edge_rows, eqtp_interaction, eqtp_interaction_workspace_bytes, eqtp_linear,
                   eqtp_num_paths, eqtp_path_table, eqtp_set_debug, eqtp_sh, eqtp_sort_edges, eqtp_sort_edges_stable, eqtp_sort_workspace_bytes,
                   eqtp_status_string,
                   eqtp_test_segment_probe, load_library)
