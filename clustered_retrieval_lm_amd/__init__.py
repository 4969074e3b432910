"""FlashHead output head for AMD Instinct MI355X (gfx950).

The compute path is libflashhead.so (hand-written HIP kernels behind a C ABI declared in
include/flashhead.h); this package holds its ctypes binding (``flashhead``), a
device-resident convenience wrapper (``head.DeviceHead``) and the build step (``build``).
"""
from .flashhead import (  # noqa: F401
    FH_BF16, FH_F32, FH_GREEDY, FH_INT4_G128, FH_SAMPLE, FlashHeadError, fh_desc, fh_outputs,
    flashhead_build_clusters, flashhead_build_clusters_workspace_bytes, flashhead_centroid_scores, flashhead_centroids,
    flashhead_centroids_bytes, flashhead_dense_forward, flashhead_dense_workspace_bytes, flashhead_forward,
    flashhead_last_error, flashhead_mc_marginal, flashhead_mc_marginal_workspace_bytes, flashhead_pack, flashhead_probe_logits, flashhead_select_and_probe, flashhead_select_probes,
    flashhead_version,
    flashhead_workspace_bytes, load_library, make_desc, make_outputs,
)
