"""MI355X (gfx950) implementation of SparsePR's per-call sparse attention operator.

The operator runs in libsparsepr (HIP kernels behind the C ABI of include/sparsepr.h);
this package holds the build script and a thin ctypes binding with the same call names.
"""
from .sparsepr import (  # noqa: F401
    OperatorConfig, Partition, Route, SparsePR, SparsePRError, dense_workspace, library, make_desc,
    probe_workspace, sparsepr_attn_dense, sparsepr_attn_dense_noalloc,
    sparsepr_attn_sparse, sparsepr_fit_correct, sparsepr_kmeans, sparsepr_partition, sparsepr_probe_exact,
    sparsepr_route, sparsepr_workspace_size, warm_state,
)
