"""The allocation-free dense call against sparsepr_attn_dense, through the C ABI (GPU).

sparsepr_attn_dense_noalloc runs the dense kernels on the library's fixed device scratch; its
output must match the workspace entry point's on the same inputs, within the attention parity bar
(2e-3 relative L2 per row), on two calls in a row of which the second is smaller, so that it
also runs on scratch the first call left behind."""
import numpy as np
import pytest
import torch

import free_block_sparse_sampled_amd as spr
from tests.gpu_pipeline import row_rel_err
from workloads import batch_inputs, config

pytestmark = pytest.mark.gpu

ROW_TOL = 2e-3


def _case(cfg, step):
    q, k, v = batch_inputs(cfg, step=step)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return tuple(torch.from_numpy(x).to(dt).cuda() for x in (q, k, v))


def test_dense_noalloc_matches_dense_on_two_calls():
    big = config("small").with_(H=8)                                   # 8 heads, N = 8192, d = 128
    small = config("small").with_(H=2, grid=(2, 25, 40), d=64)         # 2 heads, N = 2000, d = 64
    for cfg, step in ((big, 0), (small, 1)):
        q, k, v = _case(cfg, step)
        desc = spr.make_desc(q)
        assert spr.sparsepr.library().sparsepr_dense_workspace_size(desc) <= spr.sparsepr.NOALLOC_SCRATCH_BYTES
        shape = (cfg.B, cfg.H, cfg.N, cfg.d)
        out_ref = torch.empty(shape, dtype=torch.float32, device="cuda")
        spr.sparsepr_attn_dense(desc, q, k, v, out_ref)
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        spr.sparsepr_attn_dense_noalloc(desc, q, k, v, out)
        torch.cuda.synchronize()
        a = out.reshape(-1, cfg.d).cpu().numpy().astype(np.float64)
        b = out_ref.reshape(-1, cfg.d).cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a))
        err = row_rel_err(a, b)
        assert err.max() < ROW_TOL, (cfg.name, cfg.H, cfg.N, cfg.d, err.max())
