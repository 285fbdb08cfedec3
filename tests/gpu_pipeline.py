"""Helpers of the GPU parity tests: run the HIP operator on a workload and bring every
intermediate back as numpy arrays.  Imports the binding only; oracle calls stay in the
tests themselves."""
from __future__ import annotations

import numpy as np
import torch

import free_block_sparse_sampled_amd as spr
from workloads import WorkloadConfig, batch_inputs


def op_config(cfg: WorkloadConfig, **kw) -> spr.OperatorConfig:
    base = dict(Ck=cfg.Ck, Cq=cfg.Cq, rK=cfg.rK, rQ=min(cfg.rQ, cfg.d), Ms=cfg.Ms, max_iters=cfg.max_iters,
                tol=cfg.tol, M=cfg.M, rho=cfg.rho, lam=cfg.lam, seed=0)
    base.update(kw)
    return spr.OperatorConfig(**base)


def device_inputs(cfg: WorkloadConfig, heads=None, step: int = 0):
    q, k, v = batch_inputs(cfg, heads, step)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    to = lambda x: torch.from_numpy(x).to(dt).cuda()  # noqa: E731
    return (q, k, v), (to(q), to(k), to(v))


def run_operator(cfg: WorkloadConfig, opc: spr.OperatorConfig, tq, tk, tv):
    op = spr.SparsePR(tq, opc, n_text=cfg.n_text, diagnostics=True, keep_scores=True, k=tk)
    op.run(tq, tk, tv)
    torch.cuda.synchronize()
    return op


def pull(op: spr.SparsePR) -> dict:
    """Everything the operator produced, as numpy (per flattened head on axis 0)."""
    out = {}
    for obj in (op.part, op.route):
        for name, val in vars(obj).items():
            if isinstance(val, torch.Tensor):
                out[name] = val.float().cpu().numpy() if val.dtype == torch.bfloat16 else val.cpu().numpy()
    out["o_sp"] = op.o_sp.cpu().numpy()
    out["o_probe"] = op.o_probe.cpu().numpy()
    out["out"] = op.out.float().cpu().numpy().reshape(op.o_sp.shape)
    out["head_status"] = op.head_status.cpu().numpy()
    out["fit_state"] = op.fit_state.cpu().numpy()
    return out


def row_rel_err(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row relative L2 error |a - b| / |b|."""
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)
