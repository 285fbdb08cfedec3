"""ctypes binding of libsparsepr (include/sparsepr.h).

Argument marshalling only: torch tensors provide device memory and the current HIP
stream; every step of the operator runs in the library's HIP kernels.  The library must
have been built (``python -m free_block_sparse_sampled_amd.build``); nothing here falls
back to another implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparsepr.so")

SPR_BF16, SPR_F32 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP launch failed",
          5: "problem exceeds the fixed scratch of the allocation-free call"}
HS_BITS = {1: "cholesky_fallback", 2: "budget_unreached", 4: "kv_groups_empty", 8: "q_groups_empty", 16: "rms_floor",
           32: "eigen_noconv"}

P = ctypes.c_void_p


class spr_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("n_text", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("sn", ctypes.c_int64),
                ("Hkv", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("ksb", ctypes.c_int64), ("ksh", ctypes.c_int64), ("ksn", ctypes.c_int64)]


class spr_part_params(ctypes.Structure):
    _fields_ = [("Ck", ctypes.c_int32), ("Cq", ctypes.c_int32), ("rK", ctypes.c_int32), ("rQ", ctypes.c_int32),
                ("Ms", ctypes.c_int32), ("max_iters", ctypes.c_int32), ("tol", ctypes.c_double),
                ("rms_eps", ctypes.c_double), ("eig_clamp", ctypes.c_double), ("seed", ctypes.c_uint64),
                ("mode", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_PART_FIELDS = ["kv_label", "q_label", "kv_perm", "q_perm", "q_pos", "kv_off", "q_off", "n_kv", "n_q", "kbar",
                "vbar", "qbar", "qdist", "FK", "FQ", "Qp", "Kp", "Vp", "phiK", "phiQ", "cK_last", "cQ_last", "passes"]
_ROUTE_FIELDS = ["sel_cnt", "sel_kv", "probe_idx", "probe_w", "pairs", "rho_exec", "scores", "score_err"]


class spr_partition(ctypes.Structure):
    _fields_ = [(n, P) for n in _PART_FIELDS]


class spr_route(ctypes.Structure):
    _fields_ = [(n, P) for n in _ROUTE_FIELDS]


_WARM_FIELDS = ["FK", "FQ", "kbar", "qbar", "n_kv", "n_q"]


class spr_warm(ctypes.Structure):
    _fields_ = [(n, P) for n in _WARM_FIELDS]


class spr_probe_options(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class spr_fit_options(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("out_rank", ctypes.c_int32)]


# spr_probe_mode and spr_fit_family of include/sparsepr.h
PROBE_MODES = {"stratified": 0, "random": 1, "uniform": 2}
FIT_FAMILIES = {"full": 0, "mean": 1, "scalar": 2, "diag": 3}
PART_MODES = {"response": 0, "semantic": 1, "key_response": 2}


class SparsePRError(RuntimeError):
    pass


_lib = None


def library():
    """Load libsparsepr.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SparsePRError(f"{LIB_PATH} is missing: build it with `python -m free_block_sparse_sampled_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        lib.sparsepr_workspace_size.argtypes = [ctypes.POINTER(spr_desc), ctypes.POINTER(spr_part_params), ctypes.c_int32]
        lib.sparsepr_workspace_size.restype = ctypes.c_size_t
        lib.sparsepr_partition.argtypes = [ctypes.POINTER(spr_desc), P, P, P, ctypes.POINTER(spr_part_params),
                                           ctypes.POINTER(spr_warm), ctypes.POINTER(spr_partition), P,
                                           ctypes.c_size_t, P]
        lib.sparsepr_partition.restype = st
        lib.sparsepr_route.argtypes = [ctypes.POINTER(spr_desc), ctypes.POINTER(spr_part_params),
                                       ctypes.POINTER(spr_partition), ctypes.c_double, ctypes.c_int32,
                                       ctypes.POINTER(spr_probe_options), ctypes.POINTER(spr_route), P,
                                       ctypes.c_size_t, P]
        lib.sparsepr_route.restype = st
        lib.sparsepr_attn_sparse.argtypes = [ctypes.POINTER(spr_desc), ctypes.POINTER(spr_part_params),
                                             ctypes.POINTER(spr_partition), ctypes.POINTER(spr_route), P, P,
                                             ctypes.c_size_t, P]
        lib.sparsepr_attn_sparse.restype = st
        lib.sparsepr_probe_exact.argtypes = [ctypes.POINTER(spr_desc), P, P, P, P, ctypes.c_int32, P, P,
                                             ctypes.c_size_t, P]
        lib.sparsepr_probe_exact.restype = st
        lib.sparsepr_fit_correct.argtypes = [ctypes.POINTER(spr_desc), ctypes.POINTER(spr_part_params),
                                             ctypes.POINTER(spr_partition), ctypes.POINTER(spr_route), P, P,
                                             ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                             ctypes.POINTER(spr_fit_options), P, ctypes.c_int32, P, P, P,
                                             ctypes.c_size_t, P]
        lib.sparsepr_fit_correct.restype = st
        lib.sparsepr_attn_dense.argtypes = [ctypes.POINTER(spr_desc), P, P, P, P, ctypes.c_int32, P, ctypes.c_size_t,
                                            P]
        lib.sparsepr_attn_dense.restype = st
        lib.sparsepr_attn_dense_noalloc.argtypes = [ctypes.POINTER(spr_desc), P, P, P, P, ctypes.c_int32, P]
        lib.sparsepr_attn_dense_noalloc.restype = st
        lib.sparsepr_dense_workspace_size.argtypes = [ctypes.POINTER(spr_desc)]
        lib.sparsepr_dense_workspace_size.restype = ctypes.c_size_t
        lib.sparsepr_probe_workspace_size.argtypes = [ctypes.POINTER(spr_desc), ctypes.c_int32]
        lib.sparsepr_probe_workspace_size.restype = ctypes.c_size_t
        lib.sparsepr_kmeans.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                        ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P, P, P, P,
                                        ctypes.c_size_t, P]
        lib.sparsepr_kmeans.restype = st
        lib.sparsepr_kmeans_workspace_size.argtypes = [ctypes.c_int32] * 4
        lib.sparsepr_kmeans_workspace_size.restype = ctypes.c_size_t
        lib.sparsepr_status_string.argtypes = [ctypes.c_int]
        lib.sparsepr_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


EXPORTED = ["sparsepr_workspace_size", "sparsepr_partition", "sparsepr_route", "sparsepr_attn_sparse",
            "sparsepr_probe_exact", "sparsepr_probe_workspace_size", "sparsepr_fit_correct", "sparsepr_attn_dense",
            "sparsepr_dense_workspace_size", "sparsepr_attn_dense_noalloc", "sparsepr_kmeans",
            "sparsepr_kmeans_workspace_size", "sparsepr_status_string"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # SPR_NOALLOC_SCRATCH_BYTES


def _check(status: int, what: str):
    if status != 0:
        raise SparsePRError(f"{what}: {STATUS.get(status, status)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclasses.dataclass
class OperatorConfig:
    """Hyperparameters of one operator call (defaults: Table C.1 of the paper's App. C.2)."""
    Ck: int = 1000
    Cq: int = 300
    rK: int = 48
    rQ: int = 64
    Ms: int = 2048
    max_iters: int = 25
    tol: float = 1e-4
    rms_eps: float = 1e-6
    eig_clamp: float = 1e-6
    seed: int = 0
    M: int = 64
    rho: float = 0.22
    lam: float = 1.0
    std_eps: float = 1e-6
    probe_mode: str = "stratified"  # Table 4: "stratified" | "random" | "uniform"
    fit_family: str = "full"        # App. D.4: "full" | "mean" | "scalar" | "diag"
    out_rank: int = 0               # App. D.3 output truncation rank; 0: none
    partition_mode: str = "response"  # Sec. 3.1, Table 2: "response" | "semantic" | "key_response"

    def coord_ranks(self, d: int):
        """Ranks of the K/V and query k-means coordinates (raw activations have rank d)."""
        rK = d if self.partition_mode == "semantic" else self.rK
        rQ = self.rQ if self.partition_mode == "response" else d
        return rK, rQ

    def probe_options(self) -> spr_probe_options:
        return spr_probe_options(PROBE_MODES[self.probe_mode], self.seed)

    def fit_options(self) -> spr_fit_options:
        return spr_fit_options(FIT_FAMILIES[self.fit_family], self.out_rank)

    def part_params(self) -> spr_part_params:
        return spr_part_params(self.Ck, self.Cq, self.rK, self.rQ, self.Ms, self.max_iters, self.tol, self.rms_eps,
                               self.eig_clamp, self.seed, PART_MODES[self.partition_mode], 0)


def make_desc(q: torch.Tensor, n_text: int = 0, k: Optional[torch.Tensor] = None) -> spr_desc:
    """Descriptor of a [B, H, N, d] tensor (any strides with a contiguous last dim).

    With ``k`` of shape [B, Hkv, N, d], Hkv < H dividing H, the descriptor is that of grouped-query
    attention: k and v (same strides as k) hold Hkv heads, each shared by H / Hkv query heads."""
    if q.dim() != 4 or q.stride(3) != 1:
        raise SparsePRError("q, k, v must be [B, H, N, d] with a contiguous last dimension")
    dt = {torch.bfloat16: SPR_BF16, torch.float32: SPR_F32}.get(q.dtype)
    if dt is None:
        raise SparsePRError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    desc = spr_desc(B, H, N, d, n_text, dt, q.stride(0), q.stride(1), q.stride(2))
    if k is not None and k.shape[1] != H:
        if k.dim() != 4 or k.stride(3) != 1 or (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d):
            raise SparsePRError("k, v must be [B, Hkv, N, d] with a contiguous last dimension")
        desc.Hkv = k.shape[1]
        desc.ksb, desc.ksh, desc.ksn = k.stride(0), k.stride(1), k.stride(2)
    return desc


def kv_heads(desc: spr_desc) -> int:
    """K/V heads per batch entry of a descriptor."""
    return desc.Hkv if 0 < desc.Hkv < desc.H else desc.H


class Partition:
    """Device buffers of sparsepr_partition's outputs."""

    def __init__(self, desc: spr_desc, cfg: OperatorConfig, device, diagnostics: bool = False):
        BH, N, d = desc.B * desc.H, desc.N, desc.d
        BHkv = desc.B * kv_heads(desc)  # K/V-side arrays are per K/V head
        Nv = N - desc.n_text
        i32, f64 = torch.int32, torch.float64
        dt = torch.bfloat16 if desc.dtype == SPR_BF16 else torch.float32
        z = lambda shape, t: torch.empty(shape, dtype=t, device=device)  # noqa: E731
        self.kv_label = z((BHkv, Nv), i32)
        self.q_label = z((BH, Nv), i32)
        self.kv_perm = z((BHkv, Nv), i32)
        self.q_perm = z((BH, Nv), i32)
        self.q_pos = z((BH, Nv), i32)
        self.kv_off = z((BHkv, cfg.Ck + 1), i32)
        self.q_off = z((BH, cfg.Cq + 1), i32)
        self.n_kv = z((BHkv,), i32)
        self.n_q = z((BH,), i32)
        self.kbar = z((BHkv, cfg.Ck, d), f64)
        self.vbar = z((BHkv, cfg.Ck, d), f64)
        self.qbar = z((BH, cfg.Cq, d), f64)
        self.qdist = z((BH, Nv), f64)
        self.FK = z((BHkv, d, cfg.rK), f64)
        self.FQ = z((BHkv, d, cfg.rQ), f64)
        self.Qp = z((BH, N, d), dt)
        self.Kp = z((BHkv, N, d), dt)
        self.Vp = z((BHkv, N, d), dt)
        self.phiK = self.phiQ = self.cK_last = self.cQ_last = self.passes = None
        if diagnostics:
            rK, rQ = cfg.coord_ranks(d)
            self.phiK = z((BHkv, Nv, rK), f64)
            self.phiQ = z((BH, Nv, rQ), f64)
            self.cK_last = z((BHkv, cfg.Ck, rK), f64)
            self.cQ_last = z((BH, cfg.Cq, rQ), f64)
            self.passes = z((BH, 2), i32)
        self.struct = spr_partition(*[_ptr(getattr(self, n)) for n in _PART_FIELDS])


class Route:
    """Device buffers of sparsepr_route's outputs."""

    def __init__(self, desc: spr_desc, cfg: OperatorConfig, device, keep_scores: bool = False):
        BH = desc.B * desc.H
        i32 = torch.int32
        z = lambda shape, t: torch.empty(shape, dtype=t, device=device)  # noqa: E731
        self.sel_cnt = z((BH, cfg.Cq + 1), i32)
        self.sel_kv = z((BH, cfg.Cq + 1, cfg.Ck + 1), i32)
        self.probe_idx = z((BH, cfg.M), i32)
        self.probe_w = z((BH, cfg.M), torch.float64)
        self.pairs = z((BH,), torch.int64)
        self.rho_exec = z((BH,), torch.float64)
        self.scores = z((BH, cfg.Cq, cfg.Ck), torch.float64) if keep_scores else None
        self.score_err = z((BH, cfg.Cq, cfg.Ck), torch.float64) if keep_scores else None
        self.struct = spr_route(*[_ptr(getattr(self, n)) for n in _ROUTE_FIELDS])


# ----------------------------------------------------------------- C-ABI calls
def sparsepr_workspace_size(desc: spr_desc, cfg: OperatorConfig) -> int:
    n = library().sparsepr_workspace_size(ctypes.byref(desc), ctypes.byref(cfg.part_params()), cfg.M)
    if n == 0:
        raise SparsePRError("sparsepr_workspace_size: invalid descriptor or parameters")
    return int(n)


def warm_state(prev: "Partition") -> spr_warm:
    """Later-call state (App. C.1) taken from a previous call's partition buffers."""
    return spr_warm(*[_ptr(getattr(prev, n)) for n in _WARM_FIELDS])


def sparsepr_partition(desc, q, k, v, cfg: OperatorConfig, part: Partition, ws: torch.Tensor, stream=None,
                       warm: Optional[spr_warm] = None):
    pp = cfg.part_params()
    _check(library().sparsepr_partition(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(pp),
                                        ctypes.byref(warm) if warm is not None else None,
                                        ctypes.byref(part.struct), _ptr(ws), ws.numel(), _stream(stream)),
           "sparsepr_partition")


def sparsepr_route(desc, cfg: OperatorConfig, part: Partition, route: Route, ws: torch.Tensor, stream=None):
    pp = cfg.part_params()
    po = cfg.probe_options()
    _check(library().sparsepr_route(ctypes.byref(desc), ctypes.byref(pp), ctypes.byref(part.struct), cfg.rho, cfg.M,
                                    ctypes.byref(po), ctypes.byref(route.struct), _ptr(ws), ws.numel(),
                                    _stream(stream)),
           "sparsepr_route")


def sparsepr_attn_sparse(desc, cfg: OperatorConfig, part: Partition, route: Route, o_sp: torch.Tensor,
                         ws: torch.Tensor, stream=None):
    pp = cfg.part_params()
    _check(library().sparsepr_attn_sparse(ctypes.byref(desc), ctypes.byref(pp), ctypes.byref(part.struct),
                                          ctypes.byref(route.struct), _ptr(o_sp), _ptr(ws), ws.numel(),
                                          _stream(stream)), "sparsepr_attn_sparse")


def sparsepr_probe_exact(desc, q, k, v, probe_idx: torch.Tensor, M: int, o_probe: torch.Tensor, ws: torch.Tensor,
                         stream=None):
    _check(library().sparsepr_probe_exact(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(probe_idx), M,
                                          _ptr(o_probe), _ptr(ws), ws.numel(), _stream(stream)),
           "sparsepr_probe_exact")


def sparsepr_fit_correct(desc, cfg: OperatorConfig, part: Partition, route: Route, o_sp, o_probe, out,
                         head_status, ws, fit_state=None, stream=None):
    pp = cfg.part_params()
    out_dt = SPR_BF16 if out.dtype == torch.bfloat16 else SPR_F32
    fo = cfg.fit_options()
    _check(library().sparsepr_fit_correct(ctypes.byref(desc), ctypes.byref(pp), ctypes.byref(part.struct),
                                          ctypes.byref(route.struct), _ptr(o_sp), _ptr(o_probe), cfg.M, cfg.lam,
                                          cfg.std_eps, ctypes.byref(fo), _ptr(out), out_dt, _ptr(fit_state),
                                          _ptr(head_status), _ptr(ws), ws.numel(), _stream(stream)),
           "sparsepr_fit_correct")


def dense_workspace(desc, device) -> torch.Tensor:
    n = library().sparsepr_dense_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise SparsePRError("sparsepr_dense_workspace_size: invalid descriptor")
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def probe_workspace(desc, M: int, device) -> torch.Tensor:
    n = library().sparsepr_probe_workspace_size(ctypes.byref(desc), M)
    if n == 0:
        raise SparsePRError("sparsepr_probe_workspace_size: invalid arguments")
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def sparsepr_attn_dense(desc, q, k, v, out, ws: Optional[torch.Tensor] = None, stream=None):
    """Dense flash attention of every row; ``ws`` (from ``dense_workspace``) is allocated when omitted."""
    out_dt = SPR_BF16 if out.dtype == torch.bfloat16 else SPR_F32
    if ws is None:
        ws = dense_workspace(desc, q.device)
    _check(library().sparsepr_attn_dense(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), out_dt,
                                         _ptr(ws), ws.numel(), _stream(stream)), "sparsepr_attn_dense")


def sparsepr_attn_dense_noalloc(desc, q, k, v, out, stream=None):
    """sparsepr_attn_dense on the library's fixed device scratch: no allocation anywhere in the call."""
    out_dt = SPR_BF16 if out.dtype == torch.bfloat16 else SPR_F32
    _check(library().sparsepr_attn_dense_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), out_dt,
                                                 _stream(stream)), "sparsepr_attn_dense_noalloc")


def sparsepr_kmeans(feat: torch.Tensor, C: int, seed: int, stage: int, max_iters: int, tol: float, stream=None):
    """k-means helper on feat [BH, n, r] fp64; returns (labels, centres of the final pass, passes)."""
    BH, n, r = feat.shape
    lib = library()
    nbytes = lib.sparsepr_kmeans_workspace_size(BH, n, r, C)
    if nbytes == 0:
        raise SparsePRError("sparsepr_kmeans_workspace_size: invalid arguments")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=feat.device)
    labels = torch.empty((BH, n), dtype=torch.int32, device=feat.device)
    cent = torch.empty((BH, C, r), dtype=torch.float64, device=feat.device)
    passes = torch.empty((BH,), dtype=torch.int32, device=feat.device)
    _check(lib.sparsepr_kmeans(BH, n, r, C, _ptr(feat), seed, stage, max_iters, tol, _ptr(labels), _ptr(cent),
                               _ptr(passes), _ptr(ws), nbytes, _stream(stream)), "sparsepr_kmeans")
    return labels, cent, passes


# ----------------------------------------------------------------- whole operator
class SparsePR:
    """The five calls of one operator invocation with buffers allocated once.

    ``run(q, k, v)`` returns the corrected output [B, H, N, d] (fp32 by default).  Passing ``k``
    (or any tensor of its shape and strides) with fewer heads than q selects grouped-query
    attention; later calls must then pass k and v of that shape."""

    def __init__(self, q: torch.Tensor, cfg: OperatorConfig, n_text: int = 0, out_dtype=torch.float32,
                 diagnostics: bool = False, keep_scores: bool = False, k: Optional[torch.Tensor] = None):
        self.cfg = cfg
        self.desc = make_desc(q, n_text, k)
        dev = q.device
        B, H, N, d = q.shape
        self.ws = torch.empty(sparsepr_workspace_size(self.desc, cfg), dtype=torch.uint8, device=dev)
        self.ws_probe = probe_workspace(self.desc, cfg.M, dev)
        self.part = Partition(self.desc, cfg, dev, diagnostics)
        self.route = Route(self.desc, cfg, dev, keep_scores)
        self.o_sp = torch.empty((B * H, N, d), dtype=torch.float32, device=dev)
        self.o_probe = torch.empty((B * H, cfg.M, d), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
        self.head_status = torch.empty((B * H,), dtype=torch.int32, device=dev)
        self.fit_state = torch.empty((B * H, 3 * d + d * d), dtype=torch.float64, device=dev) if diagnostics else None
        self.warm_iters = 2  # k-means iteration limit of later calls (Table C.1)
        self.side = None     # stream of the exact probes, beside the sparse attention

    def partition(self, q, k, v, warm: bool = False):
        """warm: later call of App. C.1 from this object's previous partition (in place), with
        the warm iteration limit ``warm_iters``."""
        if warm:
            cfg = dataclasses.replace(self.cfg, max_iters=self.warm_iters)
            sparsepr_partition(self.desc, q, k, v, cfg, self.part, self.ws, warm=warm_state(self.part))
        else:
            sparsepr_partition(self.desc, q, k, v, self.cfg, self.part, self.ws)

    def route_(self):
        sparsepr_route(self.desc, self.cfg, self.part, self.route, self.ws)

    def attn_sparse(self):
        sparsepr_attn_sparse(self.desc, self.cfg, self.part, self.route, self.o_sp, self.ws)

    def probe_exact(self, q, k, v):
        sparsepr_probe_exact(self.desc, q, k, v, self.route.probe_idx, self.cfg.M, self.o_probe, self.ws_probe)

    def fit_correct(self):
        sparsepr_fit_correct(self.desc, self.cfg, self.part, self.route, self.o_sp, self.o_probe, self.out,
                             self.head_status, self.ws, self.fit_state)

    def probes_beside(self, q, k, v):
        """Start the exact probes on a second stream (default priority) once the routing on the
        current stream is done; they need only the inputs and the probe rows, and run beside the
        sparse attention.  ``join`` makes the current stream wait for them."""
        main = torch.cuda.current_stream()
        if self.side is None:
            self.side = torch.cuda.Stream(device=q.device)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            self.probe_exact(q, k, v)

    def join(self):
        torch.cuda.current_stream().wait_stream(self.side)

    def run(self, q, k, v, warm: bool = False) -> torch.Tensor:
        self.partition(q, k, v, warm)
        self.route_()
        self.probes_beside(q, k, v)
        self.attn_sparse()
        self.join()
        self.fit_correct()
        return self.out
