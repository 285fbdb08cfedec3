"""The C ABI without a GPU: libsparsepr loads, exports every function include/sparsepr.h declares,
and its host-side validation answers before any device work (nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest
import torch

import free_block_sparse_sampled_amd as spr
from free_block_sparse_sampled_amd import sparsepr as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsepr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsepr_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libsparsepr.so is not built")
    return spr.library()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_status_strings(lib):
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace too small"),
                       (5, b"problem exceeds the fixed scratch of the allocation-free call")]:
        assert lib.sparsepr_status_string(code) == text
    assert lib.sparsepr_status_string(99) == b"unknown status"


def _desc(N=4096, d=128, dtype=B.SPR_BF16, n_text=0, H=2):
    return B.spr_desc(B=1, H=H, N=N, d=d, n_text=n_text, dtype=dtype, sb=H * N * d, sh=N * d, sn=d)


def _params(Ck=64, Cq=64, rK=48, rQ=64):
    return B.spr_part_params(Ck=Ck, Cq=Cq, rK=rK, rQ=rQ, Ms=256, max_iters=25, tol=1e-4, rms_eps=1e-6,
                             eig_clamp=1e-6, seed=0)


def test_workspace_size_validates_and_grows(lib):
    d, p = _desc(), _params()
    small = lib.sparsepr_workspace_size(ctypes.byref(d), ctypes.byref(p), 64)
    big = lib.sparsepr_workspace_size(ctypes.byref(_desc(N=8192)), ctypes.byref(p), 64)
    assert 0 < small < big
    assert small % 256 == 0
    bad = [(_desc(d=96), p), (_desc(dtype=7), p), (_desc(n_text=4095), p), (d, _params(Ck=2000)),
           (d, _params(rK=0)), (d, _params(rQ=129))]
    for dd, pp in bad:
        assert lib.sparsepr_workspace_size(ctypes.byref(dd), ctypes.byref(pp), 64) == 0
    assert lib.sparsepr_workspace_size(None, ctypes.byref(p), 64) == 0


def test_kmeans_workspace_size_limits(lib):
    assert lib.sparsepr_kmeans_workspace_size(2, 1000, 48, 64) > 0
    assert lib.sparsepr_kmeans_workspace_size(2, 1000, 48, 1025) == 0  # C above the supported 1024
    assert lib.sparsepr_kmeans_workspace_size(2, 10, 48, 11) == 0      # more centres than points
    assert lib.sparsepr_kmeans_workspace_size(2, 1000, 65, 64) == 0    # rank not built
    assert lib.sparsepr_kmeans_workspace_size(2, 1000, 128, 64) > 0    # raw 128-dimensional coordinates
    assert lib.sparsepr_kmeans_workspace_size(2, 1000, 256, 64) == 0


def test_entry_points_reject_invalid_arguments_on_the_host(lib):
    d, p = _desc(), _params()
    part, route = B.spr_partition(), B.spr_route()
    dummy = ctypes.c_void_p(16)  # never dereferenced: validation fails before any device work
    assert lib.sparsepr_partition(None, dummy, dummy, dummy, ctypes.byref(p), None, ctypes.byref(part), dummy, 0,
                                  None) == 1
    # required partition outputs missing
    assert lib.sparsepr_partition(ctypes.byref(d), dummy, dummy, dummy, ctypes.byref(p), None, ctypes.byref(part),
                                  dummy, 1 << 40, None) == 1
    # a warm state with a null member
    full = B.spr_partition(*([dummy] * len(B._PART_FIELDS)))
    warm = B.spr_warm(dummy, dummy, dummy, None, dummy, dummy)
    assert lib.sparsepr_partition(ctypes.byref(d), dummy, dummy, dummy, ctypes.byref(p), ctypes.byref(warm),
                                  ctypes.byref(full), dummy, 1 << 40, None) == 1
    # unsupported head dimension
    assert lib.sparsepr_attn_dense(ctypes.byref(_desc(d=80)), dummy, dummy, dummy, dummy, 0, dummy, 1 << 40,
                                   None) == 2
    assert lib.sparsepr_attn_dense(ctypes.byref(d), dummy, dummy, dummy, dummy, 5, dummy, 1 << 40, None) == 2
    # dense workspace: null, then too small for the fp16 copy of v
    assert lib.sparsepr_attn_dense(ctypes.byref(d), dummy, dummy, dummy, dummy, 0, None, 1 << 40, None) == 1
    need = lib.sparsepr_dense_workspace_size(ctypes.byref(d))
    assert need >= d.B * d.H * d.N * d.d * 2
    assert lib.sparsepr_attn_dense(ctypes.byref(d), dummy, dummy, dummy, dummy, 0, dummy, need - 1, None) == 3
    assert lib.sparsepr_probe_workspace_size(ctypes.byref(d), 64) >= need
    # allocation-free dense call: null pointer, unknown output dtype, a v copy beyond its fixed scratch
    assert lib.sparsepr_attn_dense_noalloc(ctypes.byref(d), None, dummy, dummy, dummy, 0, None) == 1
    assert lib.sparsepr_attn_dense_noalloc(ctypes.byref(d), dummy, dummy, dummy, dummy, 5, None) == 2
    huge = _desc(N=1 << 17, H=4)  # 4 heads x 131072 x 128 bf16 = 128 MiB of fp16 v
    assert lib.sparsepr_dense_workspace_size(ctypes.byref(huge)) > B.NOALLOC_SCRATCH_BYTES
    assert lib.sparsepr_attn_dense_noalloc(ctypes.byref(huge), dummy, dummy, dummy, dummy, 0, None) == 5
    # probes: M must lie in [1, Nv)
    assert lib.sparsepr_probe_exact(ctypes.byref(d), dummy, dummy, dummy, dummy, 0, dummy, dummy, 1 << 40, None) == 1
    assert lib.sparsepr_probe_exact(ctypes.byref(d), dummy, dummy, dummy, dummy, 4096, dummy, dummy, 1 << 40,
                                    None) == 1
    # probe workspace too small
    assert lib.sparsepr_probe_exact(ctypes.byref(d), dummy, dummy, dummy, dummy, 64, dummy, dummy, 16, None) == 3
    # route: density target out of range, and a budget below one key (rho*N^2 <= M*N)
    assert lib.sparsepr_route(ctypes.byref(d), ctypes.byref(p), ctypes.byref(part), 1.5, 64, None,
                              ctypes.byref(route), dummy, 1 << 40, None) == 1
    assert lib.sparsepr_route(ctypes.byref(d), ctypes.byref(p), ctypes.byref(part), 64 / 4096, 64, None,
                              ctypes.byref(route), dummy, 1 << 40, None) == 1
    # an unknown probe mode
    full_route = B.spr_route(*([dummy] * len(B.spr_route._fields_)))
    assert lib.sparsepr_route(ctypes.byref(d), ctypes.byref(p), ctypes.byref(full), 0.3, 64,
                              ctypes.byref(B.spr_probe_options(7, 0)), ctypes.byref(full_route), dummy, 1 << 40,
                              None) == 1
    # fit: negative lambda, then zero std_eps
    args = (ctypes.byref(part), ctypes.byref(route), dummy, dummy, 64)
    assert lib.sparsepr_fit_correct(ctypes.byref(d), ctypes.byref(p), *args, -1.0, 1e-6, None, dummy, 1, None,
                                    dummy, dummy, 1 << 40, None) == 1
    assert lib.sparsepr_fit_correct(ctypes.byref(d), ctypes.byref(p), *args, 1.0, 0.0, None, dummy, 1, None, dummy,
                                    dummy, 1 << 40, None) == 1
    # an unknown estimator family, a negative truncation rank
    for fo in [B.spr_fit_options(4, 0), B.spr_fit_options(0, -1)]:
        assert lib.sparsepr_fit_correct(ctypes.byref(d), ctypes.byref(p), *args, 1.0, 1e-6, ctypes.byref(fo), dummy,
                                        1, None, dummy, dummy, 1 << 40, None) == 1
    # k-means helper: stage outside {0, 1}, rank not built
    assert lib.sparsepr_kmeans(1, 100, 48, 8, dummy, 0, 2, 25, 1e-4, dummy, dummy, dummy, dummy, 1 << 40, None) == 1
    assert lib.sparsepr_kmeans(1, 100, 20, 8, dummy, 0, 0, 25, 1e-4, dummy, dummy, dummy, dummy, 1 << 40, None) == 2
    # workspace smaller than required
    ws_need = lib.sparsepr_workspace_size(ctypes.byref(d), ctypes.byref(p), 1)
    assert lib.sparsepr_attn_sparse(ctypes.byref(d), ctypes.byref(p), ctypes.byref(part), ctypes.byref(route), dummy,
                                    dummy, ws_need - 1, None) == 3


def test_grouped_query_descriptors_are_validated(lib):
    p = _params()
    N, d = 4096, 128

    def gqa(H=4, Hkv=2, ksn=d, reserved=0):
        dd = _desc(N=N, d=d, H=H)
        dd.Hkv, dd.reserved = Hkv, reserved
        dd.ksb, dd.ksh, dd.ksn = Hkv * N * d, N * d, ksn
        return dd

    ok = lib.sparsepr_workspace_size(ctypes.byref(gqa()), ctypes.byref(p), 64)
    assert ok > 0
    # Hkv = H is plain multi-head attention (k strides unused); Hkv = 0 likewise
    assert lib.sparsepr_workspace_size(ctypes.byref(gqa(Hkv=4, ksn=0)), ctypes.byref(p), 64) > 0
    assert lib.sparsepr_workspace_size(ctypes.byref(gqa(Hkv=0, ksn=0)), ctypes.byref(p), 64) > 0
    for bad in [gqa(Hkv=3), gqa(Hkv=5), gqa(Hkv=-1), gqa(reserved=1), gqa(ksn=d - 1), gqa(ksn=d + 1)]:
        assert lib.sparsepr_workspace_size(ctypes.byref(bad), ctypes.byref(p), 64) == 0
    # the binding builds the descriptor from tensors of H and Hkv heads
    q = torch.empty((1, 4, N, d), dtype=torch.bfloat16)
    k = torch.empty((1, 2, N, d), dtype=torch.bfloat16)
    dd = B.make_desc(q, 0, k)
    assert (dd.Hkv, dd.ksb, dd.ksh, dd.ksn) == (2, 2 * N * d, N * d, d) and B.kv_heads(dd) == 2
    assert B.make_desc(q, 0, q).Hkv == 0
