"""Host-side validation at the C ABI (CPU only: every call here is refused
before any device work, so it needs no GPU).

Each case passes one argument outside the documented range and checks the
documented return code; the pointers are placeholders that must never be
dereferenced.
"""
import ctypes

import pytest
import torch

# The placeholder pointers below must never reach a kernel; run only where
# no device exists, so that a validation gap shows up as a failed assertion.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks; a HIP device is present")

EI_OK, EI_EINVAL, EI_ERANGE, EI_ENOSPACE = 0, 1, 2, 4
FAKE = ctypes.c_void_p(0x1000)   # a non-null address that is never touched


@pytest.fixture(scope="module")
def ei():
    import exact_integer_amd
    return exact_integer_amd


def _desc(ei, n, k, fmt=1, experts=1):
    d = ei.Weights()
    d.packed = 0x10000
    d.n, d.k, d.n_pad, d.nb = n, k, (n + 31) // 32 * 32, k // 32
    d.smax, d.format, d.experts = 0, fmt, experts
    d.expert_stride = 256 + d.n_pad * k + d.n_pad * (k // 32) * 4
    return d


def test_packed_and_workspace_sizes(ei):
    L = ei.lib()
    assert L.ei_packed_bytes(100, 96) == 256 + 128 * 96 + 128 * 3 * 4 + 128 * 8   # header, codes, scales, row offsets
    assert L.ei_packed_bytes(100, 95) == 0
    assert L.ei_wide_packed_bytes(100, 96) == 256 + 128 * 96 * 3
    d = _desc(ei, 896, 4864)
    # the skinny path at T=30 splits 28 row tiles over workgroups: partials (h, r)
    assert L.ei_gemm_workspace_bytes(ctypes.byref(d), 30, 3, 0) > 3 * 32 * 4864
    assert L.ei_gemm_workspace_bytes(ctypes.byref(d), 1, 3, 0) == 0          # the GEMV needs none
    assert L.ei_wide_workspace_bytes(ctypes.byref(_desc(ei, 896, 896, 3)), 4096) == 4 * 4096 * 896
    # the skinny path splits 64 x 1024 at T=5 over two workgroups: their (h, r)
    # pairs take two int64 per output whatever the limb count up to three, so
    # one and two limbs differ only in the limb tiles (32 tokens x 1024 bytes)
    d = _desc(ei, 64, 1024)
    w1, w2 = L.ei_gemm_workspace_bytes(ctypes.byref(d), 5, 1, 0), L.ei_gemm_workspace_bytes(ctypes.byref(d), 5, 2, 0)
    assert w2 - w1 == 32 * 1024
    assert w1 >= 32 * 1024 + 2 * 2 * 5 * 64 * 8


def test_projection_arguments(ei):
    L = ei.lib()
    d = _desc(ei, 64, 128)
    assert L.int_gemm_q8(None, FAKE, FAKE, 4, 3, 0, 0, None, 0, None, None) == EI_EINVAL
    assert L.int_gemm_q8(ctypes.byref(d), None, FAKE, 4, 3, 0, 0, None, 0, None, None) == EI_EINVAL
    assert L.int_gemm_q8(ctypes.byref(d), FAKE, FAKE, 0, 3, 0, 0, None, 0, None, None) == EI_EINVAL
    assert L.int_gemm_q8(ctypes.byref(d), FAKE, FAKE, 4, 9, 0, 0, None, 0, None, None) == EI_EINVAL
    assert L.int_gemm_q8(ctypes.byref(d), FAKE, FAKE, 4, 5, 0, 0, None, 0, None, None) == EI_ERANGE
    assert L.int_gemm_q8(ctypes.byref(d), FAKE, FAKE, 4, 3, 9, 0, None, 0, None, None) == EI_EINVAL
    assert L.int_gemm_q8(ctypes.byref(d), FAKE, FAKE, 65535 * 32 + 1, 3, 0, 0, None, 0, None, None) == EI_ERANGE
    big = _desc(ei, 32, 262144 + 32)
    assert L.int_gemm_q8(ctypes.byref(big), FAKE, FAKE, 1, 3, 0, 0, None, 0, None, None) == EI_ERANGE
    # a T=30 call needs its workspace
    assert L.int_gemm_q8(ctypes.byref(d), FAKE, FAKE, 30, 3, 0, 0, None, 0, None, None) == EI_ENOSPACE
    # the 4-bit entry point refuses an 8-bit descriptor
    assert L.int_gemm_q4(ctypes.byref(d), FAKE, FAKE, 4, 3, 0, 0, None, 0, None, None) == EI_EINVAL


def test_batched_gemv_arguments(ei):
    L = ei.lib()
    WP = ctypes.POINTER(ei.Weights)
    a, b, c = _desc(ei, 64, 128), _desc(ei, 96, 128), _desc(ei, 64, 96)
    ws = (WP * 17)(*[ctypes.pointer(a)] * 17)
    ys = (ctypes.c_void_p * 17)(*[0x1000] * 17)
    assert L.int_gemm_q8_multi(ws, 0, FAKE, ys, 1, 3, None, None) == EI_EINVAL      # no matrices
    assert L.int_gemm_q8_multi(ws, 17, FAKE, ys, 1, 3, None, None) == EI_EINVAL     # more than 16
    assert L.int_gemm_q8_multi(ws, 2, FAKE, ys, 5, 3, None, None) == EI_EINVAL      # t > 4: not a decode size
    assert L.int_gemm_q8_multi(ws, 2, FAKE, ys, 0, 3, None, None) == EI_EINVAL
    assert L.int_gemm_q8_multi(ws, 2, None, ys, 1, 3, None, None) == EI_EINVAL
    assert L.int_gemm_q8_multi(ws, 2, FAKE, None, 1, 3, None, None) == EI_EINVAL
    assert L.int_gemm_q8_multi(ws, 2, FAKE, ys, 1, 5, None, None) == EI_ERANGE
    mixed = (WP * 2)(ctypes.pointer(b), ctypes.pointer(c))                          # k 128 and 96
    assert L.int_gemm_q8_multi(mixed, 2, FAKE, ys, 1, 3, None, None) == EI_EINVAL
    holes = (ctypes.c_void_p * 2)(0x1000, None)                                      # a null output
    assert L.int_gemm_q8_multi(ws, 2, FAKE, holes, 1, 3, None, None) == EI_EINVAL
    q4 = _desc(ei, 64, 128, fmt=2)
    fmt = (WP * 2)(ctypes.pointer(a), ctypes.pointer(q4))
    assert L.int_gemm_q8_multi(fmt, 2, FAKE, ys, 1, 3, None, None) == EI_EINVAL


def test_routed_and_ffn_arguments(ei):
    L = ei.lib()
    w = _desc(ei, 64, 128, experts=8)
    assert L.int_gemm_q8_grouped(ctypes.byref(w), FAKE, FAKE, 8193, 2, FAKE, 3, FAKE, 1 << 30, None, None) == EI_ERANGE
    assert L.int_gemm_q8_grouped(ctypes.byref(w), FAKE, FAKE, 4, 2, FAKE, 4, FAKE, 1 << 30, None, None) == EI_ERANGE
    assert L.int_gemm_q8_grouped(ctypes.byref(w), FAKE, FAKE, 4, 2, FAKE, 3, FAKE, 0, None, None) == EI_ENOSPACE
    g, u, dn = _desc(ei, 96, 64), _desc(ei, 96, 64), _desc(ei, 64, 96)
    bad = _desc(ei, 64, 64)
    assert L.int_ffn_q8(ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad), FAKE, FAKE, FAKE, 3, FAKE, 1 << 30,
                        None, None) == EI_EINVAL
    assert L.int_ffn_q8(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), FAKE, FAKE, FAKE, 3, FAKE, 0,
                        None, None) == EI_ENOSPACE
    assert L.int_ffn_q8_prenorm(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), FAKE, 0, FAKE, FAKE, FAKE, 3,
                                FAKE, 1 << 30, None, None) == EI_ERANGE
    WP = ctypes.POINTER(ei.Weights)
    layers = (WP * 3)(ctypes.pointer(g), ctypes.pointer(u), ctypes.pointer(dn))
    assert L.int_ffn_q8_chain(layers, 0, FAKE, FAKE, FAKE, 3, FAKE, 1 << 30, None, None) == EI_EINVAL
    assert L.int_ffn_q8_chain(layers, 1, FAKE, FAKE, FAKE, 3, FAKE, 0, None, None) == EI_ENOSPACE
    gns = (ctypes.c_void_p * 1)(0x1000)
    assert L.int_ffn_q8_prenorm_chain(layers, 0, gns, 1 << 20, FAKE, FAKE, FAKE, 3, FAKE, 1 << 30, None, None) == EI_EINVAL
    assert L.int_ffn_q8_prenorm_chain(layers, 1, None, 1 << 20, FAKE, FAKE, FAKE, 3, FAKE, 1 << 30, None, None) == EI_EINVAL
    nulls = (ctypes.c_void_p * 1)(None)
    assert L.int_ffn_q8_prenorm_chain(layers, 1, nulls, 1 << 20, FAKE, FAKE, FAKE, 3, FAKE, 1 << 30, None, None) == EI_EINVAL
    assert L.int_ffn_q8_prenorm_chain(layers, 1, gns, 0, FAKE, FAKE, FAKE, 3, FAKE, 1 << 30, None, None) == EI_ERANGE
    assert L.int_ffn_q8_prenorm_chain(layers, 1, gns, 1 << 20, FAKE, FAKE, FAKE, 3, FAKE, 0, None, None) == EI_ENOSPACE


def test_next_row_arguments(ei):
    L = ei.lib()
    assert L.ei_topk_route(FAKE, 4, 64, 65, FAKE, None) == EI_EINVAL
    assert L.ei_topk_route(FAKE, 4, 2049, 8, FAKE, None) == EI_ERANGE
    assert L.ei_topk_route(None, 4, 64, 8, FAKE, None) == EI_EINVAL
    assert L.ei_requant(FAKE, 3, 127, FAKE, 10, None, None) == EI_EINVAL
    assert L.ei_requant(FAKE, 3, -1, FAKE, 10, None, None) == EI_EINVAL
    assert L.ei_rmsnorm_q16(FAKE, FAKE, 1, FAKE, 2, 65537, None, None) == EI_ERANGE
    assert L.ei_rmsnorm_q16(FAKE, FAKE, 0, FAKE, 2, 64, None, None) == EI_ERANGE
    assert L.ei_rmsnorm_q16(FAKE, FAKE, (1 << 32) + 1, FAKE, 2, 64, None, None) == EI_ERANGE
    wd = _desc(ei, 64, 32768 + 32, 3)
    assert L.int_gemm_wide(ctypes.byref(wd), FAKE, FAKE, 4, FAKE, 1 << 40, None, None) == EI_ERANGE
    assert L.int_gemm_wide(ctypes.byref(_desc(ei, 64, 64, 1)), FAKE, FAKE, 4, FAKE, 1 << 40, None, None) == EI_EINVAL
    assert L.int_gemm_q4_table(FAKE, FAKE, FAKE, FAKE, 64, 96, 65536, None, 0, None, None) == EI_ERANGE
    assert L.int_gemm_q4_table(FAKE, FAKE, FAKE, FAKE, 64, 95, 4, None, 0, None, None) == EI_EINVAL
    assert L.int_gemm_q4_table(FAKE, FAKE, FAKE, FAKE, 64, 262144 + 32, 4, FAKE, 1 << 40, None, None) == EI_ERANGE
    # K in chunks of 256 columns: exact int128 sums per chunk, none for one chunk
    assert L.ei_q4_table_workspace_bytes(64, 256, 4) == 0
    assert L.ei_q4_table_workspace_bytes(64, 288, 4) == 2 * 4 * 64 * 16
    assert L.ei_q4_table_workspace_bytes(1030, 2048, 7) == 8 * 7 * 1030 * 16
    assert L.ei_q4_table_workspace_bytes(64, 95, 4) == 0
    assert L.int_gemm_q4_table(FAKE, FAKE, FAKE, FAKE, 64, 288, 4, None, 0, None, None) == EI_ENOSPACE
    assert L.int_gemm_q4_table(FAKE, FAKE, FAKE, FAKE, 64, 288, 4, FAKE, 2 * 4 * 64 * 16 - 1, None, None) == EI_ENOSPACE
    odd = ctypes.c_void_p(0x1008)   # int128 sums need 16-byte alignment
    assert L.int_gemm_q4_table(FAKE, FAKE, FAKE, FAKE, 64, 288, 4, odd, 1 << 20, None, None) == EI_EINVAL
    out = ei.Weights()
    assert L.ei_wide_pack(FAKE, 64, 95, FAKE, 1 << 30, ctypes.byref(out), None) == EI_EINVAL
    assert L.ei_wide_pack(FAKE, 64, 96, FAKE, 100, ctypes.byref(out), None) == EI_ENOSPACE
