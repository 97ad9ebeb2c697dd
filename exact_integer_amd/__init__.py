"""Python binding of libexact_int.so: the exact-integer block-quantized
projection on AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/exact_int.h.  PyTorch provides
device memory and streams.  There is no CPU path: without the built library
or a HIP device every compute call raises.

torch is imported before the library is loaded, so that the library binds to
the HIP runtime torch already loaded and shares its streams and allocations.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

import torch

__all__ = [
    "EIError", "PackedWeights", "lib", "pack_q8", "pack_q4", "pack_q8_stacked", "gemm_q8", "gemm_q8_noalloc", "gemm_q4",
    "gemm_q8_grouped", "fp32_shadow", "limb_split", "silu_lut", "silu_mul", "digest", "sha256_host", "workspace_bytes",
    "grouped_workspace_bytes", "SCHEDULES", "DEV_LIMB_RANGE", "DEV_OUT_RANGE", "DEV_ROUTE",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libexact_int.so")

EI_OK, EI_EINVAL, EI_ERANGE, EI_EDEVICE, EI_ENOSPACE = 0, 1, 2, 3, 4
DEV_LIMB_RANGE, DEV_OUT_RANGE, DEV_ROUTE = 1, 2, 4
SCHEDULES = {"default": 0, "canonical": 1, "reversed": 2, "tiled_shuffled": 3, "split_k": 4, "tree_walk": 5}
FORMAT_Q8, FORMAT_Q4 = 1, 2


class EIError(RuntimeError):
    """A library call failed (host-detected code, or a device status bit)."""


class Weights(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("n_pad", ctypes.c_int64), ("nb", ctypes.c_int64), ("smax", ctypes.c_uint32),
                ("format", ctypes.c_int32), ("experts", ctypes.c_int64), ("expert_stride", ctypes.c_int64)]


# name -> (restype, argtypes); mirrors include/exact_int.h
P, I64, I32, SZ, U64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64
WP = ctypes.POINTER(Weights)
SIGNATURES = {
    "ei_packed_bytes": (SZ, [I64, I64]),
    "ei_q8_pack": (I32, [P, P, I64, I64, P, SZ, WP, P]),
    "ei_q4_pack": (I32, [P, P, I64, I64, P, SZ, WP, P]),
    "ei_packed_bytes_stacked": (SZ, [I64, I64, I64]),
    "ei_q8_pack_stacked": (I32, [P, P, I64, I64, I64, P, SZ, WP, P]),
    "ei_grouped_workspace_bytes": (SZ, [WP, I64, I32, I32]),
    "int_gemm_q8_grouped": (I32, [WP, P, P, I64, I32, P, I32, P, SZ, P, P]),
    "ei_limb_split": (I32, [P, P, I64, I32, P, P]),
    "ei_gemm_workspace_bytes": (SZ, [WP, I64, I32, I32]),
    "int_gemm_q8": (I32, [WP, P, P, I64, I32, I32, U64, P, SZ, P, P]),
    "int_gemm_q8_multi": (I32, [P, I32, P, P, I64, I32, P, P]),
    "int_gemm_q8_noalloc": (I32, [WP, P, P, I64, I32, P, P]),
    "int_gemm_q4": (I32, [WP, P, P, I64, I32, I32, U64, P, SZ, P, P]),
    "ei_silu_lut_build": (I32, [P, P]),
    "silu_lut_epilogue": (I32, [P, P, P, P, I64, P, P]),
    "ei_q8_fp32_shadow": (I32, [P, P, P, P, I64, I64, I64, I32, U64, P]),
    "output_digest": (I32, [P, SZ, P, P]),
    "ei_sha256_host": (None, [P, SZ, P]),
    "ei_topk_route": (I32, [P, I64, I64, I32, P, P]),
    "int_gemm_q4_table": (I32, [P, P, P, P, I64, I64, I64, P, SZ, P, P]),
    "ei_q4_table_workspace_bytes": (SZ, [I64, I64, I64]),
    "silu_lut_epilogue_radix16": (I32, [P, P, P, P, I64, P, P]),
    "ei_wide_packed_bytes": (SZ, [I64, I64]),
    "ei_wide_pack": (I32, [P, I64, I64, P, SZ, WP, P]),
    "ei_wide_workspace_bytes": (SZ, [WP, I64]),
    "int_gemm_wide": (I32, [WP, P, P, I64, P, SZ, P, P]),
    "ei_requant": (I32, [P, I64, I32, P, I64, P, P]),
    "ei_rmsnorm_q16": (I32, [P, P, I64, P, I64, I64, P, P]),
    "ei_ffn_workspace_bytes": (SZ, [WP, WP, I64]),
    "int_ffn_q8": (I32, [WP, WP, WP, P, P, P, I64, P, SZ, P, P]),
    "int_ffn_q8_prenorm": (I32, [WP, WP, WP, P, I64, P, P, P, I64, P, SZ, P, P]),
    "int_ffn_q8_prenorm_chain": (I32, [ctypes.POINTER(WP), I32, P, I64, P, P, P, I64, P, SZ, P, P]),
    "ei_ffn_chain_workspace_bytes": (SZ, [WP, WP, I64]),
    "int_ffn_q8_chain": (I32, [ctypes.POINTER(WP), I32, P, P, P, I64, P, SZ, P, P]),
    "ei_moe_ffn_workspace_bytes": (SZ, [WP, WP, I64, I32]),
    "int_moe_ffn_q8": (I32, [WP, WP, WP, P, P, I64, I32, P, P, P, SZ, P, P]),
    "ei_status_string": (ctypes.c_char_p, [I32]),
    "ei_version": (I32, []),
}


@lru_cache(maxsize=1)
def lib() -> ctypes.CDLL:
    """Load libexact_int.so (building it first only if it is absent)."""
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def _check(code: int, what: str) -> None:
    if code != EI_OK:
        raise EIError(f"{what}: {lib().ei_status_string(code).decode()} ({code})")


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise EIError(f"{name} must be a HIP device tensor")
    if t.dtype != dtype:
        raise EIError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise EIError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    if not torch.cuda.is_available():
        raise EIError("no HIP device: the exact-integer kernels need an MI355X")
    return torch.cuda.current_stream().cuda_stream


def _raise_status(status: torch.Tensor, what: str) -> None:
    v = int(status.item())
    if v:
        bits = [n for b, n in ((DEV_LIMB_RANGE, "activation outside the declared limb range"),
                               (DEV_OUT_RANGE, "result outside int64"),
                               (DEV_ROUTE, "expert id outside [0, E)")) if v & b]
        raise EIError(f"{what}: " + "; ".join(bits))


class PackedWeights:
    """A packed weight matrix: the device buffer and its host descriptor."""

    def __init__(self, buf: torch.Tensor, desc: Weights):
        self.buf = buf          # keeps the device memory alive
        self.desc = desc

    @property
    def n(self) -> int:
        return self.desc.n

    @property
    def k(self) -> int:
        return self.desc.k

    @property
    def fmt(self) -> int:
        return self.desc.format


def _pack(fn: str, codes: torch.Tensor, scales: torch.Tensor, n: int, k: int, cdt, sdt) -> PackedWeights:
    s = _stream()
    pc, ps = _dev(codes, cdt, "codes"), _dev(scales, sdt, "scales")
    nbytes = lib().ei_packed_bytes(n, k)
    if nbytes == 0:
        raise EIError(f"{fn}: bad shape n={n} k={k}")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    desc = Weights()
    _check(getattr(lib(), fn)(pc, ps, n, k, buf.data_ptr(), nbytes, ctypes.byref(desc), s), fn)
    return PackedWeights(buf, desc)


def pack_q8(codes: torch.Tensor, scales: torch.Tensor) -> PackedWeights:
    """codes int8 [n][k], scales int32 [n][k/32] (device) -> packed weights."""
    n, k = codes.shape
    return _pack("ei_q8_pack", codes, scales, n, k, torch.int8, torch.int32)


def pack_q4(nib: torch.Tensor, sme: torch.Tensor) -> PackedWeights:
    """nibbles uint8 [n][k/2], scale bytes uint8 [n][k/32] (device) -> packed weights."""
    n, kh = nib.shape
    return _pack("ei_q4_pack", nib, sme, n, 2 * kh, torch.uint8, torch.uint8)


def pack_q8_stacked(codes: torch.Tensor, scales: torch.Tensor) -> PackedWeights:
    """codes int8 [E][n][k], scales int32 [E][n][k/32] (device) -> E packed experts in one buffer."""
    s = _stream()
    e, n, k = codes.shape
    pc, ps = _dev(codes, torch.int8, "codes"), _dev(scales, torch.int32, "scales")
    nbytes = lib().ei_packed_bytes_stacked(e, n, k)
    if nbytes == 0:
        raise EIError(f"ei_q8_pack_stacked: bad shape e={e} n={n} k={k}")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    desc = Weights()
    _check(lib().ei_q8_pack_stacked(pc, ps, e, n, k, buf.data_ptr(), nbytes, ctypes.byref(desc), s),
           "ei_q8_pack_stacked")
    return PackedWeights(buf, desc)


def grouped_workspace_bytes(w: PackedWeights, rows: int, topk: int, limbs: int = 3) -> int:
    return int(lib().ei_grouped_workspace_bytes(ctypes.byref(w.desc), rows, topk, limbs))


def gemm_q8_grouped(w: PackedWeights, x: torch.Tensor, route: torch.Tensor, limbs: int = 3, out=None,
                    workspace=None, status=None) -> torch.Tensor:
    """Routed projection: y[r*topk + s] = Q8 projection of expert route[r][s] on x[r] (int64 [rows*topk][n])."""
    s = _stream()
    rows, k = x.shape
    if k != w.k:
        raise EIError(f"int_gemm_q8_grouped: x has k={k}, weights k={w.k}")
    if route.dim() != 2 or route.shape[0] != rows:
        raise EIError("int_gemm_q8_grouped: route must be [rows][topk]")
    topk = route.shape[1]
    px, pr = _dev(x, torch.int64, "x"), _dev(route, torch.int32, "route")
    y = out if out is not None else torch.empty((rows * topk, w.n), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    if tuple(y.shape) != (rows * topk, w.n):
        raise EIError(f"int_gemm_q8_grouped: y must be [{rows * topk}][{w.n}]")
    need = grouped_workspace_bytes(w, rows, topk, limbs)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_gemm_q8_grouped(ctypes.byref(w.desc), px, pr, rows, topk, py, limbs, workspace.data_ptr(),
                                     workspace.numel(), status.data_ptr(), s), "int_gemm_q8_grouped")
    if check:
        _raise_status(status, "int_gemm_q8_grouped")
    return y


def requant(c: torch.Tensor, m: int, k: int, out=None, status=None) -> torch.Tensor:
    """y = round_half_away(c * m / 2^k), int64, elementwise."""
    s = _stream()
    pc = _dev(c, torch.int64, "c")
    y = out if out is not None else torch.empty_like(c)
    py = _dev(y, torch.int64, "y")
    if y.numel() != c.numel():
        raise EIError("ei_requant: y must have c's size")
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=c.device)
    _check(lib().ei_requant(pc, m, k, py, c.numel(), status.data_ptr(), s), "ei_requant")
    if check:
        _raise_status(status, "ei_requant")
    return y


def rmsnorm_q16(x: torch.Tensor, g: torch.Tensor, eps_q32: int, out=None, status=None) -> torch.Tensor:
    """Integer RMSNorm of Q16 rows with a Q16 weight g and eps in Q32 (int64 [t][d])."""
    s = _stream()
    t, d = x.shape
    px, pg = _dev(x, torch.int64, "x"), _dev(g, torch.int32, "g")
    if g.numel() != d:
        raise EIError(f"ei_rmsnorm_q16: g must have {d} entries")
    y = out if out is not None else torch.empty_like(x)
    py = _dev(y, torch.int64, "y")
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().ei_rmsnorm_q16(px, pg, eps_q32, py, t, d, status.data_ptr(), s), "ei_rmsnorm_q16")
    if check:
        _raise_status(status, "ei_rmsnorm_q16")
    return y


def q4_table_workspace_bytes(n: int, k: int, t: int) -> int:
    return int(lib().ei_q4_table_workspace_bytes(n, k, t))


def gemm_q4_table(nib: torch.Tensor, sme: torch.Tensor, x: torch.Tensor, out=None, workspace=None,
                  status=None) -> torch.Tensor:
    """The 4-bit projection by table reads, from the export format (int64 [t][n])."""
    s = _stream()
    n = nib.shape[0]
    t, k = x.shape
    if tuple(nib.shape) != (n, k // 2) or tuple(sme.shape) != (n, k // 32):
        raise EIError("int_gemm_q4_table: nib [n][k/2], sme [n][k/32], x [t][k]")
    pn, ps, px = _dev(nib, torch.uint8, "nib"), _dev(sme, torch.uint8, "sme"), _dev(x, torch.int32, "x")
    y = out if out is not None else torch.empty((t, n), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    need = q4_table_workspace_bytes(n, k, t)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    pw, wb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None else (None, 0)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_gemm_q4_table(pn, ps, px, py, n, k, t, pw, wb, status.data_ptr(), s), "int_gemm_q4_table")
    if check:
        _raise_status(status, "int_gemm_q4_table")
    return y


def silu_mul_radix16(g: torch.Tensor, u: torch.Tensor, lut: torch.Tensor, out=None, status=None) -> torch.Tensor:
    """silu_mul with the runtime product by base-16 table reads."""
    s = _stream()
    pg, pu, pl = _dev(g, torch.int64, "g"), _dev(u, torch.int64, "u"), _dev(lut, torch.int32, "lut")
    h = out if out is not None else torch.empty_like(g)
    ph = _dev(h, torch.int64, "h")
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=g.device)
    _check(lib().silu_lut_epilogue_radix16(pg, pu, pl, ph, g.numel(), status.data_ptr(), s),
           "silu_lut_epilogue_radix16")
    if check:
        _raise_status(status, "silu_lut_epilogue_radix16")
    return h


def pack_wide(codes: torch.Tensor) -> PackedWeights:
    """Repack wide integer codes (int32 [n][k], |c| <= 8,355,711) into digit tiles."""
    s = _stream()
    n, k = codes.shape
    pc = _dev(codes, torch.int32, "codes")
    nbytes = int(lib().ei_wide_packed_bytes(n, k))
    if nbytes == 0:
        raise EIError(f"ei_wide_pack: bad shape {n}x{k}")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    desc = Weights()
    _check(lib().ei_wide_pack(pc, n, k, buf.data_ptr(), nbytes, ctypes.byref(desc), s), "ei_wide_pack")
    return PackedWeights(buf, desc)


def gemm_wide(w: PackedWeights, x: torch.Tensor, out=None, workspace=None, status=None) -> torch.Tensor:
    """y = x @ codes^T exactly (int32 [t][k] activations, int64 [t][n] result)."""
    s = _stream()
    t, k = x.shape
    if k != w.k:
        raise EIError(f"int_gemm_wide: x has k={k}, weights k={w.k}")
    px = _dev(x, torch.int32, "x")
    y = out if out is not None else torch.empty((t, w.n), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    if workspace is None:
        workspace = torch.empty(int(lib().ei_wide_workspace_bytes(ctypes.byref(w.desc), t)), dtype=torch.uint8,
                                device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_gemm_wide(ctypes.byref(w.desc), px, py, t, workspace.data_ptr(), workspace.numel(),
                               status.data_ptr(), s), "int_gemm_wide")
    if check:
        _raise_status(status, "int_gemm_wide")
    return y


def topk_route(scores: torch.Tensor, k: int, out=None) -> torch.Tensor:
    """Integer top-k: route[t][s] = expert of rank s (score descending, index ascending), int32 [t][k]."""
    s = _stream()
    if scores.dim() != 2:
        raise EIError("ei_topk_route: scores must be [t][e]")
    t, e = scores.shape
    ps = _dev(scores, torch.int64, "scores")
    route = out if out is not None else torch.empty((t, k), dtype=torch.int32, device=scores.device)
    pr = _dev(route, torch.int32, "route")
    if tuple(route.shape) != (t, k):
        raise EIError(f"ei_topk_route: route must be [{t}][{k}]")
    _check(lib().ei_topk_route(ps, t, e, k, pr, s), "ei_topk_route")
    return route


def ffn_workspace_bytes(wg: PackedWeights, wd: PackedWeights, t: int) -> int:
    return int(lib().ei_ffn_workspace_bytes(ctypes.byref(wg.desc), ctypes.byref(wd.desc), t))


def ffn_q8(wg: PackedWeights, wu: PackedWeights, wd: PackedWeights, x: torch.Tensor, lut: torch.Tensor, out=None,
           workspace=None, status=None) -> torch.Tensor:
    """One FFN layer: y = x + Q8(wd, silu_mul(Q8(wg, x), Q8(wu, x))) (int64 [t][d])."""
    s = _stream()
    t, d = x.shape
    if d != wg.k or wu.k != wg.k or wu.n != wg.n or wd.k != wg.n or wd.n != wg.k:
        raise EIError("int_ffn_q8: shapes must be wg, wu [f][d], wd [d][f], x [t][d]")
    px, pl = _dev(x, torch.int64, "x"), _dev(lut, torch.int32, "lut")
    y = out if out is not None else torch.empty((t, d), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    if tuple(y.shape) != (t, d):
        raise EIError(f"int_ffn_q8: y must be [{t}][{d}]")
    if workspace is None:
        workspace = torch.empty(max(ffn_workspace_bytes(wg, wd, t), 1), dtype=torch.uint8, device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_ffn_q8(ctypes.byref(wg.desc), ctypes.byref(wu.desc), ctypes.byref(wd.desc), px, pl, py, t,
                            workspace.data_ptr(), workspace.numel(), status.data_ptr(), s), "int_ffn_q8")
    if check:
        _raise_status(status, "int_ffn_q8")
    return y


def ffn_chain_workspace_bytes(wg: PackedWeights, wd: PackedWeights, t: int) -> int:
    return int(lib().ei_ffn_chain_workspace_bytes(ctypes.byref(wg.desc), ctypes.byref(wd.desc), t))


def ffn_q8_chain(layers, x: torch.Tensor, lut: torch.Tensor, out=None, workspace=None, status=None) -> torch.Tensor:
    """A stack of FFN layers (a list of (gate, up, down) PackedWeights): x_{l+1} = ffn_q8(layer l, x_l)."""
    s = _stream()
    t, d = x.shape
    wg0, _, wd0 = layers[0]
    for wg, wu, wd in layers:
        if d != wg.k or wu.k != wg.k or wu.n != wg.n or wd.k != wg.n or wd.n != wg.k or wg.n != wg0.n:
            raise EIError("int_ffn_q8_chain: every layer must be gate, up [f][d], down [d][f] of one shape")
    descs = (WP * (3 * len(layers)))(*[ctypes.pointer(w.desc) for layer in layers for w in layer])
    px, pl = _dev(x, torch.int64, "x"), _dev(lut, torch.int32, "lut")
    y = out if out is not None else torch.empty_like(x)
    py = _dev(y, torch.int64, "y")
    if workspace is None:
        workspace = torch.empty(max(ffn_chain_workspace_bytes(wg0, wd0, t), 1), dtype=torch.uint8, device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_ffn_q8_chain(descs, len(layers), px, pl, py, t, workspace.data_ptr(), workspace.numel(),
                                  status.data_ptr(), s), "int_ffn_q8_chain")
    if check:
        _raise_status(status, "int_ffn_q8_chain")
    return y


def ffn_q8_prenorm(wg: PackedWeights, wu: PackedWeights, wd: PackedWeights, g_norm: torch.Tensor, eps_q32: int,
                   x: torch.Tensor, lut: torch.Tensor, out=None, workspace=None, status=None) -> torch.Tensor:
    """Pre-norm FFN layer: y = x + Q8(wd, silu_mul(Q8(wg, n), Q8(wu, n))), n = rmsnorm_q16(x, g_norm, eps)."""
    s = _stream()
    t, d = x.shape
    if d != wg.k or wu.k != wg.k or wu.n != wg.n or wd.k != wg.n or wd.n != wg.k or g_norm.numel() != d:
        raise EIError("int_ffn_q8_prenorm: shapes must be wg, wu [f][d], wd [d][f], g_norm [d], x [t][d]")
    px, pl, pg = _dev(x, torch.int64, "x"), _dev(lut, torch.int32, "lut"), _dev(g_norm, torch.int32, "g_norm")
    y = out if out is not None else torch.empty((t, d), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    if workspace is None:
        workspace = torch.empty(max(ffn_workspace_bytes(wg, wd, t), 1), dtype=torch.uint8, device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_ffn_q8_prenorm(ctypes.byref(wg.desc), ctypes.byref(wu.desc), ctypes.byref(wd.desc), pg,
                                    eps_q32, px, pl, py, t, workspace.data_ptr(), workspace.numel(),
                                    status.data_ptr(), s), "int_ffn_q8_prenorm")
    if check:
        _raise_status(status, "int_ffn_q8_prenorm")
    return y


def ffn_q8_prenorm_chain(layers, g_norms, eps_q32: int, x: torch.Tensor, lut: torch.Tensor, out=None,
                         workspace=None, status=None) -> torch.Tensor:
    """A stack of pre-norm FFN layers: x_{l+1} = ffn_q8_prenorm(layer l, g_norms[l], x_l)."""
    s = _stream()
    t, d = x.shape
    wg0, _, wd0 = layers[0]
    if len(g_norms) != len(layers) or any(g.numel() != d for g in g_norms):
        raise EIError("int_ffn_q8_prenorm_chain: one g_norm [d] per layer")
    for wg, wu, wd in layers:
        if d != wg.k or wu.k != wg.k or wu.n != wg.n or wd.k != wg.n or wd.n != wg.k or wg.n != wg0.n:
            raise EIError("int_ffn_q8_prenorm_chain: every layer must be gate, up [f][d], down [d][f] of one shape")
    descs = (WP * (3 * len(layers)))(*[ctypes.pointer(w.desc) for layer in layers for w in layer])
    gptrs = (ctypes.c_void_p * len(g_norms))(*[_dev(g, torch.int32, "g_norm") for g in g_norms])
    px, pl = _dev(x, torch.int64, "x"), _dev(lut, torch.int32, "lut")
    y = out if out is not None else torch.empty_like(x)
    py = _dev(y, torch.int64, "y")
    if workspace is None:
        workspace = torch.empty(max(ffn_chain_workspace_bytes(wg0, wd0, t), 1), dtype=torch.uint8, device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_ffn_q8_prenorm_chain(descs, len(layers), ctypes.cast(gptrs, ctypes.c_void_p), eps_q32, px, pl,
                                          py, t, workspace.data_ptr(), workspace.numel(), status.data_ptr(), s),
           "int_ffn_q8_prenorm_chain")
    if check:
        _raise_status(status, "int_ffn_q8_prenorm_chain")
    return y


def moe_ffn_workspace_bytes(wg: PackedWeights, wd: PackedWeights, rows: int, topk: int) -> int:
    return int(lib().ei_moe_ffn_workspace_bytes(ctypes.byref(wg.desc), ctypes.byref(wd.desc), rows, topk))


def moe_ffn_q8(wg: PackedWeights, wu: PackedWeights, wd: PackedWeights, x: torch.Tensor, route: torch.Tensor,
               lut: torch.Tensor, out=None, workspace=None, status=None) -> torch.Tensor:
    """Routed FFN: y[r*topk + s] = expert route[r][s]'s gated MLP on x[r] (int64 [rows*topk][d])."""
    s = _stream()
    rows, d = x.shape
    if d != wg.k or wu.k != wg.k or wu.n != wg.n or wd.k != wg.n or wd.n != wg.k:
        raise EIError("int_moe_ffn_q8: shapes must be wg, wu [E][f][d], wd [E][d][f], x [rows][d]")
    if route.dim() != 2 or route.shape[0] != rows:
        raise EIError("int_moe_ffn_q8: route must be [rows][topk]")
    topk = route.shape[1]
    px, pr, pl = _dev(x, torch.int64, "x"), _dev(route, torch.int32, "route"), _dev(lut, torch.int32, "lut")
    y = out if out is not None else torch.empty((rows * topk, d), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    if tuple(y.shape) != (rows * topk, d):
        raise EIError(f"int_moe_ffn_q8: y must be [{rows * topk}][{d}]")
    if workspace is None:
        workspace = torch.empty(max(moe_ffn_workspace_bytes(wg, wd, rows, topk), 1), dtype=torch.uint8,
                                device=x.device)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_moe_ffn_q8(ctypes.byref(wg.desc), ctypes.byref(wu.desc), ctypes.byref(wd.desc), px, pr, rows,
                                topk, pl, py, workspace.data_ptr(), workspace.numel(), status.data_ptr(), s),
           "int_moe_ffn_q8")
    if check:
        _raise_status(status, "int_moe_ffn_q8")
    return y


def workspace_bytes(w: PackedWeights, t: int, limbs: int = 3, schedule: str = "default") -> int:
    return int(lib().ei_gemm_workspace_bytes(ctypes.byref(w.desc), t, limbs, SCHEDULES[schedule]))


def _gemm(fn: str, w: PackedWeights, x: torch.Tensor, xdt, limbs: int, schedule: str, seed: int,
          out, workspace, status) -> torch.Tensor:
    s = _stream()
    t, k = x.shape
    if k != w.k:
        raise EIError(f"{fn}: x has k={k}, weights k={w.k}")
    px = _dev(x, xdt, "x")
    y = out if out is not None else torch.empty((t, w.n), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    if tuple(y.shape) != (t, w.n):
        raise EIError(f"{fn}: y must be [{t}][{w.n}]")
    need = workspace_bytes(w, t, limbs, schedule)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    pw = workspace.data_ptr() if workspace is not None else None
    wsz = workspace.numel() if workspace is not None else 0
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(getattr(lib(), fn)(ctypes.byref(w.desc), px, py, t, limbs, SCHEDULES[schedule], seed,
                              pw, wsz, status.data_ptr(), s), fn)
    if check:
        _raise_status(status, fn)
    return y


def gemm_q8(w: PackedWeights, x: torch.Tensor, limbs: int = 3, schedule: str = "default", seed: int = 0xE1,
            out=None, workspace=None, status=None) -> torch.Tensor:
    """y = (sum_b S sum_j q x + 2^23) >> 24 for Q16 int64 activations x [t][k]."""
    return _gemm("int_gemm_q8", w, x, torch.int64, limbs, schedule, seed, out, workspace, status)


def gemm_q8_noalloc(w: PackedWeights, x: torch.Tensor, limbs: int = 3, out=None, status=None) -> torch.Tensor:
    """gemm_q8 under the default schedule with the library's own scratch array
    (int_gemm_q8_noalloc): no workspace argument, nothing allocated by the call."""
    s = _stream()
    t, k = x.shape
    if k != w.k:
        raise EIError(f"int_gemm_q8_noalloc: x has k={k}, weights k={w.k}")
    px = _dev(x, torch.int64, "x")
    y = out if out is not None else torch.empty((t, w.n), dtype=torch.int64, device=x.device)
    py = _dev(y, torch.int64, "y")
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_gemm_q8_noalloc(ctypes.byref(w.desc), px, py, t, limbs, status.data_ptr(), s),
           "int_gemm_q8_noalloc")
    if check:
        _raise_status(status, "int_gemm_q8_noalloc")
    return y


def gemm_q8_multi(ws, x: torch.Tensor, limbs: int = 3, outs=None, status=None):
    """Several Q8 projections of the same x [t][k] (t <= 4) in one launch:
    returns [gemm_q8(w, x) for w in ws] (list of int64 [t][w.n])."""
    s = _stream()
    t, k = x.shape
    count = len(ws)
    if any(w.k != k for w in ws):
        raise EIError("int_gemm_q8_multi: every matrix must have x's k")
    px = _dev(x, torch.int64, "x")
    ys = outs if outs is not None else [torch.empty((t, w.n), dtype=torch.int64, device=x.device) for w in ws]
    if len(ys) != count or any(tuple(y.shape) != (t, w.n) for y, w in zip(ys, ws)):
        raise EIError("int_gemm_q8_multi: outs must be [t][n] per matrix")
    descs = (Weights * max(count, 1))(*[w.desc for w in ws])
    dptrs = (ctypes.POINTER(Weights) * max(count, 1))(*[ctypes.pointer(descs[m]) for m in range(count)])
    yptrs = (ctypes.c_void_p * max(count, 1))(*[_dev(y, torch.int64, "y") for y in ys])
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().int_gemm_q8_multi(ctypes.cast(dptrs, ctypes.c_void_p), count, px, ctypes.cast(yptrs, ctypes.c_void_p),
                                   t, limbs, status.data_ptr(), s), "int_gemm_q8_multi")
    if check:
        _raise_status(status, "int_gemm_q8_multi")
    return ys


def gemm_q4(w: PackedWeights, x: torch.Tensor, limbs: int = 2, schedule: str = "default", seed: int = 0xE1,
            out=None, workspace=None, status=None) -> torch.Tensor:
    """y = sum_g m 2^e sum_j q x (exact) for int32 activations x [t][k].

    limbs 2 (the default) is the two-limb form for x in [-2^15, 2^15)."""
    return _gemm("int_gemm_q4", w, x, torch.int32, limbs, schedule, seed, out, workspace, status)


def limb_split(x: torch.Tensor, limbs: int = 3):
    """Balanced base-256 limbs of int64 x: (d int8 [limbs][n], status int32 [1])."""
    s = _stream()
    xf = x.reshape(-1)
    d = torch.empty((limbs, xf.numel()), dtype=torch.int8, device=x.device)
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().ei_limb_split(_dev(xf, torch.int64, "x"), d.data_ptr(), xf.numel(), limbs, status.data_ptr(), s),
           "ei_limb_split")
    return d, status


def silu_lut(device="cuda") -> torch.Tensor:
    """The 65537-entry SiLU table, built on the device."""
    s = _stream()
    lut = torch.empty(65537, dtype=torch.int32, device=device)
    _check(lib().ei_silu_lut_build(lut.data_ptr(), s), "ei_silu_lut_build")
    return lut


def silu_mul(g: torch.Tensor, u: torch.Tensor, lut: torch.Tensor, out=None, status=None) -> torch.Tensor:
    """h = (lut[clamp((g + 16) >> 5)] * u) >> 16, elementwise (int64)."""
    s = _stream()
    if g.shape != u.shape:
        raise EIError("silu_mul: gate and up shapes differ")
    h = out if out is not None else torch.empty_like(g)
    check = status is None
    if check:
        status = torch.zeros(1, dtype=torch.int32, device=g.device)
    _check(lib().silu_lut_epilogue(_dev(g, torch.int64, "gate"), _dev(u, torch.int64, "up"),
                                   _dev(lut, torch.int32, "lut"), _dev(h, torch.int64, "h"), g.numel(),
                                   status.data_ptr(), s), "silu_lut_epilogue")
    if check:
        _raise_status(status, "silu_lut_epilogue")
    return h


def fp32_shadow(codes: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, schedule: str = "canonical",
                seed: int = 0xE1) -> torch.Tensor:
    """The float32 shadow of the Q8 projection in one schedule's order (contrast only)."""
    s = _stream()
    n, k = codes.shape
    t = x.shape[0]
    y = torch.empty((t, n), dtype=torch.float32, device=x.device)
    _check(lib().ei_q8_fp32_shadow(_dev(codes, torch.int8, "codes"), _dev(scales, torch.int32, "scales"),
                                   _dev(x, torch.int64, "x"), y.data_ptr(), n, k, t, SCHEDULES[schedule], seed, s),
           "ei_q8_fp32_shadow")
    return y


def digest(t: torch.Tensor) -> str:
    """SHA-256 (hex) of a device tensor's raw little-endian bytes (synchronises)."""
    s = _stream()
    if not t.is_contiguous():
        raise EIError("digest: tensor must be contiguous")
    out = (ctypes.c_uint8 * 32)()
    _check(lib().output_digest(t.data_ptr(), t.numel() * t.element_size(), out, s), "output_digest")
    return bytes(out).hex()


def sha256_host(data: bytes) -> str:
    """The library's SHA-256 of a host byte string (host-only)."""
    out = (ctypes.c_uint8 * 32)()
    buf = ctypes.create_string_buffer(data, len(data))
    lib().ei_sha256_host(buf, len(data), out)
    return bytes(out).hex()
