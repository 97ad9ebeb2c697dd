"""Seeded synthetic inputs for the exact-integer block-quantized projection.

This module is the only code shared by the CPU oracle and the GPU path: it
draws input bytes (weight codes, block scales, activations, routing indices)
from seeded numpy generators and holds none of the projection's arithmetic.

Every tensor comes from its own generator, seeded by the first 8 bytes
(little-endian) of SHA-256("ei/v1/{workload}/{layer}/{tensor}"), so any
tensor of any layer can be regenerated alone, on any host, bit-identically.

The recipes follow the workloads' statement of the inputs:
  * 8-bit codes uniform in [-127, 127], one int32 scale per 32-wide block
    along K, S = rint(|N(0, 0.02)| / 127 * 2**24) (a Q24 integer);
  * Q16 activations rint(N(0, 1) * 2**16) clipped to +-2**22, as int64;
  * 4-bit codes uniform in [-8, 7] (two's-complement nibbles, element 2k in
    the low nibble of byte k), one scale byte per group of 32 holding the
    mantissa m in [1, 15] in the low nibble and the exponent e in [0, 15] in
    the high nibble; int32 activations uniform in [-2**15, 2**15);
  * routing: per token, top-k distinct experts drawn uniformly without
    replacement, listed in ascending expert id.
"rint" is numpy's round-half-to-even on float64; it belongs to input
generation only.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

__all__ = [
    "rng_for", "q8_codes", "q8_scales", "q16_acts", "q4_codes_packed",
    "q4_scale_bytes", "i32_acts", "routing", "WORKLOADS", "Workload",
    "q8_matrix", "q4_matrix", "input_sha256",
]


def rng_for(workload: str, layer: int, tensor: str) -> np.random.Generator:
    """Generator for one tensor of one layer of one workload."""
    h = hashlib.sha256(f"ei/v1/{workload}/{layer}/{tensor}".encode()).digest()
    return np.random.default_rng(int.from_bytes(h[:8], "little"))


def q8_codes(r: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 [n][k], uniform in [-127, 127]."""
    return r.integers(-127, 128, size=(n, k), dtype=np.int8)


def q8_scales(r: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int32 [n][k/32]: rint(|N(0, 0.02)| / 127 * 2**24)."""
    assert k % 32 == 0
    s = np.rint(np.abs(r.normal(0.0, 0.02, size=(n, k // 32))) / 127.0 * 2.0**24)
    return s.astype(np.int32)


def q16_acts(r: np.random.Generator, t: int, k: int) -> np.ndarray:
    """int64 [t][k]: rint(N(0, 1) * 2**16) clipped to +-2**22."""
    x = np.rint(r.normal(0.0, 1.0, size=(t, k)) * 2.0**16)
    return np.clip(x, -(2.0**22), 2.0**22).astype(np.int64)


def q4_codes_packed(r: np.random.Generator, n: int, k: int) -> np.ndarray:
    """uint8 [n][k/2]: codes uniform in [-8, 7] as nibbles, element 2j low."""
    assert k % 2 == 0
    c = r.integers(-8, 8, size=(n, k), dtype=np.int8)
    nib = (c.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def q4_scale_bytes(r: np.random.Generator, n: int, k: int) -> np.ndarray:
    """uint8 [n][k/32]: m in [1, 15] low nibble, e in [0, 15] high nibble."""
    assert k % 32 == 0
    m = r.integers(1, 16, size=(n, k // 32), dtype=np.int16)
    e = r.integers(0, 16, size=(n, k // 32), dtype=np.int16)
    return (m | (e << 4)).astype(np.uint8)


def i32_acts(r: np.random.Generator, t: int, k: int) -> np.ndarray:
    """int32 [t][k], uniform in [-2**15, 2**15)."""
    return r.integers(-(2**15), 2**15, size=(t, k), dtype=np.int32)


def routing(r: np.random.Generator, t: int, n_experts: int, top_k: int) -> np.ndarray:
    """int32 [t][top_k]: distinct experts per token, ascending."""
    out = np.empty((t, top_k), dtype=np.int32)
    for i in range(t):
        out[i] = np.sort(r.choice(n_experts, top_k, replace=False))
    return out


def q8_matrix(workload: str, layer: int, name: str, n: int, k: int):
    """(codes int8 [n][k], scales int32 [n][k/32]) of one named projection."""
    return (q8_codes(rng_for(workload, layer, name + ".codes"), n, k),
            q8_scales(rng_for(workload, layer, name + ".scales"), n, k))


def q4_matrix(workload: str, layer: int, name: str, n: int, k: int):
    """(nibbles uint8 [n][k/2], scale bytes uint8 [n][k/32]) of one projection."""
    return (q4_codes_packed(rng_for(workload, layer, name + ".codes"), n, k),
            q4_scale_bytes(rng_for(workload, layer, name + ".scales"), n, k))


def input_sha256(*arrays: np.ndarray) -> str:
    """SHA-256 over the little-endian bytes of the given arrays, in order."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).astype(a.dtype.newbyteorder("<"), copy=False).tobytes())
    return h.hexdigest()


@dataclass(frozen=True)
class Workload:
    name: str
    description: str


# The synthetic workloads. They stand in for the pages' real checkpoints
# (Qwen2.5-0.5B Q8_0, OLMoE-1B-7B, a 7B-class dense model), which are not
# available; only their shapes are used.
WORKLOADS = {
    "q8_896x896": Workload("q8_896x896", "single Q8 GEMV, W 896x896, T=1"),
    "qwen05b_ffn": Workload("qwen05b_ffn", "Qwen2.5-0.5B-shaped Q8 FFN, gate/up 4864x896, down 896x4864, T=30, 24 layers"),
    "q4_d512": Workload("q4_d512", "4-bit projections 512x512, 2048x512, 512x2048 at T=1 and T=64"),
    "qkv_gate": Workload("qkv_gate", "layer-0 Q 896x896, K 128x896, V 128x896 on a 4-token prefix"),
    "olmoe_grouped": Workload("olmoe_grouped", "64 experts, hidden 2048, expert intermediate 1024, top-8 of 64, T=512"),
    "dense_14336x4096": Workload("dense_14336x4096", "dense 14336x4096 Q8 at T=1 and T=512"),
}


# ------------------------------------------------------------------------
# Named workload builders (inputs only).

def q8_896_inputs():
    """W 896x896 Q8 and one Q16 token."""
    w = q8_matrix("q8_896x896", 0, "w", 896, 896)
    x = q16_acts(rng_for("q8_896x896", 0, "x"), 1, 896)
    return w, x


QWEN_D, QWEN_F, QWEN_T, QWEN_LAYERS = 896, 4864, 30, 24


def qwen_ffn_layer(layer: int):
    """(gate, up, down) of one Qwen2.5-0.5B-shaped FFN layer, fresh per layer."""
    return (q8_matrix("qwen05b_ffn", layer, "gate", QWEN_F, QWEN_D),
            q8_matrix("qwen05b_ffn", layer, "up", QWEN_F, QWEN_D),
            q8_matrix("qwen05b_ffn", layer, "down", QWEN_D, QWEN_F))


def qwen_ffn_x0(t: int = QWEN_T):
    return q16_acts(rng_for("qwen05b_ffn", 0, "x"), t, QWEN_D)


Q4_SHAPES = {"p512x512": (512, 512), "p2048x512": (2048, 512), "p512x2048": (512, 2048)}


def q4_d512_matrix(name: str):
    n, k = Q4_SHAPES[name]
    return q4_matrix("q4_d512", 0, name, n, k)


def q4_d512_x(k: int, t: int):
    return i32_acts(rng_for("q4_d512", 0, f"x_k{k}_t{t}"), t, k)


QKV_SHAPES = {"q": (896, 896), "k": (128, 896), "v": (128, 896)}


def qkv_inputs():
    mats = {name: q8_matrix("qkv_gate", 0, name, n, k) for name, (n, k) in QKV_SHAPES.items()}
    x = q16_acts(rng_for("qkv_gate", 0, "x"), 4, 896)
    return mats, x


OLMOE_E, OLMOE_H, OLMOE_I, OLMOE_TOPK, OLMOE_T = 64, 2048, 1024, 8, 512


def olmoe_expert(e: int):
    """(gate, up, down) of expert e: gate/up 1024x2048, down 2048x1024."""
    return (q8_matrix("olmoe_grouped", e, "gate", OLMOE_I, OLMOE_H),
            q8_matrix("olmoe_grouped", e, "up", OLMOE_I, OLMOE_H),
            q8_matrix("olmoe_grouped", e, "down", OLMOE_H, OLMOE_I))


def olmoe_x(t: int = OLMOE_T):
    return q16_acts(rng_for("olmoe_grouped", 0, "x"), t, OLMOE_H)


WIDE_N, WIDE_K, WIDE_T = 896, 896, 4096   # the wide-code hot kernel: 896x896 weights, 4096 rows


def wide_trits(r: np.random.Generator, n: int, k: int) -> np.ndarray:
    """12 balanced trits per weight, uniform in {-1, 0, 1}: int8 [12][n][k]."""
    return r.integers(-1, 2, (12, n, k)).astype(np.int8)


def wide_codes_from_trits(trits: np.ndarray) -> np.ndarray:
    """code = sum_i 3^i trit_i (the balanced-ternary value), int32 [n][k]."""
    w = np.zeros(trits.shape[1:], np.int64)
    for i in range(trits.shape[0]):
        w += (3 ** i) * trits[i].astype(np.int64)
    return w.astype(np.int32)


def wide_acts(r: np.random.Generator, t: int, k: int) -> np.ndarray:
    """Activations quantized per tensor by their own maximum to the
    interchange level 2^28: rint(v / max|v| * 2^28), v ~ N(0, 1); int32 [t][k]."""
    v = r.normal(0.0, 1.0, (t, k))
    return np.rint(v / np.abs(v).max() * 2**28).astype(np.int32)


def wide_inputs(t: int = WIDE_T):
    trits = wide_trits(rng_for("wide_gemm", 0, "w"), WIDE_N, WIDE_K)
    return wide_codes_from_trits(trits), wide_acts(rng_for("wide_gemm", 0, "x"), t, WIDE_K)


QWEN_RMS_EPS_Q32 = 4295   # eps = 1e-6 (the Qwen2.5 family's norm epsilon) in Q32


def qwen_norm_weight(layer: int):
    """The layer's RMSNorm weight in Q16: rint(N(1, 0.1) * 2^16) as int32 [896]."""
    r = rng_for("qwen05b_ffn", layer, "norm")
    return np.rint(r.normal(1.0, 0.1, QWEN_D) * 2**16).astype(np.int32)


def olmoe_router():
    """The router's Q8 weights [64 experts][2048] (integer router scores)."""
    return q8_matrix("olmoe_grouped", 0, "router", OLMOE_E, OLMOE_H)


def olmoe_route(t: int = OLMOE_T):
    return routing(rng_for("olmoe_grouped", 0, "route"), t, OLMOE_E, OLMOE_TOPK)


DENSE_N, DENSE_K = 14336, 4096


def dense_w(copy: int = 0):
    """The 14336x4096 Q8 matrix; copy > 0 gives independent same-shape copies."""
    return q8_matrix("dense_14336x4096", copy, "w", DENSE_N, DENSE_K)


def dense_x(t: int):
    return q16_acts(rng_for("dense_14336x4096", 0, f"x_t{t}"), t, DENSE_K)
