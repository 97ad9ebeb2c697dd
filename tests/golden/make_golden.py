"""Write the stored expected values under tests/golden/ (CPU only).

Calls only the oracle (and the shared seeded input generators): no value
written here comes from the GPU path.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main(threads: int = 8) -> None:
    lut = oracle.silu_lut()
    with open(os.path.join(HERE, "silu_lut.sha256"), "w") as f:
        f.write(oracle.digest(lut) + "  silu_lut int32[65537] little-endian\n")

    out = {}
    (w, s), x = synth.q8_896_inputs()
    out["q8_896x896"] = {"inputs": synth.input_sha256(w, s, x), "y": oracle.digest(oracle.q8(w, s, x))}

    mats, x = synth.qkv_inputs()
    rec = {"inputs_x": synth.input_sha256(x)}
    for name, (c, sc) in mats.items():
        rec[name] = oracle.digest(oracle.q8(c, sc, x))
        rec[name + "_fp32"] = {o: oracle.digest(oracle.q8_fp32(c, sc, x, o)) for o in oracle.SCHEDULES}
    out["qkv_gate"] = rec

    rec = {}
    for name, (n, k) in synth.Q4_SHAPES.items():
        nib, sme = synth.q4_d512_matrix(name)
        for t in (1, 64):
            rec[f"{name}_t{t}"] = oracle.digest(oracle.q4(nib, sme, synth.q4_d512_x(k, t), threads=threads))
    out["q4_d512"] = rec

    x = synth.qwen_ffn_x0()
    layers = []
    for layer in range(synth.QWEN_LAYERS):
        wg, wu, wd = synth.qwen_ffn_layer(layer)
        g, u, h, d, x = oracle.ffn_layer(x, wg, wu, wd, lut, threads=threads)
        layers.append({"g": oracle.digest(g), "u": oracle.digest(u), "h": oracle.digest(h),
                       "d": oracle.digest(d), "x_next": oracle.digest(x)})
        print("ffn layer", layer, layers[-1]["x_next"][:16], flush=True)
    out["qwen05b_ffn"] = {"layers": layers}

    x = synth.qwen_ffn_x0()
    layers = []
    for layer in range(synth.QWEN_LAYERS):
        wg, wu, wd = synth.qwen_ffn_layer(layer)
        _, d, x = oracle.ffn_layer_prenorm(x, synth.qwen_norm_weight(layer), synth.QWEN_RMS_EPS_Q32, wg, wu, wd,
                                           lut, threads=threads)
        layers.append({"d": oracle.digest(d), "x_next": oracle.digest(x)})
        print("prenorm ffn layer", layer, layers[-1]["x_next"][:16], flush=True)
    out["qwen05b_ffn_prenorm"] = {"eps_q32": synth.QWEN_RMS_EPS_Q32, "layers": layers}

    c, a = synth.wide_inputs()
    out["wide_896x896_t4096"] = {"inputs": synth.input_sha256(c, a), "y": oracle.digest(oracle.wide_gemm(c, a))}

    (rc, rs), xo = synth.olmoe_router(), synth.olmoe_x()
    scores = oracle.q8(rc, rs, xo, threads=threads)
    iroute = oracle.topk_route(scores, synth.OLMOE_TOPK)
    print("olmoe step, integer route", flush=True)
    out["olmoe_router"] = {"scores": oracle.digest(scores), "route": oracle.digest(iroute),
                           "y": oracle.digest(oracle.moe_pairs(xo, iroute, synth.olmoe_expert, lut,
                                                               threads=threads))}
    # the whole routed step (every one of the 4096 token-expert pairs), with
    # the seeded route
    print("olmoe step, seeded route", flush=True)
    out["olmoe_step"] = {"y": oracle.digest(oracle.moe_pairs(xo, synth.olmoe_route(), synth.olmoe_expert, lut,
                                                             threads=threads))}

    w, s = synth.dense_w()
    x1 = synth.dense_x(1)
    print("dense 14336x4096, T = 1 and 512", flush=True)
    out["dense_14336x4096"] = {"t1_y": oracle.digest(oracle.q8(w, s, x1, threads=threads)),
                               "t512_y": oracle.digest(oracle.q8(w, s, synth.dense_x(512), threads=threads))}

    with open(os.path.join(HERE, "oracle_digests.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
