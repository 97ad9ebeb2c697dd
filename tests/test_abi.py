"""The C ABI library loads and exports every symbol its header declares (CPU).

No device compute is called here; the host-only SHA-256 is checked against
Python's hashlib.
"""
import glob
import hashlib
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            if not text[m.start():].startswith(("typedef", "enum", "struct", "#")):
                names.add(m.group(1))
    return names


def test_header_declares_the_entry_points():
    names = _declared()
    for required in ("int_gemm_q8", "int_gemm_q4", "silu_lut_epilogue", "output_digest", "ei_q8_pack",
                     "ei_q4_pack", "ei_limb_split", "ei_silu_lut_build"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import exact_integer_amd as ei
    lib = ei.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(ei.SIGNATURES) >= _declared(), sorted(_declared() - set(ei.SIGNATURES))
    assert lib.ei_version() == 109


def test_host_sha256_matches_hashlib():
    import exact_integer_amd as ei
    r = np.random.default_rng(3)
    for n in (0, 1, 55, 56, 63, 64, 65, 119, 120, 128, 1000, 4099):
        data = r.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert ei.sha256_host(data) == hashlib.sha256(data).hexdigest()


def test_status_strings():
    import exact_integer_amd as ei
    assert ei.lib().ei_status_string(0) == b"ok"
    assert ei.lib().ei_status_string(2) == b"outside the exactness envelope"


def test_compute_calls_refuse_without_a_device():
    import pytest
    import torch
    import exact_integer_amd as ei
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present")
    with pytest.raises(ei.EIError):
        ei.silu_lut()
