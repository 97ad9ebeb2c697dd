"""The allocation-free projection (int_gemm_q8_noalloc) against the projection
with a caller workspace (int_gemm_q8), through the C ABI (GPU).

The allocation-free call keeps its scratch in one array per device that every
call shares, so the test makes calls in a row: a large one, then smaller ones
that reuse the array with different sizes and paths, each compared bit for bit
with int_gemm_q8 under the default schedule and, at small sizes, with the
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ei():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import exact_integer_amd
    return exact_integer_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(ei, seed, n, k, t):
    r = np.random.default_rng(seed)
    q, s, x = synth.q8_codes(r, n, k), synth.q8_scales(r, n, k), synth.q16_acts(r, t, k)
    return q, s, x, ei.pack_q8(dev(q), dev(s))


def test_noalloc_equals_workspace_projection_in_a_row(ei):
    # 1: the tiled prefill path (6 MB of limb tiles in the scratch array);
    # 2: a smaller skinny call with workgroup partials (T=30); 3: smaller again
    # (T=5, ragged); 4: the GEMV path (no scratch); 5: the first shape again
    cases = [(1, 4096, 4096, 512), (2, 896, 4864, 30), (3, 100, 320, 5), (4, 37, 96, 1), (1, 4096, 4096, 512)]
    for seed, n, k, t in cases:
        q, s, x, w = _case(ei, seed, n, k, t)
        xd = dev(x)
        print("noalloc", (n, k, t), flush=True)
        want = ei.gemm_q8(w, xd)
        got = ei.gemm_q8_noalloc(w, xd)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (n, k, t)
        if n * k * t <= 2_000_000:
            assert (got.cpu().numpy() == oracle.q8(q, s, x)).all(), (n, k, t)


def test_noalloc_rejects_work_beyond_its_scratch(ei):
    # 3 limbs x 3072 tokens x 4096 columns of limb tiles = 36 MiB > 32 MiB
    _, _, _, w = _case(ei, 5, 64, 4096, 1)
    x = torch.zeros((3072, 4096), dtype=torch.int64, device="cuda")
    with pytest.raises(ei.EIError, match="int_gemm_q8_noalloc"):
        ei.gemm_q8_noalloc(w, x)
    # the array is still usable afterwards
    q, s, x2, w2 = _case(ei, 6, 70, 160, 9)
    assert (ei.gemm_q8_noalloc(w2, dev(x2)).cpu().numpy() == oracle.q8(q, s, x2)).all()
