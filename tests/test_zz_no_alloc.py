"""nvfp4_gemv_ws_static, the no-allocation form of nvfp4_gemv_ws, through the
C ABI: its partials live in the library's fixed scratch memory, and its
results equal nvfp4_gemv_ws's (caller workspace) bit for bit.  Two calls in a
row on one stream, the second with a smaller input, then the first again;
sampled rows also against the CPU oracle."""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def case(N, K, n, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x28, 0x48, size=(N, K // 16), dtype=np.uint8)
    g = 1.0 / 64
    pw = nv.PackedWeight.from_canonical(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), g, N, K)
    X = inputs.activations_bf16(n, K, seed + 1)
    Xd = torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)
    return codes, scales, g, pw, X, Xd


def bits(Y):
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def test_static_scratch_equals_caller_workspace():
    assert torch.cuda.is_available()
    assert nv.gemv_static_scratch_bytes() == 8 << 20
    big = (5120, 17408, 16, 0)     # dense FFN down, the library's 4 parts: 1.3 MB of partials
    small = (1000, 9008, 3, 2)     # smaller second call, 2 parts, ragged K
    cases = {key: case(*key[:3], seed=900 + i) for i, key in enumerate((big, small))}
    results = {}
    for key in (big, small, big):
        N, K, n, ks = key
        say("ws_static", N, K, n, ks)
        codes, scales, g, pw, X, Xd = cases[key]
        Yst = bits(nv.gemv_ws_static(pw, Xd, ks))
        Yws = bits(nv.gemv_ws(pw, Xd, ks))
        assert np.array_equal(Yst, Yws), key
        rows = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
        Yref, Aref = O.gemv(codes[rows], scales[rows], g, X)
        err = np.abs(O.bf16_bits_to_f64(Yst[:, rows]) - Yref)
        assert (err <= O.tolerance(Yref, Aref)).all(), key
        if key in results:
            assert np.array_equal(results[key], Yst)
        results[key] = Yst
    # one part: no scratch touched, the plain GEMV's result
    codes, scales, g, pw, X, Xd = cases[small]
    assert np.array_equal(bits(nv.gemv_ws_static(pw, Xd, 1)), bits(nv.gemv(pw, Xd)))
