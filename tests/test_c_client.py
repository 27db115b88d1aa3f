"""The library from plain C (tests/c_client/gemv_client.c): only include/nvfp4.h
and the HIP runtime, no Python in the caller.  Without a GPU the client is
compiled and linked against the built libnvfp4.so with gcc; on the GPU it
packs a weight, runs nvfp4_gemv and nvfp4_gemv_qkv, and its outputs are
checked against the oracle (same bar as the Python-side tests)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
from nvfp4_weight_only_02_amd import build, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "gemv_client.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compile_client(out_dir):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not found")
    if not os.path.exists(build.LIB):
        pytest.skip("library not built")
    exe = os.path.join(str(out_dir), "gemv_client")
    pkg = os.path.dirname(build.LIB)
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", exe,
           "-L", pkg, "-lnvfp4", "-Wl,-rpath," + pkg,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_client_compiles_and_links(tmp_path):
    exe = compile_client(tmp_path)
    assert os.access(exe, os.X_OK)
    # wrong usage is reported without touching the GPU
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 1 and "usage" in res.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("N,K,n", [(1000, 5120, 16), (333, 2000, 5)])
def test_client_results_match_oracle(tmp_path, N, K, n):
    exe = compile_client(tmp_path)
    W = inputs.weights_f32(N, K, 31 + N)
    codes, scales, g = O.quantize(W)
    X = inputs.activations_bf16(n, K, 37 + K)
    files = {k: os.path.join(str(tmp_path), k + ".bin") for k in ("codes", "scales", "x", "y", "yq")}
    codes.tofile(files["codes"])
    scales.tofile(files["scales"])
    np.ascontiguousarray(X).tofile(files["x"])
    print("c client", N, K, n, flush=True)
    res = subprocess.run([exe, str(N), str(K), str(n), repr(float(g)), files["codes"], files["scales"],
                          files["x"], files["y"], files["yq"]], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr + res.stdout
    Y = np.fromfile(files["y"], dtype=np.uint16).reshape(n, N)
    YQ = np.fromfile(files["yq"], dtype=np.uint16).reshape(n, N + 32)
    Yref, Aref = O.gemv(codes, scales, g, X)
    err = np.abs(O.bf16_bits_to_f64(Y) - Yref)
    tol = O.tolerance(Yref, Aref)
    assert (err <= tol).all(), float((err / tol).max())
    # the fused-QKV output is the same bits, rearranged: v, then q, then k
    q, k = N // 2, N // 4
    assert (YQ[:, :32] == 0).all()
    assert np.array_equal(YQ[:, 32:32 + (N - q - k)], Y[:, q + k:])
    assert np.array_equal(YQ[:, 32 + (N - q - k):32 + (N - k)], Y[:, :q])
    assert np.array_equal(YQ[:, 32 + (N - k):], Y[:, q:q + k])
