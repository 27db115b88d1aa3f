"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every comparison uses the same seeded inputs on both sides.  The bar:
  * quantiser: codes, scales and gscale bit-exact with the oracle;
  * GEMV: |y - y_ref| <= 1e-3 * sum_k |w x| + one bf16 ulp of y_ref, with y_ref
    the oracle's fp64 sum;
  * invariants: bit-exact (a token's result in an n-token launch equals the
    n = 1 launch and every tile schedule; permutation, negation, exact 2^j
    scaling; fused QKV equals the three slices of the plain GEMV).
"""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_02_amd as nv
import oracle as O
from nvfp4_weight_only_02_amd import inputs, probes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    nv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


# ---- helpers -----------------------------------------------------------------

def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def y_bits(Y: torch.Tensor) -> np.ndarray:
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def packed_from_canonical(codes, scales, g, N, K) -> nv.PackedWeight:
    return nv.PackedWeight.from_canonical(to_dev_u8(codes), to_dev_u8(scales), g, N, K)


_cases = {}


def weight_case(N, K, seed, zero_outlier=False):
    key = (N, K, seed, zero_outlier)
    if key not in _cases:
        if len(_cases) > 4:
            _cases.clear()
        W = inputs.weights_f32(N, K, seed)
        if zero_outlier:
            W = inputs.add_zero_and_outlier_blocks(W, seed + 7)
        codes, scales, g = O.quantize(W)
        _cases[key] = (W, codes, scales, g)
    return _cases[key]


def assert_parity(Ybits, Yref, Aref, what=""):
    y = O.bf16_bits_to_f64(Ybits)
    tol = O.tolerance(Yref, Aref)
    err = np.abs(y - Yref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), bad.size, float(np.max(err / tol)))


# ---- quantiser -----------------------------------------------------------------

@pytest.mark.parametrize("N,K,kind", [
    (1024, 1024, "plain"), (37, 144, "plain"), (1, 16, "plain"), (300, 6144, "zero_outlier"),
    (64, 64, "zeros"), (8, 32, "tiny"), (16, 48, "signed_zero")])
def test_quantize_matches_oracle(N, K, kind):
    say("quantize", N, K, kind)
    if kind == "zeros":
        W = np.zeros((N, K), dtype=np.float32)
    elif kind == "tiny":
        W = inputs.weights_f32(N, K, 3) * np.float32(1e-30)
        W[0, 0] = np.float32(3e38)
    elif kind == "signed_zero":
        W = inputs.weights_f32(N, K, 4)
        W[::3] = -0.0
        W[1, :16] = 0.0
    else:
        W = inputs.weights_f32(N, K, 5)
        if kind == "zero_outlier":
            W = inputs.add_zero_and_outlier_blocks(W, 6)
    codes, scales, g = O.quantize(W)
    c, s, ts = nv.quantize(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), codes)
    assert np.array_equal(s.cpu().numpy().reshape(scales.shape), scales)
    assert float(ts[0].item()) == g
    assert float(ts[1].item()) == float(np.abs(W).max())


@pytest.mark.parametrize("N,K,kind", [
    (1024, 1024, "f32"), (37, 144, "f32"), (1, 16, "f32"), (300, 6160, "f32_zero_outlier"),
    (64, 64, "zeros"), (45, 656, "bf16"), (1024, 1024, "bf16")])
def test_quantize_packed_equals_quantize_then_pack(N, K, kind):
    """The fused quantiser writes the packed layout byte for byte as
    pack(quantize(W)) would (padding included), and quantize(W) is the
    oracle's recipe bit for bit (test above); bf16 input is the recipe on
    the exactly widened values."""
    say("quantize_packed", N, K, kind)
    if kind == "zeros":
        W = np.zeros((N, K), dtype=np.float32)
    else:
        W = inputs.weights_f32(N, K, 11)
        if kind == "f32_zero_outlier":
            W = inputs.add_zero_and_outlier_blocks(W, 12)
    if kind == "bf16":
        Wd = torch.from_numpy(W).cuda().to(torch.bfloat16)
        W32 = inputs.bf16_bits_to_f32(Wd.view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        Wd = torch.from_numpy(W).cuda()
        W32 = W
    cp, sp, ts = nv.quantize_packed(Wd)
    codes, scales, g = O.quantize(W32)
    pw = packed_from_canonical(codes, scales, g, N, K)
    torch.cuda.synchronize()
    assert torch.equal(cp, pw.codes)
    assert torch.equal(sp, pw.scales)
    assert float(ts[0].item()) == g
    assert float(ts[1].item()) == float(np.abs(W32).max())


# ---- GEMV parity -----------------------------------------------------------------

@pytest.mark.parametrize("n", list(range(1, 17)))
def test_gemv_parity_1024(n):
    say("gemv 1024x1024 n", n)
    W, codes, scales, g = weight_case(1024, 1024, inputs.weight_seed(0))
    pw = packed_from_canonical(codes, scales, g, 1024, 1024)
    X = inputs.activations_bf16(n, 1024, inputs.act_seed(0, n))
    Y = nv.gemv(pw, x_to_dev(X))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(Y), Yref, Aref, "1024x1024 n=%d" % n)


@pytest.mark.parametrize("N,K", [(1, 16), (37, 144), (100, 272), (16, 128), (33, 1040),
                                 (50, 8192), (300, 640), (2049, 96),
                                 # K split into chunks (several X slices per wave):
                                 # ragged last chunk, exact chunks, ragged K tile
                                 (40, 8208), (64, 14336), (37, 12304),
                                 # one-pass kernels with exactly 3 and 7 tiles per wave
                                 (4100, 3072), (2000, 7168)])
@pytest.mark.parametrize("n", [1, 5, 16])
def test_gemv_parity_ragged(N, K, n):
    say("gemv ragged", N, K, n)
    W, codes, scales, g = weight_case(N, K, 100 + N + K)
    pw = packed_from_canonical(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, 200 + n)
    Y = nv.gemv(pw, x_to_dev(X))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(Y), Yref, Aref, "%dx%d n=%d" % (N, K, n))


def test_product_path_from_float_matches_oracle():
    say("from_float 512x2048")
    W = inputs.weights_f32(512, 2048, 9)
    pw = nv.PackedWeight.from_float(torch.from_numpy(W).cuda())
    codes, scales, g = O.quantize(W)
    assert pw.gscale == g
    X = inputs.activations_bf16(7, 2048, 10)
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(y_bits(nv.gemv(pw, x_to_dev(X))), Yref, Aref, "from_float")


def test_one_hot_is_exact_dequant():
    """gscale = 1 and X one-hot at column k make Y[t][r] = E2M1 * E4M3 exactly."""
    say("one-hot 64x256")
    rng = np.random.default_rng(21)
    N, K = 64, 256
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    pw = packed_from_canonical(codes, scales, 1.0, N, K)
    Wd = O.dequant(codes, scales, 1.0)
    for k0 in range(0, K, 16):
        X = np.zeros((16, K), dtype=np.float32)
        X[np.arange(16), k0 + np.arange(16)] = 1.0
        Y = O.bf16_bits_to_f64(y_bits(nv.gemv(pw, x_to_dev(inputs.f32_to_bf16_bits(X)))))
        assert np.array_equal(Y, Wd[:, k0:k0 + 16].T), k0


# ---- bit-identity invariants at a full decode shape ---------------------------------

@pytest.fixture(scope="module")
def qkvz():
    say("build ssm_qkvz 16384x5120")
    N, K = 16384, 5120
    W, codes, scales, g = weight_case(N, K, inputs.weight_seed(3))
    pw = packed_from_canonical(codes, scales, g, N, K)
    X = inputs.activations_bf16(16, K, inputs.act_seed(3, 16), row_scale=True)
    return pw, codes, scales, g, X


def test_qkvz_full_parity_n16(qkvz):
    say("qkvz full parity n=16")
    pw, codes, scales, g, X = qkvz
    Y = y_bits(nv.gemv(pw, x_to_dev(X)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "qkvz n=16")


def test_token_result_independent_of_n(qkvz):
    say("identity across n")
    pw, _, _, _, X = qkvz
    Xd = x_to_dev(X)
    full = y_bits(nv.gemv(pw, Xd))
    for t in range(16):
        one = y_bits(nv.gemv(pw, Xd[t:t + 1].contiguous()))
        assert np.array_equal(one[0], full[t]), t
    for n in range(1, 16):
        part = y_bits(nv.gemv(pw, Xd[:n].contiguous()))
        assert np.array_equal(part, full[:n]), n
    for a in (3, 9):   # a window of tokens that does not start at token 0
        part = y_bits(nv.gemv(pw, Xd[a:16].contiguous()))
        assert np.array_equal(part, full[a:16]), a


@pytest.mark.parametrize("sched", [[3, 3, 3, 3, 3, 1], [16], [8, 8], [4, 4, 4, 4], [1] * 16, [5, 11]])
def test_schedule_independence(qkvz, sched):
    say("schedule", sched)
    pw, _, _, _, X = qkvz
    Xd = x_to_dev(X)
    ref = y_bits(nv.gemv(pw, Xd))
    assert np.array_equal(y_bits(nv.gemv_sched(pw, Xd, sched)), ref)


def test_permutation_negation_scaling(qkvz):
    say("permutation / negation / scaling")
    pw, _, _, _, X = qkvz
    ref = y_bits(nv.gemv(pw, x_to_dev(X)))
    perm = np.random.default_rng(3).permutation(16)
    assert np.array_equal(y_bits(nv.gemv(pw, x_to_dev(X[perm]))), ref[perm])
    neg = y_bits(nv.gemv(pw, x_to_dev(X ^ np.uint16(0x8000))))
    assert np.array_equal(neg, ref ^ np.uint16(0x8000))
    X8 = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(X) * np.float32(8))
    y8 = O.bf16_bits_to_f64(y_bits(nv.gemv(pw, x_to_dev(X8))))
    assert np.array_equal(y8, 8 * O.bf16_bits_to_f64(ref))
    pw4 = nv.PackedWeight(pw.codes, pw.scales, pw.gscale * 0.25, pw.N, pw.K)
    y4 = O.bf16_bits_to_f64(y_bits(nv.gemv(pw4, x_to_dev(X))))
    assert np.array_equal(y4, 0.25 * O.bf16_bits_to_f64(ref))


def test_zero_weight_gives_zero():
    say("zero weight")
    N, K = 96, 512
    pw = packed_from_canonical(np.zeros((N, K // 2), np.uint8), np.full((N, K // 16), 0x38, np.uint8),
                               1.0, N, K)
    X = inputs.activations_bf16(16, K, 5)
    assert not O.bf16_bits_to_f64(y_bits(nv.gemv(pw, x_to_dev(X)))).any()


# ---- fused QKV and output bounds ------------------------------------------------------

def test_fused_qkv_equals_slices_and_respects_offsets():
    say("fused QKV 14336x5120")
    N, K, rows = 14336, 5120, inputs.QKV_ROWS
    W, codes, scales, g = weight_case(N, K, inputs.weight_seed(1))
    pw = packed_from_canonical(codes, scales, g, N, K)
    for n in (1, 4, 16):
        X = x_to_dev(inputs.activations_bf16(n, K, inputs.act_seed(1, n)))
        plain = y_bits(nv.gemv(pw, X))
        off = (0, 8192 + 64, 8192 + 64 + 3072 + 32)
        ldy = off[2] + 3072 + 48
        canary = torch.full((n, ldy), -7.0, dtype=torch.bfloat16, device="cuda")
        out = y_bits(nv.gemv_qkv(pw, X, rows, off, ldy, out=canary))
        start = 0
        mask = np.ones(ldy, dtype=bool)
        for p in range(3):
            assert np.array_equal(out[:, off[p]:off[p] + rows[p]], plain[:, start:start + rows[p]])
            mask[off[p]:off[p] + rows[p]] = False
            start += rows[p]
        assert (O.bf16_bits_to_f64(out[:, mask]) == -7.0).all()


def test_guard_band_untouched():
    say("guard band 1000x1024")
    N, K, n, G = 1000, 1024, 13, 4096
    W, codes, scales, g = weight_case(N, K, 31)
    pw = packed_from_canonical(codes, scales, g, N, K)
    X = x_to_dev(inputs.activations_bf16(n, K, 32))
    buf = torch.full((G + n * N + G,), 3.0, dtype=torch.bfloat16, device="cuda")
    nv.gemv(pw, X, out=buf[G:G + n * N].view(n, N))
    b = O.bf16_bits_to_f64(y_bits(buf))
    assert (b[:G] == 3.0).all() and (b[G + n * N:] == 3.0).all()


# ---- full-size parity of every workload ------------------------------------------------

@pytest.mark.parametrize("name,N,K,cfg,zero_outlier,row_scale", [
    ("fused_qkv", 14336, 5120, 1, False, False),
    ("ssm_out_proj", 5120, 6144, 3, True, False),
    ("ssm_out_proj_plain", 5120, 6144, 3, False, False),
])
@pytest.mark.parametrize("n", [1, 3, 16])
def test_full_size_parity(name, N, K, cfg, zero_outlier, row_scale, n):
    say("full size", name, n)
    W, codes, scales, g = weight_case(N, K, inputs.weight_seed(cfg), zero_outlier)
    pw = packed_from_canonical(codes, scales, g, N, K)
    X = inputs.activations_bf16(n, K, inputs.act_seed(cfg, n), row_scale=row_scale)
    Y = y_bits(nv.gemv(pw, x_to_dev(X)))
    Yref, Aref = O.gemv(codes, scales, g, X)
    assert_parity(Y, Yref, Aref, "%s n=%d" % (name, n))


@pytest.fixture(scope="module")
def out_proj():
    say("build ssm_out_proj 5120x6144 (1% zero + 1% outlier blocks)")
    N, K = 5120, 6144
    W, codes, scales, g = weight_case(N, K, inputs.weight_seed(4), zero_outlier=True)
    pw = packed_from_canonical(codes, scales, g, N, K)
    X = inputs.activations_bf16(16, K, inputs.act_seed(4, 16))
    Yref, Aref = O.gemv(codes, scales, g, X)
    return pw, X, Yref, Aref


def test_out_proj_every_n(out_proj):
    """ssm_out_proj 5120x6144 at every n = 1..16 (each n of a quad runs its own
    kernel instantiation): every output against the oracle, and each token
    bit-identical with the 16-token launch."""
    pw, X, Yref, Aref = out_proj
    Xd = x_to_dev(X)
    full = y_bits(nv.gemv(pw, Xd))
    assert_parity(full, Yref, Aref, "out_proj n=16")
    for n in range(1, 16):
        say("out_proj n", n)
        Y = y_bits(nv.gemv(pw, Xd[:n].contiguous()))
        assert_parity(Y, Yref[:n], Aref[:n], "out_proj n=%d" % n)
        assert np.array_equal(Y, full[:n]), n


def test_gemv_sched_rejects_a_wrong_output_shape():
    W, codes, scales, g = weight_case(1024, 1024, inputs.weight_seed(0))
    pw = packed_from_canonical(codes, scales, g, 1024, 1024)
    X = x_to_dev(inputs.activations_bf16(4, 1024, 5))
    with pytest.raises(ValueError):
        nv.gemv_sched(pw, X, [3, 1], out=torch.empty((3, 1024), dtype=torch.bfloat16, device="cuda"))


def test_gemv_qkv_needs_three_projections():
    W, codes, scales, g = weight_case(1024, 1024, inputs.weight_seed(0))
    pw = packed_from_canonical(codes, scales, g, 1024, 1024)
    X = x_to_dev(inputs.activations_bf16(4, 1024, 5))
    with pytest.raises(ValueError):
        nv.gemv_qkv(pw, X, (512, 512), (0, 512), 1024)
    with pytest.raises(ValueError):
        nv.gemv_qkv(pw, X, (512, 256, 256), (0, 512), 1024)


def test_block_rate_probe_runs():
    """The MFMA-vs-VALU arithmetic-rate probe launches for every n it takes
    and writes its sink (its values carry no meaning)."""
    sink = torch.full((256 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    for path in (probes.RATE_MFMA, probes.RATE_VALU):
        for n in (1, 2, 4, 8, 12, 16):
            sink.fill_(float("nan"))
            probes.block_rate(path, n, 64, sink)
            torch.cuda.synchronize()
            assert not bool(torch.isnan(sink).all()), (path, n)


def test_empty_launch_probe_runs():
    for wg in (1, 256, 4096):
        probes.empty(wg)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [probes.XSTAGE_LOADS, probes.XSTAGE_FULL])
def test_x_stage_probe_runs_and_leaves_data(mode):
    X = x_to_dev(inputs.activations_bf16(16, 5120, 11))
    before = X.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    probes.x_stage(X, 256, 4, mode, sink)
    torch.cuda.synchronize()
    assert torch.equal(X.view(torch.int16), before.view(torch.int16))
    assert int(sink.item()) == 0


def test_read_stream_runs_and_leaves_data():
    """The read-ceiling aid reads a buffer without changing it (sink written
    only on a checksum value the data below cannot produce)."""
    say("read_stream 1 MiB + 48 B")
    buf = torch.arange((1 << 20) + 48, dtype=torch.int32, device="cuda").to(torch.uint8)
    ref = buf.clone()
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    probes.read_stream(buf, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
    assert int(sink.item()) == 7


# ---- K longer than one chunk: a dense-FFN down projection -------------------------

@pytest.fixture(scope="module")
def ffn_down():
    say("build ffn down 5120x17408")
    N, K = 5120, 17408
    W, codes, scales, g = weight_case(N, K, inputs.weight_seed(6))
    pw = packed_from_canonical(codes, scales, g, N, K)
    X = inputs.activations_bf16(16, K, inputs.act_seed(6, 16))
    return pw, codes, scales, g, X


@pytest.mark.parametrize("n", [1, 5, 16])
def test_ffn_down_parity(ffn_down, n):
    say("ffn down parity n", n)
    pw, codes, scales, g, X = ffn_down
    Y = y_bits(nv.gemv(pw, x_to_dev(X[:n])))
    Yref, Aref = O.gemv(codes, scales, g, X[:n])
    assert_parity(Y, Yref, Aref, "ffn down 5120x17408 n=%d" % n)


def test_ffn_down_token_identity(ffn_down):
    say("ffn down identity across n")
    pw, _, _, _, X = ffn_down
    Xd = x_to_dev(X)
    full = y_bits(nv.gemv(pw, Xd))
    for n in (1, 3, 8):
        assert np.array_equal(y_bits(nv.gemv(pw, Xd[:n].contiguous())), full[:n]), n


# ---- the small hidden-2048 attention layer ----------------------------------------

@pytest.mark.parametrize("n", [1, 16])
def test_small_attention_shapes(n):
    """Fused q|k|v 4096|512|512 x 2048 and o_proj 2048 x 4096: fewer row groups
    than compute units (one per workgroup)."""
    say("small attention n", n)
    for N, K, rows in ((5120, 2048, (4096, 512, 512)), (2048, 4096, None)):
        W, codes, scales, g = weight_case(N, K, 500 + K)
        pw = packed_from_canonical(codes, scales, g, N, K)
        X = inputs.activations_bf16(n, K, 600 + n)
        Yref, Aref = O.gemv(codes, scales, g, X)
        if rows:
            off = (0, rows[0], rows[0] + rows[1])
            Y = y_bits(nv.gemv_qkv(pw, x_to_dev(X), rows, off, N))
        else:
            Y = y_bits(nv.gemv(pw, x_to_dev(X)))
        assert_parity(Y, Yref, Aref, "%dx%d n=%d" % (N, K, n))
