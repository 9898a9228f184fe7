"""GPU parity of the block-quantized x f32 products against the oracle:
q4_gemv / q4_gemm_ws over Q4_0 weights and q8_gemv / q8_gemm_ws over Q8_0 weights
(sections qmatvec_q4_0 and matmul_q4_0_tiled of "fuel-vulkan-kernels —
quantized (GGML) kernel contracts", whose quantized-matmul binding picks
either block format; blocks of sections dequant_q4_0 and dequant_q8_0).
Every output must satisfy |y - y_ref| <= 1e-5 * sum|a w| + 1e-6, with y_ref
the oracle's f64 sum over the dequantized weights."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
from gpu_helpers import (BLOCK_BYTES, DEV, FORMATS, Guarded, assert_within_tolerance,  # noqa: E402
                         oracle_dequant, oracle_matmul, oracle_matmul_sampled, random_blocks,
                         to_dev, weight_blob)

# "gemm" is the workspace form; "gemm_noalloc" the form with the pages' argument
# list, on the library's own scratch (the same kernels and results).
ENTRY = {("q4_0", "gemv"): binding.q4_gemv, ("q4_0", "gemm"): binding.q4_gemm_ws,
         ("q4_0", "gemm_noalloc"): binding.q4_gemm,
         ("q8_0", "gemv"): binding.q8_gemv, ("q8_0", "gemm"): binding.q8_gemm_ws,
         ("q8_0", "gemm_noalloc"): binding.q8_gemm}
WS_BYTES = {"q4_0": binding.q4_gemm_workspace_bytes, "q8_0": binding.q8_gemm_workspace_bytes}


def _run(fmt, kind, a: np.ndarray, blob: np.ndarray, N: int, K: int, w_dev=None):
    M = a.shape[0]
    y = Guarded(M * N, torch.float32)
    w = to_dev(blob) if w_dev is None else w_dev
    ENTRY[fmt, kind](to_dev(a), w, y.view, M, N, K)
    torch.cuda.synchronize()
    assert y.guards_intact()
    return y.host().reshape(M, N)


def _full_check(fmt, kind, a, blob, N, K, what, relative_only=False):
    got = _run(fmt, kind, a, blob, N, K)
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    return assert_within_tolerance(got, ref, bound, "%s %s" % (fmt, what), relative_only)


# ------------------------------------------------------------- the workloads

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", ["gemv_1x256x512", "gemv_1x4096x4096", "gemv_8x4096x4096"])
def test_gemv_workloads_full_output(fmt, name):
    s = wl.WORKLOADS[name]
    blob = weight_blob(fmt, s["N"], s["K"], s["w_seed"])
    a = wl.activations_f32(s["a_seed"], s["M"], s["K"])
    _full_check(fmt, "gemv", a, blob, s["N"], s["K"], name)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind", ["gemm", "gemm_noalloc"])
@pytest.mark.parametrize("name", ["gemm_1024x4096x4096", "gemm_2048x14336x4096"])
def test_gemm_workloads_sampled(fmt, kind, name):
    s = wl.WORKLOADS[name]
    M, N, K = s["M"], s["N"], s["K"]
    blob = weight_blob(fmt, N, K, s["w_seed"])
    a = wl.activations_f32(s["a_seed"], M, K)
    got = _run(fmt, kind, a, blob, N, K)
    # 4096 random outputs plus whole first/last rows and columns of the tiles.
    mi = np.concatenate([wl.uniform_ints(7, 0, M, 4096), np.zeros(N, np.int64),
                         np.full(N, M - 1), np.arange(M), np.arange(M)])
    ni = np.concatenate([wl.uniform_ints(8, 0, N, 4096), np.arange(N), np.arange(N),
                         np.zeros(M, np.int64), np.full(M, N - 1)])
    ref, bound = oracle_matmul_sampled(fmt)(a, blob, N, K, mi, ni)
    assert np.isfinite(got).all()
    assert_within_tolerance(got[mi, ni], ref, bound, "%s %s %s" % (fmt, kind, name))


# ------------------------------------------------------ shapes and tails

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_gemv_row_group_loop_matches_single_groups(fmt, M):
    # 9000 weight rows at K = 4096: 256 workgroups walk 563 row groups, each
    # splitting its activations once. The first and second 4096 rows run again
    # as GEMVs of their own (one row group per workgroup): every output must
    # come out with the same bits.
    N, K = 9000, 4096
    blob = weight_blob(fmt, N, K, 91 + M)
    a = wl.activations_f32(92 + M, M, K)
    w = to_dev(blob)
    a_dev = to_dev(a)
    full = torch.empty(M * N, dtype=torch.float32, device=DEV)
    binding_gemv = ENTRY[fmt, "gemv"]
    binding_gemv(a_dev, w, full, M, N, K)
    row_bytes = K // 32 * BLOCK_BYTES[fmt]
    for r0 in (0, 4096):
        part = torch.empty(M * 4096, dtype=torch.float32, device=DEV)
        binding_gemv(a_dev, w[r0 * row_bytes:(r0 + 4096) * row_bytes], part, M, 4096, K)
        torch.cuda.synchronize()
        got = full.view(M, N)[:, r0:r0 + 4096].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), part.view(M, 4096).cpu().numpy().view(np.uint32)), r0


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", [(17, 32), (300, 256), (129, 1056), (64, 4096), (33, 8192),
                                 (4097, 4096), (4200, 4096), (9000, 4096), (1000, 2048),
                                 (5000, 2048)])
def test_gemv_shapes(fmt, M, N, K):
    # More than 256 row groups at K = 4096 (one chunk per wavefront): 256
    # workgroups walk the groups, two or three each, the last one ragged (at
    # N = 4097 one workgroup takes a second group of one row).
    # K = 2048 gives one 8-block chunk per wavefront (row-group loops at
    # N = 5000); K = 8192 several chunks per wavefront, where the streaming
    # kernel reads A from LDS.
    blob = weight_blob(fmt, N, K, 10 * M + K)
    a = wl.activations_f32(20 * M + N, M, K)
    _full_check(fmt, "gemv", a, blob, N, K, "gemv %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", [(1, 300, 256), (8, 129, 64), (65, 70, 160), (5, 257, 128),
                                   (33, 6144, 2048), (128, 128, 32), (129, 129, 96),
                                   (300, 17, 4128), (257, 384, 512), (1, 1, 32),
                                   # Longer K runs in segments of at most 112 block
                                   # partials per accumulator: 2 segments at K = 14336
                                   # (the FFN down-projection), 3 at 16384; the general
                                   # kernel (K % 64 != 0) at 7200 takes 3 of 75 blocks.
                                   (96, 200, 14336), (130, 160, 16384), (40, 96, 7200),
                                   (3, 33, 7168), (17, 40, 7232),
                                   # The preparation cuts each 16-row group's K into
                                   # parts for about 256 workgroups: 3 uneven parts
                                   # (22, 22, 20 blocks) at 1500 rows, one at 4200.
                                   (1500, 64, 2048), (4200, 40, 1024)])
@pytest.mark.parametrize("kind", ["gemm", "gemm_noalloc"])
def test_gemm_shapes(fmt, M, N, K, kind):
    blob = weight_blob(fmt, N, K, 3 * M + N)
    a = wl.activations_f32(5 * M + K, M, K)
    _full_check(fmt, kind, a, blob, N, K, "%s %dx%dx%d" % (kind, M, N, K))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind,M,K", [("gemv", 1, 4096), ("gemv", 8, 2048), ("gemv", 3, 96),
                                      ("gemm", 70, 1024), ("gemm", 9, 96)])
def test_every_code_and_random_scales(fmt, kind, M, K):
    # Uniformly random block bytes: every code of the format (Q8_0's -128,
    # which no quantizer writes, included) with random finite scales.
    N = 160
    blob = random_blocks(fmt, N * K // 32, 31 + M)
    a = wl.activations_f32(32 + M, M, K)
    _full_check(fmt, kind, a, blob, N, K, "random blocks %s %dx%dx%d" % (kind, M, N, K))


# ---------------------------------------------------- degenerate inputs

ZERO_CODE_BYTE = {"q4_0": 0x88, "q8_0": 0x00}


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 8), ("gemm", 40)])
def test_zero_codes_give_zero(fmt, kind, M):
    # All nibbles 8 (Q4_0) or all bytes 0 (Q8_0): every weight is zero.
    N, K = 48, 512
    blob = weight_blob(fmt, N, K, 1).reshape(N, K // 32, -1).copy()
    blob[:, :, 2:] = ZERO_CODE_BYTE[fmt]
    a = wl.activations_f32(2, M, K)
    got = _run(fmt, kind, a, blob.reshape(-1), N, K)
    assert (got == 0).all()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 7), ("gemm", 19)])
def test_one_hot_activations_pick_weights_exactly(fmt, kind, M):
    N, K = 96, 1024
    blob = random_blocks(fmt, N * K // 32, 3)
    w = getattr(oracle, fmt + "_dequant")(blob).reshape(N, K)
    ks = wl.uniform_ints(4, 0, K, M)
    a = np.zeros((M, K), np.float32)
    a[np.arange(M), ks] = 1.0
    got = _run(fmt, kind, a, blob, N, K)
    assert (got == w[:, ks].T).all()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_zero_activations(fmt, kind):
    N, K = 40, 256
    got = _run(fmt, kind, np.zeros((3, K), np.float32), weight_blob(fmt, N, K, 5), N, K)
    assert (got == 0).all()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind", ["gemv", "gemm", "gemm_noalloc"])
@pytest.mark.parametrize("scale", [1e-38, 1e-30, 1e-8, 1e-3, 1e3, 6e4, 1e5, 1e30])
def test_activation_magnitudes(fmt, kind, scale):
    # Any finite activations, unclipped (up to 4e30 and down into the f32
    # subnormals), against weights with |d| in [1024, 8192): |y| stays far
    # from both the f32 range's ends, and the check drops the bar's absolute
    # 1e-6, which would pass anything at the small scales.
    N, K, M = 80, 2048, 4
    a = (wl.activations_f32(6, M, K) * np.float32(scale)).astype(np.float32)
    blob = random_blocks(fmt, N * K // 32, 7, 25, 28)
    _full_check(fmt, kind, a, blob, N, K, "%s scale %g" % (kind, scale), relative_only=True)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 8), ("gemm", 70)])
def test_power_of_two_row_scaling_is_exact(fmt, kind, M):
    # Row m scaled by 2^k_m (|k| up to 100, so activations reach 1.6e30)
    # scales row m of y by exactly 2^k_m, bit for bit: each row's (or K
    # stretch's) own power of two absorbs the factor before the split.
    N, K = 96, 2048
    blob = weight_blob(fmt, N, K, 61)
    a = wl.activations_f32(62, M, K)
    ks = np.array([100, -100, 37, -61, 0, 90, -1, 12] * ((M + 7) // 8))[:M]
    a2 = (a * np.ldexp(np.float32(1), ks)[:, None]).astype(np.float32)
    y1 = _run(fmt, kind, a, blob, N, K)
    y2 = _run(fmt, kind, a2, blob, N, K)
    want = (y1 * np.ldexp(np.float32(1), ks)[:, None]).astype(np.float32)
    assert np.array_equal(y2.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_tiny_activations_against_large_scales(fmt, kind):
    # Rows of very different magnitudes in one call, tiny ones included,
    # against |d| in [1024, 8192): every row must meet the relative bar on its
    # own, which rules out a scale shared across rows.
    N, K, M = 72, 1024, 5
    a = wl.activations_f32(63, M, K)
    for m, s in enumerate([1e-30, 1e-8, 1.0, 7e4, 3e29]):
        a[m] *= np.float32(s)
    blob = random_blocks(fmt, N * K // 32, 64, 25, 28)
    _full_check(fmt, kind, a, blob, N, K, "%s rows 1e-30 .. 3e29" % kind, relative_only=True)


# The binary16 floor of the two-term split that the headers state beside the
# relative bar: an activation's split is within 2^-22 of it or within FLOOR of
# its row's largest magnitude, whichever is larger. The GEMV's lo term is not
# lifted by 2^11 and Q4_0's high-nibble slots sit 2^4 below the stretch's
# largest A value; the GEMM lifts lo by 2^11 (2^-50, or 2^-46 on those slots).
SPLIT_FLOOR = {("q4_0", "gemv"): 2.0 ** -35, ("q8_0", "gemv"): 2.0 ** -39,
               ("q4_0", "gemm"): 2.0 ** -46, ("q8_0", "gemm"): 2.0 ** -46}


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("K", [1024, 992])   # streaming / split path, and the general kernels
def test_wide_span_rows_meet_the_stated_bound(fmt, kind, K):
    # Rows whose magnitudes span up to 2^60 inside one stretch of K, against
    # |d| in [1024, 8192): every output must be within 1e-5 sum|a w| + 1e-6
    # plus FLOOR * max|a[m, :]| * sum_k |w[n, k]|.
    N, M = 64, 4
    a = wl.activations_f32(71, M, K).astype(np.float64)
    e = wl.uniform_ints(72, -60, 1, (M, K))
    a[0] *= np.ldexp(1.0, e[0])                  # log-uniform over 2^-60 .. 2^0
    a[1, ::5] *= 2.0 ** -40                      # tiny elements among N(0,1) ones
    a[2] *= 2.0 ** -30
    a[2, 100] = 2.0 ** 20                        # one large element
    a[3] *= np.ldexp(1.0, e[3] + 80)             # the same span near 2^80
    a = a.astype(np.float32)
    blob = random_blocks(fmt, N * K // 32, 73, 25, 28)
    got = np.asarray(_run(fmt, kind, a, blob, N, K), dtype=np.float64)
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    w_abs = np.abs(oracle_dequant(fmt)(blob).astype(np.float64).reshape(N, K)).sum(axis=1)
    a_max = np.abs(a.astype(np.float64)).max(axis=1)
    tol = oracle.tolerance(bound) + SPLIT_FLOOR[fmt, kind] * a_max[:, None] * w_abs[None, :]
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, "%s %s K=%d: %d outputs beyond the stated bound, first %s: err %r tol %r" % (
        fmt, kind, K, len(bad), tuple(bad[0]), err[tuple(bad[0])], tol[tuple(bad[0])])


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_ffn_down_projection_sampled(fmt):
    # 512 x 4096 x 14336: the long-K GEMM (two K segments), sampled outputs.
    M, N, K = 512, 4096, 14336
    blob = weight_blob(fmt, N, K, 65)
    a = wl.activations_f32(66, M, K)
    got = _run(fmt, "gemm", a, blob, N, K)
    mi = np.concatenate([wl.uniform_ints(67, 0, M, 2048), np.arange(M), np.full(N, M - 1)])
    ni = np.concatenate([wl.uniform_ints(68, 0, N, 2048), np.full(M, N - 1), np.arange(N)])
    ref, bound = oracle_matmul_sampled(fmt)(a, blob, N, K, mi, ni)
    assert np.isfinite(got).all()
    assert_within_tolerance(got[mi, ni], ref, bound, "%s gemm %dx%dx%d" % (fmt, M, N, K))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_mixed_magnitude_rows_and_outliers(fmt, kind):
    N, K, M = 64, 1024, 6
    a = wl.activations_f32(8, M, K)
    a[1] *= np.float32(1e-4)
    a[2] *= np.float32(300.0)
    a[3, ::97] = np.float32(2000.0)               # outliers in an otherwise N(0,1) row
    a[4] = 0.0
    a[5, 5] = np.float32(1e-30)
    _full_check(fmt, kind, a, weight_blob(fmt, N, K, 9), N, K, "%s mixed rows" % kind)


def _integer_blob(fmt, codes):
    """d = 1.0 blocks holding integer codes, packed from the layout."""
    N, K = codes.shape
    nb = K // 32
    c = codes.reshape(N, nb, 32)
    if fmt == "q4_0":
        blob = np.zeros((N, nb, 18), np.uint8)
        blob[:, :, 2:] = c[:, :, :16] | (c[:, :, 16:] << 4)
    else:
        blob = np.zeros((N, nb, 34), np.uint8)
        blob[:, :, 2:] = (c & 0xFF).astype(np.uint8)
    blob[:, :, 1] = 0x3C
    return blob.reshape(-1)


@pytest.mark.parametrize("fmt", FORMATS)
def test_integer_data_is_exact(fmt):
    # d = 1 and small integer activations: every partial is an exact integer.
    N, K, M = 32, 512, 3
    lo, hi, zero = (0, 16, 8) if fmt == "q4_0" else (-128, 128, 0)
    codes = wl.uniform_ints(10, lo, hi, (N, K))
    codes[0, :] = lo                              # the extreme codes in whole rows
    codes[1, :] = hi - 1
    blob = _integer_blob(fmt, codes)
    a = wl.uniform_ints(11, -8, 9, (M, K)).astype(np.float32)
    ref = (a.astype(np.int64) @ (codes - zero).T).astype(np.float64)
    for kind in ("gemv", "gemm"):
        assert (_run(fmt, kind, a, blob, N, K) == ref).all(), kind


# ------------------------------------------------------ gates and agreement

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("kind,M", [("gemv", 3), ("gemm", 200)])
def test_repeat_is_bitwise_identical(fmt, kind, M):
    N, K = 272, 1024
    blob = weight_blob(fmt, N, K, 12)
    a = wl.activations_f32(13, M, K)
    w = to_dev(blob)
    y1 = _run(fmt, kind, a, blob, N, K, w_dev=w)
    y2 = _run(fmt, kind, a, blob, N, K, w_dev=w)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 4, 8])
def test_gemv_agrees_with_gemm(fmt, M):
    N, K = 512, 2048
    blob = weight_blob(fmt, N, K, 14)
    a = wl.activations_f32(15, M, K)
    yv = _run(fmt, "gemv", a, blob, N, K)
    ym = _run(fmt, "gemm", a, blob, N, K)
    _, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert (np.abs(yv.astype(np.float64) - ym) <= 2 * oracle.tolerance(bound)).all()


def test_q8_quantize_then_q8_gemv():
    # The device quantizer's Q8_0 blocks feed the Q8_0 product directly.
    M, N, K = 2, 300, 1024
    x = to_dev(wl.weights_f32(41, N, K))
    blob = torch.empty(N * K // 32 * 34, dtype=torch.uint8, device=DEV)
    binding.q8_quantize(x, blob)
    a = wl.activations_f32(42, M, K)
    y = torch.empty(M * N, device=DEV)
    binding.q8_gemv(to_dev(a), blob, y, M, N, K)
    torch.cuda.synchronize()
    host_blob = blob.cpu().numpy()
    assert np.array_equal(host_blob, oracle.q8_0_quantize(wl.weights_f32(41, N, K)))
    ref, bound = oracle.q8_0_matmul(a, host_blob, N, K)
    assert_within_tolerance(y.cpu().numpy().reshape(M, N), ref, bound, "quantize -> gemv")


@pytest.mark.parametrize("fmt", FORMATS)
def test_streams_are_honoured(fmt):
    N, K, M = 256, 1024, 64
    blob = weight_blob(fmt, N, K, 16)
    a = wl.activations_f32(17, M, K)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = _run(fmt, "gemm", a, blob, N, K)
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert_within_tolerance(got, ref, bound, "side stream")


@pytest.mark.parametrize("fmt", FORMATS)
def test_empty_problems_are_no_ops(fmt):
    bb = 18 if fmt == "q4_0" else 34
    for kind in ("gemv", "gemm"):
        ENTRY[fmt, kind](None, None, None, 0, 16, 64, w_bytes=16 * 2 * bb)
        ENTRY[fmt, kind](None, None, None, 3, 0, 64, w_bytes=0)


# ------------------------------------------------------- the GEMM workspace

@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_workspace_exact_size_and_garbage(fmt):
    # A workspace of exactly the *_gemm_workspace_bytes size, filled with garbage
    # and fenced by guard bytes: the result is right and nothing outside is
    # written.
    M, N, K = 130, 200, 512
    need = WS_BYTES[fmt](M, N, K)
    assert need == 768 + 256 * K * 4
    ws = Guarded(need, torch.uint8)
    ws.view.fill_(0x7F)                      # binary16 NaN patterns everywhere
    blob = weight_blob(fmt, N, K, 21)
    a = wl.activations_f32(22, M, K)
    y = Guarded(M * N, torch.float32)
    ENTRY[fmt, "gemm"](to_dev(a), to_dev(blob), y.view, M, N, K, workspace=ws.view)
    torch.cuda.synchronize()
    assert ws.guards_intact() and y.guards_intact()
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert_within_tolerance(y.host().reshape(M, N), ref, bound, "exact workspace")


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_too_small_workspace_is_rejected(fmt):
    M, N, K = 4, 16, 128
    need = WS_BYTES[fmt](M, N, K)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    y = torch.full((M * N,), 3.0, device=DEV)
    with pytest.raises(binding.Q4Error) as e:
        ENTRY[fmt, "gemm"](to_dev(wl.activations_f32(1, M, K)), to_dev(weight_blob(fmt, N, K, 2)),
                           y, M, N, K, workspace=ws)
    assert e.value.status == binding.Q4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (y == 3.0).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_graph_replays_match_eager(fmt):
    # The call allocates nothing, so it can be captured; every replay (with
    # other eager work and synchronizations in between) must equal the eager
    # result bit for bit.
    M, N, K = 96, 384, 1024
    gemm = ENTRY[fmt, "gemm"]
    blob = to_dev(weight_blob(fmt, N, K, 23))
    a = to_dev(wl.activations_f32(24, M, K))
    ws = torch.empty(WS_BYTES[fmt](M, N, K), dtype=torch.uint8, device=DEV)
    y_eager = torch.empty(M * N, device=DEV)
    gemm(a, blob, y_eager, M, N, K, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty(M * N, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gemm(a, blob, y, M, N, K, workspace=ws)   # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gemm(a, blob, y, M, N, K, workspace=ws)
    for rep in range(4):
        y.fill_(float("nan"))
        gemm(a, blob, torch.empty_like(y), M, N, K)   # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_eager.view(torch.int32)), rep
