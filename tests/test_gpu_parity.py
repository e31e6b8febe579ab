"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: packed bytes, beta, Xq, x_scale, row sums and the int32
accumulators.  fp32 Y: within 1e-5 relative of the oracle's binary64 value,
and exactly 0 where the accumulator is 0.  Every input is seeded and
synthetic (ternary_weight_linear_act_amd.workloads).
"""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import cover_rows, direct_tiles, direct_tiles_split, full_check, hip_forward, hip_pack, hip_quant, skinny_direct, to_dev

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# the five workloads at their real shapes
# ---------------------------------------------------------------------------
def test_single_1024_all_tokens():
    d = workloads.draw("single_1024")
    for M in (1, 16):
        full_check(d.W["linear"], d.X[("linear", M)], label="single_1024")


@pytest.mark.parametrize("proj", ["gate", "up", "down"])
def test_decode_ffn_2b(proj):
    d = workloads.draw("decode_ffn_2b", projs=[proj])
    full_check(d.W[proj], d.X[(proj, 1)], label="decode_ffn_2b/" + proj)


def test_prefill_2048_covering_rows():
    # every 256-row tile and every MFMA fragment row position of the full-size
    # prefill, in the kernel bench.py times
    import ternary_weight_linear_act_amd as bl
    d = workloads.draw("prefill_2048")
    full_check(d.W["up"], d.X[("up", 2048)], rows=cover_rows(2048), label="prefill_2048")
    assert bl.last_dispatch() == "gemm_dense_dma_256x256_w8_s6", bl.last_dispatch()


@pytest.mark.parametrize("nm,K,kernel", [((0, 0), 64, "gemm_dense_dma_256x256_w8_s6"),
                                         ((2, 4), 128, "gemm_nm24_smfmac_256x256"),
                                         ((6, 8), 64, "gemm_nm68_expand_dense_256x256")])
def test_prefill_2048_grid_all_rows(nm, K, kernel):
    # the exact tile grid of the 2048 x 6912 prefill (216 tiles of 256 x 256,
    # the 4 x 2 XCD regions) at small K, every output compared with the oracle
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(4100 + K, 2048, 6912, K, outlier_frac=0.001)
    full_check(W, X, nm, label="prefill-grid-all-rows")
    assert bl.last_dispatch() == kernel, bl.last_dispatch()


@pytest.mark.parametrize("proj,nm", [("dense", (0, 0)), ("nm24", (2, 4)), ("nm68", (6, 8))])
def test_sparse_ffn_1p5b(proj, nm):
    d = workloads.draw("sparse_ffn_1p5b", projs=[proj])
    full_check(d.W[proj], d.X[(proj, 1)], nm, label="sparse_ffn_1p5b/%s/M1" % proj)
    full_check(d.W[proj], d.X[(proj, 512)], nm, rows=cover_rows(512),
               label="sparse_ffn_1p5b/%s/M512" % proj)


@pytest.mark.parametrize("proj", ["q", "k", "v", "o", "gate", "up", "down"])
def test_block_3b(proj):
    d = workloads.draw("block_3b", projs=[proj])
    for M in (1, 8, 64):
        full_check(d.W[proj], d.X[(proj, M)], rows=cover_rows(M), label="block_3b/%s/M%d" % (proj, M))


# ---------------------------------------------------------------------------
# edge cases: ragged tiles, thresholds between kernels, extremes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [
    (1, 1, 64), (1, 37, 192), (2, 129, 320), (3, 200, 704), (4, 255, 1024),
    (5, 33, 128), (7, 130, 256), (17, 257, 384), (31, 64, 576), (33, 100, 640),
    (127, 129, 1088), (129, 300, 448), (200, 513, 64), (255, 31, 2048),
])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_ragged_shapes(M, N, K, nm):
    W, X = workloads.small_case(1000 + M * 7 + N, M, N, K, outlier_frac=0.01)
    full_check(W, X, nm, label="ragged")


@pytest.mark.parametrize("M,N,K", [(1000, 8000, 64), (1000, 8000, 192), (777, 9999, 320), (2048, 6912, 128),
                                   (500, 4100, 192), (512, 8960, 1536)])
def test_prefill_pipelined_gemm_edges(M, N, K):
    # the deep-pipeline dense GEMM with ragged M and N tiles and fewer K
    # slices than pipeline stages
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(77 + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, rows=cover_rows(M), label="gemm-pipeline-edge")
    assert bl.last_dispatch().startswith("gemm_dense_dma"), bl.last_dispatch()


@pytest.mark.parametrize("M,N,K,tile", [(700, 9000, 320, "128x256_w8_s4"), (1000, 8000, 2560, "128x256_w8_s4"),
                                        (256, 8960, 1536, "128x128_w4_s4"), (2048, 6912, 320, "256x256_w8_s6"),
                                        (4096, 4096, 64, "256x256_w8_s6")])
def test_dense_gemm_tile_choice(M, N, K, tile):
    # the tile-size cost model: 128 x 256 between 128 x 128 and 256 x 256
    # (ragged M and N in the first case; the six-stage 256 x 256 kernel with
    # five K slices and with one)
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1600 + M, M, N, K, outlier_frac=0.001)
    full_check(W, X, rows=cover_rows(M), label="gemm-tile-choice")
    assert bl.last_dispatch() == "gemm_dense_dma_" + tile, bl.last_dispatch()


@pytest.mark.parametrize("M", [64, 65, 255, 256, 257])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_gemm_tile_thresholds(M, nm):
    W, X = workloads.small_case(300 + M, M, 1000, 448)
    full_check(W, X, nm, rows=cover_rows(M), label="gemm-threshold")


@pytest.mark.parametrize("M,N,K,tile", [(1024, 8200, 320, "256x256"), (300, 1000, 1472, "128x128"),
                                        (40, 517, 704, "64x128")])
@pytest.mark.parametrize("nm", [(2, 4), (6, 8)])
def test_nm_gemm_tbytes(M, N, K, tile, nm):
    # (2:4 with K % 128 == 0 and at least 128 tokens runs on the sparse
    # matrix cores instead: these K leave 64 over)
    # N:M prefill: kept codes spread over their positions as 64 * t bytes by
    # byte permutes, read straight into the MFMA operand (K <= 2^18)
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1200 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, nm, rows=cover_rows(M), label="nm-gemm")
    name = bl.last_dispatch()
    if M > 64:
        # from 65 tokens the rows are expanded to dense codes for the
        # pipelined dense GEMM (these K are not multiples of 128, so 2:4 does
        # not take the sparse MFMA either)
        assert name == "gemm_nm%d%d_expand_dense_%s" % (nm[0], nm[1], expand_tile(M, N, K)), name
    elif skinny_tiles(M, N):
        assert name.startswith("skinny_mfma_nm") and name.endswith("_mt16"), name
    else:
        split = "splitk_" if tbytes_splits(M, N, K, tile) >= 2 else ""
        assert name == "gemm_nm%d%d_%s%s_tbytes" % (nm[0], nm[1], split, tile), name


@pytest.mark.parametrize("M,N,K,nm", [(2048, 6912, 2560, (6, 8)), (512, 8960, 1536, (6, 8)), (65, 777, 64, (6, 8)),
                                      (1000, 8000, 640, (6, 8)), (300, 1000, 1472, (2, 4)), (100, 4100, 192, (2, 4)),
                                      (129, 257, 11008, (6, 8)), (4096, 4096, 128, (6, 8))])
def test_nm_expand_dense_gemm(M, N, K, nm):
    # 65+ tokens with 6:8 (or 2:4 off the sparse MFMA): rows expanded to dense
    # codes in the workspace, then the pipelined dense GEMM, all three tiles,
    # ragged tiles, one K slice, deep K
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(2100 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, nm, rows=cover_rows(M), label="nm-expand-dense")
    want = "gemm_nm%d%d_expand_dense_%s" % (nm[0], nm[1], expand_tile(M, N, K))
    assert bl.last_dispatch() == want, bl.last_dispatch()


def expand_tile(M, N, K):
    t = dense_tile(M, N, K)
    return "splitk_128x128" if t.startswith("splitk") else t.split("_")[0]


@pytest.mark.parametrize("M,N,K", [(512, 2560, 6912), (129, 1000, 4096), (256, 640, 11008), (300, 2000, 512)])
def test_prefill_split_k(M, N, K):
    # past 64 tokens with fewer than 128 tiles of 128 x 128: K split over
    # workgroups, int32 partial tiles in the workspace, a second kernel adds
    # them; every covering row compared with the oracle
    import ternary_weight_linear_act_amd as bl
    assert dense_split(M, N, K) >= 2
    W, X = workloads.small_case(5100 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, rows=cover_rows(M), label="prefill-splitk")
    assert bl.last_dispatch() == "gemm_dense_splitk_128x128_w4_s4", bl.last_dispatch()
    assert bl.forward_workspace_size(M, N, K) == dense_split(M, N, K) * (-(-M // 128) * -(-N // 128)) * 65536


def dense_split(M, N, K):
    """K splits of the dense GEMM past 64 tokens: fewer than 128 tiles of
    128 x 128 and at least 8 K slices of 64 -> enough workgroups for the 256
    compute units, >= 4 slices each, partials within 32 MiB."""
    t = -(-M // 128) * -(-N // 128)
    if t >= 128 or K // 64 < 8:
        return 0
    return min(-(-256 // t), (K // 64) // 4, (32 << 20) // (t * 128 * 128 * 4))


def dense_tile(M, N, K=None):
    """Tile of the pipelined dense GEMM: rounds of tiles over the 256 compute
    units cost 4 (256 x 256), 2 (128 x 256), 1.35 (128 x 128); too few 128 x
    128 tiles split K."""
    if K is not None and dense_split(M, N, K) >= 2:
        return "splitk_128x128_w4_s4"
    rounds = lambda bm, bn: -(-(-(-M // bm) * -(-N // bn)) // 256)
    c256, c12, c128 = 4 * rounds(256, 256), 2 * rounds(128, 256), 1.35 * rounds(128, 128)
    if c256 <= c12 and c256 <= c128:
        return "256x256_w8_s6"
    return "128x256_w8_s4" if c12 <= c128 else "128x128_w4_s4"


def tbytes_splits(M, N, K, tile):
    """K splits of the N:M t-byte GEMM: enough workgroups for the 256 compute
    units, at least 4 slices of 64 each, partials within 32 MiB."""
    bm, bn = (int(v) for v in tile.split("x"))
    tiles = -(-M // bm) * -(-N // bn)
    return min(-(-256 // tiles), (K // 64) // 4, (32 << 20) // (tiles * bm * bn * 4))


@pytest.mark.parametrize("M,N,K,nm", [(32, 2560, 6912, (2, 4)), (64, 2560, 6912, (6, 8)), (16, 2560, 6912, (6, 8)),
                                      (48, 9000, 2560, (6, 8)), (17, 8300, 512, (2, 4)), (60, 3000, 1536, (2, 4)),
                                      (64, 8960, 1536, (6, 8)), (33, 2048, 11008, (6, 8))])
def test_nm_gemm_tbytes_splitk(M, N, K, nm):
    # few tokens (or few weight rows) with N:M weights: K split over enough
    # workgroups for the chip, partial 64 * t sums added by the epilogue
    # kernel; ragged M and N, 2 to 16 splits
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1800 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, nm, rows=cover_rows(M), label="nm-gemm-splitk")
    tile = "64x128"
    assert tbytes_splits(M, N, K, tile) >= 2
    assert bl.last_dispatch() == "gemm_nm%d%d_splitk_%s_tbytes" % (nm[0], nm[1], tile), bl.last_dispatch()


def nm24_sparse_tile(M, N):
    """Token tile of the 2:4 sparse-MFMA GEMM: rounds of tiles over the 256
    compute units cost 4 at 256 tokens, 2 at 128; ties take 256."""
    rounds = lambda bm: -(-(-(-M // bm) * -(-N // 256)) // 256)
    return "256x256" if 4 * rounds(256) <= 2 * rounds(128) else "128x256"


@pytest.mark.parametrize("M,N,K", [(2048, 6912, 2560), (1000, 8000, 128), (777, 9999, 256), (1025, 8000, 1536),
                                   (512, 16385, 384), (1000, 8000, 640), (300, 1000, 1536), (130, 777, 256),
                                   (3072, 6912, 2560), (2048, 2560, 6912)])
def test_nm24_sparse_mfma_gemm(M, N, K):
    # 2:4 prefill on the sparse matrix cores (K % 128 == 0, M >= 128), both
    # token tiles: ragged token and weight tiles, one and two K slices (fewer
    # than the pipeline's stages), N not a multiple of 4, prefill shapes
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1400 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, (2, 4), rows=cover_rows(M), label="nm24-smfmac")
    assert bl.last_dispatch() == "gemm_nm24_smfmac_" + nm24_sparse_tile(M, N), bl.last_dispatch()


@pytest.mark.parametrize("M", [127, 128, 129, 255, 256, 257])
def test_nm24_sparse_threshold(M):
    # below 128 tokens 2:4 takes the dense GEMM on expanded rows
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1450 + M, M, 1000, 512)
    full_check(W, X, (2, 4), rows=cover_rows(M), label="nm24-threshold")
    if M < 128:
        want = "gemm_nm24_expand_dense_" + expand_tile(M, 1000, 512)
    else:
        want = "gemm_nm24_smfmac_" + nm24_sparse_tile(M, 1000)
    assert bl.last_dispatch() == want, bl.last_dispatch()


@pytest.mark.parametrize("M,N,K", [(1024, 8192, 256), (2048, 6912, 2560)])
def test_nm24_sparse_mfma_vector_epilogue(M, N, K):
    # full tiles, N % 4 == 0 and no accumulator output: the 16-byte store path,
    # bit-identical to the element-wise one taken when acc is requested (both
    # token tiles: 128 for the first shape, 256 for the second)
    import torch

    import ternary_weight_linear_act_amd as bl
    from gpu_helpers import hip_pack, hip_quant
    W, X = workloads.small_case(1500 + M, M, N, K)
    pk, ws = hip_pack(W, (2, 4))
    Xq, xs, rs = hip_quant(X)
    Y1 = bl.forward(Xq, xs, rs, pk, ws, N, (2, 4))
    Y2, _ = bl.forward(Xq, xs, rs, pk, ws, N, (2, 4), want_acc=True)
    torch.cuda.synchronize()
    assert bl.last_dispatch() == "gemm_nm24_smfmac_" + nm24_sparse_tile(M, N)
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("nm", [(2, 4), (6, 8)])
def test_nm_gemm_past_tbytes_limit(nm):
    # K > 2^18: 64 * 127 * K could leave int32, so the superblocks are decoded
    # to dense codes instead
    import ternary_weight_linear_act_amd as bl
    M, N, K = 20, 40, (1 << 18) + 64
    W, X = workloads.small_case(1300, M, N, K)
    full_check(W, X, nm, label="nm-gemm-large-k")
    name = bl.last_dispatch()
    assert name.startswith("gemm_nm") and not name.endswith("_tbytes"), name


@pytest.mark.parametrize("M,mt,K", [(3, 4, 11008), (8, 8, 11008), (12, 16, 4096)])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_skinny_deep_k(M, mt, K, nm):
    # 2-16 tokens over deep K: token rows staged 4, 8 or 16 at a time (16 rows
    # of K = 11008 would not fit LDS)
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1400 + M, M, 300, K, outlier_frac=0.001)
    full_check(W, X, nm, label="skinny-deep-k")
    name = bl.last_dispatch()
    if nm == (2, 4) and nm24_smfmac_skinny(M, K):
        assert name == "skinny_smfmac_nm24", name
    elif skinny_direct(M, K, 300, 1, nm):
        assert name.startswith("skinny_direct_dense_") and "_mt%d_" % mt in name, name
    else:
        assert name.startswith("skinny_mfma_") and name.endswith("_mt%d" % mt), name


def nm24_smfmac_skinny(M, K):
    """2:4 at 2-16 tokens runs on the sparse MFMA for K <= 4096, or past 8
    tokens (K % 128 == 0, K <= 16384)."""
    return 2 <= M <= 16 and K % 128 == 0 and K <= 16384 and (K <= 4096 or M > 8)


@pytest.mark.parametrize("M,N,K", [(2, 1000, 640), (5, 6912, 2560), (8, 8960, 1536), (16, 2560, 6912),
                                   (16, 777, 128), (9, 3000, 8192), (12, 300, 11008), (16, 33, 16384),
                                   (3, 4095, 4096), (13, 100, 8320)])
def test_nm24_smfmac_skinny(M, N, K):
    # 2:4 at 2-16 tokens on v_smfmac_i32_16x16x128_i8: weights as the sparse
    # operand, tokens as the dense one (zero columns past M); one to 16 waves
    # of at most 4 (K <= 8192) or 8 steps of 128, uneven runs, ragged weight
    # rows, one step, the largest K
    import ternary_weight_linear_act_amd as bl
    assert nm24_smfmac_skinny(M, K)
    W, X = workloads.small_case(1900 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, (2, 4), label="nm24-smfmac-skinny")
    assert bl.last_dispatch() == "skinny_smfmac_nm24", bl.last_dispatch()


@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_gemv_fallback_very_deep_k(M, nm):
    # 1-4 tokens past the skinny kernel's K range (44 chunks x 16 waves):
    # the dot-product GEMV
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(1500 + M, M, 40, 65536, outlier_frac=0.001)
    full_check(W, X, nm, label="gemv-fallback")
    assert bl.last_dispatch().startswith("gemv_"), bl.last_dispatch()


@pytest.mark.parametrize("M,N,K", [(24, 4200, 11008), (17, 8200, 3136), (20, 4200, 3136), (33, 6000, 3200),
                                   (64, 2600, 3136), (64, 800, 11008), (40, 9000, 192), (64, 11008, 4096)])
def test_few_token_gemm(M, N, K):
    # few tokens with many weight rows (or K too deep for the skinny kernel),
    # outside the direct-load token-tile kernel's rules: K split over several
    # workgroups, partial tiles combined by a second kernel; twice in a row,
    # bit-identical
    import torch
    import ternary_weight_linear_act_amd as bl
    assert direct_tiles(M, K, N) is None and direct_tiles_split(M, K, N) is None
    W, X = workloads.small_case(900 + M + K, M, N, K, outlier_frac=0.001)
    out = full_check(W, X, rows=cover_rows(M), label="few-token")
    name = bl.last_dispatch()
    assert name.startswith("gemm_dense_splitk") or name.startswith("gemm_dense_dma"), name
    Y2, acc2 = hip_forward(out["Xq"], out["xs"], out["rs"], out["packed"], out["ws"], N, (0, 0))
    torch.cuda.synchronize()
    assert torch.equal(acc2, out["acc"])
    assert torch.equal(Y2.view(torch.int32), out["Y"].view(torch.int32))


def skinny_tiles(M, N):
    """17-64 tokens take the skinny kernel in 16-token tiles when the tiles make
    at most 512 workgroups."""
    return M <= 16 or (M <= 64 and -(-N // 16) * -(-M // 16) <= 512)


@pytest.mark.parametrize("M,N,K", [(17, 300, 2048), (33, 2040, 2048), (64, 256, 2048), (40, 1000, 192),
                                   (64, 2040, 2048), (50, 97, 4096), (32, 2048, 2048)])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_skinny_token_tiles(M, N, K, nm):
    # 17-64 tokens with few weight rows: the skinny kernel over tiles of 16
    # tokens along the grid's y (a ragged last tile, ragged weight rows)
    import ternary_weight_linear_act_amd as bl
    assert skinny_tiles(M, N) and direct_tiles(M, K, N, nm) is None
    W, X = workloads.small_case(2500 + M + K, M, N, K, outlier_frac=0.001)
    full_check(W, X, nm, rows=cover_rows(M), label="skinny-tiles")
    name = bl.last_dispatch()
    assert name.startswith("skinny_mfma_") and name.endswith("_mt16"), name


def test_zero_rows_and_zero_weights():
    W, X = workloads.small_case(5, 9, 70, 256)
    X[2] = 0.0
    X[7] = 0.0
    W[3] = 0.0
    W[10, :128] = 0.0
    full_check(W, X, label="zeros")


def test_all_zero_weight_matrix():
    W = np.zeros((64, 128), np.float32)   # beta = 0, d = 1e-5: every weight ternarises to 0
    _, X = workloads.small_case(6, 5, 64, 128)
    out = full_check(W, X, label="zero-matrix")
    assert not out["acc"].cpu().numpy().any()


def test_extreme_accumulators():
    # q = -127 (all equal) against t = -1 everywhere: acc = 127 * K at K = 11008
    K = 11008
    X = np.full((2, K), -1.0, np.float32)
    W = np.full((8, K), -0.02, np.float32)
    out = full_check(W, X, label="extreme")
    assert (out["acc"].cpu().numpy() == 127 * K).all()


def test_ties_in_ternarisation_and_masks():
    # weights on exact multiples of a power of two: many |W| ties inside N:M
    # groups and many quotients near the rounding boundaries
    rng = np.random.default_rng(77)
    W = (rng.integers(-3, 4, size=(96, 256)) * 2.0 ** -7).astype(np.float32)
    _, X = workloads.small_case(78, 6, 96, 256)
    for nm in [(0, 0), (2, 4), (6, 8)]:
        full_check(W, X, nm, label="ties")


def test_m_zero_is_noop():
    import torch
    import ternary_weight_linear_act_amd as bl
    W, _ = workloads.small_case(9, 1, 64, 128)
    packed, ws = hip_pack(W, (0, 0))
    Xq = torch.empty((0, 128), dtype=torch.int8, device="cuda")
    xs = torch.empty(0, dtype=torch.float32, device="cuda")
    rs = torch.empty(0, dtype=torch.int32, device="cuda")
    Y = bl.forward(Xq, xs, rs, packed, ws, 64)
    torch.cuda.synchronize()
    assert Y.shape == (0, 64)
    assert bl.last_dispatch() == "none"


def test_deterministic_and_dispatch():
    import torch
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(10, 300, 384, 512)
    packed, ws = hip_pack(W, (0, 0))
    for M, expect in [(1, "decode_dot4"), (4, "skinny"), (16, "skinny"), (17, "skinny"), (64, "skinny"), (65, "gemm"),
                      (300, "gemm")]:
        Xq, xs, rs = hip_quant(X[:M])
        Y1, a1 = hip_forward(Xq, xs, rs, packed, ws, 384, (0, 0))
        name = bl.last_dispatch()
        Y2, a2 = hip_forward(Xq, xs, rs, packed, ws, 384, (0, 0))
        torch.cuda.synchronize()
        assert name.startswith(expect), name
        assert torch.equal(a1, a2)
        assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))


def test_forward_without_acc_matches():
    import torch
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(11, 70, 256, 256)
    packed, ws = hip_pack(W, (0, 0))
    Xq, xs, rs = hip_quant(X)
    Y1, _ = hip_forward(Xq, xs, rs, packed, ws, 256, (0, 0))
    Y2 = bl.forward(Xq, xs, rs, packed, ws, 256, (0, 0))
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_stream_argument():
    import torch
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(12, 8, 512, 256)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        packed, ws = bl.pack_weights(to_dev(W))
        Xq, xs, rs = bl.quant_act(to_dev(X))
        Y, acc = bl.forward(Xq, xs, rs, packed, ws, 512, want_acc=True)
    s.synchronize()
    import oracle
    beta, w_eff, _ = oracle.quantize_weights(W)
    q, xs_o, _ = oracle.quant_act(X)
    acc_o, _ = oracle.forward(q, xs_o, w_eff, beta)
    assert np.array_equal(acc.cpu().numpy(), acc_o)


@pytest.mark.parametrize("nm", [(2, 4), (6, 8)])
@pytest.mark.parametrize("N,K,Ms", [(8960, 1536, (1, 8, 512)), (6912, 2560, (1, 64)), (37, 192, (1, 5, 70))])
def test_pack_masked_dense_layout(nm, N, K, Ms):
    # N:M weights stored in the dense layout (pruned positions t = 0): the
    # packed bytes are the oracle's dense packing of W_eff, and the dense
    # forward on them gives the oracle's accumulators and those of the N:M
    # format, bit for bit
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    W, _ = workloads.small_case(5300 + N + K, 1, N, K)
    print("case masked dense layout N=%d K=%d nm=%s" % (N, K, nm), flush=True)
    pk, ws = bl.pack_weights_masked(to_dev(W), nm)
    pk_nm, ws_nm = hip_pack(W, nm)
    torch.cuda.synchronize()
    beta, w_eff, _ = oracle.quantize_weights(W, *nm)
    assert np.array_equal(pk.cpu().numpy(), oracle.pack_dense(w_eff))
    assert ws.cpu().numpy().view(np.uint32)[0] == np.float32(beta).view(np.uint32)
    for M in Ms:
        _, X = workloads.small_case(5400 + M, M, 8, K, outlier_frac=0.001)
        Xq, xs, rs = hip_quant(X)
        Y, acc = hip_forward(Xq, xs, rs, pk, ws, N, (0, 0))
        Y2, acc2 = hip_forward(Xq, xs, rs, pk_nm, ws_nm, N, nm)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc2), "dense layout and N:M format differ (M=%d)" % M
        rows = cover_rows(M)
        q, xs_o, _ = oracle.quant_act(X[rows])
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy()[rows], acc_o)


@pytest.mark.parametrize("n,m", [(1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (7, 8), (8, 8), (1, 4), (3, 4),
                                 (4, 16), (12, 16)])
def test_nm_sweep_dense_layout(n, m):
    # the N:8 sweep (and other N:M) on the dense layout: packed bytes equal the
    # oracle's dense packing of its masked ternary weights; one token and 512
    # tokens through the dense kernels, accumulators bit-exact
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    N, K = 8960, 1536
    W, _ = workloads.small_case(5500 + 10 * n + m, 1, N, K)
    print("case N:M sweep %d:%d" % (n, m), flush=True)
    pk, ws = bl.pack_weights_masked(to_dev(W), (n, m))
    torch.cuda.synchronize()
    beta = oracle.absmean(W)
    w_eff = oracle.apply_mask(oracle.ternarize(W, beta), oracle.nm_keep(W, n, m))
    assert np.array_equal(pk.cpu().numpy(), oracle.pack_dense(w_eff))
    assert ws.cpu().numpy().view(np.uint32)[0] == np.float32(beta).view(np.uint32)
    for M in (1, 512):
        _, X = workloads.small_case(5600 + M, M, 8, K, outlier_frac=0.001)
        Xq, xs, rs = hip_quant(X)
        Y, acc = hip_forward(Xq, xs, rs, pk, ws, N, (0, 0))
        torch.cuda.synchronize()
        rows = cover_rows(M)
        q, xs_o, _ = oracle.quant_act(X[rows])
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy()[rows], acc_o)
