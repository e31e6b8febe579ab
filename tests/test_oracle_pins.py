"""Pins of the CPU oracle against things other than itself.

Each test fixes the oracle to a closed form, a hand-worked value, a brute-force
search, a value printed on the pages (tests/golden/) or an invariant that the
mathematics forces, so that a plausible slip in the oracle -- a dropped abs, a
wrong divisor, a transposed operand, a wrong rounding rule, a wrong tie-break
or a misplaced bit -- fails at least one of them.

Sources:
* "BitNet 논문 분석: 1-Bit LLM의 시대" (youngju.dev), sections "Absmean 양자화
  함수" (absmean ternary weights, absmax int8 activations, integer linear and
  rescale) and "bitnet.cpp 추론 프레임워크" / "I2_S 커널의 내부 동작" (2-bit
  code, TL2 pair lookup);
* "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2 and sec. 5.1;
* "Sparse-BitNet: ..." (review), sec. 3.2 (top-N |latent| per block of M,
  quant-then-mask).
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ternary_weight_linear_act_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def f32(x):
    return F32(x)


def ulp32(x):
    x = abs(F32(x))
    return float(np.nextafter(x, F32(np.inf)) - x)


# --------------------------------------------------------------------------
# independent reader of the packed layout (written from the format's text:
# code j of a 16-code word at bit 8*(j%4) + 2*(j/4), little-endian words)
# --------------------------------------------------------------------------
def read_codes(buf, ncodes):
    out = []
    for c in range(ncodes):
        word = c // 16
        j = c % 16
        w = int(buf[4 * word]) | int(buf[4 * word + 1]) << 8 | int(buf[4 * word + 2]) << 16 | int(buf[4 * word + 3]) << 24
        out.append((w >> (8 * (j % 4) + 2 * (j // 4))) & 3)
    return out


def decode_dense(buf, N, K):
    rows = []
    for r in range(N):
        codes = read_codes(buf[r * K // 4:(r + 1) * K // 4], K)
        rows.append([c - 1 for c in codes])
    return np.array(rows, dtype=np.int8)


def decode_nm(buf, N, K, n, m):
    vrow = K * n // m // 4
    mrow = K // 8
    masks = buf[N * vrow:]
    out = np.zeros((N, K), np.int8)
    for r in range(N):
        codes = read_codes(buf[r * vrow:(r + 1) * vrow], K * n // m)
        ci = 0
        for g in range(K // m):
            if m == 4:
                mask = (int(masks[r * mrow + g // 2]) >> (4 * (g % 2))) & 0xF
            else:
                mask = int(masks[r * mrow + g])
            assert bin(mask).count("1") == n
            for i in range(m):
                if mask >> i & 1:
                    out[r, g * m + i] = codes[ci] - 1
                    ci += 1
    return out


# ==========================================================================
# absmean (beta)
# ==========================================================================
class TestAbsmean:
    def test_constant(self):
        W = np.full((4, 64), 0.25, np.float32)
        assert oracle.absmean(W) == F32(0.25)

    def test_signs_are_dropped(self):
        W = np.full((4, 64), 0.5, np.float32)
        W[:, ::2] *= -1
        W[1::2] *= -1
        assert oracle.absmean(W) == F32(0.5)

    def test_divides_by_all_elements(self):
        # row n holds (n+1)/8, mean over N=8 rows = (1+...+8)/64 = 36/64
        N, K = 8, 128
        W = np.repeat((np.arange(1, N + 1, dtype=np.float32) / 8)[:, None], K, axis=1)
        W[:, 1::3] *= -1
        assert oracle.absmean(W) == F32(36 / 64)
        # a wrong divisor (N or K alone) or a missing abs would not give 0.5625

    def test_matches_exact_mean(self):
        rng = np.random.default_rng(11)
        for shape in [(3, 64), (17, 128), (64, 1024)]:
            W = (rng.standard_normal(shape) * 0.02).astype(np.float32)
            exact = sum((Fraction(float(abs(v))) for v in W.ravel()), Fraction(0)) / W.size
            beta = oracle.absmean(W)
            assert abs(Fraction(float(beta)) - exact) <= Fraction(ulp32(beta)) * Fraction(1, 2) * Fraction(1000001, 1000000)

    def test_gaussian_absmean(self):
        # E|w| = sigma * sqrt(2/pi) for w ~ N(0, sigma^2)
        W = workloads.normal_f32(np.random.default_rng(0), (1024, 1024), 0.02)
        assert abs(float(oracle.absmean(W)) / (0.02 * math.sqrt(2 / math.pi)) - 1) < 0.005

    def test_rejects_nonfinite(self):
        W = np.ones((2, 64), np.float32)
        W[1, 3] = np.nan
        with pytest.raises(ValueError):
            oracle.absmean(W)


# ==========================================================================
# ternarisation  t = clamp(round(W / (beta + 1e-5)), -1, 1)
# ==========================================================================
def beta_giving_unit_d():
    """A float32 beta with fl32(beta + 1e-5f) == 1 exactly."""
    b = F32(1) - F32(1e-5)
    for _ in range(64):
        d = F32(b + F32(1e-5))
        if d == F32(1):
            return b
        b = np.nextafter(b, F32(0) if d > 1 else F32(2))
    raise AssertionError("no beta found")


class TestTernarize:
    def test_ties_and_clamp_with_unit_d(self):
        beta = beta_giving_unit_d()
        W = np.array([0.0, 0.5, -0.5, np.nextafter(F32(0.5), F32(0)), np.nextafter(F32(0.5), F32(1)),
                      1.0, 1.5, -1.5, 2.5, -7.0, 1e-30, np.nextafter(F32(-0.5), F32(-1)), 0.75, -0.25],
                     dtype=np.float32)
        want = [0, 0, 0, 0, 1, 1, 1, -1, 1, -1, 0, -1, 1, 0]
        assert oracle.ternarize(W, beta).tolist() == want

    def test_eps_is_added_to_beta(self):
        # with beta = 0, d = 1e-5: W = 4e-6 -> 0.4 -> 0 ; W = 6e-6 -> 0.6 -> 1
        W = np.array([4e-6, 6e-6, -6e-6], np.float32)
        assert oracle.ternarize(W, 0.0).tolist() == [0, 1, -1]

    def test_gaussian_zero_fraction(self):
        # t = 0 iff |W| < d/2 with d ~= sigma*sqrt(2/pi): P = erf(sqrt(1/pi)/sqrt(2)*...) ;
        # P(|Z| < 0.5*sqrt(2/pi)) = erf(0.5*sqrt(2/pi)/sqrt(2)) = erf(0.5/sqrt(pi))
        W = workloads.normal_f32(np.random.default_rng(0), (1024, 1024), 0.02)
        t = oracle.ternarize(W, oracle.absmean(W))
        p0 = math.erf(0.5 / math.sqrt(math.pi))
        frac0 = float(np.mean(t == 0))
        assert abs(frac0 - p0) < 0.003
        assert abs(float(np.mean(t == 1)) - float(np.mean(t == -1))) < 0.005
        assert set(np.unique(t).tolist()) == {-1, 0, 1}

    def test_matches_definition_elementwise(self):
        # round-half-even on fp32 quotients, recomputed with numpy's fp32 ops
        rng = np.random.default_rng(5)
        W = (rng.standard_normal(4096) * 0.02).astype(np.float32)
        beta = F32(0.016)
        d = F32(beta + F32(1e-5))
        want = np.clip(np.rint(W / d), -1, 1).astype(np.int8)
        assert np.array_equal(oracle.ternarize(W, beta), want)


# ==========================================================================
# N:M keep mask
# ==========================================================================
def brute_keep(w, n):
    """The unique n-subset whose every member outranks every non-member.

    Rank key of position i: (|w_i|, -i): larger magnitude first, then lower i.
    """
    m = len(w)
    key = lambda i: (abs(float(w[i])), -i)
    found = []
    for S in itertools.combinations(range(m), n):
        rest = [i for i in range(m) if i not in S]
        if not rest or min(key(i) for i in S) > max(key(i) for i in rest):
            found.append(S)
    assert len(found) == 1
    return found[0]


class TestNM:
    @pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (1, 4), (3, 8), (7, 8), (2, 8), (5, 8), (1, 8), (4, 8),
                                     (4, 16), (12, 16)])
    def test_brute_force_with_ties(self, n, m):
        rng = np.random.default_rng(100 + 10 * n + m)
        # magnitudes from a small set -> many ties
        W = rng.choice(np.array([0.0, 0.01, -0.01, 0.02, -0.02, 0.03], np.float32), size=(6, 8 * m))
        keep = oracle.nm_keep(W, n, m)
        for r in range(W.shape[0]):
            for g in range(W.shape[1] // m):
                S = brute_keep(W[r, g * m:(g + 1) * m], n)
                got = tuple(np.nonzero(keep[r, g * m:(g + 1) * m])[0].tolist())
                assert got == S

    def test_hand_examples(self):
        W = np.array([[0.1, -0.3, 0.3, 0.2, 0.2, 0.2, 0.2, 0.2]], np.float32)
        assert oracle.nm_keep(W, 2, 4).tolist() == [[0, 1, 1, 0, 1, 1, 0, 0]]
        W = (np.arange(1, 9, dtype=np.float32) / 10)[None, :]
        assert oracle.nm_keep(W, 6, 8).tolist() == [[0, 0, 1, 1, 1, 1, 1, 1]]
        W = np.zeros((1, 8), np.float32)
        assert oracle.nm_keep(W, 6, 8).tolist() == [[1, 1, 1, 1, 1, 1, 0, 0]]

    def test_dense_limit(self):
        # n = m keeps everything: the N:M forward reduces to the dense one
        W = workloads.normal_f32(np.random.default_rng(1), (4, 64), 0.02)
        assert oracle.nm_keep(W, 8, 8).all()
        assert oracle.nm_keep(W, 4, 4).all()

    @pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
    def test_invariants_random(self, n, m):
        W = workloads.normal_f32(np.random.default_rng(2), (64, 256), 0.02)
        keep = oracle.nm_keep(W, n, m).reshape(64, -1, m).astype(bool)
        mag = np.abs(W).reshape(64, -1, m)
        assert (keep.sum(-1) == n).all()
        kept_min = np.where(keep, mag, np.inf).min(-1)
        pruned_max = np.where(~keep, mag, -np.inf).max(-1)
        assert (kept_min >= pruned_max).all()

    def test_ranked_by_latent_not_ternary(self):
        # 0.9 and 0.6 both ternarise to +1 (d = 1): the mask must still prefer 0.9
        beta = beta_giving_unit_d()
        W = np.array([[0.6, 0.9, 0.1, 0.0]], np.float32)
        t = oracle.ternarize(W, beta)
        assert t.tolist() == [[1, 1, 0, 0]]
        assert oracle.nm_keep(W, 1, 4).tolist() == [[0, 1, 0, 0]]


# ==========================================================================
# packed layout
# ==========================================================================
def load_code_map():
    cmap = {}
    with open(os.path.join(GOLDEN, "i2s_code_map.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            a, b = line.split()
            if a == "words":
                cmap["words"] = int(b)
            else:
                cmap[int(a)] = int(b, 2)
    return cmap


def word(buf, i):
    return int.from_bytes(bytes(buf[4 * i:4 * i + 4]), "little")


class TestPack:
    def test_code_map_from_pages(self):
        cmap = load_code_map()
        assert cmap["words"] == 16
        for v in (-1, 0, 1):
            buf = oracle.pack_dense(np.full((1, 64), v, np.int8))
            for i in range(4):
                w = word(buf, i)
                fields = [(w >> (2 * f)) & 3 for f in range(16)]
                assert fields == [cmap[v]] * 16
        assert word(oracle.pack_dense(np.full((1, 64), 1, np.int8)), 0) == 0xAAAAAAAA
        assert word(oracle.pack_dense(np.full((1, 64), 0, np.int8)), 0) == 0x55555555
        assert word(oracle.pack_dense(np.full((1, 64), -1, np.int8)), 0) == 0x00000000

    @pytest.mark.parametrize("j,val,want", [
        (0, 1, 0x55555556), (1, 1, 0x55555655), (3, 1, 0x56555555), (4, 1, 0x55555559),
        (15, 1, 0x95555555), (0, -1, 0x55555554), (5, -1, 0x55555155), (10, -1, 0x55455555),
    ])
    def test_bit_positions(self, j, val, want):
        # a single nonzero at k = 16 + j (second word); code j sits at bit 8*(j%4) + 2*(j/4)
        t = np.zeros((1, 64), np.int8)
        t[0, 16 + j] = val
        buf = oracle.pack_dense(t)
        assert word(buf, 0) == 0x55555555 and word(buf, 2) == 0x55555555
        assert word(buf, 1) == want

    def test_round_trip_and_no_code_3(self):
        rng = np.random.default_rng(3)
        t = rng.integers(-1, 2, size=(5, 192)).astype(np.int8)
        buf = oracle.pack_dense(t)
        assert buf.size == 5 * 192 // 4
        assert np.array_equal(decode_dense(buf, 5, 192), t)
        b = buf.astype(np.uint32)
        for s in range(0, 8, 2):
            assert not np.any(((b >> s) & 3) == 3)

    def test_sizes(self):
        assert oracle.packed_bytes(6912, 2560) == 4423680
        assert oracle.packed_bytes(8960, 1536, 2, 4) == 3440640
        assert oracle.packed_bytes(8960, 1536, 6, 8) == 4300800
        assert oracle.packed_bytes(10, 96) == -1       # K % 64 != 0
        assert oracle.packed_bytes(10, 128, 3, 4) == -1

    def test_nm_hand_example_2_4(self):
        # K = 64, one row: group g keeps positions (g % 4, (g % 4 + 1) % 4 ... ) chosen by magnitude
        K = 64
        W = np.zeros((1, K), np.float32)
        t = np.zeros((1, K), np.int8)
        # groups: keep positions {1,2} with values (+1, -1) in every group
        for g in range(K // 4):
            W[0, 4 * g + 1] = 0.5
            W[0, 4 * g + 2] = -0.4
            t[0, 4 * g + 1] = 1
            t[0, 4 * g + 2] = -1
        keep = oracle.nm_keep(W, 2, 4)
        buf = oracle.pack_nm(t, keep, 2, 4)
        assert buf.size == K // 8 + K // 8
        # values: 32 kept codes alternating (+1 -> 2, -1 -> 0): codes j even = 2, j odd = 0
        # word fields: code j at bit 8*(j%4) + 2*(j/4) -> bytes 0 and 2 hold 2 in every field
        for wi in range(2):
            assert word(buf, wi) == 0x00AA00AA
        # masks: nibble 0b0110 for every group -> bytes 0x66
        assert buf[K // 8:].tolist() == [0x66] * (K // 8)

    @pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
    def test_nm_decodes_to_masked_dense(self, n, m):
        W = workloads.normal_f32(np.random.default_rng(4), (3, 128), 0.02)
        beta, w_eff, buf = oracle.quantize_weights(W, n, m)
        assert buf.size == oracle.packed_bytes(3, 128, n, m)
        assert np.array_equal(decode_nm(buf, 3, 128, n, m), w_eff)
        t = oracle.ternarize(W, beta)
        keep = oracle.nm_keep(W, n, m).astype(bool)
        assert np.array_equal(w_eff, np.where(keep, t, 0))


# ==========================================================================
# activation quantisation
# ==========================================================================
class TestQuantAct:
    def test_hand_examples(self):
        X = np.array([[1.0, -0.5, 0.25, 0.0]], np.float32)
        q, xs, rs = oracle.quant_act(X)
        assert q.tolist() == [[127, -64, 32, 0]]          # -63.5 -> -64 (half to even), 31.75 -> 32
        assert xs[0] == F32(1) / F32(127) and rs[0] == 95
        q, _, _ = oracle.quant_act(np.array([[2.0, 1.0, -1.0, 0.0]], np.float32))
        assert q.tolist() == [[127, 64, -64, 0]]          # 63.5 -> 64
        q, xs, _ = oracle.quant_act(np.array([[-4.0, 1.0, 0.5, 0.0]], np.float32))
        assert q.tolist() == [[-127, 32, 16, 0]]          # s = 31.75
        assert xs[0] == F32(4) / F32(127)
        q, _, _ = oracle.quant_act(np.array([[254.0, 1.0, 3.0, -1.0]], np.float32))
        assert q.tolist() == [[127, 0, 2, 0]]            # s = 0.5: 0.5 -> 0, 1.5 -> 2, -0.5 -> 0

    def test_scale_computed_once(self):
        # g = 7.5: s = fl32(127/7.5) = 8877943 * 2^-19 = 16.933332443...;
        # 3.75 * s = 63.4999966... -> fl32 = 16646143 * 2^-18 = 63.499996... -> 63.
        # (Multiplying by 127 first and dividing by g would give exactly 63.5 -> 64.)
        q, _, _ = oracle.quant_act(np.array([[7.5, 3.75, -3.75, 0.0]], np.float32))
        assert q.tolist() == [[127, 63, -63, 0]]

    def test_zero_row(self):
        q, xs, rs = oracle.quant_act(np.zeros((2, 64), np.float32))
        assert not q.any() and not xs.any() and not rs.any()

    def test_argmax_maps_to_127_and_never_minus_128(self):
        X = workloads.activations(np.random.default_rng(6), 2000, 2560, 0.001)
        q, xs, rs = oracle.quant_act(X)
        am = np.argmax(np.abs(X), axis=1)
        assert np.array_equal(np.abs(q[np.arange(2000), am].astype(int)), np.full(2000, 127))
        assert q.min() >= -127
        assert np.array_equal(rs, q.astype(np.int64).sum(1))
        assert np.array_equal(xs, (np.abs(X).max(1) / F32(127)).astype(np.float32))

    def test_monotone(self):
        x = np.sort(np.random.default_rng(7).standard_normal(512)).astype(np.float32)[None, :]
        q, _, _ = oracle.quant_act(x)
        assert np.all(np.diff(q[0].astype(int)) >= 0)

    def test_power_of_two_invariance(self):
        X = workloads.activations(np.random.default_rng(8), 16, 256)
        q0, xs0, _ = oracle.quant_act(X)
        for e in (-3, 1, 5):
            q1, xs1, _ = oracle.quant_act((X * F32(2.0 ** e)).astype(np.float32))
            assert np.array_equal(q0, q1)
            assert np.array_equal(xs1, (xs0 * F32(2.0 ** e)).astype(np.float32))

    def test_tiny_row_hand_example(self):
        # g = 2^-125: fl32(127/g) would be 127 * 2^125 > FLT_MAX (+inf), so x*s
        # would be +-inf and 0*s NaN.  The row is taken at 2^100 times its
        # size (exact), where s = 127 * 2^25: 2^-127 / 2^-125 * 127 = 31.75 -> 32.
        X = np.array([[2.0 ** -125, -(2.0 ** -125), 0.0, 2.0 ** -127]], np.float32)
        q, xs, rs = oracle.quant_act(X)
        assert q.tolist() == [[127, -127, 0, 32]]
        assert rs[0] == 32
        assert xs[0] == np.float32(F32(2.0 ** -125) / F32(127))

    def test_power_of_two_invariance_down_to_overflow(self):
        # entries of magnitude in [1, 2) (and zeros) stay normal down to 2^-125,
        # so the scaling is exact; below g = 2^-121.3 the unscaled s overflows
        rng = np.random.default_rng(9)
        X = (rng.uniform(1.0, 2.0, (8, 256)) * rng.choice([-1.0, 1.0], (8, 256))).astype(np.float32)
        X[:, ::17] = 0.0
        q0, _, rs0 = oracle.quant_act(X)
        for e in (-90, -101, -110, -122, -125):
            q1, _, rs1 = oracle.quant_act((X * F32(2.0 ** e)).astype(np.float32))
            assert np.array_equal(q0, q1), e
            assert np.array_equal(rs0, rs1), e

    def test_listing_variant_differs(self):
        # the 128/(g+1e-5) form printed in the listing can reach -128; 127/g cannot
        X = np.array([[-1.0, 0.5]], np.float32)
        assert oracle.quant_act(X, variant=1)[0].tolist() == [[-128, 64]]
        assert oracle.quant_act(X, variant=0)[0].tolist() == [[-127, 64]]


# ==========================================================================
# transformed activation rows: ReLU^2 gate and RMSNorm before the quantiser
# ("BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2: squared ReLU in the
# feed-forward network, subln; "BitNet 논문 분석: 1-Bit LLM의 시대", section
# "Absmean 양자화 함수": BitLinear_b158 applies an RMSNorm over the inputs
# before activation_quant)
# ==========================================================================
def torch_rms_reference(X, up, gamma, eps):
    """xhat in binary64 from torch's own RMSNorm; the gated row h is formed
    by torch in binary32 (relu, square, times up)."""
    import torch
    h = torch.from_numpy(X)
    if up is not None:
        h = torch.relu(h) ** 2 * torch.from_numpy(up)
    ref = torch.nn.functional.rms_norm(h.double(), (X.shape[1],), weight=torch.from_numpy(gamma).double(),
                                       eps=float(eps))
    return h.numpy(), ref.numpy()


class TestActTransform:
    def test_gate_hand_examples(self):
        g = np.zeros((2, 64), np.float32)
        u = np.ones((2, 64), np.float32)
        g[0, :4], u[0, :4] = [-1.0, 0.0, 0.5, 2.0], [3.0, 5.0, -2.0, 0.25]
        g[1, :4], u[1, :4] = [-3.0, 1.5, -0.5, 1.0], [-1.0, 2.0, 4.0, -1.0]
        q, xs, rs = oracle.quant_act_ex(g, u)
        # row 0: h = [0, 0, 0.25 * -2, 4 * 0.25] = [0, 0, -0.5, 1]: s = 127, -63.5 -> -64
        assert q[0, :4].tolist() == [0, 0, -64, 127] and xs[0] == F32(1) / F32(127) and rs[0] == 63
        # row 1: h = [0 (not 9 * -1), 2.25 * 2, 0, -1] = [0, 4.5, 0, -1]: s = 127 / 4.5
        assert q[1, :4].tolist() == [0, 127, 0, -28] and xs[1] == F32(4.5) / F32(127)
        assert not q[:, 4:].any()

    def test_rms_closed_forms(self):
        # x = c * (+1, -1, ...): mean(x^2) = c^2, every code is +-127 and
        # x_scale = c / 127 / sqrt(c^2 + eps)
        K = 256
        alt = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
        one = np.ones(K, np.float32)
        q, xs, rs = oracle.quant_act_ex((2.0 * alt)[None, :].astype(np.float32), gamma=one, eps=0.0)
        assert np.array_equal(np.abs(q[0]), np.full(K, 127)) and rs[0] == 0
        assert xs[0] == F32(1.0 / 127.0)                    # 2 / 127 / 2
        q, xs, _ = oracle.quant_act_ex((1.5 * alt)[None, :].astype(np.float32), gamma=one, eps=0.75)
        assert xs[0] == F32(math.sqrt(3.0) / 254.0)        # 1.5 / 127 / sqrt(3)
        # gamma = 2 on even k, 1 on odd k: codes 127 and -64 (63.5 to even);
        # mean(x^2) is taken before gamma: x_scale = 2 * 1.5 / 127 / sqrt(3)
        gam = np.where(np.arange(K) % 2 == 0, 2.0, 1.0).astype(np.float32)
        q, xs, _ = oracle.quant_act_ex((1.5 * alt)[None, :].astype(np.float32), gamma=gam, eps=0.75)
        assert q[0, :2].tolist() == [127, -64]
        assert xs[0] == F32(math.sqrt(3.0) / 127.0)

    def test_unit_gamma_keeps_the_plain_codes(self):
        # the per-row factor 1/rms divides out of the absmax codes
        X = workloads.activations(np.random.default_rng(31), 12, 512, 0.01)
        q0, _, rs0 = oracle.quant_act(X)
        for eps in (0.0, 1e-5, 3.0):
            q1, _, rs1 = oracle.quant_act_ex(X, gamma=np.ones(512, np.float32), eps=eps)
            assert np.array_equal(q0, q1) and np.array_equal(rs0, rs1)

    @pytest.mark.parametrize("gated", [False, True])
    @pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-5, 0.5])
    def test_matches_torch_rms_norm(self, gated, eps):
        rng = np.random.default_rng(32 + int(gated))
        M, K = 24, 384
        X = workloads.activations(rng, M, K, 0.01)
        X[::3] *= F32(3e-3)                                 # rows where eps matters
        up = workloads.activations(rng, M, K) if gated else None
        gamma = rng.uniform(0.25, 1.75, K).astype(np.float32)
        q, xs, rs = oracle.quant_act_ex(X, up, gamma, eps)
        h, ref = torch_rms_reference(X, up, gamma, eps)
        # codes: exactly the plain quantiser's codes of fl32(h * gamma)
        qp, _, rsp = oracle.quant_act((h * gamma).astype(np.float32))
        assert np.array_equal(q, qp) and np.array_equal(rs, rsp)
        # scale: the largest |xhat| maps to 127
        gmax = np.abs(ref).max(1)
        assert np.all(np.abs(xs.astype(np.float64) * 127.0 - gmax) <= 1e-6 * gmax)
        # every dequantised value within half a step of torch's xhat
        err = np.abs(q * xs.astype(np.float64)[:, None] - ref)
        assert np.all(err <= xs.astype(np.float64)[:, None] * (0.5 + 1e-5) + 1e-6 * np.abs(ref))

    def test_listing_order_codes(self):
        # The listing's literal order: RMSNorm in fp32 first (torch's
        # rms_norm), then the absmax quantiser on the normalised row.  The
        # oracle takes the codes from fl32(h * gamma) (1/rms divides out).
        # The two differ only where a value lands on a rounding boundary:
        # measured 7 of 5,767,168 entries (K = 2560, 6912, 2048, 11008; 256
        # rows each), all by one code.
        import torch
        rng = np.random.default_rng(35)
        diff = total = 0
        for K in (2560, 6912):
            M = 256
            X = workloads.activations(rng, M, K, 0.001)
            gamma = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
            q, _, _ = oracle.quant_act_ex(X, None, gamma, 1e-5)
            xn = torch.nn.functional.rms_norm(torch.from_numpy(X), (K,), torch.from_numpy(gamma), 1e-5).numpy()
            g = np.abs(xn).max(1, keepdims=True)
            s = (np.float32(127.0) / g).astype(np.float32)
            ql = np.rint((xn * s).astype(np.float32)).astype(np.int64)
            d = q.astype(np.int64) != ql
            assert np.all(np.abs(q.astype(np.int64) - ql) <= 1)
            # each disagreement is a rounding-boundary case: the exact value
            # of v * 127 / max|v|, v = h * gamma, is within 1e-4 of a half
            v = X.astype(np.float64) * gamma.astype(np.float64)
            exact = v * 127.0 / np.abs(v).max(1, keepdims=True)
            frac = np.abs(exact[d]) - np.floor(np.abs(exact[d]))
            assert np.all(np.abs(frac - 0.5) <= 1e-4), frac
            diff += int(d.sum())
            total += d.size
        assert diff <= 1e-5 * total, (diff, total)

    def test_zero_rows(self):
        X = np.zeros((2, 128), np.float32)
        for eps in (0.0, 1e-5):
            q, xs, rs = oracle.quant_act_ex(X, X, np.ones(128, np.float32), eps)
            assert not q.any() and not rs.any() and not xs.any()
        # a gate that is never positive makes the row zero too
        g = -np.abs(workloads.activations(np.random.default_rng(33), 2, 128))
        q, xs, _ = oracle.quant_act_ex(g, np.ones_like(g), np.ones(128, np.float32), 1e-5)
        assert not q.any() and not xs.any()

    def test_identity_transform(self):
        X = workloads.activations(np.random.default_rng(34), 6, 256, 0.01)
        a, b = oracle.quant_act(X), oracle.quant_act_ex(X)
        assert all(np.array_equal(u, v) for u, v in zip(a, b))


# ==========================================================================
# 4-bit activations after an online Hadamard transform (the BitNet v2
# summary: the H-BitLinear transforms the activations, then quantises them to
# 4 bits)
# ==========================================================================
def block_hadamard_f64(X, B):
    """(H_B / sqrt(B)) applied blockwise, in binary64, from scipy's matrix."""
    import scipy.linalg
    H = scipy.linalg.hadamard(B).astype(np.float64) / math.sqrt(B)
    M, K = X.shape
    return (X.astype(np.float64).reshape(M, K // B, B) @ H.T).reshape(M, K)


class TestHadamard4:
    @pytest.mark.parametrize("B", [1, 2, 8, 256])
    def test_transform_equals_sylvester_matrix(self, B):
        # small integers: every butterfly is exact, so the result must equal
        # scipy's Hadamard matrix times each block exactly
        import scipy.linalg
        rng = np.random.default_rng(40 + B)
        K = 4 * B if B > 1 else 8
        X = rng.integers(-50, 50, (3, K)).astype(np.float32)
        H = scipy.linalg.hadamard(B)
        want = (X.reshape(3, K // B, B) @ H.T).reshape(3, K)
        assert np.array_equal(oracle.hadamard_rows(X, B), want.astype(np.float32))

    def test_involution_and_blocks(self):
        rng = np.random.default_rng(41)
        X = rng.integers(-9, 9, (2, 512)).astype(np.float32)
        # H H = B I (exact on small integers)
        assert np.array_equal(oracle.hadamard_rows(oracle.hadamard_rows(X, 128), 128), X * 128)
        # a change in one block leaves the others' transform alone
        Y = X.copy()
        Y[:, 130] += 5
        d = oracle.hadamard_rows(Y, 128) != oracle.hadamard_rows(X, 128)
        assert d[:, 128:256].all() and not d[:, :128].any() and not d[:, 256:].any()

    @pytest.mark.parametrize("B", [64, 256])
    def test_one_hot_rows(self, B):
        # e_j -> column j of H_B: every code +-7 with H's signs; scale 1/(7 sqrt(B))
        import scipy.linalg
        H = scipy.linalg.hadamard(B)
        X = np.zeros((3, B), np.float32)
        for r, j in enumerate((0, 5, B - 1)):
            X[r, j] = 2.5
        q, xs, rs = oracle.quant_act_h4(X, B)
        for r, j in enumerate((0, 5, B - 1)):
            assert np.array_equal(q[r], 7 * H[:, j])
        assert np.all(xs == F32(2.5 / 7.0 / math.sqrt(B)))
        assert np.array_equal(rs, q.astype(np.int64).sum(1))

    @pytest.mark.parametrize("K,B", [(2560, 512), (6912, 256), (1024, 1024), (192, 64)])
    def test_matches_orthonormal_transform(self, K, B):
        # against the binary64 product with scipy's matrix: the largest value
        # maps to 7 and every dequantised value is within half a step, up to the
        # binary32 butterflies' error (log2(B) roundings of partial sums bounded
        # by the block's sum of |x|)
        rng = np.random.default_rng(42 + K)
        X = workloads.activations(rng, 12, K, 0.01)
        X[5] *= F32(2.0 ** -110)                          # tiny row (prescaled)
        q, xs, rs = oracle.quant_act_h4(X, B)
        ref = block_hadamard_f64(X, B)
        l1 = np.abs(X.astype(np.float64)).reshape(12, K // B, B).sum(2)
        fp_err = (math.log2(B) + 1) * 2.0 ** -24 * np.repeat(l1, B, axis=1) / math.sqrt(B)
        xs64 = xs.astype(np.float64)[:, None]
        assert np.all(np.abs(q * xs64 - ref) <= xs64 * (0.5 + 1e-5) + fp_err)
        gmax = np.abs(ref).max(1)
        assert np.all(np.abs(7.0 * xs.astype(np.float64) - gmax) <= 1e-6 * gmax + fp_err.max(1))
        assert q.min() >= -7 and q.max() <= 7
        assert np.array_equal(rs, q.astype(np.int64).sum(1))

    def test_tiny_row_hand_example(self):
        # a one-hot row of 2^-126: every transformed value is +-2^-126, where
        # fl32(7 / g) would overflow (7 * 2^126 > FLT_MAX) -- the row is taken
        # at 2^100 times its size and the codes are 7 times H's column
        import scipy.linalg
        B = 64
        X = np.zeros((1, B), np.float32)
        X[0, 9] = np.float32(2.0 ** -126)
        q, xs, _ = oracle.quant_act_h4(X, B)
        assert np.array_equal(q[0], 7 * scipy.linalg.hadamard(B)[:, 9])
        assert xs[0] == np.float32(2.0 ** -126 / 7.0 / 8.0)

    def test_power_of_two_invariance_and_zero_rows(self):
        X = workloads.activations(np.random.default_rng(43), 6, 512)
        X[2] = 0.0
        q0, xs0, _ = oracle.quant_act_h4(X, 256)
        assert not q0[2].any() and xs0[2] == 0.0
        for e in (-7, 3):
            q1, xs1, _ = oracle.quant_act_h4((X * F32(2.0 ** e)).astype(np.float32), 256)
            assert np.array_equal(q0, q1)
            assert np.array_equal(xs1, (xs0 * F32(2.0 ** e)).astype(np.float32))


# ==========================================================================
# contraction and epilogue
# ==========================================================================
class TestForward:
    def test_exhaustive_ternary_rows(self):
        K = 8
        rows = np.array(list(itertools.product((-1, 0, 1), repeat=K)), np.int8)   # 3^8 rows
        rng = np.random.default_rng(9)
        q = rng.integers(-128, 128, size=(3, K)).astype(np.int8)
        acc, _ = oracle.forward(q, np.ones(3, np.float32), rows, 1.0)
        for m in range(3):
            for n in range(0, rows.shape[0], 97):
                assert acc[m, n] == sum(int(q[m, k]) * int(rows[n, k]) for k in range(K))
        # permutation symmetry: each column sums to 0 because +1 and -1 rows pair up
        assert not acc.sum(1).any()

    def test_closed_forms(self):
        K = 256
        q = np.random.default_rng(10).integers(-128, 128, size=(2, K)).astype(np.int8)
        W = np.zeros((4, K), np.int8)
        W[0] = 1
        W[1] = -1
        W[2, 37] = 1               # one-hot: selects q[:, 37]
        W[3, 200] = -1
        acc, _ = oracle.forward(q, np.ones(2, np.float32), W, 1.0)
        rs = q.astype(np.int64).sum(1)
        assert acc[:, 0].tolist() == rs.tolist()
        assert acc[:, 1].tolist() == (-rs).tolist()
        assert acc[:, 2].tolist() == q[:, 37].astype(int).tolist()
        assert acc[:, 3].tolist() == (-q[:, 200].astype(int)).tolist()

    def test_transposition_is_caught(self):
        # rows of W_eff are outputs: W[n] one-hot at k = n + 1
        K, N = 64, 8
        W = np.zeros((N, K), np.int8)
        for n in range(N):
            W[n, n + 1] = 1
        q = np.arange(K, dtype=np.int8)[None, :]
        acc, _ = oracle.forward(q, np.ones(1, np.float32), W, 1.0)
        assert acc[0].tolist() == list(range(1, N + 1))

    def test_extremes(self):
        K = 11008
        q = np.full((1, K), -128, np.int8)
        W = np.full((1, K), -1, np.int8)
        acc, Y = oracle.forward(q, np.ones(1, np.float32), W, 1.0)
        assert acc[0, 0] == 1409024 == 128 * K

    def test_epilogue_closed_form(self):
        q = np.array([[1, 2, 3, 4] * 16], np.int8)
        W = np.ones((1, 64), np.int8)
        acc, Y = oracle.forward(q, np.array([0.5], np.float32), W, 0.25)
        assert acc[0, 0] == 160
        assert Y[0, 0] == 160 * 0.125

    def test_tl2_pair_lookup_identity(self):
        # TL2 description: pairs (w0, w1) index a 9-entry table of a0*w0 + a1*w1
        with open(os.path.join(GOLDEN, "tl2_demo_weights.txt")) as f:
            fields = {l.split()[0]: l.split()[1:] for l in f if l.strip() and not l.startswith("#")}
        w = np.array([int(v) for v in fields["weights"]], np.int8)
        acts = np.random.RandomState(int(fields["seed"][0])).randn(len(w)).astype(np.float32)
        # the page's pair indices: (w0 + 1) * 3 + (w1 + 1)
        idx = [(w[i] + 1) * 3 + (w[i + 1] + 1) for i in range(0, len(w), 2)]
        assert idx == [2, 5, 1, 6]
        # integer version of the lookup on the oracle's int8 activations
        q, _, _ = oracle.quant_act(np.tile(acts, 8)[None, :])    # K = 64
        wrow = np.tile(w, 8)[None, :]
        acc, _ = oracle.forward(q, np.ones(1, np.float32), wrow, 1.0)
        total = 0
        qa = q[0].astype(int)
        for i in range(0, 64, 2):
            a0, a1 = qa[i], qa[i + 1]
            lut = [-(a0 + a1), -a0, -a0 + a1, -a1, 0, a1, a0 - a1, a0, a0 + a1]
            total += lut[(wrow[0, i] + 1) * 3 + (wrow[0, i + 1] + 1)]
        assert acc[0, 0] == total

    def test_end_to_end_tracks_float_linear(self):
        W, X = workloads.small_case(12, 16, 64, 1024)
        beta, w_eff, _ = oracle.quantize_weights(W)
        q, xs, _ = oracle.quant_act(X)
        _, Y = oracle.forward(q, xs, w_eff, beta)
        ref = X.astype(np.float64) @ W.astype(np.float64).T
        c = np.corrcoef(Y.ravel(), ref.ravel())[0, 1]
        assert c > 0.85
        # and the dequantised product equals the float product of the quantised operands
        deq = (q.astype(np.float64) * xs[:, None].astype(np.float64)) @ (w_eff.astype(np.float64) * float(beta)).T
        assert np.allclose(Y, deq, rtol=1e-12, atol=0)


# ==========================================================================
# BitNet a4.8's hybrid activations ("BitNet 논문 분석", section "BitNet a4.8:
# 하이브리드 양자화 전략": the top values of the activation tensor are
# separated and kept at 8 bits, the rest quantised to 4 bits, each part with
# its own scale).  T outliers per token row, given by the caller.
# ==========================================================================
class TestA48:
    def test_hand_example(self):
        # x = [0.1, -3, 0.5, 2, -0.25, 0.75, 3, 1].  T = 2: |-3| and |3| tie,
        # the lower k (1) is taken first, then k = 6.  hi: g = 3, codes
        # rne(+-3 * fl32(127/3)) = +-127.  lo: g = 2, s = 3.5, codes of
        # [0.35, 0, 1.75, 7, -0.875, 2.625, 0, 3.5] = [0, 0, 2, 7, -1, 3, 0, 4]
        # (2.625 -> 3 and 3.5 -> 4: half to even), x_scale 2/7.
        x = np.array([[0.1, -3.0, 0.5, 2.0, -0.25, 0.75, 3.0, 1.0]], np.float32)
        q, xs, rs, sel = oracle.quant_act_a48(x, 2)
        assert q[0].tolist() == [0, -127, 0, 0, 0, 0, 127, 0]
        assert q[1].tolist() == [0, 0, 2, 7, -1, 3, 0, 4]
        assert sel[0].tolist() == [0, 1, 0, 0, 0, 0, 1, 0]
        assert xs[0] == F32(3.0) / F32(127.0) and xs[1] == F32(2.0) / F32(7.0)
        assert rs.tolist() == [0, 15]
        # T = 1: only k = 1 (the tie goes to the lower k); lo's max is then 3
        # (k = 6): s = fl32(7/3), codes of [0.233, 0, 1.167, 4.667, -0.583,
        # 1.75, 7, 2.333] = [0, 0, 1, 5, -1, 2, 7, 2]
        q, xs, rs, sel = oracle.quant_act_a48(x, 1)
        assert sel[0].tolist() == [0, 1, 0, 0, 0, 0, 0, 0]
        assert q[0].tolist() == [0, -127, 0, 0, 0, 0, 0, 0]
        assert q[1].tolist() == [0, 0, 1, 5, -1, 2, 7, 2]
        assert xs[1] == F32(3.0) / F32(7.0)

    def test_selection_brute_force(self):
        # rows of few distinct magnitudes (many ties), every T: the outliers
        # are the first T indices ordered by (-|x|, k)
        rng = np.random.default_rng(41)
        for K in (1, 2, 5, 8, 13):
            X = (rng.integers(-3, 4, size=(40, K)) * 0.5).astype(np.float32)
            for T in range(K + 1):
                _, _, _, sel = oracle.quant_act_a48(X, T)
                for m in range(X.shape[0]):
                    order = sorted(range(K), key=lambda k: (-abs(float(X[m, k])), k))
                    want = np.zeros(K, np.uint8)
                    want[order[:T]] = 1
                    assert np.array_equal(sel[m], want), (K, T, X[m], sel[m])

    def test_no_outliers_is_the_4bit_quantiser(self):
        # T = 0: the hi rows are zero with scale 0; the lo rows are the 4-bit
        # absmax codes, which the H-BitLinear quantiser with blocks of 1 (an
        # identity transform) computes independently
        X = workloads.activations(np.random.default_rng(42), 16, 320, 0.01)
        q, xs, rs, _ = oracle.quant_act_a48(X, 0)
        assert not q[0::2].any() and not xs[0::2].any() and not rs[0::2].any()
        q4, xs4, rs4 = oracle.quant_act_h4(X, 1)
        assert np.array_equal(q[1::2], q4) and np.array_equal(rs[1::2], rs4)
        assert np.array_equal(xs[1::2].view(np.uint32), xs4.view(np.uint32))
        assert q[1::2].min() >= -7 and q[1::2].max() <= 7

    def test_all_outliers_is_the_8bit_quantiser(self):
        X = workloads.activations(np.random.default_rng(43), 9, 192, 0.01)
        q, xs, rs, sel = oracle.quant_act_a48(X, 192)
        q8, xs8, rs8 = oracle.quant_act(X)
        assert sel.all()
        assert np.array_equal(q[0::2], q8) and np.array_equal(rs[0::2], rs8)
        assert np.array_equal(xs[0::2].view(np.uint32), xs8.view(np.uint32))
        assert not q[1::2].any() and not xs[1::2].any()

    @pytest.mark.parametrize("T", [1, 3, 26, 100])
    def test_split_and_reconstruction(self, T):
        X = workloads.activations(np.random.default_rng(44 + T), 32, 2560, 0.001)
        q, xs, rs, sel = oracle.quant_act_a48(X, T)
        a = np.abs(X.astype(np.float64))
        s = sel.astype(bool)
        assert np.all(s.sum(1) == T)
        # every outlier at least as large as every other value of its row
        assert np.all(np.where(s, a, np.inf).min(1) >= np.where(s, -np.inf, a).max(1))
        qh, ql = q[0::2].astype(np.float64), q[1::2].astype(np.float64)
        assert not qh[~s].any() and not ql[s].any()
        assert np.abs(qh).max() == 127 and np.abs(ql).max(1).min() == 7
        # each value within half a step of its part's dequantised code
        sh, sl = xs[0::2].astype(np.float64)[:, None], xs[1::2].astype(np.float64)[:, None]
        rec = qh * sh + ql * sl
        step = np.where(s, sh, sl)
        assert np.all(np.abs(rec - X) <= step * (0.5 + 1e-5))
        assert np.array_equal(rs[0::2], q[0::2].sum(1, dtype=np.int64))
        assert np.array_equal(rs[1::2], q[1::2].sum(1, dtype=np.int64))

    def test_zero_and_tiny_rows(self):
        X = np.zeros((2, 64), np.float32)
        X[1, 5] = 2.0 ** -126
        X[1, 9] = -(2.0 ** -127)
        q, xs, rs, _ = oracle.quant_act_a48(X, 1)
        assert not q[0:2].any() and not xs[0:2].any()
        # row 1: the outlier is k = 5; the rest has max 2^-127 at k = 9 and
        # quantises to -7 (the 2^100 pre-scale keeps 7/g finite)
        assert q[2, 5] == 127 and q[3, 9] == -7 and q[3, 5] == 0
        assert xs[3] == F32(2.0 ** -127) / F32(7.0)

    def test_forward_pairs(self):
        # through an identity weight matrix (t = I), output k of token m is
        # beta * (x_hi q_hi + x_lo q_lo)[k]: the pairing of rows 2m, 2m+1
        X = workloads.activations(np.random.default_rng(45), 6, 64, 0.01)
        q, xs, _, sel = oracle.quant_act_a48(X, 5)
        w_eff = np.eye(64, dtype=np.int8)
        acc, Y, Yp = oracle.forward_a48(q, xs, w_eff, 0.5)
        want = 0.5 * (q[0::2] * xs[0::2].astype(np.float64)[:, None] + q[1::2] * xs[1::2].astype(np.float64)[:, None])
        assert np.allclose(Y, want, rtol=1e-15, atol=0)
        assert np.array_equal(acc, q.astype(np.int32))
        assert np.all(np.abs(Y - 0.5 * X) <= 0.5 * np.where(sel.astype(bool), xs[0::2][:, None], xs[1::2][:, None]) * 0.5 * (1 + 1e-5))


# ---------------------------------------------------------------------------
# 2:4 trit pack: the 2:4 weights as one 6-bit code per group of 4 (the kept
# pair of inputs and their two ternary values; TL2's 3 x 3 value index,
# "I2_S 커널의 내부 동작", times the 6 pairs a 2:4 group can keep), 16 codes
# in 12 bytes.

TRIT_PAIRS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


def _trit_example():
    # a hand-worked row of 64 inputs: groups 0, 5, 10 and 15 as listed, the
    # others keep (0, 1) with values (0, 0); pruned positions hold nonzero t
    # (the mask drops them)
    special = {0: ((1, 3), (1, -1)), 5: ((2, 3), (-1, 1)), 10: ((0, 2), (1, 1)), 15: ((0, 3), (-1, 0))}
    t = np.ones((1, 64), np.int8)
    keep = np.zeros((1, 64), np.uint8)
    for g in range(16):
        (i0, i1), (v0, v1) = special.get(g, ((0, 1), (0, 0)))
        keep[0, 4 * g + i0] = keep[0, 4 * g + i1] = 1
        t[0, 4 * g + i0], t[0, 4 * g + i1] = v0, v1
    return t, keep


def test_trit24_hand_example():
    # codes: group 0 keeps (1, 3) = pair 4 with (+1, -1): 36 + 6 + 0 = 42;
    # group 5 (2, 3) = pair 5 with (-1, +1): 45 + 0 + 2 = 47; group 10 (0, 2)
    # = pair 1 with (+1, +1): 9 + 6 + 2 = 17; group 15 (0, 3) = pair 2 with
    # (-1, 0): 18 + 0 + 1 = 19; the rest (0, 1) = pair 0 with (0, 0): 4.
    # Bits 6g..6g+5 of a little-endian 96-bit string, worked by hand: byte 0
    # = 42 = 0x2a; byte 1 = code 1's bits 2-5 (0b0001) + code 2's bits 0-3
    # (0b0100) << 4 = 0x41; byte 3 = code 4 (4) + code 5's low two bits
    # (0b11) << 6 = 0xc4, code 5 straddling bytes 3 and 4; byte 4 = code 5's
    # bits 2-5 (0b1011) + code 6's bits 0-3 << 4 = 0x4b.
    t, keep = _trit_example()
    got = oracle.pack_trit24(t, keep)
    assert got.tobytes().hex() == "2a4110c44b1004111104414c"
    assert oracle.packed_bytes_trit24(1, 64) == 12


def test_trit24_all_codes_brute_force():
    # every pair and value combination of one group, alone in a row of 64
    # (the other groups keep (0, 1) with values (0, 0), code 4): the code at
    # bits 0-5 is 9 p + 3 (v0 + 1) + (v1 + 1), the 54 codes are distinct and
    # below 64, and the bytes decode back to the masked ternary row
    seen = set()
    for p, (i0, i1) in enumerate(TRIT_PAIRS):
        for v0, v1 in itertools.product((-1, 0, 1), repeat=2):
            t = np.zeros((1, 64), np.int8)
            keep = np.zeros((1, 64), np.uint8)
            keep[0, 0::4] = keep[0, 1::4] = 1
            keep[0, 0:4] = 0
            keep[0, i0] = keep[0, i1] = 1
            t[0, i0], t[0, i1] = v0, v1
            b = oracle.pack_trit24(t, keep)
            code = int(b[0]) & 63
            assert code == 9 * p + 3 * (v0 + 1) + (v1 + 1)
            seen.add(code)
            w = oracle.unpack_trit24(b, 1, 64)
            assert np.array_equal(w, t * keep.astype(np.int8))
    assert seen == set(range(54))


def test_trit24_round_trip_against_the_2_4_path():
    # quant-then-mask through the trit bytes gives the 2:4 path's W_eff and
    # beta, at 3/4 of the dense bytes (1.5 bits per weight)
    for seed, (N, K) in enumerate([(3, 64), (17, 192), (64, 1536)]):
        W, _ = workloads.small_case(7000 + seed, 1, N, K)
        beta, w_eff, packed = oracle.quantize_weights_trit24(W)
        beta2, w_eff2, _ = oracle.quantize_weights(W, 2, 4)
        assert beta == beta2
        assert np.array_equal(w_eff, w_eff2)
        assert packed.size == 3 * N * K // 16 == 3 * oracle.packed_bytes(N, K) // 4
        assert np.array_equal(oracle.unpack_trit24(packed, N, K), w_eff)
        # exactly two kept per group, as the format assumes
        assert np.all((w_eff.reshape(N, K // 4, 4) != 0).sum(axis=2) <= 2)


def test_trit24_rejects_groups_not_2_of_4():
    t = np.zeros((1, 64), np.int8)
    keep = np.zeros((1, 64), np.uint8)
    keep[0, 0::2] = 1                       # 2 per group: fine
    oracle.pack_trit24(t, keep)
    keep[0, 1] = 1                          # 3 in group 0
    with pytest.raises(Exception):
        oracle.pack_trit24(t, keep)
    keep = np.zeros((1, 64), np.uint8)
    keep[0, 0::4] = 1                       # 1 per group
    with pytest.raises(Exception):
        oracle.pack_trit24(t, keep)
