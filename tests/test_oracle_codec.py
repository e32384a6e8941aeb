"""Pins of the oracle's tile quantiser, record layout and dequantiser.

Each test checks the oracle against something other than itself: a closed form worked by hand,
an invariant the normalisation must satisfy, a special case that reduces to a textbook
quantiser, the rounding bounds the grid construction guarantees, or an exact round trip."""

import numpy as np
import pytest

from oracle import codec, formats, hadamard
from workloads import gen

T, D = 128, 128


def _tile(seed, outliers=True, drift=False):
    rng = np.random.default_rng(seed)
    mult = np.exp(rng.standard_normal(D))
    if outliers:
        mult[rng.choice(D, 3, replace=False)] *= 15
    x = rng.standard_normal((T, D)) * mult
    if drift:
        x *= np.exp(0.5 * rng.standard_normal((T, 1)))
    return x.astype(np.float16).astype(np.float64)


# ------------------------------------------------------------------ closed-form worked example


def _permuted_hadamard_tile(seed):
    """Row t = sign_t * 2^e_t * (row kappa(t) of the +-1 Sylvester matrix): fp16-exact input
    whose rotation has exactly one nonzero per row and per column."""
    rng = np.random.default_rng(seed)
    kappa = rng.permutation(T)
    sign = np.where(rng.random(T) < 0.5, -1.0, 1.0)
    half = rng.integers(-5, 6, T // 2)
    e = rng.permutation(np.concatenate([half, -half]))   # exponents sum to zero
    pm1 = hadamard.H128 * np.sqrt(128.0)
    x = (sign * 2.0 ** e)[:, None] * pm1[kappa]
    return x, kappa, sign, e


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_closed_form_one_nonzero_per_row(seed):
    # Rotated tile: xt[t, kappa(t)] = sign_t * sqrt(128) * 2^e_t, zero elsewhere.
    # Column std over tokens of a vector with one nonzero a is |a| sqrt(127) / 128; the row step
    # then sees one nonzero of magnitude 128 / sqrt(127) per row, whose std is exactly 1, so
    # the row scales stay 1 and every round gives the same column scales. After the gauge
    # (mean log c = 0, and sum e = 0): c_j = 2^e_t for the token t with kappa(t) = j, which
    # E4M3 holds exactly. Each token of xt / c_hat is then one entry sign*sqrt(128) and zeros.
    #   sign +1: z = 0, step = sqrt(128)/(2^b - 1); s = E4M3 round-up of it
    #            K: 11.3137/15 = 0.7542 -> 0.8125; V: 11.3137/3 = 3.7712 -> 4.0
    #            codes: sqrt(128) -> rint(13.92) = 14 (K), rint(2.83) = 3 (V); zeros -> 0
    #   sign -1: z = FP16 round-down of -sqrt(128) = -1449/128 = -11.3203125
    #            K step 11.3203125/15 -> 0.8125; V 11.3203125/3 -> 4.0
    #            codes: -sqrt(128) -> 0; zeros -> 14 (K), 3 (V)
    x, kappa, sign, e = _permuted_hadamard_tile(seed)
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
    for bits, s_exp, top in ((4, 0.8125, 14), (2, 4.0, 3)):
        q = codec.quantize_tile(x, bits)
        c_exp = np.empty(D)
        c_exp[kappa] = 2.0 ** e
        assert np.array_equal(q["c_hat"], c_exp)
        assert np.array_equal(q["s_hat"], np.full(T, s_exp))
        assert np.array_equal(q["z_hat"], np.where(sign > 0, 0.0, -1449.0 / 128.0))
        codes_exp = np.where(sign[:, None] > 0, 0, top) * np.ones((T, D), int)
        codes_exp[np.arange(T), kappa] = np.where(sign > 0, top, 0)
        assert np.array_equal(q["codes"], codes_exp)


def floor_tile():
    """A tile on which both standard-deviation floors (reading R8) decide the column scales.

    Token 2k (k < 64) is m_k * (row 2k - row 2k+1 of the +-1 Sylvester matrix) with m_k = 2^-6
    for k < 32 and 2^-4 for k >= 32; every odd token is zero. fp16-exact."""
    pm1 = hadamard.H128 * np.sqrt(128.0)
    x = np.zeros((T, D))
    for k in range(64):
        x[2 * k] = (2.0 ** -6 if k < 32 else 2.0 ** -4) * (pm1[2 * k] - pm1[2 * k + 1])
    return x


def test_closed_form_floor_tile():
    # Worked by hand (s = sqrt(128), kappa = sqrt(127/128); a column or row with one nonzero w
    # among 128 entries has standard deviation |w| kappa / s; two entries +-w have w sqrt(2)/s).
    # Rotated: token 2k holds +m_k s at channel 2k and -m_k s at channel 2k+1, nothing else;
    # max |rotated| = 2^-4 s.
    # Round 1 columns (u = 1): channel of token k: std m_k kappa; floor 2^-16 * 2^-4 s * 1 is
    #   far below. Rows: token rows see +-s / kappa -> std sqrt(2) / kappa; zero rows sit at the
    #   row floor 2^-16 * 2^-4 s * max(v), max(v) = 1 / (2^-6 kappa), so their multiplier
    #   u0 = 2^-6 kappa / (2^-16 * 2^-4 s) is the largest of all multipliers.
    # Later column steps: the column floor is 2^-16 * 2^-4 s * u0 = 2^-6 kappa, while a small
    #   channel's std is 2^-6 kappa^2 / sqrt(2) below it: every small channel (64 of them) sits
    #   at the floor 2^-6 kappa from round 2 on. A large channel's row multiplier shrinks by
    #   kappa / sqrt(2) per round: in units of 2^-6 its std is 4 kappa^2 / sqrt(2), 2 kappa^3
    #   and sqrt(2) kappa^4 in rounds 2 to 4.
    # Round 4 (the last column step) and the gauge (geometric mean of c = 1):
    #   small channels c = kappa / (2^(1/4) kappa^(5/2)) = 2^(-1/4) kappa^(-3/2) = 0.845857...
    #   large channels c = 2^(1/4) kappa^(3/2) = 1.182232...
    #   E4M3 nearest: 0.845857 -> 0.875 (midpoint 0.84375); 1.182232 -> 1.125 (midpoint 1.1875).
    # Rounding per token (y = rotated / c-hat; zero rows give z = 0, s = 0, codes 0):
    #   small rows: y = +-s / 56 = +-0.2020305; z = FP16 round-down = -1656 * 2^-13;
    #     K: (0.2020305 + 0.2021484) / 15 -> E4M3 round-up 14 * 2^-9; codes 15 (+), 0 (-), 7
    #     V: (...) / 3 -> 9 * 2^-6; codes 3 (+), 0 (-), 1
    #   large rows: y = +-s / 18 = +-0.6285394; z = -1288 * 2^-11;
    #     K: (0.6285394 + 0.6289063) / 15 -> 11 * 2^-7; codes 15, 0, 7
    #     V: (...) / 3 -> 14 * 2^-5; codes 3, 0, 1 (0.62890625 / 0.4375 = 1.4375 -> 1)
    # A floor twice as large, half as large, or without its multiplier factor, in either step,
    # moves every c-hat off these values.
    x = floor_tile()
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
    kappa = np.sqrt(127.0 / 128.0)
    small = np.arange(D) < 64
    c_pre = np.where(small, 2 ** -0.25 * kappa ** -1.5, 2 ** 0.25 * kappa ** 1.5)
    live = np.arange(T) % 2 == 0
    big_row = np.arange(T) >= 64
    for bits, s_small, s_big, mid in ((4, 14 * 2.0 ** -9, 11 * 2.0 ** -7, 7),
                                      (2, 9 * 2.0 ** -6, 14 * 2.0 ** -5, 1)):
        top = 2 ** bits - 1
        q = codec.quantize_tile(x, bits)
        assert np.allclose(q["c"], c_pre, rtol=1e-12, atol=0)
        assert np.array_equal(q["c_hat"], np.where(small, 0.875, 1.125))
        assert np.array_equal(q["z_hat"], np.where(~live, 0.0,
                                                   np.where(big_row, -1288 * 2.0 ** -11,
                                                            -1656 * 2.0 ** -13)))
        assert np.array_equal(q["s_hat"], np.where(~live, 0.0, np.where(big_row, s_big, s_small)))
        codes = np.where(live[:, None], mid, 0) * np.ones((T, D), int)
        for t in np.flatnonzero(live):
            codes[t, t] = top              # +m s at channel 2k = t
            codes[t, t + 1] = 0            # -m s at channel 2k + 1
        assert np.array_equal(q["codes"], codes)


# ------------------------------------------------------------------ normalisation invariants


@pytest.mark.parametrize("iters", [1, 2, 4, 6])
def test_final_row_step_gives_unit_row_std(iters):
    xt = hadamard.rotate(_tile(3, drift=True))
    _, lc, lr = codec.normalise(xt, iters)
    z = xt * np.exp(-lr)[:, None] * np.exp(-lc)[None, :]
    assert np.allclose(z.std(axis=1), 1.0, rtol=0, atol=1e-12)


def test_column_step_gives_unit_column_std():
    xt = hadamard.rotate(_tile(4, drift=True))
    _, lc_prev, lr_prev = codec.normalise(xt, 3)
    _, lc, _ = codec.normalise(xt, 4)
    z = xt * np.exp(-lr_prev)[:, None] * np.exp(-lc)[None, :]
    assert np.allclose(z.std(axis=0), 1.0, rtol=0, atol=1e-12)


def test_alternation_converges_up_to_the_gauge():
    # With centred standard deviations the pair (row, column) scales can drift together along
    # the gauge direction from round to round; the gauged column scales converge, and the
    # column standard deviations after a full round become equal to each other.
    xt = hadamard.rotate(_tile(4, drift=True))
    spreads, steps = [], []
    prev = codec.normalise(xt, 1)[0]
    for iters in (2, 4, 8, 16):
        lcg, lc, lr = codec.normalise(xt, iters)
        z = xt * np.exp(-lr)[:, None] * np.exp(-lc)[None, :]
        cs = z.std(axis=0)
        spreads.append(cs.max() / cs.min() - 1)
        steps.append(np.abs(lcg - prev).max())
        prev = lcg
    assert all(b <= a for a, b in zip(spreads, spreads[1:])) and spreads[-1] < 1e-8
    assert all(b <= a for a, b in zip(steps, steps[1:])) and steps[-1] < 1e-8


def test_gauge_mean_log_zero_and_ddof_invariance():
    xt = hadamard.rotate(_tile(5))
    lc0, _, _ = codec.normalise(xt, 4, ddof=0)
    lc1, _, _ = codec.normalise(xt, 4, ddof=1)
    assert abs(lc0.mean()) < 1e-14
    assert np.allclose(lc0, lc1, rtol=0, atol=1e-13)


@pytest.mark.parametrize("k", [-3, 2, 4])
def test_power_of_two_scaling_covariance(k):
    x = _tile(6, drift=True)
    for bits in (4, 2):
        a = codec.quantize_tile(x, bits)
        b = codec.quantize_tile(x * 2.0 ** k, bits)
        assert np.array_equal(a["c_hat"], b["c_hat"])
        assert np.array_equal(a["s_hat"] * 2.0 ** k, b["s_hat"])
        assert np.array_equal(a["z_hat"] * 2.0 ** k, b["z_hat"])
        assert np.array_equal(a["codes"], b["codes"])


def test_token_permutation_equivariance():
    x = _tile(7)
    perm = np.random.default_rng(0).permutation(T)
    for bits in (4, 2):
        a = codec.quantize_tile(x, bits)
        b = codec.quantize_tile(x[perm], bits)
        assert np.array_equal(a["c_hat"], b["c_hat"])
        assert np.array_equal(a["s_hat"][perm], b["s_hat"])
        assert np.array_equal(a["z_hat"][perm], b["z_hat"])
        assert np.array_equal(a["codes"][perm], b["codes"])


def test_normalisation_equalises_column_spread():
    # Outlier channels: after rotation and normalisation the column stds of xt / c are closer
    # to each other than those of the raw tile ([GR] "The four-stage pipeline", stage 2).
    x = _tile(8)
    q = codec.quantize_tile(x, 4)
    spread = lambda m: np.std(np.log(m.std(axis=0)))
    assert spread(q["xt"] / q["c"][None, :]) < 0.5 * spread(x)


# ------------------------------------------------------------------ RTN stage


@pytest.mark.parametrize("seed", [9, 10, 11])
def test_rtn_bounds(seed):
    x = _tile(seed, drift=True)
    for bits in (4, 2):
        q = codec.quantize_tile(x, bits)
        qmax = 2 ** bits - 1
        codes, s, z, y = q["codes"], q["s_hat"], q["z_hat"], q["y"]
        assert codes.min() >= 0 and codes.max() <= qmax
        deq = s[:, None] * codes + z[:, None]
        assert np.all(np.abs(y - deq) <= s[:, None] / 2 * (1 + 1e-12))
        assert np.all(z <= y.min(axis=1)) and np.all(z + qmax * s >= y.max(axis=1))
        assert np.all(codes[np.arange(T), y.argmin(axis=1)] == 0)
        assert np.all(codes[np.arange(T), y.argmax(axis=1)] >= (qmax if bits == 2 else 13))
        # s-hat is the smallest E4M3 value whose grid covers the token's range
        prev = formats.E4M3_DECODE[q["s_code"].astype(int) - 1]
        assert np.all(z + qmax * prev < y.max(axis=1))


def test_zero_iterations_is_textbook_per_token_minmax():
    x = _tile(12)
    xt = hadamard.rotate(x)
    for bits in (4, 2):
        q = codec.quantize_tile(x, bits, iters=0)
        qmax = 2 ** bits - 1
        assert np.all(q["c_hat"] == 1.0)
        mn, mx = xt.min(axis=1), xt.max(axis=1)
        expect_z = np.array([np.float16(m) if np.float16(m) <= m else
                             np.nextafter(np.float16(m), np.float16(-np.inf)) for m in mn], float)
        assert np.array_equal(q["z_hat"], expect_z)
        assert np.all(q["s_hat"] * qmax >= mx - expect_z)
        expect_codes = np.clip(np.rint((xt - expect_z[:, None]) / q["s_hat"][:, None]), 0, qmax)
        assert np.array_equal(q["codes"], expect_codes)


def test_bypass_round_trip_is_exact():
    # Skipping the rounding of stage 3 (dequantising the unrounded y) must give back x.
    x = _tile(13, drift=True)
    q = codec.quantize_tile(x, 4)
    back = (q["c_hat"][None, :] * q["y"]) @ hadamard.H128
    assert np.abs(back - x).max() <= 1e-13 * np.abs(x).max()


def test_dequant_error_small_relative_to_fp16():
    x = _tile(14)
    k = codec.quantize_tile(x, 4)
    khat = codec.dequantize(k["c_hat"], k["s_hat"], k["z_hat"], k["codes"])
    assert np.linalg.norm(khat - x) / np.linalg.norm(x) < 0.12
    # the rotated, normalised error is exactly the RTN error scaled by c-hat
    err_rot = k["c_hat"][None, :] * (k["s_hat"][:, None] * k["codes"] + k["z_hat"][:, None]
                                     - k["y"])
    assert np.allclose(khat - x, err_rot @ hadamard.H128, atol=1e-10)


# ------------------------------------------------------------------ degenerate tiles


def test_all_zero_tile():
    q = codec.quantize_tile(np.zeros((T, D)), 4)
    assert np.all(q["c_hat"] == 1) and np.all(q["s_hat"] == 0) and np.all(q["z_hat"] == 0)
    assert np.all(q["codes"] == 0)
    assert np.all(q["c_code"] == 0x38)


def test_identical_tokens_tile_uses_floor_and_reconstructs():
    row = _tile(15)[0]
    x = np.repeat(row[None, :], T, axis=0)
    for bits in (4, 2):
        q = codec.quantize_tile(x, bits)
        assert np.all(np.isfinite(q["c_hat"])) and np.all(q["c_hat"] > 0)
        xh = codec.dequantize(q["c_hat"], q["s_hat"], q["z_hat"], q["codes"])
        assert np.all(np.abs(q["y"] - (q["s_hat"][:, None] * q["codes"] + q["z_hat"][:, None]))
                      <= q["s_hat"][:, None] / 2 * (1 + 1e-12))
        assert np.all(np.isfinite(xh))


def test_single_nonzero_element():
    x = np.zeros((T, D))
    x[5, 9] = 3.0
    q = codec.quantize_tile(x, 4)
    xh = codec.dequantize(q["c_hat"], q["s_hat"], q["z_hat"], q["codes"])
    assert np.abs(xh - x).max() < 0.5


# ------------------------------------------------------------------ record layout


def test_record_round_trip_and_size():
    kq = codec.quantize_tile(_tile(16), 4)
    vq = codec.quantize_tile(_tile(17), 2)
    rec = codec.pack_record(kq, vq)
    assert rec.shape == (13312,)
    u = codec.unpack_record(rec)
    for name, q in (("k", kq), ("v", vq)):
        assert np.array_equal(u[name]["codes"], q["codes"])
        assert np.array_equal(u[name]["c_hat"], q["c_hat"])
        assert np.array_equal(u[name]["s_hat"], q["s_hat"])
        assert np.array_equal(u[name]["z_hat"], q["z_hat"])


def test_value_layout_is_a_bijection_onto_the_section():
    tt, jj = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
    byte, shift = codec.v_code_position(tt, jj)
    bitaddr = (8 * byte + shift).ravel()
    assert np.all(shift % 2 == 0)
    assert len(np.unique(bitaddr)) == T * D and bitaddr.min() == 0 and bitaddr.max() == 32766


def test_layout_hand_positions():
    # key codes: token 3, channel 5 -> byte 3*64 + 2, high nibble
    kq = dict(codes=np.zeros((T, D), int), c_code=np.zeros(D, np.uint8),
              s_code=np.zeros(T, np.uint8), z_bits=np.zeros(T, np.uint16))
    vq = {k: v.copy() for k, v in kq.items()}
    kq["codes"][3, 5] = 0xB
    # value codes: token 37 (kb 1, h 0, s 1, i 1), channel 83 (nb 5, n 3):
    # word 256 + 4*(16+3) + 0 = 332, bit 10 + 16 = 26 -> byte 1328 + 3, shift 2
    vq["codes"][37, 83] = 2
    kq["z_bits"][7] = 0xABCD
    vq["s_code"][100] = 0x42
    rec = codec.pack_record(kq, vq)
    assert rec[3 * 64 + 2] == 0xB0
    assert rec[8192 + 1331] == 2 << 2
    assert rec[12544 + 14] == 0xCD and rec[12544 + 15] == 0xAB
    assert rec[12928 + 100] == 0x42
    assert np.count_nonzero(rec) == 5


# ------------------------------------------------------------------ synthetic workloads


def test_generated_tiles_quantise_without_saturation():
    sp = gen.spec("qwen3-32b-16k", batch=1, ctx=256)
    st = gen.prefill(sp)
    for h in range(2):
        for rows in (slice(0, 128), slice(128, 256)):
            for arr, bits in ((st["k"], 4), (st["v"], 2)):
                q = codec.quantize_tile(arr[rows, h].astype(np.float64), bits)
                assert q["flags"] == 0
