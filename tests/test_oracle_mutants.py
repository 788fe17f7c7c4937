"""The pins are strong enough: each plants a plausible mistake in the ORACLE (on the
CPU, via monkeypatching) and checks that at least one pin test then fails.
"""

import numpy as np
import pytest

import oracle.adamw as A
import oracle.philox as P
import oracle.rounding as R
import test_oracle_adamw as TA
import test_oracle_codebook as TC
import test_oracle_philox as TP
import test_oracle_rounding as TR


def _fails(fn, *args, **kw):
    with pytest.raises(AssertionError):
        fn(*args, **kw)


def _swap_beta_and_weight(p, g, m1, v1, s):
    m2 = (s.w1 * m1 + s.beta1 * g).astype(np.float32)
    v2 = (s.beta2 * v1 + s.w2 * (g * g)).astype(np.float32)
    den = (np.sqrt(v2) * s.rbc2 + s.eps).astype(np.float32)
    return m2, v2, ((p - s.lrwd * p) - s.step_size * (m2 / den)).astype(np.float32)


def _eps_inside_root(p, g, m1, v1, s):
    m2 = (s.beta1 * m1 + s.w1 * g).astype(np.float32)
    v2 = (s.beta2 * v1 + s.w2 * (g * g)).astype(np.float32)
    den = (np.sqrt(v2 + s.eps) * s.rbc2).astype(np.float32)
    return m2, v2, ((p - s.lrwd * p) - s.step_size * (m2 / den)).astype(np.float32)


def _decay_sign_flipped(p, g, m1, v1, s):
    m2 = (s.beta1 * m1 + s.w1 * g).astype(np.float32)
    v2 = (s.beta2 * v1 + s.w2 * (g * g)).astype(np.float32)
    den = (np.sqrt(v2) * s.rbc2 + s.eps).astype(np.float32)
    return m2, v2, ((p + s.lrwd * p) - s.step_size * (m2 / den)).astype(np.float32)


def _grad_not_squared(p, g, m1, v1, s):
    m2 = (s.beta1 * m1 + s.w1 * g).astype(np.float32)
    v2 = (s.beta2 * v1 + s.w2 * np.abs(g)).astype(np.float32)
    den = (np.sqrt(v2) * s.rbc2 + s.eps).astype(np.float32)
    return m2, v2, ((p - s.lrwd * p) - s.step_size * (m2 / den)).astype(np.float32)


@pytest.mark.parametrize("mutant", [_swap_beta_and_weight, _eps_inside_root,
                                    _decay_sign_flipped, _grad_not_squared])
def test_update_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(TA, "adamw_param_update", mutant)
    case = (4, 1e-8, 0.1) if mutant is _decay_sign_flipped else (7, 1e-3, 0.0)
    _fails(TA.test_fp32_update_matches_torch_adamw, *case)


def test_bias_correction_off_by_one_is_caught(monkeypatch):
    real = A.host_scalars

    def shifted(hp):
        return real(A.Hparams(**{**hp.__dict__, "step": hp.step + 1}))
    monkeypatch.setattr(TA, "host_scalars", shifted)
    _fails(TA.test_fp32_update_matches_torch_adamw, 4, 1e-8, 0.1)


def test_right_sided_search_is_caught(monkeypatch):
    real = np.searchsorted

    def right(a, v, side="left", sorter=None):
        return real(a, v, side="right")
    monkeypatch.setattr(A.np, "searchsorted", right)
    _fails(TC.test_midpoint_ties_take_the_lower_code)


def test_wrong_block_index_in_dequantize_is_caught(monkeypatch):
    def shifted(codes, absmax, table):
        per = np.repeat(np.roll(np.asarray(absmax, np.float32), 1), A.BLOCK)[: np.asarray(codes).size]
        return (table[np.asarray(codes, np.uint8)] * per).astype(np.float32)
    monkeypatch.setattr(TC, "dequantize_blockwise", shifted)
    _fails(TC.test_dequantize_is_table_times_block_max)


def test_fifteen_bit_sr_is_caught(monkeypatch):
    real = R.f32_to_bf16_sr
    monkeypatch.setattr(TR, "f32_to_bf16_sr", lambda x, r: real(x, np.asarray(r, np.uint32) >> 1))
    _fails(TR.test_sr_mean_over_all_random_words_is_exact)


def test_nine_round_philox_is_caught(tmp_path):
    def nine(c0, c1, c2, c3, k0, k1):
        c0, c1, c2, c3 = (np.asarray(x, np.uint64) for x in (c0, c1, c2, c3))
        k0, k1 = int(k0), int(k1)
        for rnd in range(9):
            if rnd:
                k0, k1 = (k0 + P.W0) & 0xFFFFFFFF, (k1 + P.W1) & 0xFFFFFFFF
            p0, p1 = np.uint64(P.M0) * c0, np.uint64(P.M1) * c2
            c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & np.uint64(0xFFFFFFFF),
                              (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & np.uint64(0xFFFFFFFF))
        return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))
    ref = TP.build_ref(tmp_path)
    if ref is None:
        pytest.skip("needs g++ and the rocRAND header")
    _fails(TP.check_philox, ref, nine)


def test_rne_without_ties_to_even_is_caught(monkeypatch):
    def no_even(x):
        x = np.asarray(x, np.float32)
        b = x.view(np.uint32)
        return (((b + np.uint32(0x8000)) & np.uint32(0xFFFF0000)) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(TR, "f32_to_bf16_rne", no_even)
    _fails(TR.test_rne_matches_torch_conversion)


# ----------------------------------------------------------------------------- one-state rules
import oracle.state_sr as SS  # noqa: E402
import test_oracle_onestate as TO  # noqa: E402
import test_oracle_state_sr as TS  # noqa: E402


def _lion_new_moment_direction(p, g, m1, s):
    m2 = (s.beta2 * m1 + s.w2 * g).astype(np.float32)
    c = (s.beta1 * m2 + s.w1 * g).astype(np.float32)
    return m2, ((p - s.lrwd * p) - s.lr * np.sign(c).astype(np.float32)).astype(np.float32)


def _lion_betas_swapped(p, g, m1, s):
    c = (s.beta2 * m1 + s.w2 * g).astype(np.float32)
    m2 = (s.beta1 * m1 + s.w1 * g).astype(np.float32)
    return m2, ((p - s.lrwd * p) - s.lr * np.sign(c).astype(np.float32)).astype(np.float32)


def _lion_sign_of_zero_is_one(p, g, m1, s):
    c = (s.beta1 * m1 + s.w1 * g).astype(np.float32)
    m2 = (s.beta2 * m1 + s.w2 * g).astype(np.float32)
    sgn = np.where(c >= 0, 1, -1).astype(np.float32)
    return m2, ((p - s.lrwd * p) - s.lr * sgn).astype(np.float32)


@pytest.mark.parametrize("mutant,pin", [
    (_lion_new_moment_direction, "test_lion_uses_the_old_moment_for_the_direction"),
    (_lion_betas_swapped, "test_lion_uses_the_old_moment_for_the_direction"),
    (_lion_sign_of_zero_is_one, "test_lion_step1_closed_form"),
])
def test_lion_mutants_are_caught(monkeypatch, mutant, pin):
    monkeypatch.setattr(TO, "lion_update", mutant)
    _fails(getattr(TO, pin))


def _momentum_with_dampening(p, g, m1, s):
    m2 = (s.beta1 * m1 + s.w1 * g).astype(np.float32)
    return m2, ((p - s.lrwd * p) - s.lr * m2).astype(np.float32)


def _momentum_coupled_decay(p, g, m1, s):
    wd = np.float32(s.lrwd / s.lr) if s.lr else np.float32(0)
    m2 = (s.beta1 * m1 + (g + wd * p)).astype(np.float32)
    return m2, (p - s.lr * m2).astype(np.float32)


def test_momentum_mutants_are_caught(monkeypatch):
    monkeypatch.setattr(TO, "momentum_update", _momentum_with_dampening)
    _fails(TO.test_momentum_matches_torch_sgd, 0.0)
    monkeypatch.setattr(TO, "momentum_update", _momentum_coupled_decay)
    _fails(TO.test_momentum_decoupled_decay_and_zero_gradient)


# ----------------------------------------------------------------------------- state rounding
def _sr_codes_variant(flip=False, ge=False, gap_below=False):
    def codes(n, table, weights, r16):
        n = np.asarray(n, dtype=np.float32)
        count = np.searchsorted(table, n, side="right")
        k = np.clip(count.astype(np.int64) - 1, 0, table.size - 2)
        w = weights
        if gap_below:   # gap weight of the gap below C[k] instead of above
            w = np.concatenate([[weights[0]], weights[:-1]]).astype(np.float32)
        f = ((n - table[k]).astype(np.float32) * w[k]).astype(np.float32)
        r = np.asarray(r16, dtype=np.uint32).astype(np.float32)
        up = (f >= r) if ge else (f > r)
        if flip:
            up = ~up
        code = k + up.astype(np.int64)
        return np.where(np.isnan(n), table.size - 1, code).astype(np.uint8)
    return codes


@pytest.mark.parametrize("kw,pin", [
    (dict(flip=True), "test_mean_over_all_random_words_is_the_value"),
    (dict(ge=True), "test_codes_are_the_two_neighbours_and_entries_stay"),
    (dict(gap_below=True), "test_mean_over_all_random_words_is_the_value"),
])
def test_state_rounding_mutants_are_caught(monkeypatch, kw, pin):
    monkeypatch.setattr(TS, "sr_codes", _sr_codes_variant(**kw))
    _fails(getattr(TS, pin), "signed")


def test_state_rounding_that_ignores_the_draw_is_caught(monkeypatch):
    """Nearest rounding in place of the stochastic choice: the decay pin fails."""
    real = SS.quantize_blockwise_sr

    def nearest(x, table, zero_code, r16):
        return real(x, table, zero_code, np.full(np.asarray(r16).shape, 32768, np.uint32))
    monkeypatch.setattr(SS, "quantize_blockwise_sr", nearest)
    _fails(TS.test_decaying_second_moment_is_frozen_by_nearest_and_followed_by_stochastic)
