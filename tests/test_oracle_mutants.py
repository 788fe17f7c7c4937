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
