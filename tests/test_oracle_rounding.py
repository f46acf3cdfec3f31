"""The oracle's rounding steps against library routines and the definition.

bfloat16: the oracle's own bit routine vs torch's CPU cast (round to nearest
even) and vs a from-definition Fraction rounding.  binary16: NumPy's cast
(the oracle's step) vs torch's CPU cast and the same Fraction rounding.  The
plain-C oracle's routines are held to the same results.
"""

import numpy as np
import pytest
import torch

import oracle_pins as P
from oracle import allreduce as O
from oracle import cpu as C


def stratified_f32_patterns(n_random=1 << 21, seed=5):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1000, 0xF000], dtype=np.uint32)
    grid = (hi[:, None] | lows[None, :]).ravel()
    # binary16-relevant region: exponents around the binary16 range, all
    # rounding positions (13 dropped bits) including ties
    e = np.arange(96, 146, dtype=np.uint32)
    m_lows = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x3000, 0x7FFFFF, 0x7FE000,
                       0x7FF000, 0x7FEFFF], dtype=np.uint32)
    sgn = np.array([0, 0x80000000], dtype=np.uint32)
    f16grid = (sgn[:, None, None] | (e[None, :, None] << 23) | m_lows[None, None, :]).ravel()
    rnd = np.random.default_rng(seed).integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([grid, f16grid, rnd])


def _is_nan32(u):
    return ((u & 0x7F800000) == 0x7F800000) & ((u & 0x7FFFFF) != 0)


def test_bf16_rounding_matches_torch():
    u = stratified_f32_patterns()
    a = u.view(np.float32)
    got = O.f32_to_bf16_rne(a)
    want = torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = _is_nan32(u)
    assert np.array_equal(got[~nan], want[~nan])
    g = got[nan]
    assert np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)), "NaN must stay NaN"
    assert np.array_equal(g >> 15, (u[nan] >> 31).astype(np.uint16)), "NaN keeps its sign"


def test_f16_rounding_matches_torch():
    u = stratified_f32_patterns()
    a = u.view(np.float32)
    got = O.round_to(a, "fp16").view(np.uint16)
    want = torch.from_numpy(a.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    nan = _is_nan32(u)
    assert np.array_equal(got[~nan], want[~nan])
    g = got[nan]
    assert np.all(((g & 0x7C00) == 0x7C00) & ((g & 0x3FF) != 0))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_rounding_matches_definition(dtype):
    u = stratified_f32_patterns(n_random=4000, seed=6)
    g = np.random.default_rng(7)
    u = np.concatenate([u[(1 << 16) * 8:], g.choice(u[:(1 << 16) * 8], 6000, replace=False)])
    u = u[~_is_nan32(u)]
    a = u.view(np.float32)
    got = P.bits_of(O.round_to(a, dtype), dtype)
    for i in range(len(a)):
        v = float(a[i])
        if np.isinf(v):
            want = ("inf", 1 if v < 0 else 0)
        else:
            from fractions import Fraction
            want = P.round_def(Fraction(v), dtype)
            if v == 0.0:
                want = ("num", 1 if np.signbit(a[i]) else 0, Fraction(0))
            elif want[0] == "num" and want[2] == 0:
                want = ("num", 1 if v < 0 else 0, Fraction(0))
        assert P.same_value(got[i], want, dtype), f"{dtype} {u[i]:#010x}: got {int(got[i]):#06x} want {want}"


def test_c_rounding_matches_oracle():
    u = stratified_f32_patterns(n_random=1 << 20)
    a = u.view(np.float32)
    nan = _is_nan32(u)
    cb = C.round_bf16(a)
    ob = O.f32_to_bf16_rne(a)
    assert np.array_equal(cb, ob)  # same NaN rule too
    ch = C.round_f16(a).view(np.uint16)
    oh = O.round_to(a, "fp16").view(np.uint16)
    assert np.array_equal(ch[~nan], oh[~nan])
    assert np.all(((ch[nan] & 0x7C00) == 0x7C00) & ((ch[nan] & 0x3FF) != 0))


def test_c_f16_widening_exact():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    w = C.widen_f16(h.view(np.float16))
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(w.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    assert np.all(np.isnan(w[nan]))
