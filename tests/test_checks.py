"""The GPU tests' comparison functions must reject plausible mistakes: the
mistakes are planted in a copy of the oracle's own output, on the CPU."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gpu_util import check_fp8, check_o_lse, e4m3_order  # noqa: E402
from mla_paged_kv_05_amd import workloads as W  # noqa: E402


@pytest.fixture(scope="module")
def fused_ref():
    p = W.with_fp8v32(W.make_dense("chk", [70, 300, 5], s_q=1, h_q=16, seed=3, fused=True), seed=4)
    return oracle.decode(p)


@pytest.fixture(scope="module")
def plain_ref():
    p = W.make_dense("chk", [70, 300, 0], s_q=1, h_q=16, seed=5)
    return oracle.decode(p)


def _fp8(r, codes=None, scale=None):
    return check_fp8(r["codes"] if codes is None else codes, r["oscale"] if scale is None else scale,
                     r["codes"], r["oscale"], r["o"], "planted")


def test_fp8_identical_passes(fused_ref):
    assert _fp8(fused_ref) == 0


def test_fp8_one_code_bias_fails(fused_ref):
    c = fused_ref["codes"].copy()
    big = np.abs(fused_ref["o"]) >= np.abs(fused_ref["o"]).max(-1, keepdims=True) / 16
    mag = c & 0x7F
    bump = big & (mag < 0x7E) & (mag > 0)
    c[bump] = (c[bump] & 0x80) | (mag[bump] + 1)
    with pytest.raises(AssertionError):
        _fp8(fused_ref, codes=c)


def test_fp8_two_code_error_fails(fused_ref):
    c = fused_ref["codes"].copy()
    o = np.abs(fused_ref["o"])
    i = np.unravel_index(np.argmax(np.where(o < o.max(-1, keepdims=True) / 2, o, 0)), o.shape)
    c[i] = (c[i] & 0x80) | ((c[i] & 0x7F) - 2)
    assert abs(int(e4m3_order(c[i])) - int(e4m3_order(fused_ref["codes"][i]))) == 2
    with pytest.raises(AssertionError):
        _fp8(fused_ref, codes=c)


def test_fp8_scale_error_fails(fused_ref):
    s = fused_ref["oscale"].copy()
    s[0, 0, 3] *= 1.01
    with pytest.raises(AssertionError):
        _fp8(fused_ref, scale=s)


def test_fp8_small_element_error_fails(fused_ref):
    c = fused_ref["codes"].copy()
    o = np.abs(fused_ref["o"])
    small = o < o.max(-1, keepdims=True) / 64
    i = tuple(np.argwhere(small)[0])
    c[i] = (c[i] & 0x80) | 0x48  # |code value| 4.0 where the reference is below 7
    with pytest.raises(AssertionError):
        _fp8(fused_ref, codes=c)


def test_fp8_row_max_must_be_448(fused_ref):
    c = fused_ref["codes"].copy()
    flat = c.reshape(-1, c.shape[-1])
    once = np.nonzero(((flat & 0x7F) == 0x7E).sum(-1) == 1)[0]
    row = flat[once[0]]
    j = int(np.argmax(row & 0x7F))
    row[j] = (row[j] & 0x80) | 0x7D
    with pytest.raises(AssertionError):
        _fp8(fused_ref, codes=c)


def test_o_identical_passes(plain_ref):
    check_o_lse(plain_ref["o"], plain_ref["lse"], plain_ref["o"], plain_ref["lse"], "planted")


def test_o_one_broken_row_fails(plain_ref):
    o = plain_ref["o"].copy()
    o[1, 0, 7] *= 1.05  # 5% on one row barely moves the tensor's RMS
    with pytest.raises(AssertionError):
        check_o_lse(o, plain_ref["lse"], plain_ref["o"], plain_ref["lse"], "planted")


def test_lse_error_fails(plain_ref):
    lse = plain_ref["lse"].copy()
    lse[0, 0, 0] += 2e-3
    with pytest.raises(AssertionError):
        check_o_lse(plain_ref["o"], lse, plain_ref["o"], plain_ref["lse"], "planted")


def test_empty_row_must_be_zero(plain_ref):
    o = plain_ref["o"].copy()
    assert np.isneginf(plain_ref["lse"][2]).all()
    o[2, 0, 0, 0] = 1e-3
    with pytest.raises(AssertionError):
        check_o_lse(o, plain_ref["lse"], plain_ref["o"], plain_ref["lse"], "planted")
