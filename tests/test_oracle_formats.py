"""Pins of the oracle's number formats against the framework's own casts.

e4m3 here is OCP E4M3FN (max 448), the format implied by the per-tensor
activation scale amax/448 of the fp8 workloads; bf16 rounding is to nearest
even.  torch's float8_e4m3fn and bfloat16 casts are independent library
implementations of the same formats.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours = np.isnan(ours)
    nan_ref = np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert set(np.nonzero(nan_ours)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    # spot values fixed by the format: max normal, min normal, min subnormal
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    back = oracle.e4m3_encode(vals)
    assert np.array_equal(back, codes)


def test_e4m3_encode_midpoints_go_to_even_code():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, increasing
    assert (np.diff(pos) > 0).all()
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exactly representable
    enc = oracle.e4m3_encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc.astype(np.int64), expect)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, ref)


def test_e4m3_encode_random_in_range_matches_torch():
    g = torch.Generator().manual_seed(123)
    v = (torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 2)).clamp(-448, 448)
    v = v.to(torch.float32)
    ours = oracle.e4m3_encode(v.numpy())
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch maps -0 results to 0x80 as we do
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.4e38, -500.0, -1e30], dtype=np.float32)
    enc = oracle.e4m3_encode(v)
    assert enc.tolist() == [0x7E] * 7 + [0xFE] * 2


def test_e4m3_small_values_and_zero():
    v = np.array([0.0, -0.0, 2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -9 * 1.5], dtype=np.float32)
    enc = oracle.e4m3_encode(v)
    # 2^-10 is the midpoint of 0 and 2^-9: ties to the even code 0
    assert enc.tolist() == [0x00, 0x80, 0x00, 0x01, 0x02]


def test_bf16_encode_matches_torch():
    g = torch.Generator().manual_seed(7)
    v = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 10)
    bits = v.view(torch.int32)
    # add exact ties: low half == 0x8000, both parities of the kept bit
    ties = ((bits & ~0xFFFF) | 0x8000).view(torch.float32)
    allv = torch.cat([v, ties, torch.tensor([0.0, -0.0, 3.3895314e38, -3.3895314e38, 1e-40, -1e-42])])
    ours = oracle.bf16_encode(allv.numpy())
    ref = allv.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_is_exact_widening():
    c = np.arange(0, 65536, 97, dtype=np.uint16)
    ours = oracle.bf16_decode(c)
    ref = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_scale_from_amax():
    assert oracle.scale_from_amax(0.0) == 1.0
    assert oracle.scale_from_amax(448.0) == 1.0
    a = np.float32(3.1415927)
    assert oracle.scale_from_amax(float(a)) == float(np.float32(a / np.float32(448.0)))
