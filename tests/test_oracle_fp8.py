"""Pins of the oracle's FP8 (OCP e4m3fn) encoding and per-token cast:
torch's own float8_e4m3fn conversion (an independent implementation of the
same format), exhaustive code tables, an independent tensor formulation of
the cast, closed forms of the scale and the error bound of the round trip."""
import numpy as np
import pytest
import torch

import oracle
import synth

E4M3 = torch.float8_e4m3fn


def _bf16_bits(vals) -> np.ndarray:
    return torch.from_numpy(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _torch_codes(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float32)).to(E4M3).view(torch.uint8).numpy()


def test_decode_all_256_codes_matches_torch():
    want = torch.arange(256, dtype=torch.uint8).view(E4M3).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float32)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2  # 0x7F and 0xFF
    assert (got[~nan] == want[~nan]).all()
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_encode_every_bf16_value_in_range_matches_torch():
    """Every bf16 value with |v| <= 448 (about 33 k of them), encoded."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = _bf16_f32(bits)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    v = v[keep]
    got = np.array([oracle.e4m3_encode(float(a)) for a in v], np.uint8)
    assert (got == _torch_codes(v)).all()


def test_encode_random_fp32_and_exact_ties_match_torch():
    rng = np.random.default_rng(0)
    v = (rng.uniform(-1, 1, 20000) * 2.0 ** rng.integers(-14, 9, 20000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    # midpoints between consecutive finite codes: ties go to the even code
    vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(E4M3).to(torch.float64).numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    got = np.array([oracle.e4m3_encode(float(a)) for a in v], np.uint8)
    assert (got == _torch_codes(v)).all()
    # every tie lands on an even code
    tie_codes = np.array([oracle.e4m3_encode(float(a)) for a in mids], np.uint8)
    assert (tie_codes % 2 == 0).all()


def test_encode_saturates_above_448():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E and oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x80 and oracle.e4m3_encode(2.0 ** -11) == 0


def _torch_cast(x_bits: np.ndarray, fmt: int):
    """Independent formulation with tensor ops: per (token, 128-block) amax,
    fp32 multiplier, clamp, torch's e4m3fn conversion."""
    x = torch.from_numpy(_bf16_f32(x_bits))
    T, H = x.shape
    xb = x.view(T, H // 128, 128)
    amax = xb.abs().amax(dim=-1).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    if fmt == oracle.SCALE_F32:
        mul = torch.tensor(448.0, dtype=torch.float32) / amax
        scale = amax / torch.tensor(448.0, dtype=torch.float32)
    else:
        s0 = amax / torch.tensor(448.0, dtype=torch.float32)
        m, e = torch.frexp(s0)
        k = torch.where(m == 0.5, e - 1, e)
        mul = torch.ldexp(torch.ones_like(s0), -k)
        scale = torch.ldexp(torch.ones_like(s0), k) if fmt == oracle.SCALE_POW2 else (k + 127).to(torch.uint8)
    v = (xb * mul.unsqueeze(-1)).clamp(-448.0, 448.0)
    codes = v.to(E4M3).view(torch.uint8).reshape(T, H).numpy()
    return codes, scale.numpy()


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_POW2, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("T,H,spread", [(7, 128, 1.0), (33, 1024, 30.0), (5, 7168, 1e-3)])
def test_cast_matches_independent_tensor_formulation(fmt, T, H, spread):
    rng = np.random.default_rng(T + H)
    x = rng.standard_normal((T, H)) * np.exp(rng.uniform(-np.log(spread + 1), np.log(spread + 1), (T, H // 128, 1))
                                             ).repeat(128, axis=2).reshape(T, H)
    xb = _bf16_bits(x)
    xb[0, :128] = 0  # an all-zero block
    xb[1, 5] = _bf16_bits([1e-30])[0]
    q, s = oracle.cast_to_fp8(xb, fmt)
    q2, s2 = _torch_cast(xb, fmt)
    assert (q == q2).all()
    assert (s.view(np.uint8) == np.asarray(s2).view(np.uint8)).all()


def test_cast_closed_forms():
    rng = np.random.default_rng(1)
    x = _bf16_bits(rng.standard_normal((16, 512)) * 3)
    q, s = oracle.cast_to_fp8(x, oracle.SCALE_F32)
    xf = _bf16_f32(x).reshape(16, 4, 128)
    amax = np.abs(xf).max(axis=-1)
    np.testing.assert_array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    # the block's largest magnitude maps to +-448 (code 0x7E / 0xFE)
    qb = q.reshape(16, 4, 128)
    arg = np.abs(xf).argmax(axis=-1)
    top = np.take_along_axis(qb, arg[..., None], axis=-1)[..., 0]
    assert ((top & 0x7F) == 0x7E).all()
    # power-of-two scales: amax / s in (224, 448], UE8M0 byte = log2(s) + 127
    _, sp = oracle.cast_to_fp8(x, oracle.SCALE_POW2)
    _, su = oracle.cast_to_fp8(x, oracle.SCALE_UE8M0)
    k = np.log2(sp)
    assert (k == np.round(k)).all() and ((amax / sp > 224) & (amax / sp <= 448)).all()
    assert (su.astype(np.int32) == k.astype(np.int32) + 127).all()
    # a block of zeros: codes 0, scale 1e-4 / 448
    qz, sz = oracle.cast_to_fp8(np.zeros((1, 128), np.uint16), oracle.SCALE_F32)
    assert (qz == 0).all() and sz[0, 0] == np.float32(1e-4) / np.float32(448)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_POW2, oracle.SCALE_UE8M0])
def test_round_trip_error_bound(fmt):
    """cast_back(cast(x)) errs by at most half an e4m3 spacing (2^-4 relative
    in the normal range, 2^-10 * s in the subnormal range) plus one bf16
    rounding (2^-8 relative)."""
    w = synth.Workload("fp8pin", T=64, H=1024, K=1, E=1, R=1)
    x = synth.make_x(w, seed=3)
    q, s = oracle.cast_to_fp8(x, fmt)
    back = _bf16_f32(oracle.cast_back(q, s, fmt)).astype(np.float64)
    xf = _bf16_f32(x).astype(np.float64)
    sf = (2.0 ** (s.astype(np.float64) - 127)) if fmt == oracle.SCALE_UE8M0 else s.astype(np.float64)
    sfull = np.repeat(sf, 128, axis=1)
    err = np.abs(back - xf)
    bound = 2.0 ** -4 * np.abs(xf) * (1 + 2.0 ** -7) + 2.0 ** -10 * sfull + 2.0 ** -8 * np.abs(back)
    assert (err <= bound).all()
    # and the relative L2 error is small (fp32 scales: a few percent at most)
    assert np.sqrt((err ** 2).sum() / (xf ** 2).sum()) < 0.05
    # codes decode exactly: back == bf16(decode(q) * s)
    dec = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float32)[q]
    want = _bf16_bits((dec * np.repeat(np.asarray(sf, np.float32), 128, axis=1)).astype(np.float32))
    np.testing.assert_array_equal(oracle.cast_back(q, s, fmt), want)


def test_cast_rejects_bad_hidden():
    with pytest.raises(oracle.OracleError):
        oracle.cast_to_fp8(np.zeros((2, 100), np.uint16))
