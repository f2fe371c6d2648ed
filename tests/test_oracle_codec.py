"""Pins of the oracle's prep step (K smoothing, per-block INT8, per-channel
E4M3, binary16 V) against facts that do not come from the oracle itself:
independent FP8 and binary16 implementations (torch.float8_e4m3fn, numpy's
float16), numpy's rounding and mean, and the defining error bounds of
round-to-nearest quantisation."""
import numpy as np
import pytest
import torch

import workloads


def _torch_e4m3_codes(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_every_code_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(codes[nan]) == {0x7F, 0xFF}
    assert np.isnan(mine[nan]).all()
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_on_every_midpoint(orc):
    """Every representable value, every midpoint between neighbours, and one
    float32 ulp either side of each midpoint (all below the saturation tie)."""
    vals = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = 0.5 * (vals[1:] + vals[:-1])
    mids32 = mids.astype(np.float32)
    assert np.all(mids32.astype(np.float64) == mids)  # midpoints are exact in float32
    pts = np.concatenate([vals.astype(np.float32), mids32,
                          np.nextafter(mids32, np.float32(np.inf)),
                          np.nextafter(mids32, np.float32(0))])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    np.testing.assert_array_equal(orc.e4m3_encode(pts.astype(np.float64)), _torch_e4m3_codes(pts))


def test_e4m3_encode_matches_torch_on_all_fp16_in_range(orc):
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float32)
    h = h[np.abs(h) < 464.0]  # torch does not saturate above the 448/480 tie
    np.testing.assert_array_equal(orc.e4m3_encode(h.astype(np.float64)), _torch_e4m3_codes(h))


@pytest.mark.parametrize("x,code", [
    (448.0, 0x7E), (464.0, 0x7E), (500.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (3 * 2.0 ** -10, 0x02),
    (1.0 + 1 / 16, 0x38), (1.0 + 3 / 16, 0x3A), (0.0, 0x00), (-0.0, 0x80), (240.0, 0x77)])
def test_e4m3_encode_hand_values(orc, x, code):
    """Round-half-even ties, saturation at 448 and signed zero, worked by hand
    from the E4M3FN definition (bias 7, three mantissa bits)."""
    assert int(orc.e4m3_encode(np.array([x]))[0]) == code


# ---------------------------------------------------------------- binary16

def test_f16_decode_every_code_matches_numpy(orc):
    codes = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    mine = orc.f16_decode(codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.isnan(mine[nan]).all()
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7BFF] == 65504.0 and mine[0x0001] == 2.0 ** -24 and mine[0x0400] == 2.0 ** -14


def test_f16_encode_matches_numpy_on_every_midpoint(orc):
    """Every finite binary16 value, every midpoint between neighbours and the
    next float64 either side of it, both signs: numpy's float64 -> float16
    conversion rounds to nearest even in one step."""
    vals = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = 0.5 * (vals[1:] + vals[:-1])
    pts = np.concatenate([vals, mids, np.nextafter(mids, np.inf), np.nextafter(mids, 0.0)])
    pts = np.concatenate([pts, -pts])
    pts = pts[np.abs(pts) < 65504.0]  # numpy overflows to inf at the 65504/65536 tie
    np.testing.assert_array_equal(orc.f16_encode(pts), pts.astype(np.float16).view(np.uint16))


def test_f16_encode_matches_numpy_on_random_doubles(orc):
    rng = np.random.Generator(np.random.PCG64(3))
    x = np.ldexp(rng.uniform(1.0, 2.0, 200000), rng.integers(-30, 16, 200000))
    x *= rng.choice([-1.0, 1.0], x.size)
    x = x[np.abs(x) < 65504.0]
    np.testing.assert_array_equal(orc.f16_encode(x), x.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("x,code", [
    (65504.0, 0x7BFF), (65519.0, 0x7BFF), (65520.0, 0x7BFF), (1e30, 0x7BFF), (-1e30, 0xFBFF),
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.5 * 2.0 ** -25, 0x0001), (3 * 2.0 ** -25, 0x0002),
    (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0, 0x3C00), (0.5, 0x3800)])
def test_f16_encode_hand_values(orc, x, code):
    """Ties to even, signed zero, the subnormal step 2^-24 and saturation at
    65504 (where IEEE rounding would give infinity from 65520 up), worked by
    hand from the binary16 definition (bias 15, ten fraction bits)."""
    assert int(orc.f16_encode(np.array([x]))[0]) == code


def test_quantize_f16_mode_keeps_v_as_its_binary16_rounding(orc):
    """pv="f16": V's codes are its binary16 rounding (exact for fp16 inputs),
    the INT8 Q and K parts are those of the E4M3 mode."""
    q, k, v = workloads.random_inputs(1, 2, 2, 300, 64, "f16", seed=8)
    z8 = orc.quantize(q, k, v)
    z16 = orc.quantize(q, k, v, pv="f16")
    np.testing.assert_array_equal(z16["v_f16"], v.numpy().view(np.uint16))
    for key in ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean"):
        np.testing.assert_array_equal(z16[key], z8[key])
    _, _, vb = workloads.random_inputs(1, 2, 2, 300, 64, "bf16", seed=8)
    zb = orc.quantize(q, k, vb, pv="f16")
    np.testing.assert_array_equal(zb["v_f16"],
                                  vb.to(torch.float32).numpy().astype(np.float16).view(np.uint16))


def _deq(codes, scale, blk, n):
    s = np.repeat(scale.astype(np.float64), blk, axis=-1)[..., :n]
    return codes.astype(np.float64) * s[..., None]


@pytest.mark.parametrize("qk_bits,qmax", [(8, 127), (4, 7)])
@pytest.mark.parametrize("N,d", [(300, 64), (256, 128), (1, 64), (129, 64)])
def test_int8_blocks_round_half_even_within_half_step(orc, N, d, qk_bits, qmax):
    """INT8 (and the INT4 values of the 4-bit variant): scale absmax/qmax,
    codes numpy's rint of the float32 product, the block's largest magnitude
    at +-qmax, every code within half a step."""
    q, k, v = workloads.random_inputs(2, 3, 3, N, d, "f16", seed=N + d, scale=3.0)
    z = orc.quantize(q, k, v, qk_bits=qk_bits)
    q32 = orc.to_f32(q)
    nqb = -(-N // 128)
    qm = np.float32(qmax)
    for b in range(2):
        for h in range(3):
            for t in range(nqb):
                blk = q32[b, h, t * 128:(t + 1) * 128]
                a = np.abs(blk).max()
                s = z["q_scale"][b, h, t]
                assert s == np.float32(a) / qm
                codes = z["q_i8"][b, h, t * 128:(t + 1) * 128]
                # numpy's own rint (half-even) on the float32 product
                ref = np.clip(np.rint(blk * (qm / np.float32(a))), -qmax, qmax)
                np.testing.assert_array_equal(codes, ref.astype(np.int8))
                # the largest magnitude maps to +-qmax and every code is within
                # half a step of the value (plus float32 rounding of scale and
                # reciprocal, at most qmax * 3 * 2^-24 of a step)
                assert np.abs(codes).max() == qmax
                err = np.abs(codes.astype(np.float64) * s - blk)
                assert np.all(err <= (0.5 + 1e-4) * s)


@pytest.mark.parametrize("qk_bits,qmax", [(8, 127), (4, 7)])
@pytest.mark.parametrize("bq,bk", [(1, 32), (128, 64), (1, 1)])
def test_scale_groups_of_every_granularity(orc, bq, bk, qk_bits, qmax):
    """Q scales per bq rows and K scales per bk keys, each the group's absmax /
    qmax with numpy's rint on the float32 product, for the per-block, the
    thread-level (per-row Q, 32-key K) and the token (per-row Q, per-key K)
    granularities; ragged last groups."""
    N, d = 70, 64
    q, k, v = workloads.random_inputs(1, 2, 2, N, d, "bf16", seed=bq + bk, scale=2.0)
    z = orc.quantize(q, k, v, bq=bq, bk=bk, qk_bits=qk_bits)
    qm = np.float32(qmax)
    assert z["q_scale"].shape[-1] == -(-N // bq) and z["k_scale"].shape[-1] == -(-N // bk)
    q32 = orc.to_f32(q)
    ks = orc.to_f32(k) - z["k_mean"][:, :, None, :]
    for x, codes, scales, g in ((q32, z["q_i8"], z["q_scale"], bq), (ks, z["k_i8"], z["k_scale"], bk)):
        for h in range(2):
            for t in range(-(-N // g)):
                blk = x[0, h, t * g:(t + 1) * g]
                a = np.abs(blk).max()
                assert scales[0, h, t] == np.float32(a) / qm
                ref = np.clip(np.rint(blk * (qm / np.float32(a))), -qmax, qmax)
                np.testing.assert_array_equal(codes[0, h, t * g:(t + 1) * g], ref.astype(np.int8))


def test_k_mean_is_the_token_mean_and_smoothed_codes_bound_k_minus_mean(orc):
    w = workloads.WORKLOADS[1].resized(N=333)
    q, k, v = workloads.generate(w, seed=11)
    z = orc.quantize(q, k, v)
    k32 = orc.to_f32(k)
    mean = k32.astype(np.float64).mean(axis=2).astype(np.float32)
    np.testing.assert_array_equal(z["k_mean"], mean)
    ks = (k32 - z["k_mean"][:, :, None, :]).astype(np.float64)
    kd = _deq(z["k_i8"], z["k_scale"], 64, w.N)
    step = np.repeat(z["k_scale"].astype(np.float64), 64, axis=-1)[..., :w.N, None]
    assert np.all(np.abs(kd - ks) <= (0.5 + 1e-4) * step)
    # smoothing removes the channel offsets: the smoothed K has zero mean
    assert np.abs(ks.mean(axis=2)).max() < 1e-5


def test_constant_and_zero_blocks(orc):
    N, d = 200, 64
    q = torch.full((1, 2, N, d), -2.5, dtype=torch.float16)
    q[0, 1] = 0.0
    k = torch.full((1, 2, N, d), 7.0, dtype=torch.float16)      # identical rows
    v = torch.full((1, 2, N, d), 0.3125, dtype=torch.float16)
    v[0, 1, :, 5] = 0.0
    z = orc.quantize(q, k, v)
    assert np.all(z["q_i8"][0, 0] == -127)
    assert np.all(np.abs(z["q_scale"][0, 0] * np.float32(127) - np.float32(2.5)) <= np.spacing(np.float32(2.5)))
    assert np.all(z["q_i8"][0, 1] == 0) and np.all(z["q_scale"][0, 1] == 0)
    # identical K rows: the mean is exact, smoothed K is all zero
    assert np.all(z["k_mean"] == 7.0) and np.all(z["k_i8"] == 0) and np.all(z["k_scale"] == 0)
    # constant V channel: code 448, scale * 448 is the value
    assert np.all(z["v_fp8"][0, 0] == 0x7E)
    assert np.all(np.abs(z["v_scale"][0, 0] * np.float32(448) - np.float32(0.3125)) <= np.spacing(np.float32(0.3125)))
    assert np.all(z["v_fp8"][0, 1, :, 5] == 0) and z["v_scale"][0, 1, 5] == 0


@pytest.mark.parametrize("recipe", [1, 3, 5])
def test_v_codes_within_half_e4m3_step_and_channel_max_is_448(orc, recipe):
    w = workloads.WORKLOADS[recipe].resized(B=1, Hq=2, Hkv=2, N=700)
    q, k, v = workloads.generate(w, seed=3)
    z = orc.quantize(q, k, v)
    v32 = orc.to_f32(v).astype(np.float64)
    sv = z["v_scale"].astype(np.float64)[:, :, None, :]
    vd = orc.e4m3_decode(z["v_fp8"]) * sv
    # RNE to E4M3: error at most half a step, i.e. 2^-4 relative for normals
    # and 2^-10 (times the scale) in the subnormal range
    t = np.abs(v32) / sv
    bound = np.where(t >= 2.0 ** -6, t * 2.0 ** -4, 2.0 ** -10) * sv * (1 + 1e-6)
    assert np.all(np.abs(vd - v32) <= bound + 1e-30)
    assert np.all(np.abs(orc.e4m3_decode(z["v_fp8"])).max(axis=2) == 448.0)
