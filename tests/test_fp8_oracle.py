"""Pins for the oracle's e4m3fn format table, rounding and per-head quantiser
(CPU only). The independent reference is torch's float8_e4m3fn cast, which
rounds to nearest-even; closed forms pin the descale arithmetic."""
import numpy as np
import pytest
import torch

import oracle
from tiled_attention_fa2_amd.inputs import make_qkv


def test_table_shape_of_format():
    t = oracle.e4m3_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    finite = t[np.isfinite(t)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    pos = np.sort(finite[finite > 0])
    assert len(pos) == 126
    assert pos[0] == 2.0 ** -9                     # smallest subnormal
    assert 2.0 ** -6 in pos                        # smallest normal
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    # table entries agree with torch's own decode of every finite code
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(tv, t[codes])


def _torch_codes(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_table_midpoints_and_random():
    t = oracle.e4m3_table()
    pos = np.sort(t[np.isfinite(t) & (t >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2                 # exact ties (representable in fp32)
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float64)
    rng = np.random.default_rng(0)
    rnd = rng.uniform(-448, 448, 200000)
    small = rng.uniform(-0.03, 0.03, 100000)          # subnormal range
    for x in (pos, -pos, mids, -mids, near, -near, rnd, small):
        x = x.astype(np.float32).astype(np.float64)
        assert np.array_equal(oracle.e4m3_encode(x), _torch_codes(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([np.nan]))


def test_quantize_closed_forms():
    x = np.zeros((1, 3, 4, 8), dtype=np.float32)
    x[0, 0, 1, 2] = 448.0                  # amax 448: descale 1, codes are plain e4m3
    x[0, 0, 0, 0] = -3.0
    x[0, 1] = 1.0                          # constant head: every code maps to 448
    # head 2 stays all zero: descale 1, codes 0
    codes, ds = oracle.quantize_per_head(x)
    assert ds[0, 0] == 1.0 and ds[0, 2] == 1.0
    assert codes[0, 0, 1, 2] == 0x7E and codes[0, 0, 0, 0] == _torch_codes([-3.0])[0]
    assert np.all(codes[0, 1] == 0x7E)
    assert ds[0, 1] == np.float32(1.0 / 448.0)
    assert np.all(codes[0, 2] == 0)


def test_quantize_bf16_inputs_matches_torch_pipeline():
    q, _, _ = make_qkv(1, 4, 300, 64, "bf16", seed=3)
    codes, ds = oracle.quantize_per_head(q)
    xf = q.float()
    for h in range(4):
        amax = xf[0, h].abs().max()
        ds_t = amax / 448.0
        mult = 448.0 / amax
        y = (xf[0, h] * mult).clamp(-448, 448)
        assert ds[0, h] == ds_t.item()
        assert np.array_equal(codes[0, h], y.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        # the largest-magnitude element lands on +-448
        idx = torch.argmax(xf[0, h].abs()).item()
        assert codes[0, h].ravel()[idx] & 0x7F == 0x7E


def test_dequantize_error_bound():
    q, _, _ = make_qkv(1, 2, 512, 64, "bf16", seed=4)
    codes, ds = oracle.quantize_per_head(q)
    deq = oracle.dequantize_per_head(codes, ds)
    x = q.double().numpy()
    # relative spacing of e4m3 normals is 2^-3; half of it bounds the rounding,
    # and subnormals are spaced 2^-9 (in units of the descale)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * ds[:, :, None, None].astype(np.float64)) * 1.0001
    assert np.all(np.abs(deq - x) <= bound + 1e-7 * np.abs(x))
