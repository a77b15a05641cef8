"""Pins of the oracle's q side of the attention write (per-head RMSNorm with
no weight, then the NeoX rotation of the tail; the QNorm op's q_in,
q_head_padded, eps and apply_q_norm arguments of [KV-only op] 实现拆解 1).

Nothing here calls the HIP path. Expected values: a hand-worked pair of heads
(tests/golden/worked_tokens.json, "q_side"), torch's float64 rms_norm and
rotation with a nearest-bf16 check written from the definition of rounding,
the identity case, and scale invariance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_rope_amd import workloads as W

RNG = np.random.default_rng(7070)


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _neighbours(bits: np.ndarray):
    """float64 values of the bf16 numbers just below and just above each
    code's value (codes ordered by value: sign-magnitude to signed integer)."""
    mag = (bits & 0x7FFF).astype(np.int64)
    key = np.where(bits & 0x8000, -mag, mag)

    def value(k):
        b = np.where(k >= 0, k, (-k) | 0x8000).astype(np.uint16)
        return _bf16_value(b)
    return value(key - 1), value(key + 1)


def _torch_reference(q_bits, positions, table, eps, apply_norm=True) -> np.ndarray:
    """float64 result before rounding: torch's rms_norm and rotation."""
    x = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double()
    if apply_norm:
        x = torch.nn.functional.rms_norm(x, (512,), eps=eps)
    cs = torch.from_numpy(table[positions]).double()[:, None, :]
    c, s = cs[..., :32], cs[..., 32:]
    y = x.clone()
    x1, x2 = x[..., 448:480], x[..., 480:]
    y[..., 448:480] = x1 * c - x2 * s
    y[..., 480:] = x2 * c + x1 * s
    return y.numpy()


def test_worked_heads(golden):
    gq = golden["q_side"]
    inp = gq["inputs"]
    q = np.zeros((1, inp["heads"], 512), np.float32)
    q[0, 0, :] = 2.0
    q[0, 1, 0] = 16.0
    table = np.zeros((inp["max_pos"], 64), np.float32)
    table[:, :32] = 1.0
    table[1, 0], table[1, 32] = 0.5, 0.75
    out = oracle.qnorm_rope(W.to_bf16_bits(q), np.array([inp["position"]], np.int64), table,
                            inp["eps"])
    for h in (0, 1):
        for d, v in gq[f"head{h}"]["elements"].items():
            assert int(out[0, h, int(d)]) == v, (h, d)
    assert (out[0, 0, 1:448] == 0x3F80).all()
    assert (out[0, 1, 1:] == 0).all()


@pytest.mark.parametrize("apply_norm", [True, False])
def test_vs_torch_float64_and_nearest_bf16(apply_norm):
    n, heads = 12, 5
    x = RNG.standard_normal((n, heads, 512)).astype(np.float32)
    x *= RNG.uniform(0.01, 50.0, (n, heads, 1)).astype(np.float32)
    x[0, 0, :] = 0.0  # an all-zero head: eps keeps the scale finite
    q = W.to_bf16_bits(x)
    table = W.rope_table(3000)
    pos = RNG.integers(0, 3000, n)
    eps = 1e-6
    got = oracle.qnorm_rope(q, pos, table, eps, apply_norm)
    y = _torch_reference(q, pos, table, eps, apply_norm)
    v = _bf16_value(got)
    down, up = _neighbours(got)
    err = np.abs(v - y)
    # nearest: no neighbouring bf16 value is closer to the float64 result
    # (the sums' order differs between torch and the oracle, hence the slack)
    slack = 1e-12 * np.abs(y) + 1e-300
    assert (err <= np.abs(down - y) + slack).all()
    assert (err <= np.abs(up - y) + slack).all()
    if apply_norm:
        # RMS of each normalised NoPE+tail row is sqrt(ms / (ms + eps)) up to
        # bf16 rounding (the rotation preserves the pair norms)
        xs = _bf16_value(q)
        ms = (xs ** 2).mean(axis=2)
        rms = np.sqrt((v ** 2).mean(axis=2))
        want = np.sqrt(ms / (ms + eps))
        assert np.allclose(rms, want, rtol=2 ** -8, atol=1e-6)


def test_identity_without_norm_at_position_zero():
    x = RNG.standard_normal((6, 3, 512)).astype(np.float32)
    q = W.to_bf16_bits(x)
    q[q == 0x8000] = 0  # -0 with a negative partner rotates to +0
    table = W.rope_table(4)
    out = oracle.qnorm_rope(q, np.zeros(6, np.int64), table, 1e-6, apply_norm=False)
    assert np.array_equal(out, q)


def test_scale_invariance():
    """RMSNorm output does not depend on a power-of-two scale of the input
    when eps is negligible."""
    x = RNG.standard_normal((4, 2, 512)).astype(np.float32)
    q = W.to_bf16_bits(x)
    table = W.rope_table(100)
    pos = RNG.integers(0, 100, 4)
    base = oracle.qnorm_rope(q, pos, table, 1e-30)
    for k in (-20, -3, 5, 40):
        qk = W.to_bf16_bits(_bf16_value(q).astype(np.float32) * np.float32(2.0 ** k))
        assert np.array_equal(oracle.qnorm_rope(qk, pos, table, 1e-30), base), k


def test_pairing_and_sign_with_exact_tables():
    """Without the norm and with a quarter-turn table row (cos 0, sin 1), the
    NeoX rotation maps (x1, x2) to (-x2, x1) exactly."""
    x = RNG.standard_normal((3, 2, 512)).astype(np.float32)
    q = W.to_bf16_bits(x)
    table = np.zeros((1, 64), np.float32)
    table[0, 32:] = 1.0
    out = oracle.qnorm_rope(q, np.zeros(3, np.int64), table, 1e-6, apply_norm=False)
    neg = (q[..., 480:] ^ 0x8000).astype(np.uint16)
    nz = (q[..., 480:] & 0x7FFF) != 0
    assert np.array_equal(out[..., 448:480][nz], neg[nz])
    assert np.array_equal(out[..., 480:], q[..., 448:480])
    assert np.array_equal(out[..., :448], q[..., :448])


def test_out_of_range_positions_leave_rows_unwritten():
    q = W.to_bf16_bits(RNG.standard_normal((4, 2, 512)).astype(np.float32))
    table = W.rope_table(10)
    pos = np.array([3, -1, 10, 9], np.int64)
    sentinel = np.full_like(q, 0x1234)
    out = oracle.qnorm_rope(q, pos, table, 1e-6, out=sentinel.copy())
    assert (out[1] == 0x1234).all() and (out[2] == 0x1234).all()
    assert not (out[0] == 0x1234).all() and not (out[3] == 0x1234).all()
