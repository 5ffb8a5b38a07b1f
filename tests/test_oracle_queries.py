"""Pins of the oracle's index-query preparation (QSA page: q_layernorm then
apply_qsa_rope at the query's own token) against library routines, a
hand-derived closed form and invariants."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _rope_complex(u, cos, sin):
    """Half-split rotation as complex multiplication (independent formulation)."""
    half = cos.shape[-1]
    z = (u[..., :half] + 1j * u[..., half:2 * half]) * (cos + 1j * sin)
    out = u.copy()
    out[..., :half] = z.real
    out[..., half:2 * half] = z.imag
    return out


@pytest.mark.parametrize("d_rope", [128, 64, 16, 6])
def test_equals_torch_rmsnorm_then_complex_rope(d_rope):
    rng = np.random.default_rng(31 + d_rope)
    B, S, H, D = 2, 23, 3, 128
    q = rng.standard_normal((B, S, H, D)) * rng.uniform(0.1, 5.0, (B, S, H, 1))
    gamma = rng.uniform(0.5, 1.5, D)
    cu = np.array([0, 7, 23], dtype=np.int32)
    pos = np.stack([synth.doc_positions(1, S, cu, None)[0], np.arange(S)])
    freqs = synth.rope_table(pos, d_rope).astype(np.float64)
    got = oracle.prepare_index_queries(q, gamma, freqs, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(q), (D,), torch.from_numpy(gamma), 1e-5).numpy()
    half = d_rope // 2
    ref = _rope_complex(ref, freqs[:, :, None, :half], freqs[:, :, None, half:])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_hand_derived_quarter_and_half_turns():
    """x = (1, 2, 3, 4), eps = 0, gamma = 1: u = x / sqrt(7.5).  A quarter turn
    on pair (0, 2) gives (-u2, u0); a half turn on pair (1, 3) gives (-u1, -u3)."""
    q = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 1, 4)
    freqs = np.array([math.cos(math.pi / 2), math.cos(math.pi), math.sin(math.pi / 2), math.sin(math.pi)]).reshape(1, 1, 4)
    got = oracle.prepare_index_queries(q, np.ones(4), freqs, 0.0)
    want = np.array([-3.0, -2.0, 1.0, -4.0]) / math.sqrt(7.5)
    np.testing.assert_allclose(got.reshape(4), want, rtol=1e-14, atol=1e-15)


def _table64(S, R, theta=10000.0):
    """cat(cos, sin) rows in float64 (cos^2 + sin^2 = 1 to rounding)."""
    ang = np.arange(S)[:, None] * theta ** (-np.arange(R // 2) * 2.0 / R)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=-1)[None]


def test_rotation_preserves_norm_and_position_zero_is_plain_rmsnorm():
    rng = np.random.default_rng(8)
    B, S, H, D = 1, 40, 4, 64
    q = rng.standard_normal((B, S, H, D))
    gamma = rng.uniform(0.5, 1.5, D)
    freqs = _table64(S, D)
    got = oracle.prepare_index_queries(q, gamma, freqs, 1e-5)
    plain = oracle.prepare_index_queries(q, gamma, freqs, 1e-5, d_rope=0)
    np.testing.assert_allclose(np.sum(got ** 2, axis=-1), np.sum(plain ** 2, axis=-1), rtol=1e-12)
    np.testing.assert_allclose(got[:, 0], plain[:, 0], rtol=1e-14, atol=1e-15)
    # pairs rotate independently: the pair norms match too
    h = D // 2
    np.testing.assert_allclose(got[..., :h] ** 2 + got[..., h:] ** 2, plain[..., :h] ** 2 + plain[..., h:] ** 2,
                               rtol=1e-12, atol=1e-14)


def test_partial_rotary_width_leaves_upper_dims():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 5, 2, 32))
    freqs = synth.rope_table(np.arange(5)[None], 8).astype(np.float64)
    got = oracle.prepare_index_queries(q, np.ones(32), freqs, 1e-5)
    plain = oracle.prepare_index_queries(q, np.ones(32), freqs, 1e-5, d_rope=0)
    np.testing.assert_array_equal(got[..., 8:], plain[..., 8:])
