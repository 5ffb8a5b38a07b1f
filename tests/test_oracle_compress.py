"""Pins of the oracle's key compression against library routines and invariants."""
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


@pytest.mark.parametrize("d_rope", [64, 32])
def test_c1_is_token_rmsnorm_plus_rope(d_rope):
    rng = np.random.default_rng(5)
    S, D = 37, 64
    kI = rng.standard_normal((1, S, D))
    gamma = rng.uniform(0.5, 1.5, D)
    pos = np.arange(S)[None]
    freqs = synth.rope_table(pos, d_rope).astype(np.float64)
    kc, _ = oracle.compress_keys(kI, gamma, 1e-5, freqs, 1)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(kI[0]), (D,), torch.from_numpy(gamma), 1e-5).numpy()
    half = d_rope // 2
    ref = _rope_complex(ref, freqs[0, :, :half], freqs[0, :, half:])
    np.testing.assert_allclose(kc[0], ref, rtol=1e-12, atol=1e-12)


def test_first_block_of_each_document_is_normalised_mean():
    rng = np.random.default_rng(6)
    cu = np.array([0, 13, 14, 40, 61], dtype=np.int32)
    S, D, c = 64, 32, 4
    kI = rng.standard_normal((1, S, D))
    pos = synth.doc_positions(1, S, cu, None)
    freqs = synth.rope_table(pos, D).astype(np.float64)
    kc, cu_blocks = oracle.compress_keys(kI, np.ones(D), 1e-5, freqs, c, cu_seqlens=cu)
    lens = np.diff(cu)
    assert cu_blocks.tolist() == [0] + np.cumsum(lens // c).tolist()
    for d in range(len(lens)):
        if lens[d] < c:
            continue
        m = torch.from_numpy(kI[0, cu[d]:cu[d] + c].mean(axis=0))
        ref = torch.nn.functional.rms_norm(m, (D,), None, 1e-5).numpy()
        np.testing.assert_allclose(kc[0, cu_blocks[d]], ref, rtol=1e-12, atol=1e-12)


def test_packed_equals_each_document_alone():
    rng = np.random.default_rng(7)
    cu = np.array([0, 9, 30, 31, 57], dtype=np.int32)
    S, D, c = 60, 16, 3
    kI = rng.standard_normal((1, S, D))
    gamma = rng.uniform(0.5, 1.5, D)
    pos = synth.doc_positions(1, S, cu, None)
    freqs = synth.rope_table(pos, D).astype(np.float64)
    kc, cu_blocks = oracle.compress_keys(kI, gamma, 1e-5, freqs, c, cu_seqlens=cu)
    for d in range(len(cu) - 1):
        a, e = cu[d], cu[d + 1]
        alone, _ = oracle.compress_keys(kI[:, a:e], gamma, 1e-5, freqs[:, a:e], c)
        n = (e - a) // c
        np.testing.assert_array_equal(kc[0, cu_blocks[d]:cu_blocks[d] + n], alone[0, :n])
    # slots past the last block stay zero
    assert np.all(kc[0, cu_blocks[-1]:] == 0)


def test_rotation_preserves_pair_norms_and_mean_of_repeated_rows():
    rng = np.random.default_rng(8)
    S, D, c = 40, 16, 4
    base = rng.standard_normal((S // c, D))
    kI = np.repeat(base, c, axis=0)[None]          # every group = c copies of one row
    ang = np.arange(S)[None, :, None] * (10000.0 ** (-np.arange(D // 2) * 2.0 / D))
    freqs = np.concatenate([np.cos(ang), np.sin(ang)], axis=-1)     # exact fp64 table
    kc, _ = oracle.compress_keys(kI, np.ones(D), 0.0, freqs, c)
    unrot = base / np.sqrt(np.mean(base ** 2, axis=1, keepdims=True))
    h = D // 2
    pn = lambda x: x[:, :h] ** 2 + x[:, h:] ** 2
    np.testing.assert_allclose(pn(kc[0]), pn(unrot), rtol=1e-12)


def test_right_padded_rows():
    rng = np.random.default_rng(9)
    B, S, D, c = 3, 20, 8, 4
    kI = rng.standard_normal((B, S, D))
    lens = np.array([20, 7, 0])
    freqs = synth.rope_table(synth.doc_positions(B, S, None, lens), D).astype(np.float64)
    kc, _ = oracle.compress_keys(kI, np.ones(D), 1e-5, freqs, c, row_lens=lens)
    full, _ = oracle.compress_keys(kI[1:2, :7], np.ones(D), 1e-5, freqs[1:2, :7], c)
    np.testing.assert_array_equal(kc[1, :1], full[0, :1])
    assert np.all(kc[1, 1:] == 0) and np.all(kc[2] == 0)
