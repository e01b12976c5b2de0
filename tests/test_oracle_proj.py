"""Pins for the oracle's QKV projection and its composition with QK-norm, RoPE
and the head exchange (CPU only).

The projection is tied to a library special case (numpy's float64 matmul of
x by the transposed weight) and to one-hot rows that read back single weight
columns.  The composition is tied to identity-block weights, under which the
projection hands x itself to the already pinned norm + RoPE + scatter, so a
wrong q/k/v column split, head order or weight assignment shows up there.
"""
import numpy as np
import pytest

from sequence_attention_ulysses_amd import synth


def test_linear_matches_numpy_matmul(orc):
    rng = np.random.default_rng(0)
    for M, N, K in [(1, 1, 1), (3, 5, 7), (17, 40, 64), (64, 96, 128)]:
        x = rng.standard_normal((M, K))
        w = rng.standard_normal((N, K))
        np.testing.assert_allclose(orc.linear(x, w), x @ w.T, rtol=1e-12, atol=1e-12)


def test_linear_one_hot_rows_read_weight_columns(orc):
    """x[m] = e_{k(m)} gives y[m, n] = w[n, k(m)] exactly: pins which operand is transposed."""
    rng = np.random.default_rng(1)
    M, N, K = 11, 6, 9
    ks = rng.integers(0, K, size=M)
    x = np.zeros((M, K))
    x[np.arange(M), ks] = 1.0
    w = rng.standard_normal((N, K))
    y = orc.linear(x, w)
    for m in range(M):
        np.testing.assert_array_equal(y[m], w[:, ks[m]])


def _bits16(t):
    return synth.bits(t)


@pytest.mark.parametrize("P,B,S_l,Hq,Hkv,D,dtype", [(2, 1, 6, 4, 2, 8, "bf16"), (4, 2, 3, 8, 4, 16, "f16"),
                                                   (1, 1, 5, 2, 2, 4, "bf16")])
def test_identity_block_weights_reduce_to_norm_rope_scatter(orc, P, B, S_l, Hq, Hkv, D, dtype):
    """W = [I; I_k; 2 I_v] over hidden = Hq*D: q is x itself, k the first Hkv heads of x,
    v twice those heads; each then follows the separately pinned path."""
    hidden = Hq * D
    x = synth.normal((P, B, S_l, hidden), dtype, 5)
    x_bits = _bits16(x)
    eye = np.eye(hidden)
    w = np.concatenate([eye, eye[:Hkv * D], 2.0 * eye[:Hkv * D]], axis=0)
    w_bits = _bits16(__import__("torch").from_numpy(w).to(synth.DTYPES[dtype]))
    wq = _bits16(synth.norm_weight(D, dtype, 6))
    wk = _bits16(synth.norm_weight(D, dtype, 7))
    cos, sin = orc.rope_table_1d(P * S_l, D)
    yq, yk, yv = orc.qkv_proj_norm_rope_scatter(x_bits, dtype, w_bits, Hq, Hkv, wq, wk, 1e-6, cos, sin)
    xh = x_bits.reshape(P, B, S_l, Hq, D)
    np.testing.assert_allclose(yq, orc.fused_norm_rope_scatter(xh, dtype, wq, 1e-6, cos, sin), rtol=0, atol=1e-12)
    xk = np.ascontiguousarray(xh[:, :, :, :Hkv])
    np.testing.assert_allclose(yk, orc.fused_norm_rope_scatter(xk, dtype, wk, 1e-6, cos, sin), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(yv, 2.0 * orc.scatter(orc.widen(xk, dtype)))
    # the same weights with q and k norm weights swapped must change q (asymmetric weights)
    yq2, _, _ = orc.qkv_proj_norm_rope_scatter(x_bits, dtype, w_bits, Hq, Hkv, wk, wq, 1e-6, cos, sin)
    assert np.abs(yq2 - yq).max() > 1e-3


def test_rows_entry_matches_full_composition(orc):
    """The per-row form (used for sampled checks) agrees with the full composition."""
    P, B, S_l, Hq, Hkv, D = 2, 1, 5, 4, 2, 8
    hidden = 16
    x_bits = _bits16(synth.normal((P, B, S_l, hidden), "bf16", 8))
    w_bits = _bits16(synth.normal(((Hq + 2 * Hkv) * D, hidden), "bf16", 9, std=0.25))
    wq = _bits16(synth.norm_weight(D, "bf16", 10))
    wk = _bits16(synth.norm_weight(D, "bf16", 11))
    cos, sin = orc.rope_table_1d(P * S_l, D)
    yq, yk, yv = orc.qkv_proj_norm_rope_scatter(x_bits, "bf16", w_bits, Hq, Hkv, wq, wk, 1e-6, cos, sin)
    # token s of rank r sits at global row r*S_l + s of rank q's band
    r, s = 1, 3
    q, k, v = orc.qkv_proj_norm_rope_rows(x_bits[r, 0, s][None], "bf16", w_bits, Hq, Hkv, D, wq, wk, 1e-6,
                                          cos, sin, np.array([r * S_l + s]))
    Hl, Hkl = Hq // P, Hkv // P
    for h in range(Hq):
        np.testing.assert_array_equal(yq[h // Hl, 0, r * S_l + s, h % Hl], q[0, h])
    for h in range(Hkv):
        np.testing.assert_array_equal(yk[h // Hkl, 0, r * S_l + s, h % Hkl], k[0, h])
        np.testing.assert_array_equal(yv[h // Hkl, 0, r * S_l + s, h % Hkl], v[0, h])
