"""Pins of the oracle's elementary steps against things other than itself:
library routines, float64 brute force within textbook bounds, closed forms
and invariants.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle as O


# ---------------------------------------------------------------- bf16 ----

def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_rne_vs_torch():
    hi = np.arange(65536, dtype=np.uint32)
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF],
                    dtype=np.uint32)
    u = (hi[:, None] << 16 | lows[None, :]).reshape(-1)
    rng = np.random.default_rng(5)
    u = np.concatenate([u, rng.integers(0, 2**32, 200000, dtype=np.uint64)
                        .astype(np.uint32)])
    x = u.view(np.float32)
    ours = O.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN after the round trip
    assert np.isnan(O.bf16_to_f32(ours[nan])).all()


def test_bf16_round_trip_identity():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(bits)
    ok = ~np.isnan(f)
    assert np.array_equal(O.f32_to_bf16(f)[ok], bits[ok])


# -------------------------------------------------------------- matvec ----

@pytest.mark.parametrize("n_out,n_in", [(1, 1), (3, 7), (17, 64), (5, 688)])
def test_linear_within_gamma_n_bound(n_out, n_in):
    rng = np.random.default_rng(n_out * 1000 + n_in)
    W = O.f32_to_bf16(rng.standard_normal((n_out, n_in)).astype(np.float32))
    x = rng.standard_normal(n_in).astype(np.float32)
    y = O.linear(W, x)
    Wd = O.bf16_to_f32(W).astype(np.float64)
    u = 2.0 ** -24
    gamma = n_in * u / (1 - n_in * u)
    for i in range(n_out):
        prods = [float(Wd[i, j]) * float(x[j]) for j in range(n_in)]
        exact = math.fsum(prods)
        bound = gamma * math.fsum(abs(p) for p in prods)
        assert abs(float(y[i]) - exact) <= bound + 1e-30


def test_linear_batched_rows_match_single():
    rng = np.random.default_rng(1)
    W = O.f32_to_bf16(rng.standard_normal((9, 33)).astype(np.float32))
    X = rng.standard_normal((4, 33)).astype(np.float64)
    Y = O.linear(W, X, np.float64)
    for b in range(4):
        np.testing.assert_allclose(Y[b], O.linear(W, X[b], np.float64),
                                   rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------- RMSNorm ----

@pytest.mark.parametrize("c", [-3.0, 0.25, 1.0, 7.5])
def test_rmsnorm_constant_vector(c):
    rng = np.random.default_rng(2)
    n, eps = 64, 1e-5
    w = rng.standard_normal(n)
    y = O.rmsnorm(np.full(n, c), w, eps, np.float64)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * w, rtol=1e-14)


def test_rmsnorm_zero_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(256)
    w = rng.standard_normal(256)
    assert np.all(O.rmsnorm(np.zeros(256), w, 1e-5, np.float64) == 0)
    a = O.rmsnorm(x, w, 1e-12, np.float64)
    b = O.rmsnorm(37.0 * x, w, 1e-12, np.float64)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # unit weight: mean square of the output is mean(x^2)/(mean(x^2)+eps)
    ms = np.mean(x * x)
    y = O.rmsnorm(x, np.ones(256), 0.1, np.float64)
    assert abs(np.mean(y * y) - ms / (ms + 0.1)) < 1e-12


# ---------------------------------------------------------------- RoPE ----

def test_rope_matches_complex_exponential():
    rng = np.random.default_rng(4)
    hd, theta = 64, 10000.0
    u = rng.standard_normal((3, hd))
    for p in (0, 1, 5, 511, 4095):
        c, s = O.rope_cos_sin(p, hd, theta)
        y = O.rope(u, c, s, np.float64)
        i = np.arange(hd // 2)
        ang = p * theta ** (-2.0 * i / hd)
        z = (u[:, :hd // 2] + 1j * u[:, hd // 2:]) * np.exp(1j * ang)
        ref = np.concatenate([z.real, z.imag], axis=-1)
        # cos/sin tables are float32-rounded: error <= |u| * 2^-24 * few
        np.testing.assert_allclose(y, ref, atol=1e-6 * np.abs(u).max())


def test_rope_norm_identity_relative_inverse():
    rng = np.random.default_rng(6)
    hd, theta = 128, 500000.0
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    c0, s0 = O.rope_cos_sin(0, hd, theta)
    assert np.array_equal(O.rope(q, c0, s0, np.float64), q)
    for p in (1, 17, 1023):
        c, s = O.rope_cos_sin(p, hd, theta)
        y = O.rope(q, c, s, np.float64)
        assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-6
        cn, sn = O.rope_cos_sin(-p, hd, theta)
        np.testing.assert_allclose(O.rope(y, cn, sn, np.float64), q, atol=1e-6)
    # <R_m q, R_n k> depends only on m - n
    def rot(v, p):
        c, s = O.rope_cos_sin(p, hd, theta)
        return O.rope(v, c, s, np.float64)
    a = rot(q, 40) @ rot(k, 30)
    b = rot(q, 10) @ rot(k, 0)
    assert abs(a - b) < 1e-5


# ----------------------------------------------------------- attention ----

def _attn_bruteforce(q, K, V):
    G, hd = q.shape
    out = np.zeros((G, V.shape[1]))
    for g in range(G):
        s = [math.fsum(float(q[g, d]) * float(K[t, d]) for d in range(hd))
             / math.sqrt(hd) for t in range(len(K))]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = math.fsum(e)
        for d in range(V.shape[1]):
            out[g, d] = math.fsum(e[t] * float(V[t, d]) for t in range(len(K))) / z
    return out


def test_attention_vs_bruteforce():
    rng = np.random.default_rng(7)
    q, K, V = rng.standard_normal((4, 16)), rng.standard_normal((9, 16)), \
        rng.standard_normal((9, 16))
    np.testing.assert_allclose(O.attention(q, K, V, np.float64),
                               _attn_bruteforce(q, K, V), rtol=1e-12, atol=1e-13)


def test_attention_single_key_and_identical_keys():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 64)) * 10
    K1, V1 = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    np.testing.assert_allclose(O.attention(q, K1, V1, np.float64),
                               np.repeat(V1, 4, axis=0), rtol=1e-14)
    K = np.repeat(rng.standard_normal((1, 64)), 13, axis=0)
    V = rng.standard_normal((13, 64))
    np.testing.assert_allclose(O.attention(q, K, V, np.float64),
                               np.repeat(V.mean(0, keepdims=True), 4, axis=0),
                               rtol=1e-12, atol=1e-14)


def test_attention_weights_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(9)
    q, K = rng.standard_normal((2, 32)), rng.standard_normal((50, 32))
    ones = np.ones((50, 32))
    np.testing.assert_allclose(O.attention(q, K, ones, np.float64), 1.0,
                               rtol=1e-13)
    # shifting every key along a direction orthogonal... adds the same score
    # to all keys of a query: K + t*q/|q|^2 shifts row g's scores by t/sqrt(hd)
    V = rng.standard_normal((50, 32))
    for g in range(2):
        Ks = K + 3.0 * q[g] / (q[g] @ q[g])
        np.testing.assert_allclose(O.attention(q[g:g + 1], Ks, V, np.float64),
                                   O.attention(q[g:g + 1], K, V, np.float64),
                                   rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("cuts", [[0, 100], [0, 1, 100], [0, 0, 37, 37, 99, 100],
                                  [0, 50, 50, 100]])
def test_split_lse_combine_equals_plain(cuts):
    rng = np.random.default_rng(10)
    q = rng.standard_normal((4, 64))
    K, V = rng.standard_normal((100, 64)), rng.standard_normal((100, 64))
    parts = [O.attention_partial(q, K[a:b], V[a:b], np.float64)
             for a, b in zip(cuts[:-1], cuts[1:])]
    np.testing.assert_allclose(O.attention_combine(parts, np.float64),
                               O.attention(q, K, V, np.float64),
                               rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- SiLU ----

def test_silu_identities_and_library():
    from scipy.special import expit
    x = np.linspace(-30, 30, 2001)
    y = O.silu(x, np.float64)
    assert O.silu(np.zeros(1), np.float64)[0] == 0.0
    np.testing.assert_allclose(y - O.silu(-x, np.float64), x, atol=1e-12)
    np.testing.assert_allclose(y, x * expit(x), rtol=1e-13, atol=1e-300)
