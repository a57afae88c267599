"""The arithmetic arguments behind the K/V parity tolerances, checked on the
CPU.  Batch 1: the GPU and the oracle add the same fp32 products in
different orders.  Batched: each fp32 activation x enters the matrix cores
as two bf16 terms,
hi = bf16(x) and lo = bf16(x - hi) (round to nearest even, the bf16
multi-term split of Henry, Tang and Heinecke, 2019).

* x - hi is exact in fp32 and |x - hi - lo| <= 2^-16 |x| (two roundings to
  8 significant bits) for every x whose lo is not subnormal in bf16;
* a K-term projection on hi + lo therefore moves by at most
  2^-16 sum |w_i x_i| (hard bound), which for random signs is about
  2^-16 sqrt(K) times the RMS of the outputs: the batched K/V parity bar
  takes twice that."""
import numpy as np
import pytest

import oracle as O


def _bf16(x):
    return O.bf16_to_f32(O.f32_to_bf16(np.asarray(x, np.float32)))


def _split(x):
    x = np.asarray(x, np.float32)
    hi = _bf16(x)
    r = (x - hi).astype(np.float32)
    lo = _bf16(r)
    return hi, r, lo


def test_split_residual_is_exact_and_bounded():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-60, 60, 200_000))).astype(np.float32)
    # exact bf16 values, halfway cases between neighbours, and their negatives
    b = O.bf16_to_f32(np.arange(0x0080, 0x7F00, 7, dtype=np.uint16))
    half = (b.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, b, half, -b, -half]).astype(np.float32)
    hi, r, lo = _split(x)
    # x - hi in fp32 equals the exact difference
    assert np.array_equal(r.astype(np.float64), x.astype(np.float64) - hi.astype(np.float64))
    err = np.abs(x.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64))
    # from |x| >= 2^-100 on, a nonzero residual (a multiple of x's fp32 ulp,
    # at least 2^-123) is a normal number, and the bound holds
    big = np.abs(x) >= 2.0 ** -100
    assert big.sum() > 200_000
    assert np.all(err[big] <= 2.0 ** -16 * np.abs(x[big].astype(np.float64)))
    # below it, lo may be subnormal or zero: the error stays below 2^-126
    assert np.all(err[~big] < 2.0 ** -126)
    assert np.all(lo[np.isin(x, b)] == 0)          # a bf16 value splits exactly


@pytest.mark.parametrize("K", [256, 2048, 8192])
def test_projection_error_within_the_parity_bar(K):
    rng = np.random.default_rng(K)
    W = _bf16(rng.standard_normal((512, K)).astype(np.float32) * 0.02).astype(np.float64)
    x = rng.standard_normal(K).astype(np.float32)
    hi, _, lo = _split(x)
    y = W @ x.astype(np.float64)
    ys = W @ hi.astype(np.float64) + W @ lo.astype(np.float64)
    d = np.abs(ys - y)
    assert np.all(d <= 2.0 ** -16 * (np.abs(W) @ np.abs(x.astype(np.float64))))   # hard bound
    rms = np.sqrt(np.mean(y * y))
    assert d.max() <= 2 * 2.0 ** -16 * np.sqrt(K) * rms                        # the parity bar


def _fp32_seq(W, x):
    """Row sums accumulated in fp32 one product after another."""
    acc = np.zeros(W.shape[0], np.float32)
    for k in range(W.shape[1]):
        acc = (acc + (W[:, k] * x[k]).astype(np.float32)).astype(np.float32)
    return acc


def _fp32_lanes(W, x, lanes=64):
    """The same sums in a GEMV kernel's order: lane l accumulates products
    l, l + 64, ... in fp32, then the 64 partials are added pairwise."""
    K = W.shape[1]
    p = np.zeros((W.shape[0], lanes), np.float32)
    for k0 in range(0, K, lanes):
        blk = (W[:, k0:k0 + lanes] * x[k0:k0 + lanes]).astype(np.float32)
        p[:, :blk.shape[1]] = (p[:, :blk.shape[1]] + blk).astype(np.float32)
    while p.shape[1] > 1:
        h = p.shape[1] // 2
        p = (p[:, :h] + p[:, h:]).astype(np.float32)
    return p[:, 0]


@pytest.mark.parametrize("K", [256, 2048])
def test_fp32_summation_orders_within_the_batch1_bar(K):
    """The batch-1 K/V bar's slack, 2^-20 sqrt(K) times the outputs' RMS,
    covers two fp32 summation orders of the same products (about
    2^-24 sqrt(K) RMS apart for random signs)."""
    rng = np.random.default_rng(K + 1)
    W = _bf16(rng.standard_normal((256, K)).astype(np.float32) * 0.02)
    x = rng.standard_normal(K).astype(np.float32)
    a, b = _fp32_seq(W, x), _fp32_lanes(W, x)
    y = W.astype(np.float64) @ x.astype(np.float64)
    rms = np.sqrt(np.mean(y * y))
    d = np.abs(a.astype(np.float64) - b.astype(np.float64))
    assert d.max() > 0                                   # the orders do differ
    assert d.max() <= 2.0 ** -20 * np.sqrt(K) * rms
