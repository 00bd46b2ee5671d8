"""CPU pin of the numerics of the diagonal-block inverse in the prefill kernels.

Each 16-token diagonal block needs (I + N)^-1, N = StrictTril(Diag(beta) K K^T)
on decay-referenced keys ("Glossaire", entries "Chunkwise" and "UT").  The
kernels form it on bf16 matrix-core operands with fp32 accumulation.  This test
emulates, in numpy, the rounding points of two ways of doing that:

  product form:   (I - N)(I + N^2)(I + N^4)(I + N^8), every factor rounded to
                  bf16 before it enters a product (the first design);
  recursive form: D_2b = D_b - D_b F_b D_b for b = 1, 2, 4, 8, F_b the
                  off-diagonal b x b blocks of N, the operands D_b and F_b D_b
                  rounded to bf16, D kept in fp32 (the kernels' design);

and checks them against the exact inverse in fp64, on keys that share a
direction within the block (repeated or similar tokens), with beta near 1 and
no decay, where |N| is close to 1 and the powers of N grow like 2^k before
they cancel.  The recursive form must stay within a few bf16 roundings; the
product form fails there, which is why the kernels do not use it.  No GPU and
no kernel code: a statement about the arithmetic the kernels were designed on.
"""
import numpy as np
import pytest


def bf16(x):
    """Round float32 values to the nearest bf16 (ties to even), as float32."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def product_form(N):
    I = np.eye(16, dtype=np.float32)
    n = bf16(N)
    n2 = bf16(f32(n @ n))
    n4 = bf16(f32(n2 @ n2))
    X = f32(n4 @ n4) + I                       # I + N^8
    X = f32(n4 @ bf16(X)) + X                  # (I + N^4)(I + N^8)
    X = f32(n2 @ bf16(X)) + X
    X = f32(bf16(-n) @ bf16(X)) + X
    return bf16(X)


def recursive_form(N):
    n = bf16(N)
    D = np.eye(16, dtype=np.float32)
    b = 1
    while b < 16:
        mask = np.zeros((16, 16), dtype=bool)
        for s in range(0, 16, 2 * b):
            mask[s + b:s + 2 * b, s:s + b] = True
        F = np.where(mask, n, 0).astype(np.float32)
        Dr = bf16(D)
        X = bf16(f32(F @ Dr))
        D = f32(D - f32(Dr @ X))
        b *= 2
    return bf16(D)


def correlated_block(rng, d, eps, beta_lo):
    base = rng.standard_normal(d)
    base /= np.linalg.norm(base)
    k = base[None, :] + eps * rng.standard_normal((16, d)) / np.sqrt(d)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    k = bf16(k).astype(np.float64)               # the kernels read bf16 keys
    beta = rng.uniform(beta_lo, 1.0, 16)
    return np.tril(beta[:, None] * (k @ k.T), -1)


def rel_err(T, N):
    exact = np.linalg.inv(np.eye(16) + N)
    return float(np.max(np.abs(T.astype(np.float64) - exact)) / np.max(np.abs(exact)))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("eps", [0.05, 0.2])
def test_recursive_inverse_holds_on_correlated_keys(d, eps):
    rng = np.random.default_rng(1000 + d + int(100 * eps))
    worst = 0.0
    for _ in range(20):
        N = correlated_block(rng, d, eps, 0.8)
        worst = max(worst, rel_err(recursive_form(N), N))
    # a few bf16 roundings of the inverse's own entries (2^-9 each): 6.5e-3
    # measured for every case here
    assert worst <= 1e-2, worst


def test_product_form_fails_on_correlated_keys():
    rng = np.random.default_rng(7)
    errs = [rel_err(product_form(N), N) for N in (correlated_block(rng, 128, 0.05, 0.95)
                                                   for _ in range(10))]
    assert max(errs) > 0.5, errs


def test_both_forms_agree_on_independent_keys():
    """With independent random unit keys |N| ~ 1/sqrt(d): both forms are fine,
    which is why tests with such keys alone could not tell them apart."""
    rng = np.random.default_rng(11)
    for _ in range(10):
        k = rng.standard_normal((16, 128))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        k = bf16(k).astype(np.float64)
        N = np.tril(rng.uniform(0, 1, 16)[:, None] * (k @ k.T), -1)
        assert rel_err(recursive_form(N), N) <= 4e-3
        assert rel_err(product_form(N), N) <= 4e-3
