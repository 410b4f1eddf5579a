"""Pins for the float64 oracle: checks against facts that do not come from it.

Each ``pin_*`` takes an oracle-like namespace ``O`` (the real ``oracle``
package, or a deliberately broken variant built in the tests) and raises
``AssertionError`` when ``O`` disagrees with:
* exact rational arithmetic (``fractions.Fraction`` triple loops),
* the pages' printed worked example,
* hand-derived closed forms stored under ``tests/golden`` with citations,
* library routines on special cases where they compute the same thing,
* mathematical invariants (symmetry, positive semi-definiteness).
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _frac_gram(rows):
    """Exact Gram by a triple loop written here, independent of the oracle."""
    d = len(rows[0])
    S = [[Fraction(0)] * d for _ in range(d)]
    for r in rows:
        fr = [Fraction(float(v)) for v in r]
        for i in range(d):
            for j in range(d):
                S[i][j] += fr[i] * fr[j]
    return S


def pin_bruteforce_fraction(O, seed=11):
    """Accumulated S over several tiny batches equals the exact rational sum."""
    rng = np.random.default_rng(seed)
    d = 5
    sizes = [3, 0, 4, 1]
    batches = [rng.standard_normal((n, d)).astype(np.float32) for n in sizes]
    acc = O.GramAccumulator(d)
    for b in batches:
        acc.add_batch(b, "f32")
    rows = [r for b in batches for r in b.tolist()]
    S_exact = _frac_gram(rows)
    assert acc.N == sum(sizes), f"token count {acc.N} != {sum(sizes)}"
    for i in range(d):
        for j in range(d):
            ref = float(S_exact[i][j])
            assert abs(acc.S[i, j] - ref) <= 1e-14 * max(1.0, abs(ref)), (i, j, acc.S[i, j], ref)
    # the scaled Hessian, exactly: H = 2/N S
    H, dead, damp = acc.materialize(0.0, neutralize=False)
    for i in range(d):
        for j in range(d):
            ref = float(Fraction(2, acc.N) * S_exact[i][j])
            assert abs(H[i, j] - ref) <= 1e-14 * max(1.0, abs(ref))
    assert damp == 0.0 and not dead.any()


def pin_orientation_hand(O):
    g = _load("orientation_hand.json")
    X = np.asarray(g["X"], dtype=np.float32)
    acc = O.GramAccumulator(X.shape[1])
    acc.add_batch(X, "f32")
    assert acc.S.shape == (2, 2)
    assert np.array_equal(acc.S, np.asarray(g["expected_S"], dtype=np.float64))
    assert acc.N == g["expected_N"]
    H, _, _ = acc.materialize(0.0, neutralize=False)
    assert np.allclose(3.0 * H, np.asarray(g["expected_H_times_3"], dtype=np.float64), rtol=0, atol=1e-13)


def pin_worked_example(O):
    """The pages' printed fp32-vs-bf16 staging example, to the last bit."""
    g = _load("worked_example_staging.json")
    x = np.asarray(g["tokens"], dtype=np.float32)
    acc = O.GramAccumulator(1)
    acc.add_batch(x, "f32")
    H, _, _ = acc.materialize(0.0, neutralize=False)
    assert float(np.float32(H[0, 0])) == g["expected_diag_f32_input"]
    assert H[0, 0] == g["expected_diag_f32_input"]  # exact in float32 and float64
    acc = O.GramAccumulator(1)
    acc.add_batch(W.to_bf16_bits(x), "bf16")
    H, _, _ = acc.materialize(0.0, neutralize=False)
    assert H[0, 0] == g["expected_diag_bf16_input"]


def pin_worked_example_f16_staging(O):
    """The same example with fp16 activations and the staging type chosen per accumulator."""
    g = _load("worked_example_staging.json")
    f = g["f16_staging"]
    x = np.asarray(g["tokens"], dtype=np.float16)
    assert float(x[0, 0]) == g["tokens"][0][0]  # exact in fp16
    for staging, want in (("f32", f["expected_diag_f32_staging"]), (None, f["expected_diag_f32_staging"]),
                          ("bf16", f["expected_diag_bf16_staging"])):
        acc = O.GramAccumulator(1, staging=staging)
        acc.add_batch(x, "f16")
        H, _, _ = acc.materialize(0.0, neutralize=False)
        assert H[0, 0] == want, (staging, H[0, 0])


def _bf16_by_bits(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 by integer arithmetic on the bit
    patterns (drop the low 16 bits, round half to even; NaN kept NaN), a
    second derivation independent of the oracle's."""
    u = x32.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    hi = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((hi & 1) == 1))
    hi = hi + up.astype(np.uint64)
    out = (hi << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    out[np.isnan(x32)] = np.nan
    return out


def pin_bf16_rounding(O, seed=11):
    """Rounding to bf16 agrees with torch's CPU conversion and with an integer derivation on
    random bit patterns (all exponents, subnormals, ties, overflow), and with hand values."""
    import torch
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near_max = np.uint32(0x7F7F0000) + rng.integers(0, 2 ** 16, size=2_000, dtype=np.uint64).astype(np.uint32)
    x32 = np.concatenate([bits, ties, near_max, np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000,
                                                           0x00018000, 0x80000000], dtype=np.uint32)]).view(np.float32)
    got = O.round_to_bf16(x32.astype(np.float64))
    ref_t = torch.from_numpy(x32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    ref_b = _bf16_by_bits(x32)
    for ref in (ref_t, ref_b):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # hand values: ties go to the even significand; fp16's largest value rounds up to 2^16
    hand = {1 + 2.0 ** -8: 1.0, 1 + 3 * 2.0 ** -8: 1 + 2.0 ** -6, 1 + 2.0 ** -7: 1 + 2.0 ** -7,
            65504.0: 65536.0, -(1 + 2.0 ** -10): -1.0, 2.0 ** -134: 0.0}
    for v, want in hand.items():
        assert O.round_to_bf16(np.array([v]))[0] == want, (v, want)
    # staged values of every fp16 bit pattern: fp32 staging keeps them, bf16 staging rounds them
    h = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16).view(np.float16).reshape(1, -1)
    f32 = O.staged_values(h, "f16", "f32")
    exact = h.astype(np.float32)
    fin = np.isfinite(exact)
    assert np.array_equal(f32[fin], exact[fin].astype(np.float64))
    b = O.staged_values(h, "f16", "bf16")
    rb = torch.from_numpy(exact.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(b[fin], rb[fin])


def pin_neutralize_damp_hand(O):
    g = _load("neutralize_damp_hand.json")
    X = np.asarray(g["X"], dtype=np.float32)
    acc = O.GramAccumulator(X.shape[1])
    acc.add_batch(X, "f32")
    H, dead, damp = acc.materialize(g["damp_percent"])
    assert np.allclose(np.diag(H), g["expected_diag"], rtol=0, atol=1e-15)
    assert np.array_equal(dead, np.asarray(g["expected_dead"]))
    assert abs(damp - g["expected_damp"]) <= 1e-17
    off = H - np.diag(np.diag(H))
    assert not off.any()
    e = g["empty_accumulator"]
    acc = O.GramAccumulator(e["d"])
    acc.add_batch(np.zeros((0, e["d"]), dtype=np.float32), "f32")
    H, dead, damp = acc.materialize(e["damp_percent"])
    assert acc.N == 0
    assert np.allclose(np.diag(H), e["expected_diag"], rtol=0, atol=1e-15)
    assert dead.all() and abs(damp - e["expected_damp"]) <= 1e-17
    assert not (H - np.diag(np.diag(H))).any()


def pin_multi_batch_is_concatenation(O, seed=3):
    """Batches accumulate like one concatenated batch; N counts tokens."""
    rng = np.random.default_rng(seed)
    d = 7
    sizes = [5, 1, 0, 9, 2]
    batches = [rng.standard_normal((n, d)).astype(np.float32) for n in sizes]
    a = O.GramAccumulator(d)
    for b in batches:
        a.add_batch(b, "f32")
    c = O.GramAccumulator(d)
    c.add_batch(np.concatenate(batches, axis=0), "f32")
    assert a.N == c.N == sum(sizes)
    assert np.allclose(a.S, c.S, rtol=1e-14, atol=1e-14)
    Ha, _, _ = a.materialize(0.01)
    Hc, _, _ = c.materialize(0.01)
    assert np.allclose(Ha, Hc, rtol=1e-14, atol=1e-14)


def pin_empty_batch_noop(O, seed=4):
    rng = np.random.default_rng(seed)
    d = 6
    a = O.GramAccumulator(d)
    a.add_batch(rng.standard_normal((4, d)).astype(np.float32), "f32")
    S0, N0 = a.S.copy(), a.N
    a.add_batch(np.zeros((0, d), dtype=np.float32), "f32")
    a.add_batch(np.zeros((0, d), dtype=np.uint16), "bf16")
    assert a.N == N0 and np.array_equal(a.S, S0)


def pin_covariance_special_case(O, seed=5):
    """For zero-mean columns, 2/N X^T X is twice numpy's biased covariance."""
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal((50, 6)).astype(np.float32)
    X = np.concatenate([Y, -Y], axis=0)  # every column sums to exactly zero
    a = O.GramAccumulator(6)
    a.add_batch(X, "f32")
    H, _, _ = a.materialize(0.0, neutralize=False)
    ref = 2.0 * np.cov(X.astype(np.float64), rowvar=False, bias=True)
    assert np.allclose(H, ref, rtol=1e-12, atol=1e-12)


def pin_symmetric_psd_cholesky(O, seed=6):
    rng = np.random.default_rng(seed)
    d = 24
    a = O.GramAccumulator(d)
    for n in (3, 8, 5):  # N = 16 < d: rank-deficient before damping
        a.add_batch(rng.standard_normal((n, d)).astype(np.float32), "f32")
    H, _, damp = a.materialize(0.0, neutralize=False)
    assert np.array_equal(H, H.T)
    w = np.linalg.eigvalsh(H)
    assert w.min() >= -1e-12 * np.trace(H)
    Hd, _, damp = a.materialize(0.01)
    assert damp > 0
    np.linalg.cholesky(Hd)  # raises if the damped Hessian is not positive definite


def pin_unit_variance_diagonal(O, seed=7):
    """N(0,1) inputs give a diagonal close to 2 (E[2/N sum x^2] = 2)."""
    rng = np.random.default_rng(seed)
    d, n = 8, 100_000
    a = O.GramAccumulator(d)
    a.add_batch(rng.standard_normal((n, d)).astype(np.float32), "f32")
    H, _, _ = a.materialize(0.0, neutralize=False)
    # std of each diagonal entry is 2*sqrt(2/n) ~ 0.009; allow 6 sigma
    assert np.all(np.abs(np.diag(H) - 2.0) < 0.054)


def pin_dead_mask_matches_zeroed_columns(O, seed=8):
    rng = np.random.default_rng(seed)
    d = 40
    dead = np.array([0, 7, 13, 39])
    X = rng.standard_normal((30, d)).astype(np.float32)
    X[:, dead] = 0.0
    a = O.GramAccumulator(d)
    a.add_batch(W.to_bf16_bits(X), "bf16")
    H, mask, damp = a.materialize(0.05)
    assert np.array_equal(np.flatnonzero(mask), dead)
    H0, _, _ = a.materialize(0.0)
    assert np.allclose(H - H0, damp * np.eye(d), rtol=0, atol=1e-13)
    assert np.all(np.diag(H0)[dead] == 1.0)


def pin_bf16_decode(O):
    import torch
    known = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0078125, 0x0000: 0.0, 0x8000: -0.0,
             0x7F7F: 3.3895313892515355e38, 0x0001: 9.183549615799121e-41}
    for bits, val in known.items():
        got = O.decode_bf16(np.array([bits], dtype=np.uint16))[0]
        assert got == val, (hex(bits), got, val)
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values only
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(O.decode_bf16(bits), ref)


def pin_local_blocks(O, seed=10):
    """Per-block Grams: exact rational check, and equal to the full Gram's diagonal blocks."""
    rng = np.random.default_rng(seed)
    n, d = 6, 48
    X = rng.standard_normal((n, d)).astype(np.float32)
    Xb = W.to_bf16_bits(X)
    B = O.local_blocks(Xb, "bf16")
    assert B.shape == (3, 16, 16)
    vals = W.bf16_bits_to_float32(Xb).astype(np.float64)
    for b in range(3):
        cols = vals[:, 16 * b: 16 * b + 16]
        S_exact = _frac_gram(cols.tolist())
        for i in range(16):
            for j in range(16):
                assert abs(B[b, i, j] - float(S_exact[i][j])) <= 1e-14 * max(1.0, abs(float(S_exact[i][j])))
    a = O.GramAccumulator(d)
    a.add_batch(Xb, "bf16")
    for b in range(3):
        sl = slice(16 * b, 16 * b + 16)
        assert np.allclose(B[b], a.S[sl, sl], rtol=1e-14, atol=1e-14)


def pin_grouped(O, seed=12):
    rng = np.random.default_rng(seed)
    T, d, E, k = 200, 16, 12, 3
    X = rng.standard_normal((T, d)).astype(np.float32)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=k)
    assert offsets[-1] == T * k
    out = O.grouped_grams(X, "f32", row_idx, offsets)
    assert len(out) == E
    assert sum(N for _, N in out) == T * k
    for e, (S, N) in enumerate(out):
        rows = row_idx[offsets[e]:offsets[e + 1]]
        sub = X[rows].astype(np.float64).tolist()
        assert N == len(rows)
        if N == 0:
            assert not S.any()
            continue
        S_exact = _frac_gram(sub)
        for i in range(0, d, 5):
            for j in range(0, d, 3):
                assert abs(S[i, j] - float(S_exact[i][j])) <= 1e-13 * max(1.0, abs(float(S_exact[i][j])))


def pin_gram_entries(O, seed=13):
    rng = np.random.default_rng(seed)
    d = 9
    batches = [rng.standard_normal((n, d)).astype(np.float32) for n in (4, 0, 3)]
    rows = np.array([0, 3, 8, 8])
    cols = np.array([0, 5, 2, 8])
    got = O.gram_entries(batches, "f32", rows, cols)
    allrows = [r for b in batches for r in b.tolist()]
    S_exact = _frac_gram(allrows)
    for k in range(4):
        assert abs(got[k] - float(S_exact[rows[k]][cols[k]])) <= 1e-14 * max(1, abs(float(S_exact[rows[k]][cols[k]])))


def pin_imatrix(O, seed=14):
    """Per-column sums of squares equal exact rational sums, over batches of both dtypes."""
    rng = np.random.default_rng(seed)
    d = 6
    batches = [rng.standard_normal((n, d)).astype(np.float32) for n in (3, 0, 5, 1)]
    got = O.column_sum_squares(batches, "f32")
    rows = [r for b in batches for r in b.tolist()]
    for j in range(d):
        exact = sum(Fraction(float(r[j])) ** 2 for r in rows)
        assert abs(got[j] - float(exact)) <= 1e-15 * float(exact) + 1e-300, (j, got[j], float(exact))
    # bf16 inputs are decoded exactly: 0x3F80 = 1.0, 0xC040 = -3.0, 0x3F81 = 1 + 2^-7
    bits = np.array([[0x3F80, 0xC040, 0x3F81], [0x0000, 0x3F80, 0xC040]], dtype=np.uint16)
    got = O.column_sum_squares([bits], "bf16")
    want = [1.0, 9.0 + 1.0, (1 + 2.0 ** -7) ** 2 + 9.0]
    assert np.array_equal(got, np.array(want)), (got, want)


def _frac_inverse(M):
    """Exact inverse of a small rational matrix by Gauss-Jordan elimination on Fractions."""
    n = len(M)
    A = [[Fraction(M[i][j]) for j in range(n)] + [Fraction(int(i == j)) for j in range(n)] for i in range(n)]
    for c in range(n):
        p = next(r for r in range(c, n) if A[r][c] != 0)
        A[c], A[p] = A[p], A[c]
        piv = A[c][c]
        A[c] = [v / piv for v in A[c]]
        for r in range(n):
            if r != c and A[r][c] != 0:
                f = A[r][c]
                A[r] = [a - f * b for a, b in zip(A[r], A[c])]
    return [row[n:] for row in A]


def pin_chol_inverse_upper(O, seed=21):
    """U upper with positive diagonal and U^T U = H^-1: closed forms (diagonal, 2 x 2), a factor
    known by construction, exact rational inverses, the usual three-call library route, and the
    not-positive-definite error."""
    import torch
    # diagonal H: U = diag(1 / sqrt(h))
    h = np.array([4.0, 0.25, 9.0, 2.0])
    U = O.chol_inverse_upper(np.diag(h))
    assert np.allclose(U, np.diag(1 / np.sqrt(h)), rtol=1e-15, atol=0)
    # 2 x 2 [[a, b], [b, c]]: u11 = sqrt(c / det), u12 = -b / sqrt(c det), u22 = 1 / sqrt(c)
    a, b, c = 4.0, 2.0, 3.0
    det = a * c - b * b
    U = O.chol_inverse_upper(np.array([[a, b], [b, c]]))
    want = np.array([[np.sqrt(c / det), -b / np.sqrt(c * det)], [0.0, 1 / np.sqrt(c)]])
    assert np.allclose(U, want, rtol=1e-15, atol=1e-16), (U, want)
    # H = V V^T with V upper, positive diagonal  =>  U = V^-1 (a unique factor)
    rng = np.random.default_rng(seed)
    d = 12
    V = np.triu(rng.standard_normal((d, d)) * 0.3, 1) + np.diag(rng.uniform(0.5, 2.0, d))
    U = O.chol_inverse_upper(V @ V.T)
    Vinv = np.linalg.solve(V, np.eye(d))
    assert np.allclose(U, Vinv, rtol=1e-11, atol=1e-12)
    assert np.array_equal(U, np.triu(U)) and (np.diag(U) > 0).all()
    # exact rational inverse at d = 4: U^T U matches it
    M = [[6, 2, 1, 0], [2, 5, 2, 1], [1, 2, 4, 1], [0, 1, 1, 3]]
    Minv = np.array([[float(v) for v in row] for row in _frac_inverse(M)])
    U = O.chol_inverse_upper(np.array(M, dtype=np.float64))
    assert np.allclose(U.T @ U, Minv, rtol=0, atol=1e-15)
    # the library route: upper Cholesky of the inverse formed from the lower Cholesky of H
    X = rng.standard_normal((200, 40))
    H = 2.0 / 200 * X.T @ X
    H += 0.01 * np.mean(np.diag(H)) * np.eye(40)
    Ht = torch.from_numpy(H)
    Ut = torch.linalg.cholesky(torch.cholesky_inverse(torch.linalg.cholesky(Ht)), upper=True).numpy()
    U = O.chol_inverse_upper(H)
    assert np.allclose(U, Ut, rtol=1e-10, atol=1e-12)
    assert np.allclose(U.T @ U @ H, np.eye(40), atol=1e-10)
    # not positive definite: an error, no silent result
    for bad in (np.array([[1.0, 2.0], [2.0, 1.0]]), np.zeros((3, 3)), np.diag([1.0, -1e-3, 2.0])):
        try:
            O.chol_inverse_upper(bad)
        except np.linalg.LinAlgError:
            pass
        else:
            raise AssertionError("non-positive-definite input accepted")


def _obs_quantize(W, H, group, bits=4):
    """GPTQ as optimal brain surgery, written independently of the oracle: at column i the
    remaining weights F = i..K-1 move by -(w_i - deq_i) / [inv(H_FF)]_00 inv(H_FF)[0, :], with the
    inverse of the remaining block recomputed by a library inverse at every step."""
    W = np.array(W, dtype=np.float64)
    N, K = W.shape
    g = K if group in (-1, K) else group
    Q = np.zeros_like(W)
    codes = np.zeros((N, K), dtype=np.int64)
    loss = 0.0
    for i in range(K):
        if i % g == 0:
            a = np.max(np.abs(W[:, i:i + g]), axis=1)
            scale = 2.0 * np.where(a == 0, 1.0, a) / (2 ** bits - 1)
        Hinv = np.linalg.inv(H[i:, i:])
        w = W[:, i].copy()
        q = np.clip(np.rint(w / scale) + 2 ** (bits - 1), 0, 2 ** bits - 1)
        deq = scale * (q - 2 ** (bits - 1))
        W[:, i:] -= np.outer((w - deq) / Hinv[0, 0], Hinv[0, :])
        loss += float(np.sum((w - deq) ** 2 / Hinv[0, 0]))
        Q[:, i] = deq
        codes[:, i] = q
    return Q, codes, loss


def pin_gptq_quantize(O, seed=31):
    """Quantizer hand values; identity Hessian = plain rounding; the factor-row propagation equals
    optimal-brain-surgery updates with explicit inverses (whole rows and groups); dead columns
    quantize to zero and move nothing."""
    g = _load("quantizer_hand.json")
    row = np.asarray([g["row"]])
    assert abs(O.quant_scale(row)[0] - g["scale"]) <= 1e-15
    assert abs(O.quant_scale(np.zeros((1, 3)))[0] - g["zero_row_scale"]) <= 1e-15
    Q, codes, scales, loss = O.gptq_quantize(row, np.eye(row.shape[1]))
    assert codes[0].tolist() == g["codes"], codes
    assert np.allclose(Q[0], g["dequantized"], rtol=0, atol=1e-15)
    assert abs(loss - float(np.sum((row[0] - np.asarray(g["dequantized"])) ** 2))) <= 1e-14
    rng = np.random.default_rng(seed)
    for N, K, group in ((5, 6, -1), (4, 12, 4), (3, 9, 3), (6, 16, 8)):
        X = rng.standard_normal((3 * K, K))
        H = 2.0 / (3 * K) * X.T @ X
        H += 0.01 * np.mean(np.diag(H)) * np.eye(K)
        W = rng.standard_normal((N, K))
        U = O.chol_inverse_upper(H)
        Q, codes, scales, loss = O.gptq_quantize(W, U, group_size=group, nsamples=7)
        Qr, codes_r, loss_r = _obs_quantize(W, H, group)
        assert np.array_equal(codes, codes_r), (N, K, group)
        assert np.allclose(Q, Qr, rtol=1e-12, atol=1e-12)
        assert abs(loss * 7 - loss_r) <= 1e-10 * max(1.0, loss_r)
        assert scales.shape == (N, 1 if group == -1 else -(-K // group))
    # a tie decision that returns the default changes nothing, and every reported tie holds the
    # default code between its two neighbours
    ties = []
    Q2, codes2, _, _ = O.gptq_quantize(W, U, group_size=group, nsamples=7, tie_tol=1e-12, ties=ties,
                                       tie_break=lambda i, rows, lo, hi, dflt: dflt)
    assert np.array_equal(codes2, codes) and np.array_equal(Q2, Q)
    for i, rows, lo, hi in ties:
        assert np.all(hi.astype(int) - lo.astype(int) <= 1) and np.all(
            (codes[rows, i] == lo) | (codes[rows, i] == hi))
    # a tie decision that is not a neighbour code is refused
    try:
        O.gptq_quantize(W, U, group_size=group, tie_tol=1e-12, tie_break=lambda i, rows, lo, hi, dflt: dflt + 3)
        raise AssertionError("a non-neighbour tie decision must be refused")
    except ValueError:
        pass
    # an exact tie: w / step = -7.5 rounds to the even -8 (code 0); the other neighbour (code 1)
    # may be taken there, and the error it leaves propagates
    row = np.array([[-3.75, 1.0]])
    _, c_tie, _, _ = O.gptq_quantize(row, np.eye(2))
    assert c_tie[0, 0] == 0
    ties = []
    _, c_f, _, _ = O.gptq_quantize(row, np.eye(2), tie_tol=1e-12, ties=ties,
                                   tie_break=lambda i, rows, lo, hi, dflt: hi)
    assert c_f[0, 0] == 1
    assert [(t[0], t[1].tolist(), t[2].tolist(), t[3].tolist()) for t in ties][0] == (0, [0], [0], [1])
    # dead columns: zero weights, centre codes, no error to move
    W = rng.standard_normal((4, 8))
    X = rng.standard_normal((30, 8))
    H = X.T @ X / 15 + 0.05 * np.eye(8)
    U = O.chol_inverse_upper(H)
    dead = np.zeros(8, dtype=bool)
    dead[[2, 5]] = True
    Q, codes, _, _ = O.gptq_quantize(W, U, dead=dead)
    assert (codes[:, dead] == 8).all() and not Q[:, dead].any()
    W2 = W.copy()
    W2[:, dead] = 0.0
    Q2, codes2, _, _ = O.gptq_quantize(W2, U)
    assert np.array_equal(codes, codes2) and np.array_equal(Q, Q2)


ALL_PINS = [
    pin_gptq_quantize,
    pin_chol_inverse_upper,
    pin_imatrix,
    pin_bruteforce_fraction,
    pin_orientation_hand,
    pin_worked_example,
    pin_worked_example_f16_staging,
    pin_bf16_rounding,
    pin_neutralize_damp_hand,
    pin_multi_batch_is_concatenation,
    pin_empty_batch_noop,
    pin_covariance_special_case,
    pin_symmetric_psd_cholesky,
    pin_unit_variance_diagonal,
    pin_dead_mask_matches_zeroed_columns,
    pin_bf16_decode,
    pin_local_blocks,
    pin_grouped,
    pin_gram_entries,
]
