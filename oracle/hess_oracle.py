"""Plain float64 NumPy oracle for GPTQ/QQQ calibration-Hessian accumulation.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.

What it computes, and where the pages define it
-----------------------------------------------
* Per-batch Gram accumulation ``S += X^T X`` with X laid out tokens x
  features, and the token count ``N += n`` (GPTQModel PR 2979, "fix(qqq):
  per-device Hessian partials ...", Summary and What Changed: the count is
  of flattened token vectors, not batches; GPTQModel wiki "QQQ", Concepts >
  Quadratic error compensation).  The pages write the same matrix as
  ``X X^T`` for X laid out features x tokens.
* In-place accumulation into one persistent buffer (GPTQModel PR 2981,
  "fix(qqq): accumulate Hessian in-place per device", Changes).  Here the
  buffer is float64 and exact to ~1e-16; the library keeps float32.
* ``materialize``: scale the sum by 2 / total tokens (PR 2979, What Changed;
  wiki "QQQ", Concepts), then the quantization pass's steps 2 and 3 (wiki
  "QQQ", Concepts > Quadratic error compensation): neutralize dead input
  columns, then add ``damp_percent * mean(diag(H))`` to the diagonal.  The
  damping value returned is that absolute amount (wiki "QQQ", Implementation
  internals > Quantizer API and results).
* ``local_blocks``: per contiguous 16-feature block b, ``X_b^T X_b`` as a
  batched product (NVIDIA Model-Optimizer PR 3002 page, "What does this PR
  do?", the ``local_hessian`` bullet).
* ``grouped_grams``: one independent (S_e, N_e) per routed expert over the
  rows routed to it (Model-Optimizer PR 3002 page, "What does this PR do?":
  the option applies to every GPTQ Hessian, fused MoE experts included).
* ``column_sum_squares``: the imatrix statistic, a per-column sum of squares
  of the inputs (Model-Optimizer PR 3002 page, "What does this PR do?").
* ``chol_inverse_upper``: the upper-triangular Cholesky factor of the inverse
  of the damped Hessian, the quantization pass's step 4 (GPTQModel wiki
  "QQQ", Concepts > Quadratic error compensation): U upper triangular with a
  positive diagonal and U^T U = H^-1, which fixes U uniquely.  A damped H
  that is not positive definite is a factorization error; there is no
  automatic damping retry (wiki "QQQ", Pitfalls and the Quantizer API
  notes on damp_auto_increment).
* ``gptq_quantize``: the quantization pass's step 5 (wiki "QQQ", Concepts >
  Quadratic error compensation): columns are quantized in order and each
  column's error, divided by the factor's diagonal entry, is propagated into
  the columns not yet quantized through the row of the factor; the
  quantizer is symmetric 4-bit, one per output row (group_size -1) or per
  group of contiguous input columns (wiki "QQQ", Whole-row and grouped
  weight quantization), with group parameters taken when a group is reached
  (static_groups off, wiki "QQQ" configuration table); the loss is the
  summed squared scaled error over the token count (wiki "QQQ",
  Implementation internals > Quantizer API and results).  The pages process
  128-column blocks; blocking changes only the order of the float64
  additions, so the oracle propagates column by column.
* Staging dtype: activations are first put into the accumulator's staging
  type, then multiplied (GPTQModel PR 3052, "Shared-input Hessian dedup",
  review finding P2: an fp16 activation of 1 + 2^-10 stays exact when staged
  in fp32 and becomes 1.0 when staged in bf16; Model-Optimizer PR 3002 page,
  "What does this PR do?": ``hessian_input_dtype`` bfloat16 versus the
  float32 default).  ``round_to_bf16`` is IEEE round-to-nearest-even onto the
  bf16 value set; fp16 and bf16 values are float32 values, so fp32 staging
  changes nothing.

Readings where the pages leave a step open (each is also listed in the
design notes):
* dead column  <=>  its Hessian diagonal is exactly zero, i.e. the column
  is all zero for any input whose nonzero squares do not underflow; the
  neutralized diagonal entry becomes 1 (its row and column are already 0).
* N = 0 gives a zero scaled H, so every column is dead.
* neutralization happens before damping, so the mean diagonal includes the
  1s written for dead columns (the order of steps 2 and 3 on the wiki).
* the mean of the diagonal is taken in float64.
* local blocks are unscaled and accumulate across calls.

The input decoding is exact: bf16 values are given as their uint16 bit
patterns and widened bit-for-bit; float32 and float16 values widen exactly to
float64.
Products of two such values are exact in float64 (<= 48 significant bits)
and the sums carry only float64 rounding, about 1e-16 relative per add.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "decode_bf16",
    "exact_float64",
    "GramAccumulator",
    "materialize",
    "local_blocks",
    "grouped_grams",
    "gram_entries",
    "gram_exact_fraction",
    "column_sum_squares",
    "round_to_bf16",
    "staged_values",
    "chol_inverse_upper",
    "quant_scale",
    "gptq_quantize",
]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers given as uint16 bit patterns, as float64.

    A bf16 number is the upper half of a float32 bit pattern, so shifting the
    16 bits up by 16 and reading the result as float32 is exact.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 input must be given as uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def exact_float64(X: np.ndarray, in_dtype: str) -> np.ndarray:
    """The stored input values as float64, exactly.

    ``in_dtype`` is ``"bf16"`` (X holds uint16 bit patterns), ``"f32"`` or
    ``"f16"`` (numpy float16).
    """
    if in_dtype == "bf16":
        return decode_bf16(X)
    if in_dtype in ("f32", "f16"):
        X = np.asarray(X)
        want = np.float32 if in_dtype == "f32" else np.float16
        if X.dtype != want:
            raise TypeError(f"{in_dtype} input must be a {np.dtype(want).name} array")
        return X.astype(np.float64)
    raise ValueError(f"unknown input dtype {in_dtype!r}")


# bf16: 8 significant bits, exponents as float32 (normal numbers from 2^-126,
# subnormal spacing 2^-133), largest finite (2 - 2^-7) 2^127.
_BF16_MIN_QUANTUM = 2.0 ** -133
_BF16_OVERFLOW = (2.0 - 2.0 ** -8) * 2.0 ** 127  # halfway to 2^128: from here on, inf


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values (each exactly a float32 value) to the nearest bf16
    value, ties to the even significand; results as float64.

    The spacing of bf16 numbers in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below
    2^-126.  Dividing by that spacing is exact (a power of two), ``rint``
    rounds half to even, and multiplying back is exact.  Magnitudes at or
    beyond the midpoint between the largest finite bf16 and 2^128 become
    infinite (the tie rounds to the even significand, which is the overflow).
    NaN stays NaN and infinities stay infinite.
    """
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    a = np.abs(v[fin])
    _, e = np.frexp(a)              # a = m 2^e with m in [0.5, 1): a in [2^(e-1), 2^e)
    q = np.maximum(np.ldexp(1.0, e - 1 - 7), _BF16_MIN_QUANTUM)
    r = np.rint(a / q) * q
    r[a >= _BF16_OVERFLOW] = np.inf
    out[fin] = np.copysign(r, v[fin])
    return out


def staged_values(X: np.ndarray, in_dtype: str, staging: str | None) -> np.ndarray:
    """The float64 values a batch contributes once put into the staging type.

    ``staging`` is ``None`` (the stored type), ``"f32"`` (fp16, bf16 and
    float32 values are all float32 values: unchanged) or ``"bf16"`` (rounded
    to nearest even).
    """
    Xd = exact_float64(X, in_dtype)
    if staging is None or staging == "f32" or (staging == "bf16" and in_dtype == "bf16"):
        return Xd
    if staging == "bf16":
        return round_to_bf16(Xd)
    raise ValueError(f"unknown staging dtype {staging!r}")


class GramAccumulator:
    """Running Gram sum S and token count N of one Hessian.

    ``add_batch`` takes one calibration batch, tokens x features; an empty
    batch changes nothing (GPTQModel PR 2981, Validation: empty batches).
    ``staging`` (``None``, ``"f32"`` or ``"bf16"``) is the type every batch is
    put into before its products are formed.
    """

    def __init__(self, d: int, staging: str | None = None):
        if d < 1:
            raise ValueError("d must be positive")
        self.d = int(d)
        self.staging = staging
        self.S = np.zeros((self.d, self.d), dtype=np.float64)
        self.N = 0

    def add_batch(self, X: np.ndarray, in_dtype: str) -> None:
        Xd = staged_values(X, in_dtype, self.staging)
        if Xd.ndim != 2 or Xd.shape[1] != self.d:
            raise ValueError(f"batch must be (tokens, {self.d})")
        n = Xd.shape[0]
        if n == 0:
            return
        self.S += Xd.T @ Xd
        self.N += n

    def materialize(self, damp_percent: float, neutralize: bool = True):
        return materialize(self.S, self.N, damp_percent, neutralize)


def materialize(S: np.ndarray, N: int, damp_percent: float, neutralize: bool = True):
    """Final Hessian from the Gram sum: scale, neutralize, damp.

    Returns ``(H, dead, damp)``: H float64 (d, d), ``dead`` a bool mask of
    the neutralized columns (all False when ``neutralize`` is off), ``damp``
    the absolute amount added to every diagonal entry.
    """
    S = np.asarray(S, dtype=np.float64)
    d = S.shape[0]
    # Scale by 2 / total tokens, once, at the end; nothing accumulated -> 0.
    H = (2.0 / N) * S if N > 0 else np.zeros((d, d), dtype=np.float64)
    diag = np.diag(H).copy()
    if neutralize:
        dead = diag == 0.0
        H[dead, :] = 0.0
        H[:, dead] = 0.0
        H[dead, dead] = 1.0
    else:
        dead = np.zeros(d, dtype=bool)
    damp = float(damp_percent) * float(np.mean(np.diag(H)))
    H[np.arange(d), np.arange(d)] += damp
    return H, dead, damp


def local_blocks(X: np.ndarray, in_dtype: str, block: int = 16) -> np.ndarray:
    """Per-block Gram matrices of contiguous feature blocks, unscaled.

    out[b] = X[:, block*b : block*(b+1)]^T  X[:, block*b : block*(b+1)]
    """
    Xd = exact_float64(X, in_dtype)
    n, d = Xd.shape
    if d % block != 0:
        raise ValueError("feature count must be a multiple of the block size")
    nb = d // block
    out = np.empty((nb, block, block), dtype=np.float64)
    for b in range(nb):
        Xb = Xd[:, block * b: block * (b + 1)]
        out[b] = Xb.T @ Xb
    return out


def grouped_grams(X: np.ndarray, in_dtype: str, row_idx: np.ndarray, offsets: np.ndarray):
    """Independent Gram sums per group of rows (one group per routed expert).

    Group e consists of rows ``row_idx[offsets[e]:offsets[e+1]]`` of X.
    Returns a list of ``(S_e, N_e)``.  A group with no rows gets S = 0, N = 0.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    row_idx = np.asarray(row_idx)
    out = []
    for e in range(len(offsets) - 1):
        acc = GramAccumulator(np.asarray(X).shape[1])
        rows = row_idx[offsets[e]:offsets[e + 1]]
        acc.add_batch(np.asarray(X)[rows], in_dtype)
        out.append((acc.S, acc.N))
    return out


def gram_entries(batches, in_dtype: str, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Selected entries S[rows[k], cols[k]] of the Gram sum over ``batches``.

    Each entry is the float64 dot product of two feature columns over every
    token of every batch; used to check full-size results at sampled points.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    acc = np.zeros(rows.shape[0], dtype=np.float64)
    for X in batches:
        Xd = exact_float64(X, in_dtype)
        if Xd.shape[0] == 0:
            continue
        acc += np.einsum("tk,tk->k", Xd[:, rows], Xd[:, cols])
    return acc


def column_sum_squares(batches, in_dtype: str) -> np.ndarray:
    """The imatrix statistic: per-column sum over every token of x_j^2.

    The imatrix method keeps a float32 per-column sum of squares of the layer
    inputs instead of a Gram matrix (NVIDIA Model-Optimizer PR 3002 page,
    "What does this PR do?").  Here it is the float64 sum of the exact
    squares of the stored values.
    """
    acc = None
    for X in batches:
        Xd = exact_float64(X, in_dtype)
        if acc is None:
            acc = np.zeros(Xd.shape[1], dtype=np.float64)
        for t in range(Xd.shape[0]):
            acc += Xd[t] * Xd[t]
    return acc


def gram_exact_fraction(rows_of_values) -> list:
    """Exact rational Gram sum by a plain triple loop (tiny inputs only).

    ``rows_of_values`` is a sequence of tokens, each a sequence of d Python
    numbers (floats are converted exactly with ``Fraction``).  Returns a
    d x d list of lists of ``Fraction``.
    """
    rows = [[Fraction(v) for v in r] for r in rows_of_values]
    if not rows:
        return []
    d = len(rows[0])
    S = [[Fraction(0) for _ in range(d)] for _ in range(d)]
    for r in rows:
        for i in range(d):
            for j in range(d):
                S[i][j] += r[i] * r[j]
    return S


def chol_inverse_upper(H: np.ndarray) -> np.ndarray:
    """Upper-triangular U, positive diagonal, with U^T U = H^-1 (float64).

    H is the damped Hessian (symmetric).  The definition is applied as
    written: invert H, then take the Cholesky factor of the inverse; numpy's
    factor is the lower L with L L^T = H^-1, so U = L^T.  Raises
    ``numpy.linalg.LinAlgError`` when H (hence H^-1) is not positive
    definite.
    """
    H = np.asarray(H, dtype=np.float64)
    np.linalg.cholesky(H)            # H itself must be positive definite
    Hinv = np.linalg.inv(H)
    L = np.linalg.cholesky(Hinv)     # reads the lower triangle of H^-1
    return L.T.copy()


def quant_scale(x: np.ndarray, bits: int = 4) -> np.ndarray:
    """Symmetric quantizer step per row of x: 2 max|x| / (2^bits - 1).

    Codes are q = clip(rint(w / scale) + 2^(bits-1), 0, 2^bits - 1), i.e.
    signed values q - 2^(bits-1) in [-2^(bits-1), 2^(bits-1) - 1] around the
    fixed centre, dequantized as scale (q - 2^(bits-1)).  A row that is all
    zero takes max|x| = 1.
    """
    a = np.max(np.abs(np.asarray(x, dtype=np.float64)), axis=1)
    a = np.where(a == 0.0, 1.0, a)
    return 2.0 * a / float(2 ** bits - 1)


def gptq_quantize(W: np.ndarray, U: np.ndarray, group_size: int = -1, bits: int = 4, dead=None,
                  nsamples: int = 1, tie_tol: float = 0.0, ties=None, tie_break=None):
    """Error-propagating quantization of W (rows = outputs, columns = inputs).

    U is the upper Cholesky factor of the inverse damped Hessian (only its
    upper triangle is used).  Returns ``(Q, codes, scales, loss)``: Q the
    dequantized weights (float64), codes uint8 in [0, 2^bits - 1], scales
    (rows, groups) float64 (one column for group_size -1), loss the summed
    squared scaled error over ``nsamples``.

    Rounding ties: the largest magnitude of a group sits at 7.5 steps, so
    ties between two codes are part of the method, and a run whose float64
    additions come in another order may round such a tie the other way.  Both
    codes are then correct, and the choice decides the errors propagated
    after it.  The oracle therefore reports every position where w / step
    lies within ``tie_tol`` (relative) of a half-integer: when ``ties`` is a
    list, one record ``(column, rows, lower code, upper code)`` per column
    with such positions is appended to it.  The code taken there is
    round-half-to-even unless ``tie_break`` is given: a function
    ``tie_break(column, rows, lower, upper, default)`` returning one of the
    two neighbour codes for each listed row (the method's decision at a tie,
    passed in as an input).
    """
    W = np.array(W, dtype=np.float64)
    U = np.triu(np.asarray(U, dtype=np.float64))
    N, K = W.shape
    if dead is not None:
        W[:, np.asarray(dead, dtype=bool)] = 0.0   # the weight side of dead-column neutralization
    maxq = 2 ** bits - 1
    centre = 2 ** (bits - 1)
    g = K if group_size in (-1, K) else int(group_size)
    ngroups = -(-K // g)
    scales = np.zeros((N, ngroups), dtype=np.float64)
    codes = np.zeros((N, K), dtype=np.uint8)
    Q = np.zeros((N, K), dtype=np.float64)
    loss = 0.0
    scale = None
    for i in range(K):
        if i % g == 0:
            # parameters from the group's current (already error-updated) weights
            scale = quant_scale(W[:, i:i + g], bits)
            scales[:, i // g] = scale
        w = W[:, i].copy()
        x = w / scale
        q = np.clip(np.rint(x) + centre, 0, maxq)
        if tie_tol > 0.0 and (ties is not None or tie_break is not None):
            rows = np.flatnonzero(np.abs(x - np.floor(x) - 0.5) <= tie_tol * np.maximum(1.0, np.abs(x)))
            if rows.size:
                lo = np.clip(np.floor(x[rows]) + centre, 0, maxq)
                hi = np.clip(np.floor(x[rows]) + 1.0 + centre, 0, maxq)
                if ties is not None:
                    ties.append((i, rows, lo.astype(np.uint8), hi.astype(np.uint8)))
                if tie_break is not None:
                    pick = np.asarray(tie_break(i, rows, lo, hi, q[rows].copy()), dtype=np.float64)
                    if not np.all((pick == lo) | (pick == hi)):
                        raise ValueError(f"tie_break returned a code that is not a neighbour (column {i})")
                    q[rows] = pick
        deq = scale * (q - centre)
        err = (w - deq) / U[i, i]
        W[:, i + 1:] -= np.outer(err, U[i, i + 1:])
        codes[:, i] = q.astype(np.uint8)
        Q[:, i] = deq
        loss += float(np.sum(err * err))
    return Q, codes, scales, loss / nsamples
