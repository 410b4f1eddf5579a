"""The oracle against its pins, and planted mistakes that the pins must catch.

CPU only.  Each mutant below is a copy of the oracle with one plausible
mistake planted (a dropped term, a wrong scale, a transposed operand, a wrong
index or order); every mutant has to fail at least one pin, which shows the
pins constrain each part of the oracle.
"""

import types

import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle import hess_oracle as HO
from tests.oracle_pins import ALL_PINS

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


# ---------------------------------------------------------------- mutants --

def _ns(**over):
    base = dict(
        GramAccumulator=HO.GramAccumulator,
        materialize=HO.materialize,
        local_blocks=HO.local_blocks,
        grouped_grams=HO.grouped_grams,
        decode_bf16=HO.decode_bf16,
        exact_float64=HO.exact_float64,
        gram_entries=HO.gram_entries,
        column_sum_squares=HO.column_sum_squares,
        round_to_bf16=HO.round_to_bf16,
        staged_values=HO.staged_values,
        chol_inverse_upper=HO.chol_inverse_upper,
        quant_scale=HO.quant_scale,
        gptq_quantize=HO.gptq_quantize,
    )
    base.update(over)
    return types.SimpleNamespace(**base)


def _acc_class(add=None, mat=None):
    class Acc(HO.GramAccumulator):
        pass
    if add is not None:
        Acc.add_batch = add
    if mat is not None:
        Acc.materialize = lambda self, p, neutralize=True: mat(self.S, self.N, p, neutralize)
    return Acc


def _add_counts_batches(self, X, in_dtype):
    Xd = HO.exact_float64(X, in_dtype)
    if Xd.shape[0] == 0:
        return
    self.S += Xd.T @ Xd
    self.N += 1  # mistake: counts batches, not tokens


def _add_overwrites(self, X, in_dtype):
    Xd = HO.exact_float64(X, in_dtype)
    if Xd.shape[0] == 0:
        return
    self.S = Xd.T @ Xd  # mistake: drops the running sum
    self.N += Xd.shape[0]


def _add_transposed(self, X, in_dtype):
    Xd = HO.exact_float64(X, in_dtype)
    if Xd.shape[0] == 0:
        return
    if Xd.shape[0] > 2048:
        raise ValueError("token Gram too large")  # keeps the mutant cheap on big inputs
    G = Xd @ Xd.T  # mistake: token Gram instead of feature Gram
    if G.shape == self.S.shape:
        self.S += G
    else:
        self.S = G
    self.N += Xd.shape[0]


def _add_drops_last_token(self, X, in_dtype):
    Xd = HO.exact_float64(X, in_dtype)
    if Xd.shape[0] == 0:
        return
    Xd = Xd[:-1]  # mistake: off-by-one in the token loop
    self.S += Xd.T @ Xd
    self.N += Xd.shape[0] + 1


def _mat_scale_one_over_n(S, N, p, neutralize=True):
    H, dead, damp = HO.materialize(S, N, p, neutralize)
    if N > 0:
        H = H - damp * np.eye(len(H))
        H = H / 2.0  # mistake: 1/N instead of 2/N
        damp = p * float(np.mean(np.diag(H)))
        H = H + damp * np.eye(len(H))
    return H, dead, damp


def _mat_damp_before_neutralize(S, N, p, neutralize=True):
    d = S.shape[0]
    H = (2.0 / N) * S if N > 0 else np.zeros((d, d))
    damp = p * float(np.mean(np.diag(H)))  # mistake: damping computed first
    dead = np.diag(H) == 0.0
    if neutralize:
        H[dead, :] = 0.0
        H[:, dead] = 0.0
        H[dead, dead] = 1.0
    H = H + damp * np.eye(d)
    return H, dead, damp


def _mat_damp_max(S, N, p, neutralize=True):
    H, dead, damp = HO.materialize(S, N, 0.0, neutralize)
    damp = p * float(np.max(np.diag(H)))  # mistake: max instead of mean
    return H + damp * np.eye(len(H)), dead, damp


def _mat_no_neutralize(S, N, p, neutralize=True):
    return HO.materialize(S, N, p, neutralize=False)  # mistake: never neutralizes


def _mat_dead_zero_diag(S, N, p, neutralize=True):
    d = S.shape[0]
    H = (2.0 / N) * S if N > 0 else np.zeros((d, d))
    dead = np.diag(H) == 0.0
    # mistake: dead columns keep a zero diagonal instead of 1
    damp = p * float(np.mean(np.diag(H)))
    return H + damp * np.eye(d), dead, damp


def _local_shifted(X, in_dtype, block=16):
    Xd = HO.exact_float64(X, in_dtype)
    n, d = Xd.shape
    out = np.empty((d // block, block, block))
    for b in range(d // block):
        s = min(block * b + 1, d - block)  # mistake: block offset off by one
        Xb = Xd[:, s:s + block]
        out[b] = Xb.T @ Xb
    return out


def _local_cross(X, in_dtype, block=16):
    Xd = HO.exact_float64(X, in_dtype)
    n, d = Xd.shape
    nb = d // block
    out = np.empty((nb, block, block))
    for b in range(nb):
        A = Xd[:, block * b: block * (b + 1)]
        B = Xd[:, block * ((b + 1) % nb): block * ((b + 1) % nb + 1)]
        out[b] = A.T @ B  # mistake: pairs block b with its neighbour
    return out


def _decode_truncates(bits):
    v = HO.decode_bf16(bits)
    return np.trunc(v * 64.0) / 64.0  # mistake: loses low mantissa bits


def _grouped_shares(X, in_dtype, row_idx, offsets):
    out = HO.grouped_grams(X, in_dtype, row_idx, offsets)
    S0 = sum(S for S, _ in out)
    return [(S0, N) for _, N in out]  # mistake: experts share one Gram


def _entries_swapped(batches, in_dtype, rows, cols):
    return HO.gram_entries(batches, in_dtype, rows, (np.asarray(cols) + 1) % 9)  # wrong column index


def _imx_not_squared(batches, in_dtype):
    return sum(HO.exact_float64(X, in_dtype).sum(axis=0) for X in batches if len(X))  # mistake: sums x, not x^2


def _imx_skips_last_row(batches, in_dtype):
    return HO.column_sum_squares([X[:-1] if len(X) else X for X in batches], in_dtype)  # mistake: drops a token


def _imx_shifted(batches, in_dtype):
    return np.roll(HO.column_sum_squares(batches, in_dtype), 1)  # mistake: column index off by one


def _round_truncates(v):
    v = np.asarray(v, dtype=np.float64)
    x32 = v.astype(np.float32)
    return ((x32.view(np.uint32) >> 16) << 16).view(np.float32).astype(np.float64)  # mistake: rounds toward zero


def _round_half_away(v):
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    a = np.abs(v[fin])
    _, e = np.frexp(a)
    q = np.maximum(np.ldexp(1.0, e - 8), 2.0 ** -133)
    out[fin] = np.copysign(np.floor(a / q + 0.5) * q, v[fin])  # mistake: ties away from zero
    return out


def _round_keeps_8_fraction_bits(v):
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    a = np.abs(v[fin])
    _, e = np.frexp(a)
    q = np.ldexp(1.0, e - 9)  # mistake: one bit too many
    out[fin] = np.copysign(np.rint(a / q) * q, v[fin])
    return out


def _staging_mutant(rounder):
    def staged(X, in_dtype, staging):
        Xd = HO.exact_float64(X, in_dtype)
        return rounder(Xd) if staging == "bf16" else Xd

    class Acc(HO.GramAccumulator):
        def add_batch(self, X, in_dtype):
            Xd = staged(X, in_dtype, self.staging)
            if Xd.shape[0] == 0:
                return
            self.S += Xd.T @ Xd
            self.N += Xd.shape[0]
    return dict(GramAccumulator=Acc, round_to_bf16=rounder, staged_values=staged)


def _staging_ignored():
    class Acc(HO.GramAccumulator):
        def add_batch(self, X, in_dtype):
            Xd = HO.exact_float64(X, in_dtype)  # mistake: never rounds to the staging type
            if Xd.shape[0] == 0:
                return
            self.S += Xd.T @ Xd
            self.N += Xd.shape[0]
    return dict(GramAccumulator=Acc, staged_values=lambda X, t, s: HO.exact_float64(X, t))


def _chol_lower_returned(H):
    return np.linalg.cholesky(np.linalg.inv(np.asarray(H, dtype=np.float64)))  # mistake: the lower factor


def _chol_of_h(H):
    return np.linalg.cholesky(np.asarray(H, dtype=np.float64)).T.copy()  # mistake: factor of H, not of H^-1


def _chol_inverse_of_factor(H):
    L = np.linalg.cholesky(np.asarray(H, dtype=np.float64))
    return np.linalg.inv(L).T.copy()  # mistake: U = L^-T gives U^T U = (L^T L)^-1, not (L L^T)^-1


def _gptq_mutant(kind):
    def run(W, U, group_size=-1, bits=4, dead=None, nsamples=1):
        W = np.array(W, dtype=np.float64)
        U = np.triu(np.asarray(U, dtype=np.float64))
        N, K = W.shape
        if dead is not None:
            W[:, np.asarray(dead, dtype=bool)] = 0.0
        W0 = W.copy()
        g = K if group_size in (-1, K) else group_size
        scales = np.zeros((N, -(-K // g)))
        codes = np.zeros((N, K), dtype=np.uint8)
        Q = np.zeros((N, K))
        loss = 0.0
        for i in range(K):
            if i % g == 0:
                src = W0 if kind == "static_groups" else W   # mistake: parameters from the untouched weights
                a = np.max(np.abs(src[:, i:i + g]), axis=1)
                a = np.where(a == 0, 1.0, a)
                scale = a / 7.0 if kind == "scale_absmax_over_7" else 2 * a / 15.0  # mistake: other step
                scales[:, i // g] = scale
            w = W[:, i].copy()
            x = w / scale
            r = np.floor(x + 0.5) if kind == "ties_away" else np.rint(x)  # mistake: ties not to even
            q = np.clip(r + 8, 0, 15)
            deq = scale * (q - 8)
            err = (w - deq) if kind == "no_diag_division" else (w - deq) / U[i, i]  # mistake: unscaled
            if kind == "column_of_factor":
                W[:, i + 1:] -= np.outer(err, U[i + 1:, i])   # mistake: the factor's column, not its row
            else:
                W[:, i + 1:] -= np.outer(err, U[i, i + 1:])
            codes[:, i] = q
            Q[:, i] = deq
            loss += float(np.sum((w - deq) ** 2)) if kind == "loss_unscaled" else float(np.sum(err * err))
        return Q, codes, scales, loss / nsamples
    return run


MUTANTS = {
    **{f"gptq_{k}": _ns(gptq_quantize=_gptq_mutant(k)) for k in
       ("static_groups", "scale_absmax_over_7", "ties_away", "no_diag_division", "column_of_factor",
        "loss_unscaled")},
    "chol_lower_factor": _ns(chol_inverse_upper=_chol_lower_returned),
    "chol_of_h": _ns(chol_inverse_upper=_chol_of_h),
    "chol_inverse_of_h_factor": _ns(chol_inverse_upper=_chol_inverse_of_factor),
    "bf16_round_truncates": _ns(**_staging_mutant(_round_truncates)),
    "bf16_round_half_away": _ns(**_staging_mutant(_round_half_away)),
    "bf16_round_9_bits": _ns(**_staging_mutant(_round_keeps_8_fraction_bits)),
    "staging_ignored": _ns(**_staging_ignored()),
    "imatrix_not_squared": _ns(column_sum_squares=_imx_not_squared),
    "imatrix_skips_last_row": _ns(column_sum_squares=_imx_skips_last_row),
    "imatrix_shifted": _ns(column_sum_squares=_imx_shifted),
    "counts_batches": _ns(GramAccumulator=_acc_class(add=_add_counts_batches)),
    "overwrites_sum": _ns(GramAccumulator=_acc_class(add=_add_overwrites)),
    "transposed_operand": _ns(GramAccumulator=_acc_class(add=_add_transposed)),
    "drops_last_token": _ns(GramAccumulator=_acc_class(add=_add_drops_last_token)),
    "scale_1_over_N": _ns(GramAccumulator=_acc_class(mat=_mat_scale_one_over_n)),
    "damp_before_neutralize": _ns(GramAccumulator=_acc_class(mat=_mat_damp_before_neutralize)),
    "damp_uses_max": _ns(GramAccumulator=_acc_class(mat=_mat_damp_max)),
    "never_neutralizes": _ns(GramAccumulator=_acc_class(mat=_mat_no_neutralize)),
    "dead_diag_stays_zero": _ns(GramAccumulator=_acc_class(mat=_mat_dead_zero_diag)),
    "local_block_offset": _ns(local_blocks=_local_shifted),
    "local_cross_block": _ns(local_blocks=_local_cross),
    "bf16_decode_truncates": _ns(decode_bf16=_decode_truncates),
    "grouped_shared_gram": _ns(grouped_grams=_grouped_shares),
    "entries_wrong_column": _ns(gram_entries=_entries_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mutant = MUTANTS[name]
    failures = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # AssertionError, or a shape error from a wrong operand
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake {name!r}"


# ------------------------------------------------------- generator checks --

def test_bf16_rounding_matches_torch():
    """The generator's float32 -> bf16 rounding is round-to-nearest-even, as torch's."""
    import torch
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(1 << 16) * np.exp(rng.uniform(-20, 20, 1 << 16))).astype(np.float32)
    x[:4] = [1.0009765625, 1.00390625, 1.01171875, -0.0]  # includes exact ties
    ours = W.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_moe_routing_structure():
    rng = np.random.default_rng(3)
    T = 4096
    row_idx, offsets = W.moe_routing(rng, T, experts=64, topk=8)
    assert offsets[0] == 0 and offsets[-1] == 8 * T
    assert np.all(np.diff(offsets) >= 0)
    # every token appears in exactly 8 distinct experts
    counts = np.bincount(row_idx, minlength=T)
    assert np.all(counts == 8)
    for e in range(64):
        seg = row_idx[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)  # ascending, distinct within an expert
    # Zipf popularity: expert 0 is routed far more often than expert 63
    sizes = np.diff(offsets)
    assert sizes[0] > 4 * sizes[63]


def test_tiny_case_recipe():
    w = W.tiny_case()
    assert w.d == 256 and [b.shape[0] for b in w.batches] == [100, 37, 0]
    assert w.total_tokens == 137
    acc = O.GramAccumulator(256)
    for b in w.batches:
        acc.add_batch(b, "f32")
    H, dead, damp = acc.materialize(0.01)
    assert acc.N == 137 and not dead.any()
    assert 1.5 < np.mean(np.diag(H)) - damp < 2.5
