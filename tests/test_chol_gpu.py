"""Upper Cholesky factor of the inverse damped Hessian: HIP path vs the float64 oracle.

The factor is unique (upper triangular, positive diagonal), so the comparison is element by
element.  The HIP path works in float64 and rounds once to float32, so each entry may differ
from the oracle's by its own float32 rounding (2^-24 relative) plus the float64 error of either
side, bounded by d * cond(H) * 2^-53 relative to the largest entry.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import gptq_hessian_accumulation_amd as hs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def damped_hessian(d, n, seed, damp=0.01, dead_frac=0.0):
    """A float32 damped Hessian from seeded activations, built by the oracle (2/N X^T X,
    neutralized, damped), then rounded to float32: the input both sides receive."""
    rng = np.random.default_rng(seed)
    x = W.normal_rows(rng, n, d, W.column_scales(rng, d))
    dead = W.dead_columns(rng, d, dead_frac)
    x[:, dead] = 0.0
    acc = O.GramAccumulator(d)
    acc.add_batch(x, "f32")
    H, _, _ = acc.materialize(damp)
    return H.astype(np.float32)


def check_factor(H32, U):
    """U (float32, from the GPU) against the oracle's factor of the same float32 H."""
    H = H32.astype(np.float64)
    d = H.shape[0]
    U_ref = O.chol_inverse_upper(H)
    Ug = U.astype(np.float64)
    assert np.array_equal(np.tril(Ug, -1), np.zeros_like(Ug)), "U must be zero below the diagonal"
    assert (np.diag(Ug) > 0).all()
    cond = np.linalg.cond(H)
    scale = float(np.max(np.abs(U_ref)))
    bound = 2.0 ** -23 * np.abs(U_ref) + d * cond * 2.0 ** -53 * scale
    err = np.abs(Ug - U_ref)
    worst = float(np.max(err / bound))
    print(f"  d={d} cond={cond:.3e} max|dU|/max|U|={float(err.max()) / scale:.3e} worst/bound={worst:.3f}")
    assert worst <= 1.0, worst
    return worst


@pytest.mark.parametrize("d", [1, 5, 63, 64, 65, 130, 257, 700])
def test_chol_inverse_upper_parity(d):
    _say(f"chol inverse upper d={d}")
    H32 = damped_hessian(d, 2 * d + 7, seed=300 + d, dead_frac=0.05 if d > 60 else 0.0)
    U = hs.chol_inverse_upper(torch.from_numpy(H32).cuda())
    check_factor(H32, U.cpu().numpy())


@pytest.mark.parametrize("d,n", [(2560, 5120), (4096, 8192)])
def test_chol_inverse_upper_full_size(d, n):
    """The widths of the ragged-batch Hessians, every entry compared."""
    _say(f"chol inverse upper full size d={d}")
    H32 = damped_hessian(d, n, seed=7 + d)
    U = hs.chol_inverse_upper(torch.from_numpy(H32).cuda())
    check_factor(H32, U.cpu().numpy())


def test_chol_in_place_and_strided():
    """U written over H itself; H read through a row stride larger than d."""
    _say("chol in place / strided")
    d = 200
    H32 = damped_hessian(d, 500, seed=41)
    big = torch.zeros((d, d + 24), dtype=torch.float32, device="cuda")
    big[:, :d] = torch.from_numpy(H32).cuda()
    view = big[:, :d]
    U = hs.chol_inverse_upper(view, out=view)
    assert U.data_ptr() == view.data_ptr()
    check_factor(H32, U.cpu().numpy())
    assert not big[:, d:].any(), "columns past d must be left alone"
    # only the upper triangle of H is read: garbage below it changes nothing
    Hg = torch.from_numpy(H32).cuda()
    Hl = Hg.clone()
    Hl.view(-1)[torch.tril(torch.ones(d, d, dtype=torch.bool, device="cuda"), -1).view(-1)] = float("nan")
    assert torch.equal(hs.chol_inverse_upper(Hg), hs.chol_inverse_upper(Hl))


def test_chol_not_positive_definite():
    """A failed pivot is reported (1 + the largest failing H column) and raised; nothing hangs."""
    _say("chol not positive definite")
    d = 100
    H = np.eye(d, dtype=np.float32)
    H[37, 37] = -1.0
    U, info = hs.chol_inverse_upper(torch.from_numpy(H).cuda(), check=False)
    assert int(info.item()) == 38
    with pytest.raises(hs.HessError) as ei:
        hs.chol_inverse_upper(torch.from_numpy(H).cuda())
    assert ei.value.code == -6
    # an all-zero H (nothing accumulated, no damping): the first pivot taken, H's last column, fails
    _, info = hs.chol_inverse_upper(torch.zeros((70, 70), dtype=torch.float32, device="cuda"), check=False)
    assert int(info.item()) == 70
    # indefinite 2 x 2 block at the end of H: its last column fails first... or the one before
    H = np.eye(d, dtype=np.float32)
    H[98:, 98:] = [[1.0, 2.0], [2.0, 1.0]]
    _, info = hs.chol_inverse_upper(torch.from_numpy(H).cuda(), check=False)
    assert int(info.item()) == 99   # H[99,99] = 1 passes; the Schur complement at column 98 is -3
    # a good call after failed ones still succeeds
    H32 = damped_hessian(64, 300, seed=5)
    check_factor(H32, hs.chol_inverse_upper(torch.from_numpy(H32).cuda()).cpu().numpy())
