"""Error-propagating 4-bit block quantization: HIP path vs the float64 oracle.

Both sides work in float64, so every code decision is the same float64 division and rounding;
the only difference is the order in which the propagated updates are added (blocks of 128
columns on the GPU, one column at a time in the oracle), about 1e-16 relative, which could flip
a code only at a rounding tie that close.  Codes are therefore compared exactly; dequantized
weights and steps to their float32 rounding; the loss to 1e-9 relative.  Rows are independent,
so at full size a sample of rows is compared in full.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import gptq_hessian_accumulation_amd as hs
from tests.helpers import quantize_against_gpu_ties

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def factor_for(K, seed, dead=()):
    """float32 upper factor of the inverse damped Hessian of seeded activations (from the oracle)."""
    rng = np.random.default_rng(seed)
    x = W.normal_rows(rng, 2 * K + 11, K, W.column_scales(rng, K))
    x[:, list(dead)] = 0.0
    acc = O.GramAccumulator(K)
    acc.add_batch(x, "f32")
    H, _, _ = acc.materialize(0.01)
    return O.chol_inverse_upper(H).astype(np.float32)


def weights(N, K, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)) * 0.02).astype(np.float32)


def compare(Wt, U, group, got, dead=None, nsamples=1, rows=None):
    """Codes exactly, except at rounding ties (both neighbours correct): the oracle reports each
    tie, the checker takes the GPU's code there when it is one of the two neighbours, and both
    sides must then agree on everything after it."""
    Q, codes, scales, loss = got
    Wr = Wt if rows is None else Wt[rows]
    Qg = Q.cpu().numpy().astype(np.float64)
    cg = codes.cpu().numpy()
    sg = scales.cpu().numpy().astype(np.float64)
    if rows is not None:
        Qg, cg, sg = Qg[rows], cg[rows], sg[rows]
    (Qr, cr, sr, lr), (ties, taken) = quantize_against_gpu_ties(Wr.astype(np.float64), U.astype(np.float64), group,
                                                               cg, dead=dead, nsamples=nsamples)
    print(f"  rounding ties: {ties}; the GPU took the other neighbour at {taken} of them; {cr.size} codes")
    assert np.array_equal(cg, cr), f"{int((cg != cr).sum())} codes differ"
    assert np.all(np.abs(Qg - Qr) <= 2.0 ** -23 * np.abs(Qr)), float(np.max(np.abs(Qg - Qr)))
    assert np.all(np.abs(sg - sr) <= 2.0 ** -23 * np.abs(sr))
    if rows is None:
        lg = float(loss.cpu()[0])
        assert abs(lg - lr) <= 1e-9 * max(abs(lr), 1e-300), (lg, lr)


@pytest.mark.parametrize("N,K,group", [(5, 6, -1), (17, 130, -1), (64, 128, 128), (100, 300, 32), (33, 257, 64),
                                       (70, 1024, 128), (65, 384, 384), (3, 200, 1)])
def test_gptq_quantize_parity(N, K, group):
    _say(f"gptq quantize N={N} K={K} group={group}")
    U = factor_for(K, seed=500 + K)
    Wt = weights(N, K, seed=600 + N)
    got = hs.gptq_quantize(torch.from_numpy(Wt).cuda(), torch.from_numpy(U).cuda(), group_size=group, nsamples=13)
    compare(Wt, U, group, got, nsamples=13)


def test_gptq_quantize_dead_columns_and_in_place():
    """Dead columns are zeroed first (centre codes, zero weights); Q written over W itself."""
    _say("gptq quantize dead columns / in place")
    N, K = 48, 256
    dead = [3, 100, 255]
    U = factor_for(K, seed=77, dead=dead)
    Wt = weights(N, K, seed=78)
    mask = np.zeros(K, dtype=bool)
    mask[dead] = True
    Wd = torch.from_numpy(Wt).cuda()
    got = hs.gptq_quantize(Wd, torch.from_numpy(U).cuda(), group_size=128, dead=torch.from_numpy(mask), out=Wd)
    assert got[0].data_ptr() == Wd.data_ptr()
    compare(Wt, U, 128, got, dead=mask)
    assert (got[1].cpu().numpy()[:, dead] == 8).all()


@pytest.mark.parametrize("group", [128, -1])
def test_gptq_quantize_full_size_sampled_rows(group):
    """A 4,096 x 4,096 layer: rows are independent, so sampled rows are checked against the oracle
    in full (every column), and every code is in range."""
    _say(f"gptq quantize 4096 x 4096 group={group}")
    K = 4096
    rng = np.random.default_rng(9)
    x = W.normal_rows(rng, 2 * K, K, W.column_scales(rng, K))
    acc = O.GramAccumulator(K)
    acc.add_batch(x, "f32")
    H, _, _ = acc.materialize(0.01)
    U = O.chol_inverse_upper(H).astype(np.float32)
    Wt = weights(4096, K, seed=10)
    got = hs.gptq_quantize(torch.from_numpy(Wt).cuda(), torch.from_numpy(U).cuda(), group_size=group)
    rows = np.array([0, 1, 777, 2048, 4095])
    compare(Wt, U, group, got, rows=rows)
    assert int(got[1].max()) <= 15
