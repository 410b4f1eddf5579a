"""HIP path vs the float64 oracle, element by element, through the C ABI.

Small and medium shapes that span several tiles and ragged tails are compared
in full; the edge cases of the method (empty batches, N = 0, dead columns,
odd widths, unaligned rows) are covered; exactness cases (the pages' worked
example, dyadic inputs whose every float32 sum is exact) are compared bitwise.
"""

import ctypes
import gc
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import gptq_hessian_accumulation_amd as hs
from tests.helpers import TOL, agreement, block_agreement, quantize_against_gpu_ties, to_device, torch_dtype

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _defaults():
    hs.set_tile_override(0)
    hs.set_staging(True)
    hs.set_group_direct(True)
    yield
    hs.set_tile_override(0)
    hs.set_staging(True)
    hs.set_group_direct(True)


def run_lib(wl: W.Workload, damp=0.01, neutralize=True):
    h = hs.Hessian(wl.d, torch_dtype(wl.dtype))
    for b in wl.batches:
        h.add_batch(to_device(b, wl.dtype))
    H, dead, dmp = h.materialize(damp, neutralize=neutralize)
    torch.cuda.synchronize()
    out = H.cpu().numpy(), dead.cpu().numpy(), float(dmp.cpu()[0]), h.nsamples
    h.close()
    return out


def run_oracle(wl: W.Workload, damp=0.01, neutralize=True):
    acc = O.GramAccumulator(wl.d)
    for b in wl.batches:
        acc.add_batch(b, wl.dtype)
    H, dead, dmp = acc.materialize(damp, neutralize)
    return H, dead, dmp, acc.N


def check_against_oracle(wl: W.Workload, tol=None):
    tol = TOL[wl.dtype] if tol is None else tol
    for damp, neut in ((0.0, False), (0.01, True)):
        H, dead, dmp, N = run_lib(wl, damp, neut)
        Hr, deadr, dmpr, Nr = run_oracle(wl, damp, neut)
        assert N == Nr
        assert np.array_equal(dead, deadr)
        err = agreement(H, Hr)
        assert err <= tol, f"agreement {err:.3e} > {tol:.1e} (damp={damp}, neutralize={neut})"
        assert np.array_equal(H, H.T), "H must be bitwise symmetric"
        assert abs(dmp - dmpr) <= 1e-6 * max(abs(dmpr), 1e-30) + 1e-30
    return err


# ------------------------------------------------------------ small cases --

def test_tiny_case_fp32():
    _say("tiny d=256 fp32 100/37/0")
    wl = W.tiny_case()
    check_against_oracle(wl)


@pytest.mark.parametrize("staging", [True, False])
@pytest.mark.parametrize("d", [384, 520, 700])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_ragged_batches(d, dtype, staging):
    """Short batches go through the staging buffer (when enabled), long ones straight to the SYRK."""
    _say(f"ragged d={d} {dtype} staging={staging}")
    hs.set_staging(staging)
    sizes = [1, 63, 64, 65, 777, 0, 1500]
    wl = W.ragged_case(d, sizes, seed=100 + d, dtype=dtype, dead_frac=0.02)
    check_against_oracle(wl)


@pytest.mark.parametrize("d", [1, 17, 255, 257])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_edge_widths(d, dtype):
    _say(f"edge width d={d} {dtype}")
    wl = W.ragged_case(d, [3, 129, 1], seed=7 + d, dtype=dtype)
    check_against_oracle(wl)


@pytest.mark.parametrize("edge", [64, 128, 256])
def test_forced_tile_edges(edge):
    _say(f"forced tile {edge}")
    hs.set_tile_override(edge)
    wl = W.ragged_case(1000, [300, 2000], seed=55, dtype=W.BF16)
    check_against_oracle(wl)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("override", [0, 64])
@pytest.mark.parametrize("d", [8, 64, 72, 264, 1000, 2056])
def test_thin_tiles(d, override, dtype):
    """Batches added straight into S: the 64-tile kernel up to 512 tokens (edge
    and diagonal tiles, partial 32-token steps), the 128- or 256-tile kernels
    from 513 on."""
    _say(f"thin 64-tile d={d} override={override} {dtype}")
    hs.set_tile_override(override)
    hs.set_staging(False)
    wl = W.ragged_case(d, [1, 5, 31, 32, 33, 100, 0, 511, 512, 513], seed=900 + d, dtype=dtype, dead_frac=0.02)
    check_against_oracle(wl)


def test_thin_tiles_full_width_and_strided_rows():
    """Width 4,096 with 64-token batches straight into S (the thin-batch
    measurement's shape), one of them with a row stride wider than d."""
    _say("thin 64-tile d=4096, strided rows")
    hs.set_staging(False)
    d = 4096
    wl = W.ragged_case(d, [64, 1, 64, 200], seed=77, dtype=W.BF16, dead_frac=0.01)
    h = hs.Hessian(d, torch.bfloat16)
    for i, b in enumerate(wl.batches):
        xb = to_device(b, wl.dtype)
        if i == 2:
            wide = torch.zeros((xb.shape[0], d + 8), dtype=xb.dtype, device=xb.device)
            wide[:, :d] = xb
            xb = wide[:, :d]
        h.add_batch(xb)
    H, dead, _ = h.materialize(0.01)
    Hr, deadr, _, Nr = run_oracle(wl)
    assert h.nsamples == Nr
    assert np.array_equal(dead.cpu().numpy(), deadr)
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    h.close()


@pytest.mark.parametrize("staging", [True, False])
@pytest.mark.parametrize("d", [8, 256, 264, 520, 696, 1032])
def test_big_tiles_ragged(d, staging):
    """The 256-tile kernel at any batch length: one-token tiles, partial stream-K shares, edge tiles."""
    _say(f"256-tile ragged d={d} staging={staging}")
    hs.set_tile_override(256)
    hs.set_staging(staging)
    wl = W.ragged_case(d, [1, 31, 33, 100, 1000, 0, 3000], seed=300 + d, dtype=W.BF16, dead_frac=0.02)
    check_against_oracle(wl)


@pytest.mark.parametrize("d", [1032, 2048])
def test_transposed_staging_ragged(d):
    """bf16 at widths >= 1,024 with the default staging buffer stages in the 256-tile kernel's
    transposed layout: batch lengths that are not multiples of 8 (zero-padded blocks), a long
    batch between staged ones (the staged rows are flushed first), and a final partial flush."""
    _say(f"transposed staging ragged d={d}")
    sizes = [1, 7, 9, 500, d - 1, 3, 2 * d + 5, 17, 800, 8, 0, 255]
    wl = W.ragged_case(d, sizes, seed=500 + d, dtype=W.BF16, dead_frac=0.02)
    check_against_oracle(wl)


def test_transposed_staging_overflow():
    """A 256-token transposed staging buffer (tile override 256 at create) overflows and is
    flushed again and again; padded batch lengths count toward its capacity."""
    _say("transposed staging overflow d=520")
    hs.set_tile_override(256)
    d = 520
    wl = W.ragged_case(d, [100, 101, 99, 7, 250, 1, 249, 64, 65, 0, 200], seed=77, dtype=W.BF16, dead_frac=0.02)
    H = None
    for damp, neut in ((0.0, False), (0.01, True)):
        h = hs.Hessian(d, torch.bfloat16, staging_bytes=300 * 2 * d)
        for b in wl.batches:
            h.add_batch(to_device(b, W.BF16))
        H, dead, dmp = h.materialize(damp, neutralize=neut)
        torch.cuda.synchronize()
        Hr, deadr, dmpr, Nr = run_oracle(wl, damp, neut)
        assert h.nsamples == Nr
        assert np.array_equal(dead.cpu().numpy(), deadr)
        err = agreement(H.cpu().numpy(), Hr)
        assert err <= TOL[W.BF16], err
        h.close()


def test_transposed_staging_unaligned_rows():
    """Rows that are not 16-byte aligned (odd row stride) take the element-wise transposed copy."""
    _say("transposed staging unaligned rows d=1032")
    d = 1032
    wl = W.ragged_case(d, [5, 300, 41], seed=91, dtype=W.BF16, dead_frac=0.0)
    h = hs.Hessian(d, torch.bfloat16)
    for b in wl.batches:
        xb = to_device(b, W.BF16)
        wide = torch.zeros((xb.shape[0], d + 1), dtype=torch.bfloat16, device=xb.device)
        wide[:, :d] = xb
        h.add_batch(wide[:, :d])                       # row stride d + 1 elements
    H, dead, dmp = h.materialize(0.01)
    torch.cuda.synchronize()
    Hr, deadr, dmpr, Nr = run_oracle(wl, 0.01, True)
    assert h.nsamples == Nr
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    h.close()


def _sampled_gram_check(h, wl, n_samples=400, seed=0):
    """Compare sampled upper entries and the whole diagonal of S with the oracle's exact sums."""
    d = wl.d
    h.flush()
    S = h.state_tensor()
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, d, n_samples)
    cols = rng.integers(0, d, n_samples)
    # always include the corners of the last (edge) tile and a diagonal-tile pair
    rows = np.concatenate([rows, [d - 1, 0, d - 1, d // 2]])
    cols = np.concatenate([cols, [d - 1, d - 1, 0, d // 2 + 1]])
    up_r, up_c = np.minimum(rows, cols), np.maximum(rows, cols)
    diag = np.arange(d)
    r_all, c_all = np.concatenate([up_r, diag]), np.concatenate([up_c, diag])
    ref = O.gram_entries(wl.batches, wl.dtype, r_all, c_all)
    got = S[torch.from_numpy(r_all).cuda(), torch.from_numpy(c_all).cuda()].double().cpu().numpy()
    N = wl.total_tokens
    mean_diag = float(np.mean(ref[len(up_r):])) * 2.0 / N
    return float(np.max(np.abs(got - ref))) * 2.0 / N / mean_diag


@pytest.mark.parametrize("d,n", [(2560, 13056), (4096, 16384), (5888, 700)])
def test_big_tiles_full_size_sampled(d, n):
    """Full-width batches on the 256-tile kernel: a staged flush at width 2,560, a long batch at
    4,096, and width 5,888 (256 whole tiles plus stream-K tiles), on sampled entries."""
    _say(f"256-tile sampled d={d} n={n}")
    hs.set_tile_override(256)
    hs.set_staging(False)
    wl = W.ragged_case(d, [n], seed=400 + d, dtype=W.BF16, dead_frac=0.0)
    h = hs.Hessian(d, torch.bfloat16)
    h.add_batch(to_device(wl.batches[0], W.BF16))
    err = _sampled_gram_check(h, wl)
    assert h.nsamples == n
    assert err <= TOL[W.BF16], err
    h.close()


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_thin_tiles_widest_sampled(dtype):
    """The thin-batch kernel at width 32,768 (131,328 tiles of 64, a 4 GiB sum):
    batches of 1, 64 and 300 tokens straight into S, on sampled entries."""
    _say(f"thin 64-tile d=32768 {dtype}")
    hs.set_staging(False)
    d = 32768
    wl = W.ragged_case(d, [1, 64, 300], seed=3276, dtype=dtype, dead_frac=0.0)
    h = hs.Hessian(d, torch_dtype(dtype), staging_bytes=0)
    for b in wl.batches:
        h.add_batch(to_device(b, dtype))
    err = _sampled_gram_check(h, wl)
    assert h.nsamples == 365
    assert err <= TOL[dtype], err
    h.close()
    torch.cuda.empty_cache()


def test_widest_handle_sampled():
    """The widest handle the API accepts (d = 65,536: a 16 GiB sum, 524,800 tiles of 64) with 1%
    zeroed columns: 1- and 64-token bf16 batches straight into S (64-tile kernel) and a 600-token
    one (128-tile kernel), on sampled entries and the whole diagonal; then the materialize: dead
    mask bitwise, the damping, and sampled H entries, from the oracle's exact sums through the
    oracle's materialize rule (2/N, neutralized dead columns, p * mean(diag H) on the diagonal)."""
    _say("widest handle d=65536")
    hs.set_staging(False)
    d = 65536
    wl = W.ragged_case(d, [1, 64, 600], seed=6553, dtype=W.BF16, dead_frac=0.01)
    h = hs.Hessian(d, torch.bfloat16, staging_bytes=0)
    for b in wl.batches:
        h.add_batch(to_device(b, W.BF16))
    err = _sampled_gram_check(h, wl, n_samples=300, seed=65)
    assert h.nsamples == 665
    assert err <= TOL[W.BF16], err
    H, dead, damp = h.materialize(0.01)
    torch.cuda.synchronize()
    diag = np.arange(d)
    sdiag = O.gram_entries(wl.batches, W.BF16, diag, diag)
    N = wl.total_tokens
    dead_r = sdiag == 0.0
    assert np.array_equal(dead.cpu().numpy(), dead_r)
    assert np.array_equal(np.flatnonzero(dead_r), wl.dead_cols)
    hdiag = np.where(dead_r, 1.0, sdiag * (2.0 / N))
    damp_r = 0.01 * float(np.mean(hdiag))
    assert abs(float(damp.cpu()[0]) - damp_r) <= 1e-6 * damp_r
    rng = np.random.default_rng(66)
    r = rng.integers(0, d, 300)
    c = rng.integers(0, d, 300)
    r = np.concatenate([r, wl.dead_cols[:3], diag[:3]])
    c = np.concatenate([c, rng.integers(0, d, 3), diag[:3]])
    sv = O.gram_entries(wl.batches, W.BF16, np.minimum(r, c), np.maximum(r, c)) * (2.0 / N)
    sv = np.where(dead_r[r] | dead_r[c], 0.0, sv)
    sv = np.where(r == c, np.where(dead_r[r], 1.0, sv) + damp_r, sv)
    got = H[torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda()].double().cpu().numpy()
    assert np.max(np.abs(got - sv)) / float(np.mean(hdiag)) <= TOL[W.BF16]
    del H
    h.close()
    torch.cuda.empty_cache()


def test_transposed_staging_full_flush_sampled():
    """One full default staging buffer at width 2,560 (209,664 tokens in 2,000-token batches,
    the longest staged flush at this width) against the oracle's exact sums."""
    _say("transposed staging full flush d=2560")
    d = 2560
    sizes = [2000] * 104 + [1664]
    wl = W.ragged_case(d, sizes, seed=2560, dtype=W.BF16, dead_frac=0.0)
    h = hs.Hessian(d, torch.bfloat16)
    for b in wl.batches:
        h.add_batch(to_device(b, W.BF16))
    err = _sampled_gram_check(h, wl)
    assert h.nsamples == sum(sizes)
    assert err <= TOL[W.BF16], err
    h.close()


def test_big_tiles_chosen_automatically():
    """Width 4,096 with 24,576 tokens (408 iterations per workgroup) takes the 256-tile kernel
    without an override; the result is checked on sampled entries."""
    _say("256-tile automatic choice d=4096 n=24576")
    hs.set_staging(False)
    wl = W.ragged_case(4096, [24576], seed=78, dtype=W.BF16, dead_frac=0.0)
    h = hs.Hessian(4096, torch.bfloat16)
    h.add_batch(to_device(wl.batches[0], W.BF16))
    err = _sampled_gram_check(h, wl)
    assert err <= TOL[W.BF16], err
    h.close()


def test_staging_buffer_overflow_and_flush():
    """d=8192 bf16 with a 64 MiB staging buffer: 4,096 staged tokens fill it; later batches flush it first."""
    _say("staging overflow d=8192")
    d = 8192
    wl = W.ragged_case(d, [1500, 1500, 1500, 1500, 100], seed=61, dtype=W.BF16, dead_frac=0.0)
    h = hs.Hessian(d, torch.bfloat16, staging_bytes=64 << 20)
    for b in wl.batches:
        h.add_batch(to_device(b, W.BF16))
    h.flush()
    S = h.state_tensor()
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = rng.integers(0, d, 400)
    cols = rng.integers(0, d, 400)
    up_r, up_c = np.minimum(rows, cols), np.maximum(rows, cols)
    diag = np.arange(d)
    ref_s = O.gram_entries(wl.batches, W.BF16, np.concatenate([up_r, diag]), np.concatenate([up_c, diag]))
    got = S[torch.from_numpy(np.concatenate([up_r, diag])).cuda(), torch.from_numpy(np.concatenate([up_c, diag])).cuda()]
    got = got.double().cpu().numpy()
    N = wl.total_tokens
    mean_diag = float(np.mean(ref_s[len(up_r):])) * 2.0 / N
    err = float(np.max(np.abs(got - ref_s))) * 2.0 / N / mean_diag
    assert h.nsamples == N
    assert err <= TOL[W.BF16], err
    h.close()


def test_worked_example_bitwise():
    """One token with component 1 + 2^-10: fp32 input gives 2.003908157348633, bf16 input 2.0."""
    _say("worked example")
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = 1.0009765625
    for dtype, expect in ((W.F32, 2.003908157348633), (W.BF16, 2.0)):
        wl = W.Workload(d=16, dtype=dtype, batches=[W.encode(x, dtype)])
        H, dead, dmp, N = run_lib(wl, damp=0.0, neutralize=False)
        assert N == 1
        assert H[0, 0] == np.float32(expect)
        assert not H[1:, :].any() and not H[0, 1:].any()


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_dyadic_inputs_exact(dtype):
    """Values in {-2..2}/4 keep every float32 partial sum exact, so S is unique; N = 256 makes 2/N exact."""
    _say(f"dyadic exact {dtype}")
    rng = np.random.default_rng(31)
    d = 300
    batches = [(rng.integers(-2, 3, size=(n, d)) / 4.0).astype(np.float32) for n in (100, 0, 156)]
    wl = W.Workload(d=d, dtype=dtype, batches=[W.encode(b, dtype) for b in batches])
    H, dead, dmp, N = run_lib(wl, damp=0.0, neutralize=False)
    Hr, _, _, Nr = run_oracle(wl, damp=0.0, neutralize=False)
    assert N == Nr == 256
    assert np.array_equal(H.astype(np.float64), Hr)


def test_empty_accumulator():
    _say("N = 0")
    for dtype in (W.BF16, W.F32):
        wl = W.Workload(d=70, dtype=dtype, batches=[np.zeros((0, 70), dtype=np.uint16 if dtype == W.BF16
                                                            else np.float32)])
        H, dead, dmp, N = run_lib(wl, damp=0.01)
        assert N == 0 and dead.all()
        assert np.array_equal(H, np.float32(1.01) * np.eye(70, dtype=np.float32))
        assert dmp == np.float32(0.01)


def test_dead_columns_and_damping():
    _say("dead columns and damping")
    wl = W.ragged_case(600, [500, 300], seed=9, dtype=W.BF16, dead_frac=0.05)
    H1, dead1, d1, _ = run_lib(wl, damp=0.05)
    H0, dead0, d0, _ = run_lib(wl, damp=0.0)
    assert np.array_equal(np.flatnonzero(dead1), wl.dead_cols)
    assert np.array_equal(dead0, dead1)
    assert d0 == 0.0
    # H(p) - H(0) is the damping on the diagonal only
    diff = H1.astype(np.float64) - H0.astype(np.float64)
    assert np.array_equal(diff - np.diag(np.diag(diff)), np.zeros_like(diff))
    # (h + damp) is rounded once in float32: within half an ulp of the largest diagonal
    ulp = float(np.spacing(np.float32(np.max(np.diag(H1)))))
    assert np.allclose(np.diag(diff), d1, rtol=0, atol=ulp)
    assert np.all(np.diag(H0)[wl.dead_cols] == 1.0)
    assert not H0[wl.dead_cols][:, np.setdiff1d(np.arange(600), wl.dead_cols)].any()
    np.linalg.cholesky(H1.astype(np.float64))


def test_materialize_repeatable_and_accumulation_continues():
    _say("materialize twice, continue")
    wl = W.ragged_case(256, [200, 100, 50], seed=12, dtype=W.BF16)
    h = hs.Hessian(256, torch.bfloat16)
    h.add_batch(to_device(wl.batches[0], W.BF16))
    A, _, _ = h.materialize(0.01)
    B, _, _ = h.materialize(0.01)
    assert torch.equal(A, B)
    for b in wl.batches[1:]:
        h.add_batch(to_device(b, W.BF16))
    C, _, _ = h.materialize(0.01)
    Hr, _, _, _ = run_oracle(wl, 0.01)
    assert agreement(C.cpu().numpy(), Hr) <= TOL[W.BF16]
    assert h.nsamples == 350
    h.close()


@pytest.mark.parametrize("d,n,dtype", [(200, 150, W.F32), (264, 100, W.BF16), (1032, 1000, W.BF16)])
def test_in_place_materialize_consumes_handle(d, n, dtype):
    """After an in-place materialize the buffer holds H (both triangles); reset
    clears the sum's region only, and a new accumulation over it is exact
    again (128-tile, 64-tile and 256-tile kernels)."""
    _say(f"in-place materialize d={d} n={n} {dtype}")
    wl = W.ragged_case(d, [n], seed=13, dtype=dtype)
    h = hs.Hessian(d, torch_dtype(dtype))
    h.add_batch(to_device(wl.batches[0], dtype))
    ref, _, _ = h.materialize(0.01)
    dead, damp = h.materialize_in_place(0.01)
    torch.cuda.synchronize()
    with pytest.raises(hs.HessError) as e:
        h.add_batch(to_device(wl.batches[0], dtype))
    assert e.value.code == -4
    # the state buffer now holds H
    buf = h.state_tensor().clone()
    assert torch.equal(buf, ref)
    h.reset()
    h.add_batch(to_device(wl.batches[0], dtype))
    again, _, _ = h.materialize(0.01)
    assert torch.equal(again, ref)
    h.close()


def test_two_streams_are_ordered():
    _say("two streams")
    wl = W.ragged_case(512, [800, 800, 800, 800], seed=14, dtype=W.BF16)
    xs = [to_device(b, W.BF16) for b in wl.batches]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    h = hs.Hessian(512, torch.bfloat16)
    for i, x in enumerate(xs):
        h.add_batch(x, stream=s1 if i % 2 == 0 else s2)
    H, _, _ = h.materialize(0.01, stream=s1)
    s1.synchronize()
    Hr, _, _, _ = run_oracle(wl, 0.01)
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    h.close()


def test_staging_size_zero_disables_staging():
    _say("staging_bytes=0")
    wl = W.ragged_case(520, [3, 200, 1], seed=91, dtype=W.BF16)
    h = hs.Hessian(520, torch.bfloat16, staging_bytes=0)
    h.set_timing(True)
    for b in wl.batches:
        h.add_batch(to_device(b, W.BF16))
    launches, tokens, _ = h.timing()
    assert (launches, tokens) == (3, 204)   # every batch had its own pass
    H, _, _ = h.materialize(0.0, neutralize=False)
    Hr, _, _, _ = run_oracle(wl, 0.0, False)
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    h.close()


def test_add_batch_allocates_nothing():
    _say("zero allocation")
    h = hs.Hessian(1024, torch.bfloat16)
    x = torch.randn(1500, 1024, device="cuda").to(torch.bfloat16)
    thin = x[:300]                      # fewer tokens than d: goes through the staging buffer
    # Warm every path once (code objects load lazily), and drop garbage left by
    # earlier tests so that torch frees nothing during the measured loop.
    h.add_batch(x)
    h.add_batch(thin)
    h.flush()
    gc.collect()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(30):
        h.add_batch(x)
        h.add_batch(thin)
    h.flush()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0
    h.close()


def test_flattened_leading_dims_and_strided_rows():
    _say("3-D input and strided rows")
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 50, 96)).astype(np.float32)
    big = np.zeros((200, 128), dtype=np.float32)
    big[:, :96] = x.reshape(200, 96)
    h = hs.Hessian(96, torch.float32)
    h.add_batch(torch.from_numpy(x).cuda())                 # (4, 50, 96) -> 200 tokens
    h.add_batch(torch.from_numpy(big).cuda()[:, :96])       # row stride 128
    H, _, _ = h.materialize(0.0, neutralize=False)
    acc = O.GramAccumulator(96)
    acc.add_batch(x.reshape(200, 96), W.F32)
    acc.add_batch(big[:, :96].copy(), W.F32)
    Hr, _, _ = acc.materialize(0.0, neutralize=False)
    assert h.nsamples == 400
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.F32]
    h.close()


def test_nan_propagates():
    _say("NaN input")
    x = np.ones((4, 32), dtype=np.float32)
    x[2, 5] = np.nan
    h = hs.Hessian(32, torch.float32)
    h.add_batch(torch.from_numpy(x).cuda())
    H, dead, damp = h.materialize(0.01)
    Hn = H.cpu().numpy()
    assert np.isnan(Hn[5, 5]) and np.isnan(Hn[5, 0]) and not dead.cpu().numpy()[5]
    h.close()


# ----------------------------------------------------------- local blocks --

@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("n,d", [(1000, 512), (77, 48), (4096, 272), (300, 65536)])
def test_local_blocks(dtype, n, d):
    _say(f"local blocks n={n} d={d} {dtype}")
    rng = np.random.default_rng(40 + n)
    x = W.encode(W.normal_rows(rng, n, d, W.column_scales(rng, d)), dtype)
    x2 = W.encode(W.normal_rows(rng, n // 2 + 1, d), dtype)
    xt = to_device(x, dtype)
    out = hs.local_blocks(xt, accumulate=False)
    hs.local_blocks(to_device(x2, dtype), out=out, accumulate=True)
    torch.cuda.synchronize()
    ref = O.local_blocks(x, dtype) + O.local_blocks(x2, dtype)
    assert block_agreement(out.cpu().numpy(), ref) <= TOL[dtype]


def test_local_blocks_fixed_order_bitwise_repeatable():
    """Block sums go through per-workgroup partials added in a fixed order: two runs give the
    same bits (bf16 and float32, accumulate and overwrite)."""
    _say("local blocks repeatable")
    rng = np.random.default_rng(44)
    for dtype in (W.BF16, W.F32):
        x = to_device(W.encode(W.normal_rows(rng, 20000, 1024, W.column_scales(rng, 1024)), dtype), dtype)
        a = hs.local_blocks(x, accumulate=False)
        b = hs.local_blocks(x, accumulate=False)
        hs.local_blocks(x, out=a)
        hs.local_blocks(x, out=b)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("n", [100000, 300001, 600000])
def test_local_blocks_fp32_constant_column_and_long_chains(n):
    """float32 rows through exact-product float32 matrix instructions: a constant-valued column
    (every product the same, so a split into bf16 parts would err systematically) and long
    batches whose per-wave sums pass through a second accumulator every 2,048 tokens."""
    _say(f"local blocks fp32 constant column n={n}")
    rng = np.random.default_rng(45)
    d = 64
    x = W.normal_rows(rng, n, d, W.column_scales(rng, d))
    x[:, 5] = np.float32(1.2345679)
    x[:, 40] = np.float32(-3.0000002)
    ref = O.local_blocks(x, W.F32)
    out = hs.local_blocks(to_device(x, W.F32), accumulate=False)
    torch.cuda.synchronize()
    err = block_agreement(out.cpu().numpy(), ref)
    print(f"  fp32 local n={n}: {err:.3e}")
    assert err <= TOL[W.F32]
    xb = W.encode(x, W.BF16)
    outb = hs.local_blocks(to_device(xb, W.BF16), accumulate=False)
    torch.cuda.synchronize()
    errb = block_agreement(outb.cpu().numpy(), O.local_blocks(xb, W.BF16))
    print(f"  bf16 local n={n}: {errb:.3e}")
    assert errb <= TOL[W.BF16]


def test_local_blocks_match_full_path_diagonal_blocks():
    _say("local vs full diagonal blocks")
    rng = np.random.default_rng(41)
    x = W.encode(W.normal_rows(rng, 3000, 256), W.BF16)
    xt = to_device(x, W.BF16)
    B = hs.local_blocks(xt, accumulate=False)
    h = hs.Hessian(256, torch.bfloat16)
    h.add_batch(xt)
    H, _, _ = h.materialize(0.0, neutralize=False)
    S = H.double() * (3000 / 2.0)
    for b in range(16):
        sl = slice(16 * b, 16 * b + 16)
        ref = S[sl, sl]
        assert torch.allclose(B[b].double(), ref, rtol=2e-5, atol=1e-3)
    h.close()


# ---------------------------------------------------------------- grouped --

@pytest.mark.parametrize("gather", [True, False])
def test_grouped_experts(gather):
    _say(f"grouped experts gather={gather}")
    rng = np.random.default_rng(50)
    T, d, E, k = 1500, 384, 12, 3
    x = W.encode(W.normal_rows(rng, T, d, W.column_scales(rng, d)), W.BF16)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=k)
    hsx = [hs.Hessian(d, torch.bfloat16) for _ in range(E)]
    if gather:
        hs.add_batch_grouped(hsx, to_device(x, W.BF16), offsets, torch.from_numpy(row_idx).cuda())
        src, idx = x, row_idx
    else:
        xg = x[row_idx]
        hs.add_batch_grouped(hsx, to_device(xg, W.BF16), offsets)
        src, idx = xg, np.arange(xg.shape[0], dtype=np.int32)
    ref = O.grouped_grams(src, W.BF16, idx, offsets)
    for e in range(E):
        S_e, N_e = ref[e]
        assert hsx[e].nsamples == N_e
        H, _, _ = hsx[e].materialize(0.0, neutralize=False)
        Hr, _, _ = O.materialize(S_e, N_e, 0.0, neutralize=False)
        if N_e == 0:
            assert not H.cpu().numpy().any()
        else:
            assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
        hsx[e].close()


def _grouped_check(d, T, E, topk, seed, gather, chunk=0, empty=(), tol=None, direct=True):
    """Grouped update of E experts against the oracle's per-expert Gram sums (direct: the
    256-tile path reads the routed rows in place; otherwise it gathers them, in fills of at
    most chunk bytes when chunk > 0)."""
    rng = np.random.default_rng(seed)
    x = W.encode(W.normal_rows(rng, T, d, W.column_scales(rng, d)), W.BF16)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=topk)
    for e in empty:  # drop expert e's rows: an empty group
        n_e = offsets[e + 1] - offsets[e]
        row_idx = np.concatenate([row_idx[:offsets[e]], row_idx[offsets[e + 1]:]])
        offsets[e + 1:] -= n_e
    hsx = [hs.Hessian(d, torch.bfloat16, staging_bytes=0) for _ in range(E)]
    hs.set_group_chunk(chunk)
    hs.set_group_direct(direct)
    try:
        if gather:
            hs.add_batch_grouped(hsx, to_device(x, W.BF16), offsets, torch.from_numpy(row_idx).cuda())
            src, idx = x, row_idx
        else:
            xg = x[row_idx]
            hs.add_batch_grouped(hsx, to_device(xg, W.BF16), offsets)
            src, idx = xg, np.arange(xg.shape[0], dtype=np.int32)
    finally:
        hs.set_group_chunk(0)
        hs.set_group_direct(True)
    ref = O.grouped_grams(src, W.BF16, idx, offsets)
    for e in range(E):
        S_e, N_e = ref[e]
        assert hsx[e].nsamples == N_e
        H, _, _ = hsx[e].materialize(0.0, neutralize=False)
        Hr, _, _ = O.materialize(S_e, N_e, 0.0, neutralize=False)
        if N_e == 0:
            assert not H.cpu().numpy().any()
        else:
            assert agreement(H.cpu().numpy(), Hr) <= (TOL[W.BF16] if tol is None else tol), e
        hsx[e].close()


@pytest.mark.parametrize("direct", [True, False])
@pytest.mark.parametrize("gather", [True, False])
def test_grouped_big_tiles(gather, direct):
    """Width 1,032 (edge tiles) on the 256-tile grouped path: 9 experts, one of them empty,
    group sizes not multiples of 8 or 32; rows read in place or gathered first."""
    _say(f"grouped 256-tile gather={gather} direct={direct}")
    _grouped_check(1032, 700, 9, 3, seed=52, gather=gather, empty=(4,), direct=direct)


@pytest.mark.parametrize("chunk", [1032 * 16 * 3, 1032 * 16 * 40])
def test_grouped_big_tiles_refills(chunk):
    """A gather buffer of 3 (or 40) 8-row blocks: groups are split over many fills."""
    _say(f"grouped 256-tile refills chunk={chunk}")
    _grouped_check(1032, 500, 6, 2, seed=53, gather=True, chunk=chunk, direct=False)


def _grouped_states(d, x, offsets, ridx, direct):
    """Every expert's raw Gram sum after one grouped update on a given path."""
    E = len(offsets) - 1
    hsx = [hs.Hessian(d, torch.bfloat16, staging_bytes=0) for _ in range(E)]
    hs.set_group_direct(direct)
    try:
        hs.add_batch_grouped(hsx, x, offsets, ridx)
    finally:
        hs.set_group_direct(True)
    torch.cuda.synchronize()
    out = [(h.state_tensor().clone(), h.nsamples) for h in hsx]
    for h in hsx:
        h.close()
    return out


@pytest.mark.parametrize("d,T,E,topk", [(1032, 600, 70, 2), (2048, 3000, 16, 4), (2560, 2000, 9, 2)])
def test_grouped_direct_equals_gathered_bitwise(d, T, E, topk):
    """The rows read in place through the row table give the gathered path's bits exactly (the
    same operands in the same order): with row indices and without (rows already grouped),
    with an empty expert, and with more than 64 experts (two launches)."""
    _say(f"grouped direct == gathered d={d} T={T} E={E}")
    rng = np.random.default_rng(70 + d)
    x = W.encode(W.normal_rows(rng, T, d, W.column_scales(rng, d)), W.BF16)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=topk)
    n2 = offsets[3] - offsets[2]                               # expert 2: no tokens
    row_idx = np.concatenate([row_idx[:offsets[2]], row_idx[offsets[3]:]])
    offsets[3:] -= n2
    xt = to_device(x, W.BF16)
    ridx = torch.from_numpy(row_idx).cuda()
    a = _grouped_states(d, xt, offsets, ridx, direct=True)
    b = _grouped_states(d, xt, offsets, ridx, direct=False)
    for e in range(E):
        assert a[e][1] == b[e][1] == int(offsets[e + 1] - offsets[e])
        assert torch.equal(a[e][0], b[e][0]), e
    # rows already grouped (no row_idx): the table is the identity
    xg = xt[ridx.long()].contiguous()
    c = _grouped_states(d, xg, offsets, None, direct=True)
    for e in range(E):
        assert torch.equal(c[e][0], b[e][0]), e
    # and the oracle agrees
    ref = O.grouped_grams(x, W.BF16, row_idx, offsets)
    for e in range(E):
        S_e, N_e = ref[e]
        if N_e:
            Sg = np.triu(a[e][0].double().cpu().numpy())
            assert agreement(Sg * (2.0 / N_e), np.triu(S_e) * (2.0 / N_e)) <= TOL[W.BF16], e


def test_grouped_direct_long_group_chunks():
    """An expert with 40,000 routed rows (1,250 iterations: two chains of at most 1,024) beside a
    small one, read in place: the gathered path's bits, and the oracle's sums."""
    _say("grouped direct: a 40,000-row expert")
    rng = np.random.default_rng(75)
    d, T = 1032, 40000
    x = W.encode(W.normal_rows(rng, T, d, W.column_scales(rng, d)), W.BF16)
    big = rng.permutation(T).astype(np.int32)
    small = rng.integers(0, T, size=3000).astype(np.int32)
    row_idx = np.concatenate([big, small])
    offsets = np.array([0, T, T + 3000], dtype=np.int64)
    xt = to_device(x, W.BF16)
    ridx = torch.from_numpy(row_idx).cuda()
    a = _grouped_states(d, xt, offsets, ridx, direct=True)
    b = _grouped_states(d, xt, offsets, ridx, direct=False)
    ref = O.grouped_grams(x, W.BF16, row_idx, offsets)
    for e in range(2):
        assert torch.equal(a[e][0], b[e][0]), e
        S_e, N_e = ref[e]
        assert a[e][1] == N_e
        Sg = np.triu(a[e][0].double().cpu().numpy())
        assert agreement(Sg * (2.0 / N_e), np.triu(S_e) * (2.0 / N_e)) <= TOL[W.BF16], e


@pytest.mark.parametrize("rows", [(1 << 19) - 1, 1 << 19])
def test_grouped_rows_near_two_gib(rows):
    """X of 2,048 bf16 features and 2^19 - 1 rows (just under 2 GiB: read in place, row offsets up
    to 2^31 - 8 KiB) or 2^19 rows (2 GiB: gathered first), with the routed rows taken from both
    ends of X: the oracle's sums either way."""
    _say(f"grouped rows near 2 GiB: {rows} rows")
    d = 2048
    g = torch.Generator(device="cuda").manual_seed(76)
    x = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 1 << 16):
        r1 = min(rows, r0 + (1 << 16))
        x[r0:r1] = torch.randn((r1 - r0, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    rng = np.random.default_rng(76)
    ends = np.concatenate([np.arange(rows - 300, rows), np.arange(0, 200)]).astype(np.int32)
    rows_e = [rng.permutation(ends)[:350], rng.permutation(ends)[:90]]
    row_idx = np.concatenate(rows_e).astype(np.int32)
    offsets = np.array([0, 350, 440], dtype=np.int64)
    hsx = [hs.Hessian(d, torch.bfloat16, staging_bytes=0) for _ in range(2)]
    hs.add_batch_grouped(hsx, x, offsets, torch.from_numpy(row_idx).cuda())
    torch.cuda.synchronize()
    for e in range(2):
        xe = W.host_copy(x[torch.from_numpy(rows_e[e].astype(np.int64)).cuda()], W.BF16)
        ref = O.grouped_grams(xe, W.BF16, np.arange(xe.shape[0], dtype=np.int32),
                              np.array([0, xe.shape[0]], dtype=np.int64))[0][0]
        Sg = np.triu(hsx[e].state_tensor().double().cpu().numpy())
        assert hsx[e].nsamples == len(rows_e[e])
        assert agreement(Sg, np.triu(ref)) <= TOL[W.BF16], e
        hsx[e].close()
    del x
    torch.cuda.empty_cache()


def test_grouped_direct_rows_outside_x_read_as_zero():
    """Given X's row count, the in-place path reads a row index outside [0, n_rows) as a zero
    row (through the bounds of its buffer descriptor; it still counts toward N_e)."""
    _say("grouped direct: rows outside X")
    rng = np.random.default_rng(74)
    d, T, E = 1032, 400, 3
    x = W.encode(W.normal_rows(rng, T, d, W.column_scales(rng, d)), W.BF16)
    rows = [rng.integers(0, T, size=150).astype(np.int32) for _ in range(E)]
    rows[1][[0, 7, 149]] = [-1, T, 1 << 30]                   # three rows outside X
    row_idx = np.concatenate(rows)
    offsets = np.array([0, 150, 300, 450], dtype=np.int64)
    hsx = [hs.Hessian(d, torch.bfloat16, staging_bytes=0) for _ in range(E)]
    xt = to_device(x, W.BF16)
    # the in-place path only: bf16, d % 8 == 0, d >= 1,024, 16-byte aligned rows, X's row count known
    assert d >= 1024 and d % 8 == 0 and xt.data_ptr() % 16 == 0 and xt.stride(0) * 2 % 16 == 0
    hs.add_batch_grouped(hsx, xt, offsets, torch.from_numpy(row_idx).cuda())
    torch.cuda.synchronize()
    for e in range(E):
        keep = rows[e][(rows[e] >= 0) & (rows[e] < T)]
        ref = O.grouped_grams(x, W.BF16, keep, np.array([0, keep.size], dtype=np.int64))[0][0]
        assert hsx[e].nsamples == 150
        Sg = np.triu(hsx[e].state_tensor().double().cpu().numpy())
        assert agreement(Sg, np.triu(ref)) <= TOL[W.BF16], e
        hsx[e].close()


def test_grouped_moe_full_size_sampled():
    """The MoE workload at full size (32,768 tokens, top-8 of 64 experts, width 2,048): sampled
    entries and the whole diagonal of the largest, the smallest and two middle experts."""
    _say("grouped MoE full size")
    rng = np.random.default_rng(3)
    d, T, E = 2048, 32768, 64
    x = W.encode(W.normal_rows(rng, T, d, W.column_scales(rng, d)), W.BF16)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=8)
    hsx = [hs.Hessian(d, torch.bfloat16, staging_bytes=0) for _ in range(E)]
    hs.add_batch_grouped(hsx, to_device(x, W.BF16), offsets, torch.from_numpy(row_idx).cuda())
    sizes = np.diff(offsets)
    order = np.argsort(-sizes, kind="stable")
    for e in [int(order[0]), int(order[-1]), int(order[E // 3]), int(order[2 * E // 3])]:
        rows = row_idx[offsets[e]:offsets[e + 1]]
        wl = W.Workload(d=d, dtype=W.BF16, batches=[x[rows]], dead_cols=np.zeros(0, dtype=np.int64),
                        scales=np.ones(d))
        err = _sampled_gram_check(hsx[e], wl, n_samples=300, seed=e)
        assert hsx[e].nsamples == len(rows)
        assert err <= TOL[W.BF16], (e, err)
    for h in hsx:
        h.close()


@pytest.mark.parametrize("d", [1032, 2048, 2560])
def test_grouped_materialize_and_reset_equal_per_handle(d):
    """hess_materialize_grouped equals one hess_materialize_ex per handle bit for bit (H, dead
    mask, damping), with empty experts and dead columns, out of place and in place;
    hess_reset_grouped leaves every handle as a fresh one."""
    _say(f"grouped materialize / reset d={d}")
    rng = np.random.default_rng(60 + d)
    E, T = 9, 900
    scales = W.column_scales(rng, d)
    scales[[3, d - 1]] = 0.0                                   # dead columns
    x = to_device(W.encode(W.normal_rows(rng, T, d, scales), W.BF16), W.BF16)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=2)
    n4 = offsets[5] - offsets[4]                               # expert 4: no tokens
    row_idx = np.concatenate([row_idx[:offsets[4]], row_idx[offsets[5]:]])
    offsets[5:] -= n4
    ridx = torch.from_numpy(row_idx).cuda()
    hsx = [hs.Hessian(d, torch.bfloat16, staging_bytes=0) for _ in range(E)]
    for flags_neut in (True, False):
        hs.reset_grouped(hsx)
        hs.add_batch_grouped(hsx, x, offsets, ridx)
        got = hs.materialize_grouped(hsx, 0.01, neutralize=flags_neut)
        for e in range(E):
            H, dead, damp = hsx[e].materialize(0.01, neutralize=flags_neut)
            assert torch.equal(got[e][0], H), e
            assert torch.equal(got[e][1], dead), e
            assert torch.equal(got[e][2], damp), e
            assert hsx[e].nsamples == int(offsets[e + 1] - offsets[e])
        Hr, _, _ = O.materialize(np.zeros((d, d)), 0, 0.01, flags_neut)
        assert np.array_equal(got[4][0].cpu().numpy(), Hr.astype(np.float32))
    # in place for every other handle (NULL entries of H_out), through the C ABI
    refs = [hsx[e].materialize(0.01)[0].clone() for e in range(E)]
    lib = hs._load()
    outs = [torch.empty((d, d), dtype=torch.float32, device="cuda") for _ in range(E)]
    arr = (ctypes.c_void_p * E)(*[h._h.value for h in hsx])
    harr = (ctypes.c_void_p * E)(*[None if e % 2 else outs[e].data_ptr() for e in range(E)])
    assert lib.hess_materialize_grouped(arr, E, ctypes.c_float(0.01), 0, harr, None, None,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    for e in range(E):
        got_e = hsx[e].state_tensor() if e % 2 else outs[e]
        assert torch.equal(got_e, refs[e]), e
    with pytest.raises(hs.HessError):
        hsx[1].add_batch(x[:10])                               # consumed in place
    # reset clears consumed handles; accumulation starts over
    hs.reset_grouped(hsx)
    hs.add_batch_grouped(hsx, x, offsets, ridx)
    again = hs.materialize_grouped(hsx, 0.01)
    for e in range(E):
        assert torch.equal(again[e][0], refs[e]), e
    for h in hsx:
        h.close()


def test_grouped_equals_single_handle_runs():
    _say("grouped equals single")
    rng = np.random.default_rng(51)
    T, d, E = 900, 256, 5
    x = W.encode(W.normal_rows(rng, T, d), W.BF16)
    row_idx, offsets = W.moe_routing(rng, T, experts=E, topk=2)
    xt = to_device(x, W.BF16)
    ridx = torch.from_numpy(row_idx).cuda()
    grouped = [hs.Hessian(d, torch.bfloat16) for _ in range(E)]
    hs.add_batch_grouped(grouped, xt, offsets, ridx)
    for e in range(E):
        rows = ridx[offsets[e]:offsets[e + 1]].long()
        single = hs.Hessian(d, torch.bfloat16)
        single.add_batch(xt[rows])
        A, _, _ = grouped[e].materialize(0.01)
        B, _, _ = single.materialize(0.01)
        assert agreement(A.cpu().numpy(), B.cpu().numpy().astype(np.float64)) <= 1e-6
        single.close()
        grouped[e].close()


@pytest.mark.parametrize("d,sizes", [(1032, [100, 700, 1, 2000, 5]), (264, [30, 1, 300])])
def test_graph_capture_replays_equal_eager(d, sizes):
    """A whole Hessian (reset, staged and long batches, materialize) captured in
    a graph: every replay, with eager work and synchronizations between the
    replays, equals the eager result bit for bit."""
    _say(f"graph capture d={d}")
    wl = W.ragged_case(d, sizes, seed=41 + d, dtype=W.BF16, dead_frac=0.02)
    xs = [to_device(b, W.BF16) for b in wl.batches]
    out = torch.empty((d, d), dtype=torch.float32, device="cuda")
    h = hs.Hessian(d, torch.bfloat16)

    def one():
        h.reset()
        for x in xs:
            h.add_batch(x)
        h.materialize(0.01, out=out)

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        one()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    ref = out.clone()
    Hr, _, _, _ = run_oracle(wl)
    assert agreement(ref.cpu().numpy(), Hr) <= TOL[W.BF16]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        one()
    other = hs.Hessian(d, torch.bfloat16, staging_bytes=0)
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}"
        other.add_batch(xs[0])              # eager work between replays
        other.materialize(0.0)
        torch.cuda.synchronize()
    other.close()
    del graph
    h.close()


def test_kernel_timing_counts_launches():
    _say("SYRK launch timing")
    h = hs.Hessian(512, torch.bfloat16)
    x = torch.randn(3000, 512, device="cuda").to(torch.bfloat16)
    h.set_timing(True)
    h.add_batch(x)                      # long batch: its own SYRK pass
    h.add_batch(x[:100])                # short: staged
    h.add_batch(x[:200])
    h.flush()                           # one pass over the 300 staged tokens
    launches, tokens, ms = h.timing()
    assert (launches, tokens) == (2, 3300)
    assert ms > 0.0
    assert h.timing() == (0, 0, 0.0)    # a read starts a new window
    h.set_timing(False)
    h.add_batch(x)
    assert h.timing() == (0, 0, 0.0)
    h.close()
    # transposed staging pads each batch to 8 rows; the record counts batch rows
    h = hs.Hessian(1032, torch.bfloat16)
    x = torch.randn(300, 1032, device="cuda").to(torch.bfloat16)
    h.set_timing(True)
    h.add_batch(x[:101])
    h.add_batch(x[:5])
    h.flush()
    launches, tokens, ms = h.timing()
    assert (launches, tokens) == (1, 106)
    h.close()


# ------------------------------------------------------------- imatrix --

def _imatrix_check(d, sizes, dtype, seed, strided=False):
    rng = np.random.default_rng(seed)
    wl = W.ragged_case(d, sizes, seed=seed, dtype=dtype, dead_frac=0.0)
    m = hs.ImatrixStat(d, torch_dtype(dtype))
    for b in wl.batches:
        xb = to_device(b, dtype)
        if strided and xb.shape[0] > 0:
            wide = torch.zeros((xb.shape[0], d + 3), dtype=xb.dtype, device=xb.device)
            wide[:, :d] = xb
            xb = wide[:, :d]
        m.add_batch(xb)
    got, n = m.read()
    torch.cuda.synchronize()
    ref = O.column_sum_squares(wl.batches, dtype)
    assert n == sum(sizes)
    got = got.double().cpu().numpy()
    # every term is positive: a float32 sum of k terms is within k * 2^-24 of the column's value;
    # here k <= rows per split + splits + batches < 850
    rel = np.abs(got - ref) / np.maximum(ref, 1e-30)
    assert rel.max() <= 5e-5, rel.max()
    m.close()
    return rng


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("d", [8, 17, 1032, 4096])
def test_imatrix_parity(d, dtype):
    """Per-column float32 sums of squares against the oracle: vector and element paths,
    ragged batches including empty and 1-token ones."""
    _say(f"imatrix d={d} {dtype}")
    _imatrix_check(d, [1, 0, 700, 33, 4000], dtype, seed=600 + d)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_imatrix_widest(dtype):
    """Width 65,536 (128 column groups of 512 bf16 or 256 of 256 float32 features), batches of
    1, 300 and 65 tokens."""
    _say(f"imatrix d=65536 {dtype}")
    _imatrix_check(65536, [1, 300, 65], dtype, seed=640)


def test_imatrix_strided_rows_and_reset():
    _say("imatrix strided rows, reset")
    _imatrix_check(1032, [300, 41], W.BF16, seed=610, strided=True)
    m = hs.ImatrixStat(64, torch.float32)
    x = torch.randn(100, 64, device="cuda")
    m.add_batch(x)
    m.reset()
    m.add_batch(x[:10])
    got, n = m.read()
    torch.cuda.synchronize()
    assert n == 10
    ref = (x[:10].double() ** 2).sum(0).cpu().numpy()
    assert np.max(np.abs(got.double().cpu().numpy() - ref) / ref) <= 5e-5
    m.close()


def test_imatrix_full_size():
    """32,768 tokens x 4,096 features bf16 (the local-blocks workload's shape) against the oracle."""
    _say("imatrix full size 32768x4096")
    _imatrix_check(4096, [32768], W.BF16, seed=620)


# --------------------------------------------------------------- adopt --

def test_adopt_is_private_copy():
    """A follower adopts the leader's sum and token count (staged rows included), then diverges
    without touching the leader; bad widths and consumed leaders are refused."""
    _say("adopt")
    d = 1032
    wl = W.ragged_case(d, [5, 700, 3000, 17], seed=700, dtype=W.BF16, dead_frac=0.02)
    more = W.ragged_case(d, [400, 9], seed=701, dtype=W.BF16)
    leader, follower = hs.Hessian(d, torch.bfloat16), hs.Hessian(d, torch.bfloat16)
    for b in wl.batches:
        leader.add_batch(to_device(b, W.BF16))
    follower.add_batch(to_device(more.batches[0], W.BF16))   # dropped by the adopt
    follower.adopt_from(leader)
    assert follower.nsamples == leader.nsamples == wl.total_tokens
    A, _, _ = leader.materialize(0.01)
    B, _, _ = follower.materialize(0.01)
    torch.cuda.synchronize()
    assert torch.equal(A, B)
    for b in more.batches:
        follower.add_batch(to_device(b, W.BF16))
    A2, _, _ = leader.materialize(0.01)
    torch.cuda.synchronize()
    assert torch.equal(A, A2), "the leader changed"
    both = W.Workload(d=d, dtype=W.BF16, batches=list(wl.batches) + list(more.batches))
    H, dead, dmp = follower.materialize(0.01)
    Hr, deadr, dmpr, Nr = run_oracle(both, 0.01, True)
    assert follower.nsamples == Nr
    assert np.array_equal(dead.cpu().numpy(), deadr)
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    follower.adopt_from(follower)   # no-op
    other = hs.Hessian(d + 8, torch.bfloat16)
    with pytest.raises(hs.HessError):
        other.adopt_from(leader)
    leader.materialize_in_place()
    with pytest.raises(hs.HessError):
        follower.adopt_from(leader)
    for h in (leader, follower, other):
        h.close()


# ------------------------------------------------- staging dtype (casts) --

def test_cast_worked_example_bitwise():
    """The pages' fp16 example: one token 1 + 2^-10 gives a scaled diagonal of
    2.003908157348633 staged in float32 and exactly 2.0 staged in bf16."""
    _say("cast worked example")
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_staging.json")))
    f = g["f16_staging"]
    x = torch.tensor(g["tokens"], dtype=torch.float16, device="cuda")
    for staging, want in ((torch.float32, f["expected_diag_f32_staging"]),
                          (torch.bfloat16, f["expected_diag_bf16_staging"])):
        for d in (1, 1024):   # row-major staging; transposed bf16 staging at d = 1,024 under the 256 override
            hs.set_tile_override(256 if d == 1024 else 0)
            h = hs.Hessian(d, staging)
            xx = torch.zeros((1, d), dtype=torch.float16, device="cuda")
            xx[0, 0] = x[0, 0]
            h.add_batch(xx)
            H, _, _ = h.materialize(0.0, neutralize=False)
            assert float(H[0, 0].cpu()) == want, (staging, d, float(H[0, 0].cpu()))
            h.close()


def _diag_batch(vals: np.ndarray, dtype: str) -> np.ndarray:
    """Tokens t < len(vals): token t holds vals[t] at feature t, zeros elsewhere."""
    n = vals.shape[0]
    X = np.zeros((n, n), dtype=vals.dtype)
    X[np.arange(n), np.arange(n)] = vals
    return X


@pytest.mark.parametrize("staging,src,t8", [(W.BF16, W.F16, False), (W.BF16, W.F16, True),
                                             (W.BF16, W.F32, False), (W.BF16, W.F32, True),
                                             (W.F32, W.F16, False), (W.F32, W.BF16, False)])
def test_cast_rounding_bit_exact(staging, src, t8):
    """The conversion itself, value by value: a batch of one-hot tokens puts each converted value's
    square, a single exact product, on the diagonal of S.  f16 sources: every finite fp16 value;
    f32 sources: random bit patterns with exponents in [-60, 60], ties, and values that round up
    into the next binade."""
    _say(f"cast rounding staging={staging} src={src} t8={t8}")
    d = 2048
    if src == W.F16:
        allv = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
        allv = allv[np.isfinite(allv)]
    elif src == W.F32:
        rng = np.random.default_rng(17)
        m = rng.integers(0, 2 ** 23, size=3 * d, dtype=np.int64)
        e = rng.integers(127 - 60, 127 + 61, size=3 * d, dtype=np.int64)
        sg = rng.integers(0, 2, size=3 * d, dtype=np.int64)
        u = (sg << 31) | (e << 23) | m
        u[d:2 * d] = (u[d:2 * d] & ~0xFFFF) | 0x8000      # exact ties
        u[2 * d:2 * d + 256] |= 0x7FFFFF                   # all-ones fraction: rounds into the next binade
        allv = u.astype(np.uint32).view(np.float32)
    else:
        rng = np.random.default_rng(18)
        allv = W.encode(rng.standard_normal(2 * d).astype(np.float32) * 8, W.BF16)
    hs.set_tile_override(256 if t8 else 128)
    h = hs.Hessian(d, torch_dtype(staging))
    want = np.zeros(d, dtype=np.float64)
    got = np.zeros(d, dtype=np.float64)
    for s0 in range(0, allv.shape[0], d):
        vals = allv[s0:s0 + d]
        k = vals.shape[0]
        X = _diag_batch(vals, src)
        if k < d:
            X = np.concatenate([X, np.zeros((k, d - k), dtype=X.dtype)], axis=1)
        h.reset()
        h.add_batch(to_device(X, src))
        h.flush()
        S = h.state_tensor()
        torch.cuda.synchronize()
        got = torch.diagonal(S).cpu().numpy().astype(np.float64)[:k]
        v = O.staged_values(X[np.arange(k), np.arange(k)].reshape(1, -1), src, staging)[0]
        want = v * v
        assert np.array_equal(got, want), (s0, np.flatnonzero(got != want)[:8], got[got != want][:4],
                                           want[got != want][:4])
    h.close()


@pytest.mark.parametrize("staging,src,d,sbytes,override", [
    (W.BF16, W.F16, 1032, None, 256),        # transposed staging, 256-tile flushes
    (W.BF16, W.F32, 1032, 2 << 20, 256),     # small buffer: long batches split over many flushes
    (W.BF16, W.F16, 520, None, 0),           # row-major bf16 staging
    (W.BF16, W.F32, 17, None, 0),            # odd width: element copies
    (W.F32, W.F16, 264, None, 0),
    (W.F32, W.BF16, 100, 1 << 20, 0),        # width not a multiple of 8, small buffer
])
def test_cast_parity(staging, src, d, sbytes, override):
    """Ragged batches (long ones included) of another type than the staging dtype, against the
    oracle that rounds into the staging dtype first; plain batches mixed in."""
    _say(f"cast parity staging={staging} src={src} d={d} sbytes={sbytes} override={override}")
    hs.set_tile_override(override)
    rng = np.random.default_rng(900 + d)
    sc = W.column_scales(rng, d)
    sizes = [5, 700, 3000, 1, 17, 2500, 64]
    h = hs.Hessian(d, torch_dtype(staging), staging_bytes=sbytes)
    acc = O.GramAccumulator(d, staging=staging)
    for i, n in enumerate(sizes):
        t = staging if i == 3 else src   # one batch already in the staging dtype
        X = W.encode(W.normal_rows(rng, n, d, sc), t)
        h.add_batch(to_device(X, t))
        acc.add_batch(X, t)
    assert h.nsamples == acc.N == sum(sizes)
    for damp, neut in ((0.0, False), (0.01, True)):
        H, dead, dmp = h.materialize(damp, neutralize=neut)
        Hr, deadr, dmpr = acc.materialize(damp, neut)
        torch.cuda.synchronize()
        assert np.array_equal(dead.cpu().numpy(), deadr)
        err = agreement(H.cpu().numpy(), Hr)
        assert err <= TOL[staging], err
    h.close()


def test_cast_errors_and_adopt_settings():
    """Conversion needs a staging buffer; adopt refuses handles whose staging dtype or staging
    buffer differ (the accumulation settings) and accepts equal ones."""
    _say("cast errors / adopt settings")
    x = torch.ones((4, 64), dtype=torch.float16, device="cuda")
    h0 = hs.Hessian(64, torch.bfloat16, staging_bytes=0)
    with pytest.raises(hs.HessError):
        h0.add_batch(x)
    with pytest.raises(TypeError):
        h0.add_batch(x.double())
    a = hs.Hessian(64, torch.bfloat16)
    b = hs.Hessian(64, torch.float32)
    c = hs.Hessian(64, torch.bfloat16, staging_bytes=1 << 20)
    e = hs.Hessian(64, torch.bfloat16)
    a.add_batch(x)
    with pytest.raises(hs.HessError):
        b.adopt_from(a)
    with pytest.raises(hs.HessError):
        c.adopt_from(a)
    e.adopt_from(a)
    assert e.nsamples == 4
    for hh in (h0, a, b, c, e):
        hh.close()


def test_new_entry_points_on_a_side_stream():
    """Cast, adopt, the imatrix statistic, the Cholesky factor and the block quantize all run on a
    non-default stream with their inputs produced on that stream, and agree with the oracle."""
    _say("side stream: cast / adopt / imatrix / chol / quantize")
    side = torch.cuda.Stream()
    d = 264
    rng = np.random.default_rng(77)
    x16 = W.encode(W.normal_rows(rng, 900, d, W.column_scales(rng, d)), W.F16)
    with torch.cuda.stream(side):
        xd = torch.from_numpy(x16).to("cuda", non_blocking=False)
        xd = xd * 1.0                     # produced on the side stream
        h = hs.Hessian(d, torch.bfloat16)
        h.add_batch(xd, stream=side)
        f = hs.Hessian(d, torch.bfloat16)
        f.adopt_from(h, stream=side)
        m = hs.ImatrixStat(d, torch.bfloat16)
        m.add_batch(xd.to(torch.bfloat16), stream=side)
        H, dead, _ = f.materialize(0.01, stream=side)
        U = hs.chol_inverse_upper(H, stream=side)
        Wt = torch.randn((40, d), device="cuda", dtype=torch.float32) * 0.02
        Q, codes, _, _ = hs.gptq_quantize(Wt, U, group_size=-1, stream=side)
        sums, n = m.read(stream=side)
    side.synchronize()
    acc = O.GramAccumulator(d, staging="bf16")
    acc.add_batch(x16, W.F16)
    Hr, deadr, _ = acc.materialize(0.01)
    assert f.nsamples == acc.N == 900
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    xb = W.to_bf16_bits(x16.astype(np.float32))
    sr = O.column_sum_squares([xb], W.BF16)
    assert n == 900 and np.all(np.abs(sums.cpu().numpy() - sr) <= 5e-5 * sr + 1e-30)
    U32 = U.cpu().numpy()
    assert np.allclose(U32, O.chol_inverse_upper(H.cpu().numpy().astype(np.float64)), rtol=1e-5, atol=1e-9)
    (Qr, cr, _, _), _ = quantize_against_gpu_ties(Wt.cpu().numpy().astype(np.float64), U32.astype(np.float64), -1,
                                                  codes.cpu().numpy())
    assert np.array_equal(codes.cpu().numpy(), cr)
    for o in (h, f, m):
        o.close()


# ------------------------------------------------------ asynchronous flush --

ASYNC_D = 2048
ASYNC_STAGING = 540 << 20      # halves of 69,120 tokens: each flush long enough for the 256-tile kernel
ASYNC_HALF = 69120


def _async_workload(seed, count=150, long_at=None):
    """Batches of U[500, 2000] tokens (all staged at width 2,048), optionally a 5,000-token one."""
    rng = np.random.default_rng(seed)
    sizes = [int(v) for v in rng.integers(500, 2001, count)]
    if long_at is not None:
        sizes.insert(long_at, 5000)        # 5,000 tokens: a pass of its own straight into S
    return W.ragged_case(ASYNC_D, sizes, seed=seed, dtype=W.BF16, dead_frac=0.02)


def test_async_flush_streams_and_long_batch():
    """Full halves are folded in on the handle's own stream while staging goes on; batches arrive
    on two streams in turn, a long batch in the middle takes its own pass (after the pending
    flush), and the result matches the oracle (token count exact, dead mask bit for bit)."""
    _say("async flush: two streams and a long batch")
    hs.set_async_flush(True)
    wl = _async_workload(71, count=200, long_at=100)
    xs = [to_device(b, W.BF16) for b in wl.batches]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    h = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)
    for i, x in enumerate(xs):
        h.add_batch(x, stream=s1 if (i // 40) % 2 == 0 else s2)
    H, dead, dmp = h.materialize(0.01, stream=s2)
    s2.synchronize()
    Hr, deadr, dmpr, Nr = run_oracle(wl, 0.01, True)
    assert h.nsamples == Nr > 2 * ASYNC_HALF   # at least two halves filled: two asynchronous flushes
    assert np.array_equal(dead.cpu().numpy(), deadr)
    err = agreement(H.cpu().numpy(), Hr)
    print(f"  async: {err:.3e}")
    assert err <= TOL[W.BF16]
    h.close()


def test_async_flush_two_handles_share_the_workspace():
    """Two handles flush asynchronously, interleaved on one stream (their flushes share the
    device's split workspace); a third adopts one of them while its flush is pending; a reset
    and a destroy meet pending flushes too."""
    _say("async flush: two handles, adopt, reset, destroy")
    hs.set_async_flush(True)
    wa, wb = _async_workload(72, count=150), _async_workload(73, count=150)
    xa = [to_device(b, W.BF16) for b in wa.batches]
    xb = [to_device(b, W.BF16) for b in wb.batches]
    torch.cuda.synchronize()
    ha = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)
    hb = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)
    for x1, x2 in zip(xa, xb):
        ha.add_batch(x1)
        hb.add_batch(x2)
    hc = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)
    hc.adopt_from(ha)                                  # ha's flush may be pending here
    for h, wl in ((ha, wa), (hb, wb), (hc, wa)):
        H, dead, _ = h.materialize(0.01)
        Hr, deadr, _, Nr = run_oracle(wl, 0.01, True)
        assert h.nsamples == Nr
        assert np.array_equal(dead.cpu().numpy(), deadr)
        assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    # reset with a flush pending, then a fresh accumulation
    for x in xa:
        hb.add_batch(x)
    hb.reset()
    for x in xa[:30]:
        hb.add_batch(x)
    H, _, _ = hb.materialize(0.0, neutralize=False)
    sub = W.Workload(d=ASYNC_D, dtype=W.BF16, batches=wa.batches[:30])
    Hr, _, _, _ = run_oracle(sub, 0.0, False)
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    for x in xa:
        ha.add_batch(x)
    ha.close()                                         # a flush may be pending: destroy waits for it
    hb.close()
    hc.close()


def test_async_flush_pending_is_refused_under_capture():
    """With an asynchronous flush pending, a captured call that needs the sum is refused
    (HESS_ESTATE); after an eager flush, a whole Hessian whose halves fill captures (its flushes
    then run on the capturing stream with the same workgroups) and every replay equals the eager
    run, whose flushes went on the handle's own stream, bit for bit."""
    _say("async flush: capture")
    hs.set_async_flush(True)
    wl = _async_workload(74, count=120)
    xs = [to_device(b, W.BF16) for b in wl.batches]
    out = torch.empty((ASYNC_D, ASYNC_D), dtype=torch.float32, device="cuda")
    h = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        for x in xs:
            h.add_batch(x)                              # a flush of the first half is now pending
    torch.cuda.current_stream().wait_stream(cs)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(hs.HessError) as e:
        with torch.cuda.graph(g, stream=cs):
            h.materialize(0.01, out=out)
    assert e.value.code == -4
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        h.flush()
    torch.cuda.synchronize()

    def one():                                          # fills two halves: flushes inside the sequence
        h.reset()
        for x in xs:
            h.add_batch(x)
        h.materialize(0.01, out=out)

    with torch.cuda.stream(cs):
        one()
    torch.cuda.synchronize()
    ref = out.clone()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=cs):
        one()
    for _ in range(2):
        out.zero_()
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    h.close()


def test_async_destroy_returns_staging_memory():
    """A handle destroyed while it stages into its second half frees its whole staging
    allocation (the allocation starts at the first half)."""
    _say("async flush: destroy frees staging")
    hs.set_async_flush(True)
    wl = _async_workload(75, count=60)
    xs = [to_device(b, W.BF16) for b in wl.batches]
    warm = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)   # device workspaces
    warm.close()
    gc.collect()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    h = hs.Hessian(ASYNC_D, torch.bfloat16, staging_bytes=ASYNC_STAGING)
    for x in xs:
        h.add_batch(x)                  # 60 batches of ~1,250 tokens: past the first half
    assert h.nsamples > ASYNC_HALF
    h.close()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0, (free0, free1)


def test_one_handle_from_two_host_threads():
    """Two host threads add batches to one handle at the same time: the per-handle lock keeps
    every call whole, so the token count is exact and H matches the oracle."""
    import threading
    _say("one handle, two host threads")
    d = 1032
    wl = W.ragged_case(d, [int(v) for v in np.random.default_rng(76).integers(1, 800, 200)], seed=76,
                       dtype=W.BF16, dead_frac=0.02)
    xs = [to_device(b, W.BF16) for b in wl.batches]
    torch.cuda.synchronize()
    h = hs.Hessian(d, torch.bfloat16)
    errors = []

    def worker(part):
        try:
            for x in part:
                h.add_batch(x)
        except Exception as exc:       # reported below
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(xs[k::2],)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    H, dead, _ = h.materialize(0.01)
    Hr, deadr, _, Nr = run_oracle(wl, 0.01, True)
    assert h.nsamples == Nr
    assert np.array_equal(dead.cpu().numpy(), deadr)
    assert agreement(H.cpu().numpy(), Hr) <= TOL[W.BF16]
    h.close()
