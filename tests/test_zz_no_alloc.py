"""The allocation-free local-block call, through the C ABI, against the allocating one.

hess_local_blocks_noalloc keeps its partial sums in a fixed device array of the
library instead of memory it allocates.  It takes the same plan and summation
order as hess_local_blocks_ex, so the two agree bit for bit; both are checked
against the float64 oracle to the bf16 / float32 bars.  Two calls in a row, the
second on a smaller input, exercise the array's reuse (it keeps the first call's
contents), and the device's free memory must not change across them.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import gptq_hessian_accumulation_amd as hs
from tests.helpers import TOL, block_agreement, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DT = {W.BF16: 0, W.F32: 1}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _call(fn, x, n, d, out, accumulate):
    lib = hs._load()
    rc = getattr(lib, fn)(ctypes.c_void_p(x.data_ptr()), DT[W.BF16 if x.dtype == torch.bfloat16 else W.F32], n, d,
                          x.stride(0), 16, ctypes.c_void_p(out.data_ptr()), accumulate,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.hess_last_error()


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_noalloc_matches_allocating_call_twice(dtype):
    _say(f"local blocks without allocation {dtype}")
    rng = np.random.default_rng(70)
    cases = [(9000, 2048), (700, 512)]      # the second call is smaller
    xs = [W.encode(W.normal_rows(rng, n, d, W.column_scales(rng, d)), dtype) for n, d in cases]
    xd = [to_device(x, dtype) for x in xs]
    outs_a = [torch.zeros((d // 16, 16, 16), dtype=torch.float32, device="cuda") for _, d in cases]
    outs_b = [torch.zeros((d // 16, 16, 16), dtype=torch.float32, device="cuda") for _, d in cases]
    warm = torch.zeros((8, 16, 16), dtype=torch.float32, device="cuda")
    _call("hess_local_blocks_noalloc", xd[1][:, :128], 700, 128, warm, 0)   # first call on the device
    _call("hess_local_blocks_ex", xd[1][:, :128], 700, 128, warm, 0)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for (n, d), x, a in zip(cases, xd, outs_a):
        _call("hess_local_blocks_noalloc", x, n, d, a, 0)
        _call("hess_local_blocks_noalloc", x, n, d, a, 1)    # accumulate: twice the sums
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, "the allocation-free call changed the device's free memory"
    for (n, d), x, b in zip(cases, xd, outs_b):
        _call("hess_local_blocks_ex", x, n, d, b, 0)
        _call("hess_local_blocks_ex", x, n, d, b, 1)
    torch.cuda.synchronize()
    for (n, d), xh, a, b in zip(cases, xs, outs_a, outs_b):
        assert torch.equal(a, b), f"n={n} d={d}: differs from the allocating call"
        ref = 2.0 * O.local_blocks(xh, dtype)
        err = block_agreement(a.cpu().numpy(), ref)
        print(f"  n={n} d={d}: {err:.3e}")
        assert err <= TOL[dtype]


def test_noalloc_rejects_widths_past_its_array():
    lib = hs._load()
    d = 262144 + 16
    # buffers as large as the call describes, although it must return before any launch
    out = torch.zeros(d * 16, dtype=torch.float32, device="cuda")
    x = torch.zeros(d, dtype=torch.bfloat16, device="cuda")
    rc = lib.hess_local_blocks_noalloc(ctypes.c_void_p(x.data_ptr()), 0, 1, d, d, 16,
                                       ctypes.c_void_p(out.data_ptr()), 0, None)
    assert rc == -1 and b"allocation-free" in lib.hess_last_error()
