"""The C-ABI library loads and exports every declared symbol; argument checks
that return before touching the GPU behave as declared.  CPU only."""

import ctypes
import os

import pytest

import gptq_hessian_accumulation_amd as hs

LIB = hs.library_path()
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhess.so not built")


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    names = hs.exported_symbols()
    assert len(names) >= 14
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_required_entry_points_declared():
    names = set(hs.exported_symbols())
    for n in ("hess_create", "hess_add_batch", "hess_materialize", "hess_local_blocks",
              "hess_materialize_ex", "hess_add_batch_grouped", "hess_local_blocks_ex", "hess_reset",
              "hess_destroy", "hess_token_count"):
        assert n in names


def test_version_and_status_strings():
    lib = hs._load()
    assert lib.hess_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.hess_strerror(code)
    assert lib.hess_strerror(-99) == b"unknown status"


def test_invalid_arguments_rejected_without_gpu():
    lib = hs._load()
    assert not lib.hess_create(0, 0)
    assert b"outside" in lib.hess_last_error()
    assert not lib.hess_create(16, 7)
    assert lib.hess_add_batch(None, None, 1, 16, None) == -1
    assert lib.hess_materialize(None, 0.01, None) == -1
    assert lib.hess_token_count(None, None) == -1
    # local blocks: block must be 16, d a multiple of 16, ld >= d
    assert lib.hess_local_blocks(None, 0, 32, 8, ctypes.c_void_p(16)) == -1
    assert lib.hess_local_blocks(None, 0, 40, 16, ctypes.c_void_p(16)) == -1
    assert lib.hess_local_blocks_ex(None, 0, 0, 32, 16, 16, ctypes.c_void_p(16), 1, None) == -1
    assert lib.hess_local_blocks_ex(None, 0, 5, 32, 32, 16, ctypes.c_void_p(16), 1, None) == -1
    assert lib.hess_set_tile_override(100) == -1
    assert lib.hess_set_tile_override(64) == 0 and lib.hess_set_tile_override(0) == 0
    assert not lib.hess_create_ex(16, 0, -1)
    assert b"staging_bytes" in lib.hess_last_error()
    offs = (ctypes.c_int64 * 2)(0, 1)
    assert lib.hess_add_batch_grouped(None, 1, None, 16, None, offs, None) == -1
    assert lib.hess_add_batch_grouped_ex(None, 1, None, 4, 16, None, offs, None) == -1
    assert lib.hess_set_group_direct(0) == 0 and lib.hess_set_group_direct(1) == 0
    # Cholesky of the inverse: workspace size rule and argument checks (no device work)
    assert lib.hess_chol_inverse_workspace(0) == -1
    assert lib.hess_chol_inverse_workspace(1) == (2 * 64 * 64 + 64 * 64) * 8
    assert lib.hess_chol_inverse_workspace(65) == (2 * 128 * 128 + 128 * 64) * 8
    p = lambda a: ctypes.c_void_p(a)  # noqa: E731  (fake, never dereferenced)
    base = 1 << 40
    need = lib.hess_chol_inverse_workspace(100)
    assert lib.hess_chol_inverse_upper(p(base), 100, 100, p(base + (1 << 30)), 100, p(base + (2 << 30)), need - 1,
                                       None, None) == -1
    assert b"workspace" in lib.hess_last_error()
    assert lib.hess_chol_inverse_upper(p(base), 100, 99, p(base + (1 << 30)), 100, p(base + (2 << 30)), need,
                                       None, None) == -1
    assert lib.hess_chol_inverse_upper(p(base), 100, 100, p(base + 400), 100, p(base + (2 << 30)), need,
                                       None, None) == -1
    assert b"overlaps" in lib.hess_last_error()
    assert lib.hess_chol_inverse_upper(p(base), 100, 100, p(base + (1 << 30)), 100, p(base + 16), need,
                                       None, None) == -1
    assert lib.hess_chol_inverse_upper(p(base), 40000, 40000, p(base + (1 << 30)), 40000, p(base + (2 << 30)),
                                       need, None, None) == -1
    # the staging dtype of a handle is bf16 or f32; fp16 is an activation type only
    assert not lib.hess_create(16, 2)
    assert lib.hess_add_batch_cast(None, None, 2, 1, 16, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(hs, "_lib", None)
    monkeypatch.setattr(hs, "_LIB_PATH", "/nonexistent/libhess.so")
    with pytest.raises(RuntimeError, match="not built"):
        hs._load()


def test_quantize_arguments_rejected_without_gpu():
    lib = hs._load()
    p = lambda a: ctypes.c_void_p(a)  # noqa: E731  (fake, never dereferenced)
    base = 1 << 40
    assert lib.hess_gptq_quantize_workspace(0, 5) == -1
    need = lib.hess_gptq_quantize_workspace(10, 200)
    assert need == (128 * 256 + 128 * 128 + 10 + 10 * 2) * 8

    def call(group=-1, ldw=200, work_bytes=None, q=None, n=10):
        return lib.hess_gptq_quantize(p(base), n, 200, ldw, p(base + (1 << 30)), 200, None, group,
                                      p(q if q is not None else base + (2 << 30)), 200, p(base + (3 << 30)), 200,
                                      p(base + (4 << 30)), None, 1, p(base + (5 << 30)),
                                      need if work_bytes is None else work_bytes, None)
    assert call(group=48) == -1 and b"group_size" in lib.hess_last_error()
    assert call(group=0) == -1
    assert call(ldw=199) == -1
    assert call(work_bytes=need - 8) == -1 and b"workspace" in lib.hess_last_error()
    assert call(q=base + 64) == -1 and b"overlaps" in lib.hess_last_error()
    assert call(n=70000) == -1


def _span_elems(x2, n, ld, d):
    """Elements the library reads from the returned view's start: (n - 1) * ld + d."""
    return 0 if n == 0 else (n - 1) * ld + d


@pytest.mark.parametrize("make", ["expand", "unfold", "strided", "contig", "transposed", "one_row", "empty"])
def test_as_rows_never_reads_past_storage(make):
    """The rows handed to the library lie inside the tensor's storage and hold its values,
    for broadcast (stride 0) and overlapping (stride < d) views too."""
    import torch
    d = 8
    base = torch.arange(5 * d, dtype=torch.float32).reshape(5, d)
    if make == "expand":
        x = base[0][None].expand(5, d)                     # row stride 0
    elif make == "unfold":
        x = torch.arange(40, dtype=torch.float32).unfold(0, d, 2)   # (17, 8), row stride 2 < d
    elif make == "strided":
        x = torch.zeros(5, d + 4)[:, :d]
        x.copy_(base)
    elif make == "contig":
        x = base
    elif make == "transposed":
        x = base.reshape(d, 5).t()                         # feature stride 5
    elif make == "one_row":
        x = base[:1]
    else:
        x = base[:0]
    x2, n, ld = hs._as_rows(x, d)
    assert n == x.shape[0] and ld >= d
    assert x2.stride(1) == 1 or n == 0
    storage = x2.untyped_storage().nbytes() // 4 - x2.storage_offset()
    assert _span_elems(x2, n, ld, d) <= storage
    if n > 0:
        flat = torch.as_strided(x2, (n, d), (ld, 1))
        assert torch.equal(flat, x)
