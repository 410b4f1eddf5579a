"""Calibration-Hessian accumulation on AMD Instinct MI355X (gfx950).

Python binding of ``libhess.so`` (C ABI in ``include/hess.h``).  The binding
only marshals arguments: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.

    H = (2/N) * sum_t x_t x_t^T         (GPTQModel PR 2979, What Changed)

``Hessian.add_batch`` accumulates one calibration batch in place,
``Hessian.materialize`` scales by 2/N, neutralizes dead columns and adds
``damp_percent * mean(diag)`` to the diagonal (GPTQModel wiki "QQQ",
Concepts > Quadratic error compensation), ``local_blocks`` builds the 16 x 16
per-block Gram matrices and ``add_batch_grouped`` updates many routed-expert
Hessians in one launch (Model-Optimizer PR 3002 page, "What does this PR do?").

There is no CPU fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "Hessian",
    "HessError",
    "local_blocks",
    "add_batch_grouped",
    "reset_grouped",
    "materialize_grouped",
    "chol_inverse_upper",
    "gptq_quantize",
    "set_tile_override",
    "set_staging",
    "library_path",
    "exported_symbols",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libhess.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "hess.h")

HESS_BF16 = 0
HESS_F32 = 1
HESS_F16 = 2
HESS_NO_NEUTRALIZE = 1

_STATUS = {0: "HESS_OK", -1: "HESS_EINVAL", -2: "HESS_ENOMEM", -3: "HESS_EHIP", -4: "HESS_ESTATE",
           -5: "HESS_EALIGN", -6: "HESS_ENOTPD"}


class HessError(RuntimeError):
    """A libhess call returned an error status."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{_STATUS.get(code, code)}: {message}")
        self.code = code


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libhess.so is not built ({_LIB_PATH}); run `python gptq_hessian_accumulation_amd/build.py` "
            "(or __graft_entry__.build()).  There is no CPU fallback.")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "hess_abi_version": (c_int, []),
        "hess_strerror": (ctypes.c_char_p, [c_int]),
        "hess_last_error": (ctypes.c_char_p, []),
        "hess_create": (vp, [i64, c_int]),
        "hess_create_ex": (vp, [i64, c_int, i64]),
        "hess_destroy": (c_int, [vp]),
        "hess_add_batch": (c_int, [vp, vp, i64, i64, vp]),
        "hess_add_batch_cast": (c_int, [vp, vp, c_int, i64, i64, vp]),
        "hess_materialize": (c_int, [vp, ctypes.c_float, vp]),
        "hess_materialize_ex": (c_int, [vp, ctypes.c_float, ctypes.c_uint, vp, vp, vp, vp]),
        "hess_reset": (c_int, [vp, vp]),
        "hess_token_count": (c_int, [vp, ctypes.POINTER(i64)]),
        "hess_set_tile_override": (c_int, [c_int]),
        "hess_set_staging": (c_int, [c_int]),
        "hess_set_async_flush": (c_int, [c_int]),
        "hess_set_group_chunk": (c_int, [i64]),
        "hess_flush": (c_int, [vp, vp]),
        "hess_set_timing": (c_int, [vp, c_int]),
        "hess_timing": (c_int, [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]),
        "hess_info": (c_int, [vp, ctypes.POINTER(i64), ctypes.POINTER(c_int)]),
        "hess_state_buffer": (c_int, [vp, ctypes.POINTER(vp)]),
        "hess_local_blocks": (c_int, [vp, i64, i64, c_int, vp]),
        "hess_local_blocks_ex": (c_int, [vp, c_int, i64, i64, i64, c_int, vp, c_int, vp]),
        "hess_local_blocks_noalloc": (c_int, [vp, c_int, i64, i64, i64, c_int, vp, c_int, vp]),
        "hess_add_batch_grouped": (c_int, [ctypes.POINTER(vp), c_int, vp, i64, vp, ctypes.POINTER(i64), vp]),
        "hess_add_batch_grouped_ex": (c_int, [ctypes.POINTER(vp), c_int, vp, i64, i64, vp, ctypes.POINTER(i64), vp]),
        "hess_set_group_direct": (c_int, [c_int]),
        "hess_adopt": (c_int, [vp, vp, vp]),
        "hess_reset_grouped": (c_int, [ctypes.POINTER(vp), c_int, vp]),
        "hess_materialize_grouped": (c_int, [ctypes.POINTER(vp), c_int, ctypes.c_float, ctypes.c_uint,
                                             ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), vp]),
        "hess_chol_inverse_workspace": (i64, [i64]),
        "hess_gptq_quantize_workspace": (i64, [i64, i64]),
        "hess_gptq_quantize": (c_int, [vp, i64, i64, i64, vp, i64, vp, c_int, vp, i64, vp, i64, vp, vp, i64, vp,
                                       i64, vp]),
        "hess_chol_inverse_upper": (c_int, [vp, i64, i64, vp, i64, vp, i64, vp, vp]),
        "hess_imatrix_create": (vp, [i64, c_int]),
        "hess_imatrix_destroy": (c_int, [vp]),
        "hess_imatrix_add_batch": (c_int, [vp, vp, i64, i64, vp]),
        "hess_imatrix_read": (c_int, [vp, vp, ctypes.POINTER(i64), vp]),
        "hess_imatrix_reset": (c_int, [vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int) -> None:
    if code != 0:
        lib = _load()
        raise HessError(code, lib.hess_last_error().decode(errors="replace"))


def exported_symbols() -> list:
    """Names of the functions declared in include/hess.h."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hess_[a-z0-9_]+)\s*\(", text)))


# The current stream's raw handle without building a Stream object (about 2.5 us
# per call saved, which matters at one call per short calibration batch).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream=None, device=None) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device() if device is None else device)
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return HESS_BF16
    if dtype == torch.float32:
        return HESS_F32
    raise TypeError(f"unsupported activation dtype {dtype}; use torch.bfloat16 or torch.float32")


def _act_code(dtype) -> int:
    if dtype == torch.float16:
        return HESS_F16
    return _dtype_code(dtype)


def _as_rows(x: torch.Tensor, d: int):
    """(tokens, d) view of x whose rows are d contiguous elements at a stride ld >= d.

    Returns (tensor, n, ld).  A view whose rows overlap or repeat (a broadcast
    row, stride 0, or a sliding window, stride < d) or whose features are not
    contiguous is copied first, so the library never reads past the storage.
    """
    if x.shape[-1] != d:
        raise ValueError(f"last dimension {x.shape[-1]} != d = {d}")
    x2 = x.reshape(-1, d) if x.dim() != 2 else x
    n = x2.shape[0]
    if n > 0 and d > 1 and x2.stride(1) != 1:
        x2 = x2.contiguous()
    if n > 1 and x2.stride(0) < d:
        x2 = x2.contiguous()
    ld = x2.stride(0) if n > 1 else d
    return x2, n, ld


def set_staging(enable: bool) -> None:
    """Enable (default) or disable the staging of short batches; process-wide."""
    _check(_load().hess_set_staging(1 if enable else 0))


def set_async_flush(enable: bool) -> None:
    """Enable (default) or disable asynchronous staging flushes for Hessians created afterwards; process-wide."""
    _check(_load().hess_set_async_flush(1 if enable else 0))


def set_group_chunk(nbytes: int) -> None:
    """Cap the rows gathered per 256-tile grouped launch (bytes; 0 = the whole buffer); process-wide."""
    _check(_load().hess_set_group_chunk(int(nbytes)))


def set_group_direct(enable: bool) -> None:
    """Grouped 256-tile updates read the routed rows in place (default) or gather them first; process-wide."""
    _check(_load().hess_set_group_direct(1 if enable else 0))


def set_tile_override(edge: int) -> None:
    """Force the SYRK tile edge (0 = automatic, 64, 128 or 256); process-wide."""
    _check(_load().hess_set_tile_override(int(edge)))


class Hessian:
    """One calibration-Hessian accumulator of width ``d`` on the current GPU.

    ``dtype`` is the staging dtype (``torch.bfloat16`` or ``torch.float32``):
    the type the products are formed in.  Batches of that type are read as
    they are; float16, bfloat16 or float32 batches of another type are
    converted on their way into the staging buffer (rounded to nearest even
    when narrowing).  The Hessian is always float32.  ``staging_bytes`` sizes
    the buffer that collects short batches (default: 1 GiB at
    d >= 1024, else 64 MiB; 0 disables staging and conversion).
    """

    def __init__(self, d: int, dtype=torch.bfloat16, staging_bytes: int | None = None):
        lib = _load()
        self.d = int(d)
        self.dtype = dtype
        self._code = _dtype_code(dtype)
        if staging_bytes is None:
            h = lib.hess_create(self.d, self._code)
        else:
            h = lib.hess_create_ex(self.d, self._code, int(staging_bytes))
        if not h:
            raise HessError(-1, lib.hess_last_error().decode(errors="replace"))
        self._h = ctypes.c_void_p(h)
        self._device = torch.cuda.current_device()
        self._add = lib.hess_add_batch

    # -- accumulation ----------------------------------------------------
    def add_batch(self, x: torch.Tensor, stream=None) -> None:
        """S += X^T X, N += tokens; leading dimensions of x are flattened to tokens."""
        if not x.is_cuda:
            raise ValueError("activations must be on the GPU")
        code = _act_code(x.dtype)
        x2, n, ld = _as_rows(x, self.d)
        ptr = x2.data_ptr() if n > 0 else None
        if code == self._code:
            rc = self._add(self._h, ptr, n, ld, _stream(stream))
        else:
            rc = _load().hess_add_batch_cast(self._h, ptr, code, n, ld, _stream(stream))
        if rc != 0:
            _check(rc)

    def materialize(self, damp_percent: float = 0.01, out: torch.Tensor | None = None, neutralize: bool = True,
                    stream=None):
        """Return ``(H, dead, damp)``: H float32 (d, d), dead bool (d,), damp float32 (1,), all on the GPU."""
        dev = torch.device("cuda", self._device)
        if out is None:
            out = torch.empty((self.d, self.d), dtype=torch.float32, device=dev)
        elif out.dtype != torch.float32 or tuple(out.shape) != (self.d, self.d) or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 (d, d) GPU tensor")
        dead = torch.empty(self.d, dtype=torch.uint8, device=dev)
        damp = torch.empty(1, dtype=torch.float32, device=dev)
        flags = 0 if neutralize else HESS_NO_NEUTRALIZE
        _check(_load().hess_materialize_ex(self._h, float(damp_percent), flags, out.data_ptr(), dead.data_ptr(),
                                           damp.data_ptr(), _stream(stream)))
        return out, dead.view(torch.bool), damp

    def materialize_in_place(self, damp_percent: float = 0.01, neutralize: bool = True, stream=None):
        """Materialize into the accumulator's own buffer; the handle then needs reset()."""
        dev = torch.device("cuda", self._device)
        dead = torch.empty(self.d, dtype=torch.uint8, device=dev)
        damp = torch.empty(1, dtype=torch.float32, device=dev)
        flags = 0 if neutralize else HESS_NO_NEUTRALIZE
        _check(_load().hess_materialize_ex(self._h, float(damp_percent), flags, None, dead.data_ptr(),
                                           damp.data_ptr(), _stream(stream)))
        return dead.view(torch.bool), damp

    def state_buffer_ptr(self) -> int:
        p = ctypes.c_void_p()
        _check(_load().hess_state_buffer(self._h, ctypes.byref(p)))
        return p.value

    def flush(self, stream=None) -> None:
        """Fold staged short batches into the Gram sum."""
        _check(_load().hess_flush(self._h, _stream(stream)))

    def state_tensor(self) -> torch.Tensor:
        """A (d, d) float32 view of the accumulator's device buffer (S, or H after an in-place materialize).

        Call flush() first when reading S, so that staged batches are included.
        """
        ptr, d = self.state_buffer_ptr(), self.d

        class _View:
            __cuda_array_interface__ = {"shape": (d, d), "typestr": "<f4", "data": (ptr, False), "version": 2,
                                        "strides": None}

        return torch.as_tensor(_View(), device=torch.device("cuda", self._device))

    def reset(self, stream=None) -> None:
        _check(_load().hess_reset(self._h, _stream(stream)))

    def adopt_from(self, leader: "Hessian", stream=None) -> None:
        """Replace this Hessian's statistics with a private copy of leader's (sum and token count)."""
        _check(_load().hess_adopt(self._h, leader._h, _stream(stream)))

    def set_timing(self, on: bool) -> None:
        """Bracket every SYRK launch of this handle with HIP events on its stream."""
        _check(_load().hess_set_timing(self._h, 1 if on else 0))

    def timing(self):
        """``(launches, tokens, ms)`` of the SYRK launches timed since the last read (waits for them)."""
        n, t, ms = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_double()
        _check(_load().hess_timing(self._h, ctypes.byref(n), ctypes.byref(t), ctypes.byref(ms)))
        return n.value, t.value, ms.value

    @property
    def nsamples(self) -> int:
        n = ctypes.c_int64()
        _check(_load().hess_token_count(self._h, ctypes.byref(n)))
        return n.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(_load().hess_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def local_blocks(x: torch.Tensor, out: torch.Tensor | None = None, accumulate: bool = True, block: int = 16,
                 stream=None) -> torch.Tensor:
    """out[b] (+)= X_b^T X_b for every 16-feature block b; float32 (d/16, 16, 16)."""
    if not x.is_cuda:
        raise ValueError("activations must be on the GPU")
    d = x.shape[-1]
    x2, n, ld = _as_rows(x, d)
    if out is None:
        out = torch.zeros((d // block, block, block), dtype=torch.float32, device=x.device)
    elif out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != (d // block) * block * block:
        raise ValueError("out must be a contiguous float32 (d/16, 16, 16) GPU tensor")
    ptr = x2.data_ptr() if n > 0 else None
    _check(_load().hess_local_blocks_ex(ptr, _dtype_code(x.dtype), n, d, ld, block, out.data_ptr(),
                                        1 if accumulate else 0, _stream(stream)))
    return out


def chol_inverse_upper(H: torch.Tensor, out: torch.Tensor | None = None, check: bool = True,
                       workspace: torch.Tensor | None = None, stream=None):
    """U (float32, upper triangular, positive diagonal) with U^T U = H^-1, for a damped Hessian H.

    Only H's upper triangle is read; ``out`` may be H itself.  With ``check``
    the call waits for the result and raises HessError(HESS_ENOTPD) when H
    is not positive definite; otherwise it returns ``(U, info)`` with info a
    device int32 tensor (0, or 1 + the failing column).
    """
    if not H.is_cuda or H.dtype != torch.float32 or H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be a square float32 GPU tensor")
    if H.stride(1) != 1:
        raise ValueError("H must have unit column stride")
    lib = _load()
    d = H.shape[0]
    if out is None:
        out = torch.empty((d, d), dtype=torch.float32, device=H.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (d, d) or out.stride(1) != 1:
        raise ValueError("out must be a float32 (d, d) GPU tensor with unit column stride")
    need = int(lib.hess_chol_inverse_workspace(d))
    if need < 0:
        raise HessError(-1, f"width {d} not supported")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    _check(lib.hess_chol_inverse_upper(H.data_ptr(), d, H.stride(0), out.data_ptr(), out.stride(0),
                                       workspace.data_ptr(), need, info.data_ptr(), _stream(stream)))
    if not check:
        return out, info
    bad = int(info.item())
    if bad:
        raise HessError(-6, f"the damped Hessian is not positive definite (pivot of column {bad - 1} failed)")
    return out


def gptq_quantize(W: torch.Tensor, U: torch.Tensor, group_size: int = -1, dead: torch.Tensor | None = None,
                  nsamples: int = 1, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None):
    """4-bit error-propagating quantization of W (outputs x inputs, float32) with the factor U.

    Returns ``(Q, codes, scales, loss)``: dequantized float32 weights (``out`` may be W itself),
    uint8 codes 0..15, float32 steps (rows x groups) and a float64 device scalar loss.
    """
    for name, t in (("W", W), ("U", U)):
        if not t.is_cuda or t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a 2-D float32 GPU tensor with unit column stride")
    rows, cols = W.shape
    if tuple(U.shape) != (cols, cols):
        raise ValueError("U must be (cols, cols)")
    lib = _load()
    dev = W.device
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    groups = 1 if group_size == -1 or group_size >= cols else -(-cols // group_size)
    scales = torch.empty((rows, groups), dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    need = int(lib.hess_gptq_quantize_workspace(rows, cols))
    if need < 0:
        raise HessError(-1, f"shape {rows} x {cols} not supported")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    dptr = None
    if dead is not None:
        dead = dead.to(device=dev, dtype=torch.uint8).contiguous()
        if dead.numel() != cols:
            raise ValueError("dead must have one entry per column")
        dptr = dead.data_ptr()
    _check(lib.hess_gptq_quantize(W.data_ptr(), rows, cols, W.stride(0), U.data_ptr(), U.stride(0), dptr,
                                  int(group_size), out.data_ptr(), out.stride(0), codes.data_ptr(), codes.stride(0),
                                  scales.data_ptr(), loss.data_ptr(), int(nsamples), workspace.data_ptr(), need,
                                  _stream(stream)))
    return out, codes, scales, loss


class ImatrixStat:
    """Per-column float32 sums of squares of a layer's inputs (the imatrix statistic)."""

    def __init__(self, d: int, dtype=torch.bfloat16):
        self.d = int(d)
        self.dtype = dtype
        self._h = _load().hess_imatrix_create(self.d, _dtype_code(dtype))
        if not self._h:
            raise HessError(-1, _load().hess_last_error().decode(errors="replace"))

    def add_batch(self, x: torch.Tensor, stream=None) -> None:
        if not x.is_cuda:
            raise ValueError("activations must be on the GPU")
        if x.dtype != self.dtype:
            raise ValueError(f"expected {self.dtype} activations, got {x.dtype}")
        x2, n, ld = _as_rows(x, self.d)
        _check(_load().hess_imatrix_add_batch(self._h, x2.data_ptr() if n > 0 else None, n, ld, _stream(stream)))

    def read(self, out: torch.Tensor | None = None, stream=None):
        """(sums, tokens): the float32 per-column sums and the token count."""
        if out is None:
            out = torch.empty(self.d, dtype=torch.float32, device="cuda")
        n = ctypes.c_int64()
        _check(_load().hess_imatrix_read(self._h, out.data_ptr(), ctypes.byref(n), _stream(stream)))
        return out, int(n.value)

    def reset(self, stream=None) -> None:
        _check(_load().hess_imatrix_reset(self._h, _stream(stream)))

    def close(self) -> None:
        if getattr(self, "_h", None):
            _check(_load().hess_imatrix_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def add_batch_grouped(hessians, x: torch.Tensor, offsets, row_idx: torch.Tensor | None = None, stream=None) -> None:
    """For each e: hessians[e] accumulates rows row_idx[offsets[e]:offsets[e+1]] of x, in one launch."""
    if not hessians:
        raise ValueError("need at least one Hessian")
    d = hessians[0].d
    for h in hessians:
        if h.dtype != x.dtype:
            raise TypeError("all Hessians must take the activation dtype")
    x2, n, ld = _as_rows(x, d)
    offs = [int(o) for o in (offsets.tolist() if hasattr(offsets, "tolist") else offsets)]
    if len(offs) != len(hessians) + 1:
        raise ValueError("offsets must have len(hessians) + 1 entries")
    if row_idx is not None:
        if row_idx.dtype != torch.int32 or not row_idx.is_cuda or not row_idx.is_contiguous():
            raise ValueError("row_idx must be a contiguous int32 GPU tensor")
        if row_idx.numel() < offs[-1]:
            raise ValueError("row_idx shorter than offsets[-1]")
    elif offs[-1] > n:
        raise ValueError("offsets exceed the number of rows of x")
    arr = (ctypes.c_void_p * len(hessians))(*[h._h.value for h in hessians])
    oarr = (ctypes.c_int64 * len(offs))(*offs)
    _check(_load().hess_add_batch_grouped_ex(arr, len(hessians), x2.data_ptr() if n > 0 else None, n, ld,
                                             row_idx.data_ptr() if row_idx is not None else None, oarr,
                                             _stream(stream)))


def reset_grouped(hessians, stream=None) -> None:
    """hessians[e].reset() for every e, in one launch per 64 Hessians of one width."""
    arr = (ctypes.c_void_p * len(hessians))(*[h._h.value for h in hessians])
    _check(_load().hess_reset_grouped(arr, len(hessians), _stream(stream)))


def materialize_grouped(hessians, damp_percent: float = 0.01, outs=None, neutralize: bool = True, stream=None):
    """Materialize many Hessians of one width in two launches per 64; returns [(H, dead, damp)] as
    ``Hessian.materialize`` would for each (the same bits)."""
    if not hessians:
        return []
    d = hessians[0].d
    dev = torch.device("cuda", hessians[0]._device)
    if outs is None:
        outs = [torch.empty((d, d), dtype=torch.float32, device=dev) for _ in hessians]
    if len(outs) != len(hessians):
        raise ValueError("one output per Hessian")
    for o in outs:
        if o.dtype != torch.float32 or tuple(o.shape) != (d, d) or not o.is_contiguous():
            raise ValueError("each output must be a contiguous float32 (d, d) GPU tensor")
    dead = torch.empty((len(hessians), d), dtype=torch.uint8, device=dev)
    damp = torch.empty((len(hessians), 1), dtype=torch.float32, device=dev)
    n = len(hessians)
    hs_arr = (ctypes.c_void_p * n)(*[h._h.value for h in hessians])
    h_arr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    d_arr = (ctypes.c_void_p * n)(*[dead[e].data_ptr() for e in range(n)])
    p_arr = (ctypes.c_void_p * n)(*[damp[e].data_ptr() for e in range(n)])
    flags = 0 if neutralize else HESS_NO_NEUTRALIZE
    _check(_load().hess_materialize_grouped(hs_arr, n, float(damp_percent), flags, h_arr, d_arr, p_arr,
                                            _stream(stream)))
    return [(outs[e], dead[e].view(torch.bool), damp[e]) for e in range(n)]
