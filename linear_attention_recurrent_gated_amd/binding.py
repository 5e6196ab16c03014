"""ctypes binding of ``libdeltalog.so`` (``include/deltalog.h``).

Argument marshalling only: every computation runs in the library's gfx950
kernels.  The functions below carry the C ABI's names and take raw device
pointers (ints) and a stream handle; :class:`DecodeState` wraps them for
torch tensors (torch supplies device memory and streams, nothing else).

If the library is missing this module raises at first use; there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdeltalog.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "deltalog.h")

DL_OK, DL_ERR_INVALID, DL_ERR_UNSUPPORTED, DL_ERR_SIZE, DL_ERR_LAUNCH, DL_ERR_STATE = range(6)
DL_GDN, DL_KDA, DL_RWKV6, DL_GDN2 = 0, 1, 2, 3
DL_F32, DL_BF16 = 0, 1
DL_MERGE_FULL, DL_MERGE_ALL = 0, 1
DL_LOG_WY, DL_LOG_FACTORS = 0, 1
DL_FLAG_LOG_FULL, DL_FLAG_LOG_NONEMPTY, DL_FLAG_BAD_SLOT, DL_FLAG_BAD_KEPT = 1, 2, 4, 8
DL_BASE_F32, DL_BASE_I8 = 0, 1
DL_PROBE_READ, DL_PROBE_COPY = 0, 1


class DlDesc(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("units", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("log_len", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("merge_on_step", ctypes.c_int32), ("log_form", ctypes.c_int32),
                ("base_format", ctypes.c_int32), ("kept_channels", ctypes.c_int32)]


class DlStatePtrs(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("log_k", ctypes.c_void_p),
                ("log_v", ctypes.c_void_p), ("log_g", ctypes.c_void_p),
                ("log_beta", ctypes.c_void_p), ("log_t", ctypes.c_void_p), ("fill", ctypes.c_void_p),
                ("flags", ctypes.c_void_p), ("base_codes", ctypes.c_void_p),
                ("base_scale", ctypes.c_void_p), ("base_kept", ctypes.c_void_p),
                ("kept_idx", ctypes.c_void_p)]


class DlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"deltalog status {status}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "dl_state_bytes": (ctypes.c_size_t, [ctypes.POINTER(DlDesc)]),
    "dl_state_alloc": (_I, [ctypes.POINTER(DlDesc), _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "dl_state_free": (_I, [_P]),
    "dl_state_view": (_I, [_P, ctypes.POINTER(DlStatePtrs)]),
    "dl_decode_step_eager": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dl_decode_step_log": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dl_decode_step_eager_ordered": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dl_decode_step_log_ordered": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dl_merge": (_I, [_P, _I, _P, _I, _P]),
    "dl_merge_replay": (_I, [_P, _I, _P, _I, _P]),
    "dl_readout": (_I, [_P, _I, _P, _P, _P, _P]),
    "dl_base_import": (_I, [_P, _I, _P, _P, _P]),
    "dl_base_export": (_I, [_P, _I, _P, _P, _P]),
    "dl_state_check": (_I, [_P, _P, ctypes.POINTER(_I)]),
    "dl_time_next_launch": (_I, [_P, _P, _P]),
    "dl_last_error": (ctypes.c_char_p, []),
    "dl_version": (_I, []),
    "dl_suggest_log_len": (_I, [ctypes.POINTER(DlDesc), ctypes.POINTER(ctypes.c_int32),
                                ctypes.POINTER(ctypes.c_double)]),
    "dl_stream_probe": (_I, [_I, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "dl_state_streams": (_I, [ctypes.POINTER(DlDesc), ctypes.POINTER(_I)]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once) and declare every entry point's signature."""
    global _lib
    if _lib is None:
        # torch bundles its own HIP runtime under the same soname; loading it
        # first makes this library bind to that one runtime, so streams,
        # events and allocations are shared.
        import torch  # noqa: F401
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/deltalog.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dl_[a-z_]+)\s*\(", text)))


def _check(status: int):
    if status != DL_OK:
        raise DlError(status, load().dl_last_error().decode())


def dl_last_error() -> str:
    return load().dl_last_error().decode()


def dl_version() -> int:
    return int(load().dl_version())


def dl_suggest_log_len(desc: DlDesc):
    """(L, modeled bytes per update) with the lowest modeled cost for this shape."""
    L = ctypes.c_int32(0)
    b = ctypes.c_double(0.0)
    rc = load().dl_suggest_log_len(ctypes.byref(desc), ctypes.byref(L), ctypes.byref(b))
    if rc != DL_OK:
        raise DlError(rc, dl_last_error())
    return int(L.value), float(b.value)


def dl_state_bytes(desc: DlDesc) -> int:
    return int(load().dl_state_bytes(ctypes.byref(desc)))


def dl_state_alloc(desc: DlDesc, dev_mem: int, nbytes: int, stream: int):
    out = _P()
    _check(load().dl_state_alloc(ctypes.byref(desc), dev_mem, nbytes, stream, ctypes.byref(out)))
    return out


def dl_state_free(handle) -> None:
    _check(load().dl_state_free(handle))


def dl_state_view(handle) -> DlStatePtrs:
    out = DlStatePtrs()
    _check(load().dl_state_view(handle, ctypes.byref(out)))
    return out


def dl_decode_step_eager(handle, rows, slot_idx, q, k, v, g, beta, o, stream) -> None:
    _check(load().dl_decode_step_eager(handle, rows, slot_idx, q, k, v, g, beta, o, stream))


def dl_decode_step_log(handle, rows, slot_idx, q, k, v, g, beta, o, stream) -> None:
    _check(load().dl_decode_step_log(handle, rows, slot_idx, q, k, v, g, beta, o, stream))


def dl_decode_step_eager_ordered(handle, rows, slot_idx, row_order, q, k, v, g, beta, o,
                                 stream) -> None:
    _check(load().dl_decode_step_eager_ordered(handle, rows, slot_idx, row_order, q, k, v, g, beta,
                                               o, stream))


def dl_decode_step_log_ordered(handle, rows, slot_idx, row_order, q, k, v, g, beta, o,
                               stream) -> None:
    _check(load().dl_decode_step_log_ordered(handle, rows, slot_idx, row_order, q, k, v, g, beta,
                                             o, stream))


def dl_merge(handle, rows, slot_idx, mode, stream) -> None:
    _check(load().dl_merge(handle, rows, slot_idx, mode, stream))


def dl_merge_replay(handle, rows, slot_idx, mode, stream) -> None:
    _check(load().dl_merge_replay(handle, rows, slot_idx, mode, stream))


def dl_readout(handle, rows, slot_idx, q, o, stream) -> None:
    _check(load().dl_readout(handle, rows, slot_idx, q, o, stream))


def dl_base_import(handle, rows, slot_idx, src, stream) -> None:
    _check(load().dl_base_import(handle, rows, slot_idx, src, stream))


def dl_base_export(handle, rows, slot_idx, dst, stream) -> None:
    _check(load().dl_base_export(handle, rows, slot_idx, dst, stream))


def dl_time_next_launch(handle, start_event, stop_event) -> None:
    _check(load().dl_time_next_launch(handle, start_event, stop_event))


def dl_state_streams(desc: DlDesc) -> bool:
    """Whether a state with this descriptor streams its base (cache policy)."""
    out = _I(0)
    _check(load().dl_state_streams(ctypes.byref(desc), ctypes.byref(out)))
    return bool(out.value)


def dl_stream_probe(mode, src, dst, nbytes, stream, start_event=None, stop_event=None) -> None:
    _check(load().dl_stream_probe(mode, src, dst, nbytes, stream, start_event, stop_event))


def dl_state_check(handle, stream) -> int:
    """Returns the device flag word (and clears it); raises nothing for set flags."""
    flags = _I(0)
    st = load().dl_state_check(handle, stream, ctypes.byref(flags))
    if st not in (DL_OK, DL_ERR_STATE):
        _check(st)
    return int(flags.value)


# ---------------------------------------------------------------------------
# torch convenience layer (memory and streams only)
# ---------------------------------------------------------------------------
class DecodeState:
    """One state block in a torch uint8 device buffer, with tensor views.

    ``base`` ``[units, H, d, d]`` fp32, ``fill`` ``[units, H]`` int32, and the
    log views ``log_k``/``log_v`` ``[units, H, L, d]`` (input dtype),
    ``log_g`` ``[units, H, L]`` or ``[units, H, L, d]``, ``log_beta``
    ``[units, H, L]`` and ``log_t`` ``[units, H, L(L-1)/2]`` (the packed
    key-side factors of the delta-rule variants).  With
    ``log_form=DL_LOG_FACTORS`` (GDN, KDA) ``log_v`` holds the fp32 factors
    ``a_t`` and there is no ``log_beta`` or ``log_t``.  With
    ``base_format=DL_BASE_I8`` the base is ``base_codes`` ``[units, H, d, d]``
    int8, ``base_scale`` ``[units, H, d]``, ``base_kept`` ``[units, H, d, M]``
    and ``kept_idx`` ``[H, M]`` (``M = kept_channels``), and ``base`` is None:
    read and write it with :meth:`export_base` and :meth:`import_base`.
    """

    def __init__(self, variant: int, units: int, heads: int, d: int, log_len: int,
                 dtype: str = "bf16", device="cuda", stream=None, merge_on_step: bool = False,
                 log_form: int = DL_LOG_WY, base_format: int = DL_BASE_F32, kept_channels: int = 0):
        import torch

        self.torch = torch
        self.variant, self.units, self.heads, self.d, self.L = variant, units, heads, d, log_len
        self.dtype = dtype
        self.in_torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.merge_on_step = bool(merge_on_step)
        self.log_form = int(log_form)
        self.factors = self.log_form == DL_LOG_FACTORS and variant != DL_RWKV6
        self.base_format, self.kept_channels = int(base_format), int(kept_channels)
        self.desc = DlDesc(variant, units, heads, d, d, log_len,
                           DL_BF16 if dtype == "bf16" else DL_F32, int(self.merge_on_step),
                           self.log_form, self.base_format, self.kept_channels)
        nbytes = dl_state_bytes(self.desc)
        if nbytes == 0:
            raise DlError(DL_ERR_INVALID, dl_last_error())
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = dl_state_alloc(self.desc, self.buf.data_ptr(), nbytes, self._stream(stream))
        p = dl_state_view(self.handle)
        U, H, L = units, heads, log_len
        M = self.kept_channels
        if self.base_format == DL_BASE_I8:
            self.base = None
            self.base_codes = self._view(p.base_codes, torch.int8, (U, H, d, d))
            self.base_scale = self._view(p.base_scale, torch.float32, (U, H, d))
            self.base_kept = self._view(p.base_kept, torch.float32, (U, H, d, M)) if M else None
            self.kept_idx = self._view(p.kept_idx, torch.int32, (H, M)) if M else None
        else:
            self.base = self._view(p.base, torch.float32, (U, H, d, d))
        self.fill = self._view(p.fill, torch.int32, (U, H))
        self.flags = self._view(p.flags, torch.int32, (1,))
        if L > 0:
            self.log_k = self._view(p.log_k, self.in_torch_dtype, (U, H, L, d))
            self.log_v = self._view(p.log_v, torch.float32 if self.factors else self.in_torch_dtype,
                                    (U, H, L, d))
            gshape = (U, H, L) if variant == DL_GDN else (U, H, L, d)
            self.log_g = self._view(p.log_g, torch.float32, gshape)
            self.log_beta = (self._view(p.log_beta, torch.float32, (U, H, L))
                             if variant != DL_RWKV6 and not self.factors else None)
            nt = L * (L - 1) // 2
            self.log_t = (self._view(p.log_t, torch.float32, (U, H, nt))
                          if variant != DL_RWKV6 and nt > 0 and not self.factors else None)

    def _view(self, ptr, dtype, shape):
        torch = self.torch
        off = int(ptr) - self.buf.data_ptr()
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype).view(shape)

    def _stream(self, stream):
        if stream is None:
            return self.torch.cuda.current_stream().cuda_stream
        return getattr(stream, "cuda_stream", stream)

    def _tensor(self, name, x, dtype, shape):
        """Raise ValueError unless ``x`` is a contiguous ``dtype`` tensor of
        ``shape`` on this state's device (the library sees raw pointers only)."""
        if x is None:
            raise ValueError(f"{name} is required")
        if x.dtype != dtype or tuple(x.shape) != tuple(shape) or not x.is_contiguous() \
                or x.device != self.buf.device:
            raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)} "
                             f"on {self.buf.device}, got {x.dtype} {tuple(x.shape)} on {x.device}"
                             f"{'' if x.is_contiguous() else ' (not contiguous)'}")
        return x

    def _slots(self, slot_idx, rows):
        if slot_idx is None:
            return None
        return self._tensor("slot_idx", slot_idx, self.torch.int32, (rows,)).data_ptr()

    def _rows(self, q, slot_idx):
        rows = q.shape[0]
        self._tensor("q", q, self.in_torch_dtype, (rows, self.heads, self.d))
        return rows, self._slots(slot_idx, rows)

    def _check_inputs(self, rows, q, k, v, g, beta):
        t = self.torch
        H, d = self.heads, self.d
        for name, x in (("q", q), ("k", k), ("v", v)):
            self._tensor(name, x, self.in_torch_dtype, (rows, H, d))
        self._tensor("g", g, t.float32, (rows, H) if self.variant == DL_GDN else (rows, H, d))
        if self.variant != DL_RWKV6:
            self._tensor("beta", beta, t.float32,
                         (rows, H, 2 * d) if self.variant == DL_GDN2 else (rows, H))

    def _out(self, rows, o):
        if o is None:
            return self.torch.empty((rows, self.heads, self.d), dtype=self.torch.float32,
                                    device=self.buf.device)
        return self._tensor("o", o, self.torch.float32, (rows, self.heads, self.d))

    def _order(self, row_order, rows):
        if row_order is None:
            return None
        return self._tensor("row_order", row_order, self.torch.int32, (rows,)).data_ptr()

    def step_eager(self, q, k, v, g, beta=None, o=None, slot_idx=None, stream=None,
                   row_order=None):
        rows, sp = self._rows(q, slot_idx)
        self._check_inputs(rows, q, k, v, g, beta)
        o = self._out(rows, o)
        dl_decode_step_eager_ordered(self.handle, rows, sp, self._order(row_order, rows),
                                     q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                     None if beta is None else beta.data_ptr(), o.data_ptr(),
                                     self._stream(stream))
        return o

    def step_log(self, q, k, v, g, beta=None, o=None, slot_idx=None, stream=None,
                 row_order=None):
        rows, sp = self._rows(q, slot_idx)
        self._check_inputs(rows, q, k, v, g, beta)
        o = self._out(rows, o)
        dl_decode_step_log_ordered(self.handle, rows, sp, self._order(row_order, rows),
                                   q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                   None if beta is None else beta.data_ptr(), o.data_ptr(),
                                   self._stream(stream))
        return o

    def merge(self, mode: int = DL_MERGE_FULL, rows: int | None = None, slot_idx=None,
              replay: bool = False, stream=None):
        if rows is None:
            rows = self.units if slot_idx is None else slot_idx.shape[0]
        sp = self._slots(slot_idx, rows)
        fn = dl_merge_replay if replay else dl_merge
        fn(self.handle, rows, sp, mode, self._stream(stream))

    def import_base(self, src, slot_idx=None, stream=None):
        """Write the bases of ``src.shape[0]`` units from fp32 states ``[rows, H, d, d]``."""
        rows = src.shape[0]
        self._tensor("src", src, self.torch.float32, (rows, self.heads, self.d, self.d))
        dl_base_import(self.handle, rows, self._slots(slot_idx, rows), src.data_ptr(),
                       self._stream(stream))

    def export_base(self, rows: int | None = None, slot_idx=None, out=None, stream=None):
        """The units' bases as fp32 states ``[rows, H, d, d]``."""
        if rows is None:
            rows = self.units if slot_idx is None else slot_idx.shape[0]
        t = self.torch
        if out is None:
            out = t.empty((rows, self.heads, self.d, self.d), dtype=t.float32, device=self.buf.device)
        self._tensor("out", out, t.float32, (rows, self.heads, self.d, self.d))
        dl_base_export(self.handle, rows, self._slots(slot_idx, rows), out.data_ptr(),
                       self._stream(stream))
        return out

    def readout(self, q, o=None, slot_idx=None, stream=None):
        rows, sp = self._rows(q, slot_idx)
        o = self._out(rows, o)
        dl_readout(self.handle, rows, sp, q.data_ptr(), o.data_ptr(), self._stream(stream))
        return o

    def check(self, stream=None) -> int:
        return dl_state_check(self.handle, self._stream(stream))

    def close(self):
        if getattr(self, "handle", None) is not None:
            dl_state_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
