"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, sizes state blocks as documented and rejects bad arguments before
touching the GPU.  No kernel runs here."""
from __future__ import annotations

import ctypes
import subprocess

import pytest

from linear_attention_recurrent_gated_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    declared = B.header_functions()
    assert len(declared) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for name in declared:
        assert hasattr(lib, name)
    assert set(B._SIGS) == set(declared)


def test_library_is_gfx950_only():
    """The library embeds device code for gfx950 and for no other target."""
    out = subprocess.run(["strings", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "amdgcn-amd-amdhsa--gfx950" in out
    for other in ("gfx942", "gfx90a", "gfx908", "gfx1100", "sm_"):
        assert f"amdhsa--{other}" not in out


def _align(x):
    return (x + 255) // 256 * 256


def _expected_bytes(variant, units, heads, d, L, es, form=B.DL_LOG_WY):
    pairs = units * heads
    af = form == B.DL_LOG_FACTORS and variant != B.DL_RWKV6
    total = _align(256) + _align(pairs * 4) + _align(pairs * d * d * 4)
    total += _align(pairs * L * d * es) + _align(pairs * L * d * (4 if af else es))
    total += _align(pairs * L * (1 if variant == B.DL_GDN else d) * 4)
    total += _align(0 if variant == B.DL_RWKV6 or af else pairs * L * 4)
    total += _align(0 if variant == B.DL_RWKV6 or af else pairs * (L * (L - 1) // 2) * 4)
    return total


@pytest.mark.parametrize("form", [B.DL_LOG_WY, B.DL_LOG_FACTORS])
@pytest.mark.parametrize("variant", [B.DL_GDN, B.DL_KDA, B.DL_RWKV6, B.DL_GDN2])
@pytest.mark.parametrize("d,L,dt,es", [(128, 16, B.DL_BF16, 2), (64, 32, B.DL_F32, 4),
                                       (128, 0, B.DL_BF16, 2), (64, 64, B.DL_BF16, 2)])
def test_state_bytes(variant, d, L, dt, es, form):
    desc = B.DlDesc(variant, 7, 3, d, d, L, dt, 0, form)
    if variant == B.DL_GDN2 and form == B.DL_LOG_WY and L > 0:
        assert B.dl_state_bytes(desc) == 0          # not built: factor form only
        return
    assert B.dl_state_bytes(desc) == _expected_bytes(variant, 7, 3, d, L, es, form)


@pytest.mark.parametrize("variant", [B.DL_GDN, B.DL_KDA, B.DL_GDN2])
@pytest.mark.parametrize("d,L,M", [(128, 32, 8), (64, 16, 0), (128, 1, 16)])
def test_state_bytes_int8_base(variant, d, L, M):
    """INT8 base: codes, row scales, kept values and indices replace the fp32 base."""
    U, H = 7, 3
    desc = B.DlDesc(variant, U, H, d, d, L, B.DL_BF16, 0, B.DL_LOG_FACTORS, B.DL_BASE_I8, M)
    fp32 = _expected_bytes(variant, U, H, d, L, 2, B.DL_LOG_FACTORS)
    pairs = U * H
    q8 = _align(pairs * d * d) + _align(pairs * d * 4) + _align(pairs * d * M * 4) + _align(H * M * 4)
    assert B.dl_state_bytes(desc) == fp32 - _align(pairs * d * d * 4) + q8


def test_suggest_log_len_int8_base_models_the_smaller_base():
    """With a base a quarter the size, a step's base read weighs less, so the
    traffic model's best log is no longer (it amortises less) and costs less."""
    f = B.DlDesc(B.DL_GDN, 1, 1, 128, 128, 0, B.DL_BF16, 1, B.DL_LOG_FACTORS)
    q = B.DlDesc(B.DL_GDN, 1, 1, 128, 128, 0, B.DL_BF16, 1, B.DL_LOG_FACTORS, B.DL_BASE_I8, 8)
    Lf, bf = B.dl_suggest_log_len(f)
    Lq, bq = B.dl_suggest_log_len(q)
    assert bq < 0.5 * bf and Lq <= Lf


def test_state_bytes_full_size_configs():
    # 64 x 32 heads of 128 x 128 fp32 = 128 MiB of state plus the log
    desc = B.DlDesc(B.DL_GDN, 64, 32, 128, 128, 16, B.DL_BF16)
    assert B.dl_state_bytes(desc) >= 128 * 2**20
    desc = B.DlDesc(B.DL_GDN, 256, 32, 128, 128, 32, B.DL_BF16)
    assert B.dl_state_bytes(desc) >= 512 * 2**20


@pytest.mark.parametrize("fields,code", [
    ((0, 0, 2, 128, 128, 8, B.DL_BF16), B.DL_ERR_INVALID),      # no units
    ((0, 4, 0, 128, 128, 8, B.DL_BF16), B.DL_ERR_INVALID),      # no heads
    ((0, 4, 2, 128, 128, 8, 7), B.DL_ERR_INVALID),              # unknown dtype
    ((0, 4, 2, 128, 128, -1, B.DL_BF16), B.DL_ERR_INVALID),     # negative L
    ((0, 4, 2, 128, 64, 8, B.DL_BF16), B.DL_ERR_UNSUPPORTED),   # d_k != d_v
    ((0, 4, 2, 96, 96, 8, B.DL_BF16), B.DL_ERR_UNSUPPORTED),    # d not built
    ((0, 4, 2, 128, 128, 65, B.DL_BF16), B.DL_ERR_UNSUPPORTED), # L too long
    ((0, 4, 2, 128, 128, 8, B.DL_BF16, 2), B.DL_ERR_INVALID),   # merge_on_step not 0 / 1
    ((0, 4, 2, 128, 128, 8, B.DL_BF16, 0, 2), B.DL_ERR_INVALID),  # unknown log form
    ((4, 4, 2, 128, 128, 8, B.DL_BF16), B.DL_ERR_INVALID),        # unknown variant
    ((3, 4, 2, 128, 128, 8, B.DL_BF16, 0, 0), B.DL_ERR_UNSUPPORTED),  # gated log in WY form
    ((0, 4, 2, 128, 128, 8, B.DL_BF16, 0, 1, 2), B.DL_ERR_INVALID),   # unknown base format
    ((0, 4, 2, 128, 128, 8, B.DL_BF16, 0, 1, 0, 4), B.DL_ERR_INVALID),  # kept channels, fp32 base
    ((0, 4, 2, 128, 128, 8, B.DL_BF16, 0, 1, 1, 17), B.DL_ERR_INVALID),  # too many kept channels
    ((0, 4, 2, 128, 128, 8, B.DL_BF16, 0, 0, 1, 4), B.DL_ERR_UNSUPPORTED),  # INT8 base, WY log
    ((2, 4, 2, 64, 64, 8, B.DL_BF16, 0, 1, 1, 4), B.DL_ERR_UNSUPPORTED),  # INT8 base, RWKV6
    ((0, 4, 2, 128, 128, 0, B.DL_BF16, 0, 1, 1, 4), B.DL_ERR_UNSUPPORTED),  # INT8 base, no log
])
def test_bad_descriptors(lib, fields, code):
    desc = B.DlDesc(*fields)
    assert B.dl_state_bytes(desc) == 0
    out = ctypes.c_void_p()
    st = lib.dl_state_alloc(ctypes.byref(desc), ctypes.c_void_p(256), 1 << 30, None, ctypes.byref(out))
    assert st == code
    assert out.value is None
    assert B.dl_last_error()


def test_alloc_checks_memory_before_launching(lib):
    desc = B.DlDesc(B.DL_GDN, 4, 2, 128, 128, 8, B.DL_BF16)
    need = B.dl_state_bytes(desc)
    out = ctypes.c_void_p()
    assert lib.dl_state_alloc(ctypes.byref(desc), None, need, None, ctypes.byref(out)) == B.DL_ERR_INVALID
    assert lib.dl_state_alloc(ctypes.byref(desc), ctypes.c_void_p(4096 + 8), need, None,
                              ctypes.byref(out)) == B.DL_ERR_INVALID        # misaligned
    assert lib.dl_state_alloc(ctypes.byref(desc), ctypes.c_void_p(4096), need - 1, None,
                              ctypes.byref(out)) == B.DL_ERR_SIZE
    assert "needs" in B.dl_last_error()
    assert lib.dl_state_alloc(ctypes.byref(desc), ctypes.c_void_p(4096), need, None, None) == B.DL_ERR_INVALID


def test_null_handle_is_rejected(lib):
    p = ctypes.c_void_p(4096)
    assert lib.dl_decode_step_eager(None, 1, None, p, p, p, p, p, p, None) == B.DL_ERR_INVALID
    assert lib.dl_decode_step_log(None, 1, None, p, p, p, p, p, p, None) == B.DL_ERR_INVALID
    assert lib.dl_decode_step_eager_ordered(None, 1, None, None, p, p, p, p, p, p, None) == B.DL_ERR_INVALID
    assert lib.dl_decode_step_log_ordered(None, 1, None, None, p, p, p, p, p, p, None) == B.DL_ERR_INVALID
    assert lib.dl_merge(None, 1, None, 0, None) == B.DL_ERR_INVALID
    assert lib.dl_merge_replay(None, 1, None, 0, None) == B.DL_ERR_INVALID
    assert lib.dl_readout(None, 1, None, p, p, None) == B.DL_ERR_INVALID
    assert lib.dl_base_import(None, 1, None, p, None) == B.DL_ERR_INVALID
    assert lib.dl_base_export(None, 1, None, p, None) == B.DL_ERR_INVALID
    assert lib.dl_state_check(None, None, None) == B.DL_ERR_INVALID
    assert lib.dl_state_view(None, None) == B.DL_ERR_INVALID
    assert lib.dl_state_free(None) == B.DL_OK
    assert B.dl_version() == 100


@pytest.mark.parametrize("variant,d,dt,fuse", [(B.DL_GDN, 128, B.DL_BF16, 1), (B.DL_KDA, 128, B.DL_BF16, 1),
                                               (B.DL_KDA, 128, B.DL_BF16, 0), (B.DL_RWKV6, 64, B.DL_BF16, 0),
                                               (B.DL_GDN, 64, B.DL_F32, 0), (B.DL_GDN2, 128, B.DL_BF16, 1)])
@pytest.mark.parametrize("form", [B.DL_LOG_WY, B.DL_LOG_FACTORS])
def test_suggest_log_len(lib, variant, d, dt, fuse, form):
    """The suggested L is the argmin of the documented traffic model, and its
    modeled bytes undercut both extremes (merge every step, longest log)."""
    desc = B.DlDesc(variant, 1, 1, d, d, 0, dt, fuse, form)
    if variant == B.DL_GDN2 and form == B.DL_LOG_WY:
        with pytest.raises(B.DlError):            # the gated log exists in the factor form only
            B.dl_suggest_log_len(desc)
        return
    L, b = B.dl_suggest_log_len(desc)
    assert 1 < L < 64
    es = 2 if dt == B.DL_BF16 else 4
    af = form == B.DL_LOG_FACTORS and variant != B.DL_RWKV6
    St, g = 4 * d * d, (4 if variant == B.DL_GDN else 4 * d)
    bb = 0 if variant == B.DL_RWKV6 else (8 * d if variant == B.DL_GDN2 else 4)
    In, Out = 3 * d * es + g + bb, 4 * d
    E = d * es + d * (4 if af else es) + g + (0 if af else bb)

    def model(L):
        c = (L - 1) / 2
        rt = 4 * ((L - 1) * (L - 2) / 6 + c) if variant != B.DL_RWKV6 and not af else 0
        x = St + c * E + E + In + Out + 8 + rt
        return x + ((St - E) / L if fuse else (2 * St + L * E + 8) / L)

    assert b == pytest.approx(model(L), rel=1e-12)
    assert b < model(1) and b < model(64)


def test_suggest_log_len_errors(lib):
    with pytest.raises(B.DlError):
        B.dl_suggest_log_len(B.DlDesc(0, 1, 1, 96, 96, 0, B.DL_BF16))


def test_binding_rejects_bad_tensors():
    """The torch wrapper checks dtype, shape, layout and device before passing
    raw pointers on (the library cannot see shapes)."""
    import torch
    st = B.DecodeState.__new__(B.DecodeState)     # host logic only: no state block
    st.torch, st.buf = torch, torch.empty(0, dtype=torch.uint8)
    st.heads, st.d, st.variant, st.in_torch_dtype = 2, 64, B.DL_GDN, torch.float32
    x, g, b = torch.zeros(3, 2, 64), torch.zeros(3, 2), torch.zeros(3, 2)
    st._check_inputs(3, x, x, x, g, b)
    assert st._out(3, None).shape == (3, 2, 64)
    bad = (torch.zeros(3, 2, 32), torch.zeros(3, 2, 64, dtype=torch.float64),
           torch.zeros(3, 64, 2).transpose(1, 2))
    for y in bad:
        with pytest.raises(ValueError):
            st._check_inputs(3, x, y, x, g, b)
        with pytest.raises(ValueError):
            st._out(3, y)
    with pytest.raises(ValueError):
        st._check_inputs(3, x, x, x, torch.zeros(3, 2, 64), b)   # GDN decay is one scalar per head
    with pytest.raises(ValueError):
        st._check_inputs(3, x, x, x, g, None)                    # beta is required
    st.variant = B.DL_GDN2
    with pytest.raises(ValueError):
        st._check_inputs(3, x, x, x, torch.zeros(3, 2, 64), b)   # gated: [rows, H, d_k + d_v]
    st._check_inputs(3, x, x, x, torch.zeros(3, 2, 64), torch.zeros(3, 2, 128))
    with pytest.raises(ValueError):
        st._slots(torch.zeros(3, dtype=torch.int64), 3)
    with pytest.raises(ValueError):
        st._slots(torch.zeros(4, dtype=torch.int32), 3)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No library, no fallback: the binding raises instead of computing anything."""
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.load(str(tmp_path / "libdeltalog.so"))


def test_stream_probe_rejects_bad_arguments():
    """Argument checks of the streaming-rate probe, all before any launch."""
    buf = 4096   # a host address: never dereferenced, every call below is rejected first
    bad = [
        (7, buf, buf, 1024, B.DL_ERR_INVALID),                   # unknown mode
        (B.DL_PROBE_READ, None, buf, 1024, B.DL_ERR_INVALID),    # NULL source
        (B.DL_PROBE_COPY, buf, None, 1024, B.DL_ERR_INVALID),    # NULL destination
        (B.DL_PROBE_COPY, buf + 4, buf, 1024, B.DL_ERR_INVALID), # misaligned
        (B.DL_PROBE_READ, buf, buf, 0, B.DL_ERR_INVALID),        # empty
        (B.DL_PROBE_READ, buf, buf, 1000, B.DL_ERR_INVALID),     # not a multiple of 16
        (B.DL_PROBE_READ, buf, buf, 1 << 62, B.DL_ERR_UNSUPPORTED),
    ]
    for mode, src, dst, n, want in bad:
        with pytest.raises(B.DlError) as e:
            B.dl_stream_probe(mode, src, dst, n, None)
        assert e.value.status == want, (mode, src, dst, n)
    with pytest.raises(B.DlError) as e:
        B.dl_stream_probe(B.DL_PROBE_READ, buf, buf, 1024, None, start_event=buf)
    assert e.value.status == B.DL_ERR_INVALID


def test_streaming_rule():
    """The cache policy: an eager state streams above 256 MiB, a state with a
    log once base and log together exceed 384 MiB (the log counts: a 256 MiB
    base with a 160 MiB log streams)."""
    def desc(variant, units, d, L, form=B.DL_LOG_FACTORS, base=B.DL_BASE_F32, M=0, fuse=1):
        return B.DlDesc(variant, units, 32, d, d, L, B.DL_BF16, fuse if L else 0, form, base, M)
    cases = [
        (desc(B.DL_GDN, 64, 128, 16), False),               # 128 MiB base + 25 MiB log
        (desc(B.DL_KDA, 128, 128, 0), False),               # eager, 256 MiB
        (desc(B.DL_RWKV6, 1024, 64, 0), True),              # eager, 512 MiB (d = 64)
        (desc(B.DL_KDA, 128, 128, 16), False),              # 256 + 80 MiB
        (desc(B.DL_KDA, 128, 128, 32), True),               # 256 + 160 MiB
        (desc(B.DL_KDA, 128, 128, 64), True),               # 256 + 320 MiB
        (desc(B.DL_KDA, 128, 128, 32, form=B.DL_LOG_WY), True),   # 256 + 136 MiB
        (desc(B.DL_GDN, 256, 128, 32), True),               # 512 MiB base
        (desc(B.DL_KDA, 128, 128, 32, base=B.DL_BASE_I8, M=8), False),  # 82 + 160 MiB
    ]
    for d, want in cases:
        assert B.dl_state_streams(d) == want, (d.variant, d.units, d.log_len, d.base_format)
    with pytest.raises(B.DlError):
        B.dl_state_streams(B.DlDesc(0, 1, 1, 96, 96, 0, B.DL_BF16))
