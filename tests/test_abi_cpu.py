"""The C ABI library on the CPU: it loads, exports every function that
include/tt.h declares, and its host-side guards work without touching a GPU."""

import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "tt.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:int|void|const char \*)\s*\**\s*(tt_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import autograd_transformer_amd as tt
    return tt.lib()


def test_header_declares_the_named_entry_points():
    names = declared_functions()
    for required in ("tt_ctx_create", "tt_block_fwd", "tt_block_bwd", "tt_lmhead_ce_fwdbwd",
                     "tt_adamw_step", "tt_train_step"):
        assert required in names
    assert len(names) >= 35


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in tt.h but not exported"


def test_binding_declares_every_header_function():
    from autograd_transformer_amd import _lib
    assert sorted(_lib.SIGS) == declared_functions()


def test_only_the_c_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {os.path.join(ROOT, 'autograd_transformer_amd', 'libtt.so')}").read()
    syms = [l.split()[-1] for l in out.splitlines() if l.split() and l.split()[-2] in ("T", "W")]
    assert syms and all(s.startswith("tt_") for s in syms), syms[:10]


def test_status_strings(lib):
    for code in range(0, -8, -1):
        assert lib.tt_strerror(code)
    assert b"unknown" in lib.tt_strerror(-99)


def test_null_and_stale_handles_without_gpu(lib):
    lib.tt_ctx_destroy(None)
    lib.tt_model_destroy(None)
    lib.tt_block_saved_destroy(None)
    lib.tt_kvcache_destroy(None)
    assert lib.tt_ctx_sync(None) == -1
    fake = ctypes.create_string_buffer(512)   # zeroed memory: wrong magic word
    fp = ctypes.cast(fake, ctypes.c_void_p)
    assert lib.tt_ctx_sync(fp) == -4
    assert lib.tt_ctx_mark(fp) == -4
    assert lib.tt_linear_fwd(fp, 0, 1, 1, 1, None, None, None, None, 0, None, None) == -4
    assert lib.tt_model_refresh_shadow(fp) == -4
    assert lib.tt_model_decode(fp, fp, fp, 1, 0, fp, None, fp) == -4
    assert lib.tt_argmax(fp, 0, 1, 1, 1, fp, fp) == -4
    assert lib.tt_ctx_create(0, None, 1 << 20, None, None) == -1


def _ln_workspace(lib, n, C):
    out = ctypes.c_size_t(0)
    assert lib.tt_layernorm_bwd_workspace(n, C, ctypes.byref(out)) == 0
    return out.value


def test_layernorm_workspace_covers_every_smaller_step(lib):
    """The LayerNorm backward's partial-sum workspace, sized once for up to
    n_rows rows, must hold what any N <= n_rows needs.  Its workgroup count
    drops where a wave's rows step from 2 to 4 (N = 4096) and from 4 to 8
    (N = 8192), so the size for n_rows is the maximum over N <= n_rows and
    never shrinks as n_rows grows."""
    C = 768
    per_group = 3 * C * 4
    # row-walking kernel: 4 waves x 2 rows per workgroup up to N = 4096,
    # 4 x 4 up to 8192, 4 x 8 beyond
    def groups(n):
        r = 2 if n <= 4096 else (4 if n <= 8192 else 8)
        return -(-n // (4 * r))
    prev = 0
    for n in sorted(set(range(1, 20000, 97)) | {4095, 4096, 4097, 6144, 8192, 8193, 16384, 16385}):
        ws = _ln_workspace(lib, n, C)
        assert ws >= prev, (n, ws, prev)
        prev = ws
        assert ws == per_group * max(groups(m) for m in {n, min(n, 4096), min(n, 8192)}), n
    # the case that overran: a capacity of 6 x 1024 rows run at 4 x 1024
    assert _ln_workspace(lib, 6144, C) >= per_group * groups(4096) == per_group * 512
    assert _ln_workspace(lib, 6144, C) > per_group * groups(6144)
    # wide rows take the other kernel, whose count is monotone
    assert _ln_workspace(lib, 5000, 2048) >= _ln_workspace(lib, 4999, 2048)
    bad = ctypes.c_size_t(0)
    assert lib.tt_layernorm_bwd_workspace(10, 766, ctypes.byref(bad)) == -1
    assert lib.tt_layernorm_bwd_workspace(10, 768, None) == -1
