"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before any device work (no GPU needed: every
call here fails validation, so nothing is launched and no pointer is touched)."""
import ctypes
import os
import re

import pytest

from linear_attention_sequence_chunked_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

# Fake but 16-byte aligned, non-overlapping addresses.  They are never
# dereferenced: each call below fails a host-side check first.
BASE = 0x7F0000000000
STEP = 1 << 32


def addr(i, misalign=0):
    return ctypes.c_void_p(BASE + i * STEP + misalign)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GDN_API[^;(]*?\b(gdn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gdn.load_library()
    names = declared_symbols()
    assert "gdn_chunk_fwd" in names and "gdn_status_string" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(gdn.SIGNATURES), "binding and header disagree"


def test_abi_version_and_status_strings():
    lib = gdn.load_library()
    assert lib.gdn_abi_version() == 1
    for code in range(4):
        assert len(gdn.status_string(code)) > 0
    assert gdn.status_string(99) == "unknown status"


def call(q=0, k=1, v=2, a=3, b=4, s0=None, o=6, sf=None, B=2, T=100, H=3, K=64, V=64,
         chunk=64, dtype=gdn.GDN_DTYPE_BF16, misalign=None):
    lib = gdn.load_library()
    ptrs = {"q": q, "k": k, "v": v, "a": a, "b": b, "s0": s0, "o": o, "sf": sf}
    args = []
    for name, i in ptrs.items():
        if i is None:
            args.append(None)
        elif isinstance(i, ctypes.c_void_p):
            args.append(i)
        else:
            args.append(addr(i, 2 if misalign == name else 0))
    return lib.gdn_chunk_fwd(*args, B, T, H, K, V, chunk, dtype, None)


def test_null_required_pointers_are_invalid():
    for name in ("q", "k", "v", "a", "b", "o"):
        assert call(**{name: None}) == gdn.GDN_ERROR_INVALID_VALUE, name


def test_non_positive_sizes_are_invalid():
    for kw in ({"B": 0}, {"T": 0}, {"H": -1}, {"K": 0}, {"V": 0}, {"chunk": 0}):
        assert call(**kw) == gdn.GDN_ERROR_INVALID_VALUE, kw


def test_misaligned_pointer_is_invalid():
    for name in ("q", "k", "v", "a", "b", "o"):
        assert call(misalign=name) == gdn.GDN_ERROR_INVALID_VALUE, name
    assert call(s0=5, misalign="s0") == gdn.GDN_ERROR_INVALID_VALUE
    assert call(sf=7, misalign="sf") == gdn.GDN_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [{"K": 48}, {"V": 256}, {"K": 8}, {"chunk": 128}, {"chunk": 24},
                                {"dtype": 7}, {"B": 1 << 20, "T": 1 << 12, "H": 8}])
def test_unsupported_configurations(kw):
    assert call(**kw) == gdn.GDN_ERROR_NOT_SUPPORTED


def test_overlapping_output_is_invalid():
    # o overlapping q, final_state overlapping v, final_state overlapping o
    assert call(o=ctypes.c_void_p(BASE + 64)) == gdn.GDN_ERROR_INVALID_VALUE
    assert call(sf=ctypes.c_void_p(BASE + 2 * STEP + 4096)) == gdn.GDN_ERROR_INVALID_VALUE
    assert call(sf=ctypes.c_void_p(BASE + 6 * STEP + 4096)) == gdn.GDN_ERROR_INVALID_VALUE
    # final_state partly overlapping initial_state (not the same pointer)
    assert call(s0=5, sf=ctypes.c_void_p(BASE + 5 * STEP + 1024)) == gdn.GDN_ERROR_INVALID_VALUE


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 16)
    g = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        gdn.chunk_fwd(x, x, x, g, g)
