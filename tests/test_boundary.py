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
    assert lib.gdn_abi_version() == 8
    for code in range(5):
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
                                {"dtype": 7}, {"B": 1 << 20, "T": 1 << 12, "H": 8},
                                # state [B, H, V, K] above 2^31 elements (tokens well below)
                                {"B": 8193, "T": 1, "H": 16, "K": 128, "V": 128}])
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


def call_bwd(B=2, T=100, H=3, K=64, V=64, chunk=64, dtype=gdn.GDN_DTYPE_BF16, ws_bytes=None,
             null=None, misalign=None, ptr=None):
    """gdn_chunk_bwd on fake addresses: every case here must fail host validation."""
    lib = gdn.load_library()
    names = ["q", "k", "v", "a", "b", "s0", "do", "dsf", "dq", "dk", "dv", "da", "db", "ds0", "ws"]
    args = []
    for i, name in enumerate(names):
        if name == null:
            args.append(None)
        elif ptr and name in ptr:
            args.append(ptr[name])
        else:
            args.append(addr(i, 2 if misalign == name else 0))
    need = lib.gdn_chunk_bwd_workspace_size(B, T, H, K, V, chunk,
                                            dtype if dtype in (0, 1) else gdn.GDN_DTYPE_BF16)
    return lib.gdn_chunk_bwd(*args, need if ws_bytes is None else ws_bytes, B, T, H, K, V, chunk,
                             dtype, None)


def test_bwd_workspace_size():
    lib = gdn.load_library()
    F32, BF16 = gdn.GDN_DTYPE_F32, gdn.GDN_DTYPE_BF16

    def scalar(B, T, H, K, V, chunk, f32=True):
        # float32 path: per (b, h, chunk of min(chunk, 32) tokens) two fp32 [V,K]
        # states and 3 C x C + 3 C float32 factors, and for float32 inputs the
        # state recompute's records: 16 x 16 lower blocks of two C x C matrices,
        # two C-vectors and 4 floats
        C = min(chunk, 32)
        nb = C // 16
        rec = nb * (nb + 1) * 256 + 2 * C + 4 if f32 else 0
        return B * H * -(-T // C) * (2 * V * K + 3 * C * C + 3 * C + rec) * 4

    def mfma(B, T, H, K, V):
        # matrix-core path: per 64-token chunk two bf16 [V,K] states and a 16896-byte
        # record (Tm, P as bf16 64 x 64, gates as fp32), whatever the chunk
        return B * H * -(-T // 64) * (2 * V * K * 2 + 16896)

    assert lib.gdn_chunk_bwd_workspace_size(2, 100, 3, 64, 32, 64, F32) == scalar(2, 100, 3, 64, 32, 64)
    assert lib.gdn_chunk_bwd_workspace_size(1, 17, 1, 16, 16, 16, F32) == scalar(1, 17, 1, 16, 16, 16)
    assert lib.gdn_chunk_bwd_workspace_size(0, 17, 1, 16, 16, 16, F32) == 0
    assert lib.gdn_chunk_bwd_workspace_size(1, 17, 1, 16, 16, 16, 7) == 0
    # bf16 with K or V = 16 takes the float32 path
    assert lib.gdn_chunk_bwd_workspace_size(1, 100, 2, 16, 64, 32, BF16) == \
        scalar(1, 100, 2, 16, 64, 32, f32=False)
    assert scalar(1, 64, 1, 16, 16, 32) - scalar(1, 64, 1, 16, 16, 32, f32=False) == 2 * 1604 * 4
    # bf16 with K, V in {32, 64, 128}: the matrix-core layout alone, whatever the chunk
    for chunk in (16, 32, 64):
        assert lib.gdn_chunk_bwd_workspace_size(1, 256, 1, 128, 128, chunk, BF16) == \
            mfma(1, 256, 1, 128, 128)
        assert lib.gdn_chunk_bwd_workspace_size(1, 256, 1, 128, 128, chunk, F32) == \
            scalar(1, 256, 1, 128, 128, chunk)
    # the forward+backward workload (B4 T2048 H6 d128 bf16): about 63 MB, not the
    # 220 MB float32 layout
    ws = lib.gdn_chunk_bwd_workspace_size(4, 2048, 6, 128, 128, 64, BF16)
    assert ws == mfma(4, 2048, 6, 128, 128) == 63_307_776
    assert ws < scalar(4, 2048, 6, 128, 128, 64)


def test_bwd_rejects_bad_arguments():
    for name in ("q", "k", "v", "a", "b", "do", "dq", "dk", "dv", "da", "db", "ws"):
        assert call_bwd(null=name) == gdn.GDN_ERROR_INVALID_VALUE, name
    for name in ("q", "dq", "ws", "ds0"):
        assert call_bwd(misalign=name) == gdn.GDN_ERROR_INVALID_VALUE, name
    assert call_bwd(ws_bytes=1024) == gdn.GDN_ERROR_INVALID_VALUE
    assert call_bwd(T=0) == gdn.GDN_ERROR_INVALID_VALUE
    assert call_bwd(K=48) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert call_bwd(chunk=128) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert call_bwd(dtype=5) == gdn.GDN_ERROR_NOT_SUPPORTED
    # dk overlapping dq, workspace overlapping d_o, dv overlapping v
    assert call_bwd(ptr={"dk": ctypes.c_void_p(BASE + 8 * STEP + 64)}) == gdn.GDN_ERROR_INVALID_VALUE
    assert call_bwd(ptr={"ws": ctypes.c_void_p(BASE + 6 * STEP)}) == gdn.GDN_ERROR_INVALID_VALUE
    assert call_bwd(ptr={"dv": ctypes.c_void_p(BASE + 2 * STEP + 128)}) == gdn.GDN_ERROR_INVALID_VALUE


def test_decode_rejects_bad_arguments():
    lib = gdn.load_library()

    def dcall(null=None, misalign=None, K=64, V=64, dtype=gdn.GDN_DTYPE_BF16, same=None):
        ptrs = []
        for i, name in enumerate(["q", "k", "v", "a", "b", "s", "o"]):
            if name == null:
                ptrs.append(None)
            elif same and name == same[1]:
                ptrs.append(addr(["q", "k", "v", "a", "b", "s", "o"].index(same[0])))
            else:
                ptrs.append(addr(i, 2 if name == misalign else 0))
        return lib.gdn_decode_step(*ptrs, 2, 3, K, V, dtype, None)

    for name in ("q", "k", "v", "a", "b", "s", "o"):
        assert dcall(null=name) == gdn.GDN_ERROR_INVALID_VALUE, name
        assert dcall(misalign=name) == gdn.GDN_ERROR_INVALID_VALUE, name
    assert dcall(K=48) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert dcall(dtype=3) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert dcall(same=("s", "o")) == gdn.GDN_ERROR_INVALID_VALUE      # o aliases the state
    assert dcall(same=("q", "s")) == gdn.GDN_ERROR_INVALID_VALUE      # state aliases q


def test_varlen_rejects_bad_arguments():
    lib = gdn.load_library()

    def vcall(cu=8, N=3, misalign=None, null=None, T=100, K=64):
        names = ["q", "k", "v", "a", "b"]
        args = [None if n == null else addr(i, 2 if n == misalign else 0) for i, n in enumerate(names)]
        cu_ptr = None if cu is None else (addr(cu) if isinstance(cu, int) else cu)
        return lib.gdn_chunk_fwd_varlen(*args, cu_ptr, N, None, addr(6), None, T, 2, K, 64, 64,
                                        gdn.GDN_DTYPE_BF16, None)

    assert vcall(cu=None) == gdn.GDN_ERROR_INVALID_VALUE
    assert vcall(cu=ctypes.c_void_p(BASE + 8 * STEP + 2)) == gdn.GDN_ERROR_INVALID_VALUE  # misaligned table
    assert vcall(N=0) == gdn.GDN_ERROR_INVALID_VALUE
    assert vcall(null="q") == gdn.GDN_ERROR_INVALID_VALUE
    assert vcall(misalign="v") == gdn.GDN_ERROR_INVALID_VALUE
    assert vcall(K=48) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert vcall(cu=ctypes.c_void_p(BASE + 6 * STEP + 64)) == gdn.GDN_ERROR_INVALID_VALUE  # o overlaps the table


def test_segmented_rejects_bad_arguments():
    lib = gdn.load_library()

    def scall(segments=4, ws_bytes=None, ws=None, T=1000, K=64, null=None):
        names = ["q", "k", "v", "a", "b", "s0", "o", "sf"]
        args = [None if (n == null or n in ("s0", "sf")) else addr(i) for i, n in enumerate(names)]
        need = lib.gdn_chunk_fwd_segmented_workspace_size(2, T, 3, K, 64, 64, segments)
        wsp = addr(9) if ws is None else ws
        return lib.gdn_chunk_fwd_segmented(*args, 2, T, 3, K, 64, 64, segments, wsp,
                                           need if ws_bytes is None else ws_bytes,
                                           gdn.GDN_DTYPE_BF16, None)

    assert lib.gdn_chunk_fwd_segmented_workspace_size(2, 1000, 3, 64, 64, 64, 4) > 0
    assert lib.gdn_chunk_fwd_segmented_workspace_size(2, 1000, 3, 64, 64, 64, 0) == 0
    assert scall(segments=0) == gdn.GDN_ERROR_INVALID_VALUE
    assert scall(ws_bytes=100) == gdn.GDN_ERROR_INVALID_VALUE
    assert scall(ws=ctypes.c_void_p(BASE + 9 * STEP + 4)) == gdn.GDN_ERROR_INVALID_VALUE  # misaligned
    assert scall(ws=ctypes.c_void_p(BASE + 1 * STEP)) == gdn.GDN_ERROR_INVALID_VALUE      # overlaps k
    assert scall(null="q") == gdn.GDN_ERROR_INVALID_VALUE
    assert scall(K=48) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert scall(segments=2000) == gdn.GDN_ERROR_NOT_SUPPORTED                             # more than T


def test_segments_hint_follows_the_cost_model():
    # host only (num_cus given): the counts the cost model picks for the measured
    # shapes, 1 for a batch that fills the GPU by itself, 0 for invalid sizes
    hint = gdn.segments_hint
    assert hint(1, 32768, 2, 128, 128, 64, num_cus=256) == 32    # B1 T32768 H2: 0.138 vs 0.840 ms
    assert hint(1, 32768, 16, 128, 128, 64, num_cus=256) == 4    # B1 T32768 H16: 0.519 vs 0.850 ms
    assert hint(8, 4096, 6, 128, 128, 64, num_cus=256) == 1      # the training shape
    assert hint(2, 2048, 4, 128, 128, 64, num_cus=256) == 8      # B2 T2048 H4: 0.0554 vs 0.0594 ms plain
    assert hint(1, 100, 2, 128, 128, 64, num_cus=256) == 1       # too short to split
    assert hint(1, 32768, 2, 128, 128, 64, num_cus=512) >= 32    # more CUs, no fewer segments
    assert hint(0, 32768, 2, 128, 128, 64, num_cus=256) == 0
    assert hint(1, 32768, 2, 128, 128, -1, num_cus=256) == 0
    for args in [(1, 5000, 3, 64, 32, 32), (2, 70000, 1, 16, 16, 16), (1, 8192, 4, 128, 64, 64)]:
        P = hint(*args, num_cus=256)
        assert 1 <= P <= 256 and (P == 1 or 4 * P <= -(-args[1] // args[5]))


def test_bench_refuses_more_than_one_gpu():
    # the bench measures one GPU; a request for more exits with a message before any
    # device work (so this runs on the host)
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_noalloc_segmented_rejects_calls_beyond_its_static_scratch():
    # host checks only (fake addresses): a call that needs more than the 64 MiB
    # static scratch is refused with its own status before any device work
    lib = gdn.load_library()
    assert gdn.SEGMENTED_NOALLOC_MAX_BYTES == 64 << 20
    text = open(HEADER).read()
    assert "#define GDN_SEGMENTED_NOALLOC_MAX_BYTES ((size_t)64 << 20)" in text

    def ncall(B=1, T=32768, H=16, K=128, V=128, segments=4, null=None, dtype=gdn.GDN_DTYPE_BF16):
        names = ["q", "k", "v", "a", "b", "s0", "o", "sf"]
        args = [None if (n == null or n in ("s0", "sf")) else addr(i) for i, n in enumerate(names)]
        return lib.gdn_chunk_fwd_segmented_noalloc(*args, B, T, H, K, V, 64, segments, dtype, None)

    need = lib.gdn_chunk_fwd_segmented_workspace_size
    assert need(1, 32768, 16, 128, 128, 64, 4) <= gdn.SEGMENTED_NOALLOC_MAX_BYTES
    assert need(1, 32768, 16, 128, 128, 64, 16) > gdn.SEGMENTED_NOALLOC_MAX_BYTES
    assert ncall(segments=16) == gdn.GDN_ERROR_SCRATCH_LIMIT
    assert ncall(B=4, segments=4) == gdn.GDN_ERROR_SCRATCH_LIMIT
    assert "64 MiB" in gdn.status_string(gdn.GDN_ERROR_SCRATCH_LIMIT)
    # the other checks of the segmented call still apply, before the size check
    assert ncall(segments=0) == gdn.GDN_ERROR_INVALID_VALUE
    assert ncall(K=48) == gdn.GDN_ERROR_NOT_SUPPORTED
    assert ncall(segments=4, null="q") == gdn.GDN_ERROR_INVALID_VALUE


def test_bench_roof_follows_arithmetic_intensity():
    # bf16 inputs at d = 128 carry 134 FLOP per byte, below the bf16 ridge (2.5 PFLOP/s
    # over 8 TB/s, 312 FLOP/B): HBM-bound.  fp32 inputs move twice the bytes (68 FLOP/B)
    # but sit above the fp32 ridge (157.3 TFLOP/s over 8 TB/s, 19.7 FLOP/B): their roof
    # is the fp32 matrix cores.
    import bench
    B, T, H, K, V, C = 8, 4096, 6, 128, 128, 64
    flops = bench.algorithmic_flops(B, T, H, K, V, C)
    # per token-head: (3C-1)K + 2CV + 6KV + C^2/3 = 24,448 + 16,384 + 98,304 + 1,365.3
    assert abs(flops / (B * T * H) - 140501.333) < 1e-3
    for esz, peak, bound in ((2, bench.BF16_PEAK_TFLOPS, "hbm"), (4, bench.F32_PEAK_TFLOPS, "mfma")):
        nbytes = bench.algorithmic_bytes(B, T, H, K, V, esz=esz)
        r = bench.pick_roof(flops, nbytes, 0.1, peak)
        assert r["bound"] == bound
        if bound == "hbm":
            assert r["unit"] == "GB/s" and abs(r["achieved"] - nbytes / 1e-4 / 1e9) < 1e-6
        else:
            assert r["unit"] == "TFLOP/s" and r["peak"] == peak
            assert abs(r["frac"] - flops / 1e-4 / 1e12 / peak) < 1e-12
            assert r["hbm"]["unit"] == "GB/s"
    # the headline workload's algorithmic bytes: 1032 B per token-head plus the
    # fp32 final state
    assert bench.algorithmic_bytes(B, T, H, K, V, esz=2) == 1032 * B * T * H + B * H * V * K * 4
