"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/moe.h declares, sizes workspaces, and rejects bad
arguments before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import mixture_experts_layer_topk_amd as m
    return m


def test_header_declarations_are_exported():
    m = _lib()
    header = open(os.path.join(ROOT, "include", "moe.h")).read()
    declared = set(re.findall(r"^(?:int|const char\*)\s+(moe_\w+)\(", header, re.M))
    assert declared == set(m.EXPORTS)
    for name in declared:
        assert hasattr(m._lib, name), name


def test_workspace_size_and_layout():
    m = _lib()
    d = m.dims(4096, 7168, 2048, 32, 8)
    n = m.workspace_size(d)
    L = m.workspace_layout(d)
    assert L.total == n
    R = 4096 * 8
    assert L.o + R * 7168 * 2 <= n
    offs = [L.topk_idx, L.topk_w, L.counts, L.offsets, L.slot_src, L.slot_of, L.xq, L.xsf,
            L.hq, L.hsf, L.o]
    assert all(o % 256 == 0 for o in offs)


@pytest.mark.parametrize("bad", [
    dict(H=100), dict(I=96), dict(topk=0), dict(topk=9, E=8), dict(E=0), dict(T=-1),
    dict(score_fn=5), dict(E=2000), dict(topk=17, E=32),
    # 32-bit GEMM offsets: T*H, T*topk*I and H*I must stay below 2^32
    dict(T=1 << 19, H=8192), dict(T=1 << 18, topk=16, E=32, I=1024), dict(H=65536, I=65536)])
def test_bad_dims_rejected(bad):
    m = _lib()
    args = dict(T=16, H=256, I=128, E=8, topk=2, score_fn=0)
    args.update(bad)
    d = m.Dims(args["T"], args["H"], args["I"], args["E"], args["topk"], args["score_fn"], 1)
    n = ctypes.c_size_t()
    rc = m._lib.moe_workspace_size(ctypes.byref(d), ctypes.byref(n))
    assert rc in (m.MOE_EINVAL, m.MOE_EUNSUPPORTED)


def test_forward_rejects_null_and_small_workspace_without_gpu():
    m = _lib()
    d = m.dims(16, 256, 128, 8, 2)
    a = m.Args()
    a.dims = d
    assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EINVAL          # null pointers
    fake = ctypes.c_void_p(1 << 20)                                            # never dereferenced
    for f in ("x", "logits", "w13", "w13_sf", "w2", "w2_sf", "y"):
        setattr(a, f, fake)
    a.ws = ctypes.c_void_p(1 << 20)
    a.ws_bytes = 16
    assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EWORKSPACE
    a.ws_bytes = m.workspace_size(d)
    a.ws = ctypes.c_void_p((1 << 20) + 8)                                      # misaligned
    assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EWORKSPACE
    a.x = ctypes.c_void_p((1 << 20) + 2)                                       # misaligned x
    a.ws = ctypes.c_void_p(1 << 20)
    assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EINVAL
    a.x = fake
    for bad_flags in (m.FLAG_NARROW | m.FLAG_TILED, m.FLAG_NARROW | m.FLAG_TILED | m.FLAG_ONE_LAUNCH,
                      m.FLAG_ONE_KERNEL | m.FLAG_TILED, m.FLAG_ONE_KERNEL | m.FLAG_ONE_LAUNCH,
                      # the one-kernel layer's routing hand-off guards the tables its phases index with
                      m.FLAG_ONE_KERNEL | m.FLAG_DEBUG_SPIN_BOUND,
                      # block-FP8 weights have their own scale layout and no gate/up interleave
                      m.FLAG_WEIGHTS_FP8_BLOCK128 | m.FLAG_W13_PREINTERLEAVED,
                      m.FLAG_WEIGHTS_FP8_BLOCK128 | m.FLAG_W_SCALES_PER_ROW,
                      m.FLAG_WEIGHTS_FP8_BLOCK128 | m.FLAG_W_STAGED,
                      # the staged layout is made from the canonical gate-then-up row order
                      m.FLAG_W_STAGED | m.FLAG_W13_PREINTERLEAVED,
                      1024, 1 << 31):                                          # unknown or conflicting
        a.flags = bad_flags
        assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EINVAL
    # block-FP8 weights run on the narrow kernels in separate launches only
    for bad_flags in (m.FLAG_TILED, m.FLAG_ONE_LAUNCH, m.FLAG_ONE_KERNEL):
        a.flags = m.FLAG_WEIGHTS_FP8_BLOCK128 | bad_flags
        assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EUNSUPPORTED
    # the one-kernel layer takes at most 1024 routed pairs
    big = m.dims(129, 256, 128, 32, 8)
    a.dims = big
    a.ws_bytes = m.workspace_size(big)
    a.flags = m.FLAG_ONE_KERNEL
    assert m._lib.moe_forward(ctypes.byref(a), None) == m.MOE_EUNSUPPORTED


def test_quant_and_pack_reject_bad_sizes():
    m = _lib()
    p = ctypes.c_void_p(1 << 20)
    assert m._lib.moe_pack_weights_fp8_block128(p, 100, 128, p, p, None) == m.MOE_EINVAL   # rows % 128
    assert m._lib.moe_pack_weights_fp8_block128(p, 128, 96, p, p, None) == m.MOE_EINVAL    # cols % 128
    assert m._lib.moe_pack_weights_fp8_block128(p, 0, 128, p, p, None) == m.MOE_OK
    assert m._lib.moe_quant_act(p, 4, 48, p, p, None) == m.MOE_EINVAL
    assert m._lib.moe_pack_weights(p, 4, 0, p, p, None) == m.MOE_EINVAL
    assert m._lib.moe_quant_act(p, 0, 64, p, p, None) == m.MOE_OK            # empty is a no-op


def test_stage_weights_rejects_bad_sizes_without_gpu():
    m = _lib()
    p = ctypes.c_void_p(1 << 20)
    q = ctypes.c_void_p(1 << 28)                                               # never dereferenced
    assert m._lib.moe_stage_weights(p, 2, 192, 256, 1, q, None) == m.MOE_EINVAL    # rows % 128
    assert m._lib.moe_stage_weights(p, 2, 256, 192, 0, q, None) == m.MOE_EINVAL    # cols % 128
    assert m._lib.moe_stage_weights(p, 2, 256, 256, 1, ctypes.c_void_p((1 << 28) + 8), None) == m.MOE_EINVAL
    # output overlapping the input (2 x 256 x 128 bytes from 1 MiB)
    assert m._lib.moe_stage_weights(p, 2, 256, 256, 1, ctypes.c_void_p((1 << 20) + 65536 - 16),
                                    None) == m.MOE_EINVAL
    assert m._lib.moe_stage_weights(p, 0, 256, 256, 1, q, None) == m.MOE_OK        # empty is a no-op


def test_error_strings():
    m = _lib()
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert m._lib.moe_error_string(code)
    assert b"wait" in m._lib.moe_error_string(m.MOE_ETIMEOUT)
    assert b"scratch" in m._lib.moe_error_string(m.MOE_ESCRATCH)


def test_route_noalloc_rejects_beyond_its_scratch_without_gpu():
    m = _lib()
    p = ctypes.c_void_p(1 << 20)                                               # never dereferenced
    big = m.dims(32769, 128, 128, 64, 8)                                       # 262152 routed pairs
    assert m._lib.moe_route_noalloc(ctypes.byref(big), p, p, p, p, p, p, p, None) == m.MOE_ESCRATCH
    d = m.dims(16, 128, 128, 8, 2)
    assert m._lib.moe_route_noalloc(ctypes.byref(d), None, p, p, p, p, p, p, None) == m.MOE_EINVAL


def test_check_status_rejects_bad_workspace_without_gpu():
    m = _lib()
    assert m._lib.moe_check_status(None, None) == m.MOE_EINVAL
    assert m._lib.moe_check_status(ctypes.c_void_p((1 << 20) + 8), None) == m.MOE_EINVAL   # misaligned


def test_ctypes_structs_match_the_c_header(tmp_path):
    """The binding's ctypes structs have the header's field offsets and sizes
    (a host-only C program built against include/moe.h prints them)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs gcc and the HIP headers")
    m = _lib()
    structs = {"moe_dims_t": m.Dims, "moe_args_t": m.Args, "moe_layout_t": m.Layout}
    lines = ['#include <stdio.h>', '#include "moe.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for cname, py in structs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
