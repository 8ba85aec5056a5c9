"""The C-ABI library on a machine without a GPU: it loads, exports every
declared entry point, sizes its outputs like the oracle, and rejects invalid
arguments before any HIP call (no compute call is made here)."""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from group_scale_factor_amd import _build

    if not os.path.exists(_build.LIBRARY):
        _build.build()
    import group_scale_factor_amd as gsf

    return gsf.library()


def _header_texts():
    inc = os.path.join(ROOT, "include")
    for fname in sorted(os.listdir(inc)):
        if fname.endswith(".h"):
            yield re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, fname)).read(), flags=re.S)


def declared_functions():
    """Functions the headers declare without a body: the library's entry points."""
    names = []
    for text in _header_texts():
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M):
            names.append(m.group(1))
    return names


def inline_helpers():
    """Functions the headers define as static inline: size helpers and the status text."""
    names = []
    for text in _header_texts():
        names += re.findall(r"^static inline [\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return names


ENTRY_POINTS = ("mx_block_rearrange_M_groups", "mx_block_rearrange_K_groups", "mx_block_rearrange_3d",
                "mx_quantize_dim0_M_groups", "mx_quantize_dim1_K_groups", "mx_quantize_dim1_3d",
                "mx_pad_M_groups", "mx_unpad_M_groups", "mx_block_unrearrange_M_groups",
                "mx_block_unrearrange_K_groups")
HELPERS = ("mx_rearrange_M_groups_out_bytes", "mx_rearrange_K_groups_out_bytes", "mx_rearrange_3d_out_bytes",
           "mx_rearrange_strerror", "mx_quantize_dim0_M_groups_scale_bytes", "mx_quantize_dim1_K_groups_scale_bytes",
           "mx_quantize_dim1_3d_scale_bytes", "mx_pad_M_groups_out_rows")


def test_header_declares_entry_points():
    assert sorted(declared_functions()) == sorted(ENTRY_POINTS)
    assert sorted(inline_helpers()) == sorted(HELPERS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


@pytest.mark.skipif(shutil.which("nm") is None, reason="needs nm")
def test_library_exports_only_the_entry_points(lib):
    from group_scale_factor_amd import _build

    res = subprocess.run(["nm", "-D", "--defined-only", _build.LIBRARY], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in res.stdout.splitlines() if line.split() and
                line.split()[-1].startswith("mx_")}
    assert exported == set(ENTRY_POINTS)


def _header_probe(tmp_path, lang):
    """Compiles a program that includes every header and prints each helper's value for a list of
    arguments, and each status text; returns its output lines (a dict keyed by the call text)."""
    calls = []
    for rows, cols, G in [(0, 0, 1), (1, 1, 1), (1024, 16, 4), (131072, 44, 8), (16640, 160, 16), (7168, 4096, 8),
                          (28672, 8192, 8), (130, 10, 3), (5, 4097, 200), (-1, 4, 1), (4, -1, 1), (4, 4, 0),
                          (2147483000, 5, 4), (3, 2147483000, 7)]:
        calls += ["mx_rearrange_M_groups_out_bytes(%d, %d, %d)" % (rows, cols, G),
                  "mx_rearrange_K_groups_out_bytes(%d, %d, %d)" % (rows, cols, G),
                  "mx_pad_M_groups_out_rows(%d, %d)" % (rows, G)]
    for E, rows, cols in [(0, 0, 0), (1, 1, 1), (16, 8192, 160), (64, 8192, 160), (3, 300, 45), (7, 0, 5),
                          (-1, 4, 4), (1, 2147483520, 4), (1, 4, 2147483520), (1 << 40, 1 << 20, 1 << 10)]:
        calls.append("mx_rearrange_3d_out_bytes(%dLL, %d, %d)" % (E, rows, cols))
    for a, K, G in [(0, 32, 1), (1, 32, 1), (16640, 5120, 16), (1000, 640, 5), (7, 96, 3), (300, 0, 2), (4, 48, 1),
                    (4, 64, 0), (-1, 64, 1), (131072, 7168, 8), (2048, 300, 5)]:
        calls += ["mx_quantize_dim0_M_groups_scale_bytes(%d, %d, %d)" % (a, K, G),
                  "mx_quantize_dim1_K_groups_scale_bytes(%d, %d, %d)" % (K, a, G),
                  "mx_quantize_dim1_3d_scale_bytes(%d, %d, %d)" % (G, K, a)]
    body = "".join('  printf("%%s=%%lld\\n", "%s", (long long)%s);\n' % (c, c) for c in calls)
    body += "".join('  printf("strerror(%d)=%%s\\n", mx_rearrange_strerror(%d));\n' % (k, k) for k in range(-7, 3))
    src = tmp_path / ("probe." + lang)
    src.write_text('#include <stdio.h>\n#include "mx_rearrange.h"\n#include "mx_quantize.h"\n#include "mx_pad.h"\n'
                   "int main(void) {\n" + body + "  return 0;\n}\n")
    exe = str(tmp_path / ("probe_" + lang))
    compiler = ["gcc", "-std=c11"] if lang == "c" else ["g++", "-std=c++17"]
    res = subprocess.run(compiler + ["-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), "-o", exe,
                                     str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    return dict(line.split("=", 1) for line in out.splitlines())


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
@pytest.mark.parametrize("lang", ["c", "cpp"])
def test_header_helpers_match_the_binding(tmp_path, lang):
    """The binding restates the headers' static inline size helpers and status texts: both agree, in
    C and in C++, on ordinary, empty, invalid and overflowing sizes."""
    import group_scale_factor_amd as gsf

    got = _header_probe(tmp_path, lang)
    assert len(got) > 80
    for call, value in got.items():
        if call.startswith("strerror("):
            assert gsf.mx_rearrange_strerror(int(call[9:-1])) == value, call
            continue
        name, args = call.split("(", 1)
        args = [int(a.strip().rstrip("L")) for a in args.rstrip(")").split(",")]
        assert getattr(gsf, name)(*args) == int(value), call


def test_out_bytes_match_oracle():
    import group_scale_factor_amd as gsf
    import oracle

    rng = np.random.default_rng(5)
    shapes = [(0, 0, 1), (1, 1, 1), (1024, 16, 4), (131072, 44, 8), (16640, 160, 16), (7168, 4096, 8),
              (28672, 8192, 8), (130, 10, 3), (5, 4097, 200)]
    shapes += [(int(rng.integers(0, 5000)), int(rng.integers(0, 5000)), int(rng.integers(1, 300))) for _ in range(50)]
    for rows, cols, G in shapes:
        assert gsf.mx_rearrange_M_groups_out_bytes(rows, cols, G) == oracle.out_bytes("M", rows, cols, G)
        assert gsf.mx_rearrange_K_groups_out_bytes(rows, cols, G) == oracle.out_bytes("K", rows, cols, G)
    assert gsf.mx_rearrange_M_groups_out_bytes(-1, 4, 1) == -1
    assert gsf.mx_rearrange_K_groups_out_bytes(4, 4, 0) == -1


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("fn", ["mx_block_rearrange_M_groups", "mx_block_rearrange_K_groups"])
def test_argument_validation(lib, fn):
    f = getattr(lib, fn)
    # (scales, rows, cols, ld, offs, G, out) -> expected status
    cases = [
        ((FAKE, 4, 4, 4, None, 1, FAKE), -1),       # offsets NULL
        ((None, 4, 4, 4, FAKE, 1, FAKE), -1),       # scales NULL with data
        ((FAKE, 4, 4, 4, FAKE, 1, None), -1),       # out NULL with output bytes
        ((FAKE, -1, 4, 4, FAKE, 1, FAKE), -2),      # negative rows
        ((FAKE, 4, -4, 4, FAKE, 1, FAKE), -2),      # negative cols
        ((FAKE, 4, 8, 7, FAKE, 1, FAKE), -2),       # row stride below cols
        ((FAKE, 4, 8, (1 << 24) + 1, FAKE, 1, FAKE), -2),  # row stride too large
        ((FAKE, 1 << 31, 8, 8, FAKE, 1, FAKE), -2),  # rows past the int32 range
        ((FAKE, 4, 4, 4, FAKE, 0, FAKE), -3),       # no groups
        ((FAKE, 4, 4, 4, FAKE, -2, FAKE), -3),
        ((FAKE, 4, 4, 4, FAKE, 1, FAKE + 8), -4),   # out not 16-byte aligned
    ]
    for args, want in cases:
        assert f(*args, None) == want, (fn, args)
    # nothing to write: success without a launch
    if fn.endswith("M_groups"):
        assert f(None, 5, 0, 0, FAKE, 2, None, None) == 0
    else:
        assert f(None, 0, 9, 9, FAKE, 2, None, None) == 0


def test_3d_out_bytes_match_oracle():
    import group_scale_factor_amd as gsf
    import oracle

    rng = np.random.default_rng(6)
    shapes = [(0, 0, 0), (1, 1, 1), (16, 8192, 160), (64, 8192, 160), (3, 300, 45), (7, 0, 5), (2, 5, 0)]
    shapes += [tuple(int(x) for x in rng.integers(0, [70, 5000, 400])) for _ in range(50)]
    for E, rows, cols in shapes:
        assert gsf.mx_rearrange_3d_out_bytes(E, rows, cols) == oracle.out_bytes_3d(E, rows, cols)
    assert gsf.mx_rearrange_3d_out_bytes(-1, 4, 4) == -1
    assert gsf.mx_rearrange_3d_out_bytes(1, (1 << 31) - 128, 4) == -1
    assert gsf.mx_rearrange_3d_out_bytes(1 << 40, 1 << 20, 1 << 10) == -1   # past int64


def test_3d_argument_validation(lib):
    f = lib.mx_block_rearrange_3d
    # (scales, E, rows, cols, expert_stride, row_stride, out) -> expected status
    cases = [
        ((None, 2, 4, 4, 16, 4, FAKE), -1),          # scales NULL with data
        ((FAKE, 2, 4, 4, 16, 4, None), -1),          # out NULL with output bytes
        ((FAKE, -1, 4, 4, 16, 4, FAKE), -2),         # negative experts
        ((FAKE, 2, -4, 4, 16, 4, FAKE), -2),         # negative rows
        ((FAKE, 2, 4, -1, 16, 4, FAKE), -2),         # negative cols
        ((FAKE, 2, 4, 8, 32, 7, FAKE), -2),          # row stride below cols
        ((FAKE, 2, 4, 8, 32, (1 << 24) + 1, FAKE), -2),  # row stride too large
        ((FAKE, 2, 4, 8, -32, 8, FAKE), -2),         # negative expert stride
        ((FAKE, 4, 4, 8, 1 << 62, 8, FAKE), -2),     # expert offsets past int64
        ((FAKE, 2, 4, 4, 16, 4, FAKE + 4), -4),      # out not 16-byte aligned
    ]
    for args, want in cases:
        assert f(*args, None) == want, args
    # nothing to write: success without a launch
    assert f(None, 0, 5, 5, 25, 5, None, None) == 0
    assert f(None, 3, 0, 5, 0, 5, None, None) == 0
    assert f(None, 3, 5, 0, 0, 0, None, None) == 0


def test_quantize_sizes_match_oracle():
    import group_scale_factor_amd as gsf
    import oracle

    for rows, K, G in [(0, 32, 1), (1, 32, 1), (16640, 5120, 16), (1000, 640, 5), (7, 96, 3), (300, 0, 2)]:
        assert gsf.mx_quantize_dim0_M_groups_scale_bytes(rows, K, G) == oracle.out_bytes("M", rows, K // 32, G)
    assert gsf.mx_quantize_dim0_M_groups_scale_bytes(4, 48, 1) == -1   # K not a multiple of 32
    assert gsf.mx_quantize_dim0_M_groups_scale_bytes(4, 64, 0) == -1


def test_quantize_argument_validation(lib):
    f = lib.mx_quantize_dim0_M_groups
    A = 0x10000   # 16-byte aligned fake pointer, never dereferenced
    # (x, rows, K, ld, offs, G, q, scales) -> expected status
    cases = [
        ((A, 4, 64, 64, None, 1, A, A), -1),        # offsets NULL
        ((None, 4, 64, 64, A, 1, A, A), -1),        # x NULL with data
        ((A, 4, 64, 64, A, 1, None, A), -1),        # q NULL with data
        ((A, 4, 64, 64, A, 1, A, None), -1),        # scales NULL
        ((A, 4, 48, 48, A, 1, A, A), -2),           # K not a multiple of 32
        ((A, 4, 64, 32, A, 1, A, A), -2),           # row stride below K
        ((A, -1, 64, 64, A, 1, A, A), -2),          # negative rows
        ((A, 4, 64, (1 << 26) + 8, A, 1, A, A), -2),  # row stride too large
        ((A, 4, 64, 64, A, 0, A, A), -3),           # no groups
        ((A, 4, 64, 64, A, 4097, A, A), -3),        # too many groups
        ((A + 8, 4, 64, 64, A, 1, A, A), -4),       # x not 16-byte aligned
        ((A, 4, 64, 68, A, 1, A, A), -4),           # row stride not a multiple of 8 elements
        ((A, 4, 64, 64, A, 1, A + 8, A), -4),       # q not 16-byte aligned
        ((A, 4, 64, 64, A, 1, A, A + 4), -4),       # scales not 16-byte aligned
    ]
    for args, want in cases:
        assert f(*args, None) == want, args
    assert f(None, 5, 0, 0, A, 2, None, None, None) == 0   # K = 0: nothing to write


def test_quantize_dim1_sizes_and_validation(lib):
    import group_scale_factor_amd as gsf
    import oracle

    for T, N, G in [(0, 5, 1), (32, 1, 1), (131072, 7168, 8), (2048, 300, 5), (96, 0, 2)]:
        assert gsf.mx_quantize_dim1_K_groups_scale_bytes(T, N, G) == oracle.out_bytes("K", N, T // 32, G)
    assert gsf.mx_quantize_dim1_K_groups_scale_bytes(48, 4, 1) == -1
    f = lib.mx_quantize_dim1_K_groups
    A = 0x10000
    cases = [
        ((A, 64, 8, 8, None, 1, A, A), -1),          # offsets NULL
        ((None, 64, 8, 8, A, 1, A, A), -1),          # x NULL
        ((A, 64, 8, 8, A, 1, None, A), -1),          # qT NULL
        ((A, 64, 8, 8, A, 1, A, None), -1),          # scales NULL
        ((A, 48, 8, 8, A, 1, A, A), -2),             # T not a multiple of 32
        ((A, 64, 8, 4, A, 1, A, A), -2),             # row stride below N
        ((A, 64, 8, (1 << 23) + 8, A, 1, A, A), -2),  # row stride too large
        ((A, 64, 8, 8, A, 0, A, A), -3),             # no groups
        ((A, 64, 8, 8, A, 2049, A, A), -3),          # too many groups
        ((A + 8, 64, 8, 8, A, 1, A, A), -4),         # x misaligned
        ((A, 64, 8, 12, A, 1, A, A), -4),            # row stride not a multiple of 8
        ((A, 64, 8, 8, A, 1, A + 4, A), -4),         # qT misaligned
        ((A, 64, 8, 8, A, 1, A, A + 4), -4),         # scales misaligned
    ]
    for args, want in cases:
        assert f(*args, None) == want, args
    assert f(None, 64, 0, 0, A, 2, None, None, None) == 0   # N = 0: nothing to write


def test_quantize_dim1_3d_sizes_and_validation(lib):
    import group_scale_factor_amd as gsf
    import oracle

    for E, K, N in [(0, 64, 8), (1, 32, 1), (16, 5120, 8192), (3, 96, 130), (2, 0, 5), (4, 64, 0)]:
        assert gsf.mx_quantize_dim1_3d_scale_bytes(E, K, N) == oracle.out_bytes_3d(E, N, K // 32)
    assert gsf.mx_quantize_dim1_3d_scale_bytes(2, 48, 4) == -1
    f = lib.mx_quantize_dim1_3d
    A = 0x10000
    cases = [
        ((None, 2, 64, 8, 512, 8, A, A), -1),          # weights NULL
        ((A, 2, 64, 8, 512, 8, None, A), -1),          # codes NULL
        ((A, 2, 64, 8, 512, 8, A, None), -1),          # scales NULL
        ((A, 2, 48, 8, 512, 8, A, A), -2),             # K not a multiple of 32
        ((A, 2, 64, 8, 512, 4, A, A), -2),             # row stride below N
        ((A, 2, 64, 8, -8, 8, A, A), -2),              # negative expert stride
        ((A, -1, 64, 8, 512, 8, A, A), -2),            # negative experts
        ((A, 2049, 64, 8, 512, 8, A, A), -3),          # too many experts
        ((A + 8, 2, 64, 8, 512, 8, A, A), -4),         # weights misaligned
        ((A, 2, 64, 8, 516, 8, A, A), -4),             # expert stride not a multiple of 8
        ((A, 2, 64, 8, 512, 12, A, A), -4),            # row stride not a multiple of 8
        ((A, 2, 64, 8, 512, 8, A + 4, A), -4),         # codes misaligned
        ((A, 2, 64, 8, 512, 8, A, A + 4), -4),         # scales misaligned
    ]
    for args, want in cases:
        assert f(*args, None) == want, args
    for args in [(None, 0, 64, 8, 0, 8, None, None), (None, 3, 0, 8, 0, 8, None, None), (None, 3, 64, 0, 0, 0, None, None)]:
        assert f(*args, None) == 0, args                 # nothing to write


def test_pad_sizes_and_validation(lib):
    import group_scale_factor_amd as gsf
    import oracle

    for rows, G in [(0, 1), (5, 3), (16640, 16)]:
        assert gsf.mx_pad_M_groups_out_rows(rows, G) == oracle.default().lib.oracle_pad_M_groups_out_rows(rows, G)
    assert gsf.mx_pad_M_groups_out_rows(-1, 1) == -1 and gsf.mx_pad_M_groups_out_rows(4, 0) == -1
    A = 0x10000
    pad, unpad = lib.mx_pad_M_groups, lib.mx_unpad_M_groups
    # (data, rows, cols, ld, offs, G, padded)
    for args, want in [((A, 4, 8, 8, None, 1, A), -1), ((None, 4, 8, 8, A, 1, A), -1), ((A, 4, 8, 8, A, 1, None), -1),
                       ((A, -1, 8, 8, A, 1, A), -2), ((A, 4, 8, 7, A, 1, A), -2), ((A, 4, 8, 8, A, 0, A), -3),
                       ((A, 4, 8, 8, A, 4097, A), -3)]:
        assert pad(*args, None) == want, args
    # (padded, rows, cols, offs, G, data, ld)
    for args, want in [((A, 4, 8, None, 1, A, 8), -1), ((None, 4, 8, A, 1, A, 8), -1), ((A, 4, 8, A, 1, None, 8), -1),
                       ((A, 4, 8, A, 1, A, 7), -2), ((A, 4, 8, A, 0, A, 8), -3)]:
        assert unpad(*args, None) == want, args
    assert pad(None, 4, 0, 0, A, 1, None, None) == 0      # cols = 0: nothing to write
    assert unpad(None, 0, 8, A, 1, None, 8, None) == 0    # rows = 0: nothing to write


@pytest.mark.parametrize("fn", ["mx_block_unrearrange_M_groups", "mx_block_unrearrange_K_groups"])
def test_unrearrange_validation(lib, fn):
    f = getattr(lib, fn)
    A = 0x10000
    # (blocked, rows, cols, offs, G, out, ld) -> status
    for args, want in [((A, 4, 8, None, 1, A, 8), -1), ((None, 4, 8, A, 1, A, 8), -1), ((A, 4, 8, A, 1, None, 8), -1),
                       ((A, -1, 8, A, 1, A, 8), -2), ((A, 4, 8, A, 1, A, 7), -2), ((A, 4, 8, A, 0, A, 8), -3),
                       ((A, 4, 8, A, 4097, A, 8), -3), ((A + 4, 4, 8, A, 1, A, 8), -4)]:
        assert f(*args, None) == want, args
    assert f(None, 0, 8, A, 1, None, 8, None) == 0     # nothing to write


def test_strerror():
    import group_scale_factor_amd as gsf

    for code in (0, -1, -2, -3, -4, -5, -6, 7):   # -6 and 7: not a status, "unknown status" text
        s = gsf.mx_rearrange_strerror(code)
        assert isinstance(s, str) and len(s) > 0
    assert gsf.mx_rearrange_strerror(-6) == "unknown status"


def test_binding_has_no_cpu_path():
    # the binding refuses CPU tensors instead of computing anything itself
    import torch

    import group_scale_factor_amd as gsf

    with pytest.raises(ValueError):
        gsf.mx_block_rearrange_M_groups(torch.zeros((4, 4), dtype=torch.uint8), torch.tensor([4], dtype=torch.int32))
    with pytest.raises(TypeError):
        gsf.mx_block_rearrange_K_groups(torch.zeros((4, 4), dtype=torch.int8), torch.tensor([4], dtype=torch.int32))
    with pytest.raises(ValueError):
        gsf.mx_block_rearrange_3d(torch.zeros((2, 4, 4), dtype=torch.uint8))
    with pytest.raises(TypeError):
        gsf.mx_block_rearrange_3d(torch.zeros((4, 4), dtype=torch.uint8))
    with pytest.raises(ValueError):
        gsf.mx_quantize_dim0_M_groups(torch.zeros((4, 64), dtype=torch.bfloat16), torch.tensor([4], dtype=torch.int32))
    with pytest.raises(TypeError):
        gsf.mx_quantize_dim0_M_groups(torch.zeros((4, 64), dtype=torch.float32), torch.tensor([4], dtype=torch.int32))


def test_product_code_never_touches_the_oracle():
    # the HIP source and the binding neither include nor import the oracle
    pkg = os.path.join(ROOT, "group_scale_factor_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, f)
    src = open(os.path.join(ROOT, "oracle", "mx_rearrange_oracle.c")).read()
    includes = set(re.findall(r"#include\s*(\S+)", src))
    assert includes <= {"<stdint.h>", "<string.h>", "<math.h>", "<stdlib.h>", "<pthread.h>"}, includes


def test_no_reversed_operand_dpp_in_device_code():
    """The build refuses generated code holding v_*rev*_dpp instructions (wrong results on gfx950)."""
    from group_scale_factor_amd import _build

    _build.check_device_code()
    assert _build.REVERSED_DPP.search("\tv_subrev_u32_dpp v1, v31, v31 wave_shr:1 row_mask:0xf bank_mask:0xf")
    assert not _build.REVERSED_DPP.search("\tv_sub_u32_dpp v1, v1, v1 row_shr:1\n\tv_mov_b32_dpp v2, v1 wave_shr:1")


def test_plain_c_caller_compiles():
    """The plain C caller of tests/c_abi compiles against include/*.h as C11 (no C++ needed)."""
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    res = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                          "-I", os.path.join(rocm, "include"), "-I", os.path.join(root, "include"),
                          os.path.join(root, "tests", "c_abi", "abi_check.c")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_profile_digest_ignores_comments_only():
    """The kernel digest that ties a committed counter profile to its kernel changes with the code, not with
    comments or whitespace."""
    import bench

    src = b"// header\n#include <x>\nint f(int a) { /* sum */ return a + 1; }  // tail\n"
    assert bench.code_text(src) == bench.code_text(b"#include <x>\nint   f(int a) {\n return a + 1; }\n")
    assert bench.code_text(src) != bench.code_text(src.replace(b"a + 1", b"a + 2"))
    files = {bench.kernel_source("m_groups_skinny"): b"int k; // one\n"}
    d1 = bench.kernel_source_digest("m_groups_skinny", lambda p: files[p])
    files[bench.kernel_source("m_groups_skinny")] = b"int k; /* two */\n"
    assert bench.kernel_source_digest("m_groups_skinny", lambda p: files[p]) == d1
    files[bench.kernel_source("m_groups_skinny")] = b"long k;\n"
    assert bench.kernel_source_digest("m_groups_skinny", lambda p: files[p]) != d1


def test_counter_profiles_match_the_kernels():
    """Every committed HBM counter profile was taken from the kernel code in the tree (its digest matches),
    names the workload's own kernel source, and reads within a few percent of the algorithmic bytes on the
    workloads larger than a few fixed per-launch fetches. A kernel changed after its counters were taken
    fails here until they are taken again (bench.py would report its traffic as null meanwhile)."""
    import json

    import bench

    paths = sorted(p for p in os.listdir(bench.PROFILES) if p.startswith("pmc_") and p.endswith(".json"))
    assert len(paths) >= 14
    for fname in paths:
        with open(os.path.join(bench.PROFILES, fname)) as f:
            d = json.load(f)
        name = d["workload"]
        assert fname == "pmc_%s.json" % name
        assert d["kernel_source"] == os.path.basename(bench.kernel_source(name)), name
        assert d["kernel_source_sha256_16"] == bench.kernel_source_digest(name), name
        ratio = int(d["hbm_bytes_per_launch"]) / int(d["algorithmic_bytes_per_launch"])
        if int(d["algorithmic_bytes_per_launch"]) >= 1 << 20:
            assert 0.99 <= ratio <= 1.08, (name, ratio)


def test_grids_past_one_launch_are_rejected(lib):
    """A launch holds fewer than 2^32 work-items; entry points whose grid would not fit one launch
    (outputs of over 100 GB) return MX_REARRANGE_ESHAPE before any HIP call, and the largest sizes
    below that pass validation (checked here only up to the point of a launch: no GPU)."""
    A = 0x10000   # 16-byte aligned fake pointer, never dereferenced
    # inverse, M groups: ((2^30 / 128) + 1 row blocks) x 8 column windows > 2^32 / 128 units
    assert lib.mx_block_unrearrange_M_groups(A, 1 << 30, 1024, A, 1, A, 1024, None) == -2
    # inverse, K groups: 2^23 row blocks x 4 windows of 256 columns > 2^32 / 512 units
    assert lib.mx_block_unrearrange_K_groups(A, 1 << 30, 1024, A, 1, A, 1024, None) == -2
    # pad: 2^28 + 128 rows of one 1 KB unit, 2 units per wave, 2 waves per workgroup > 2^32 / 128
    assert lib.mx_pad_M_groups(A, 1 << 28, 1024, 1024, A, 1, A, None) == -2
    assert lib.mx_unpad_M_groups(A, 1 << 28, 1024, A, 1, A, 1024, None) == -2
    # dim1 cast: (2^30 / 128 + 2) tile columns x 2 feature blocks > 2^32 / 256 units
    assert lib.mx_quantize_dim1_K_groups(A, 1 << 30, 256, 256, A, 1, A, A, None) == -2
    # dim0 cast: 2^30 rows of one 512-element unit, 4 units per wave, 4 waves per workgroup
    assert lib.mx_quantize_dim0_M_groups(A, 1 << 30, 512, 512, A, 1, A, A, None) == -2
