"""The C ABI library on the CPU: it loads, exports what include/*.h declares,
shares torch's HIP runtime, and rejects bad arguments before any HIP call.

No test here launches a kernel; each invalid call below returns from the
host-side validation.
"""

import ctypes
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from w4a16_decode_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from w4a16_decode_amd import build

        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    from w4a16_decode_amd import _lib

    declared = _lib.header_functions()
    assert len(declared) >= 22 and "q8_gemm" in declared and "q4_gemm" in declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature in the binding"
    assert sorted(_lib.SIGNATURES) == declared


def test_single_hip_runtime(lib):
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip
    import torch

    assert os.path.dirname(next(iter(hip))) == os.path.join(os.path.dirname(torch.__file__), "lib")


def test_version_and_status_strings(lib):
    assert lib.q4_version().decode().startswith("q4 ")
    assert lib.q4_status_str(0) == b"ok"
    for st in range(1, 8):
        assert lib.q4_status_str(st) and lib.q4_status_str(st) != b"unknown status"
    assert lib.q4_status_str(99) == b"unknown status"


def test_library_built_from_this_tree(lib):
    """The loaded library carries the hash of the sources and flags it was built from,
    and it is this tree's: a library left over from other sources never runs."""
    from w4a16_decode_amd.build import source_hash

    h = source_hash()
    assert lib.q4_version().decode().endswith(" src " + h)
    assert source_hash(["-DQ4_EXTRA"]) != h


def test_source_hash_does_not_depend_on_the_tree_location(tmp_path):
    """The tree is built in one place and run from another (a copy elsewhere): the
    hash covers file contents and flags, not absolute paths."""
    import shutil
    import subprocess
    import sys

    from w4a16_decode_amd.build import ROOT, source_hash

    pkg = tmp_path / "w4a16_decode_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "w4a16_decode_amd", "build.py"), pkg / "build.py")
    (pkg / "__init__.py").write_text("")
    shutil.copytree(os.path.join(ROOT, "w4a16_decode_amd", "csrc"), pkg / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    def copy_hash():
        return subprocess.run([sys.executable, "-c", "from w4a16_decode_amd.build import source_hash; print(source_hash())"],
                              cwd=tmp_path, capture_output=True, text=True, check=True).stdout.strip()

    assert copy_hash() == source_hash()
    # comments and layout are not code: editing them keeps the hash, editing code does not
    hdr = tmp_path / "include" / "q4.h"
    text = hdr.read_text()
    hdr.write_text("/* a note */\n" + text.replace("\n", "\n\n", 5))
    assert copy_hash() == source_hash()
    hdr.write_text(text.replace("q4_version", "q4_version2", 1))
    assert copy_hash() != source_hash()


def test_sizes(lib):
    assert lib.q4_packed_bytes(4096, 4096) == 4096 * 4096 // 2
    assert lib.q4_packed_bytes(17, 96) == 32 * 128 // 2          # padded to 16 rows, 128 channels
    assert lib.q4_packed_bytes(0, 128) == 0
    assert lib.q4_groups_count(4096, 4096, 128) == 4096 * 32
    assert lib.q4_groups_count(20, 96, 32) == 32 * 4            # Gp = ceil(96/128)*128/32
    assert lib.q4_groups_count(20, 96, 64) == 0                  # 96 % 64 != 0
    for g, ok in ((32, 1), (64, 1), (128, 1), (256, 1), (4096, 1), (96, 0), (16, 0), (0, 0), (-128, 0), (192, 0)):
        assert lib.q4_group_supported(g) == ok, g


FAKE = 0x100000  # a 16-byte-aligned non-NULL address that is never dereferenced


def test_quantize_validation(lib):
    f = lib.q4_quantize_pack
    assert f(None, 16, 128, 128, FAKE, FAKE, None) == 1
    assert f(FAKE, 16, 128, 128, None, FAKE, None) == 1
    assert f(FAKE, 0, 128, 128, FAKE, FAKE, None) == 2
    assert f(FAKE, 16, -128, 128, FAKE, FAKE, None) == 2
    assert f(FAKE, 1 << 30, 128, 128, FAKE, FAKE, None) == 2
    assert f(FAKE, 16, 96, 64, FAKE, FAKE, None) == 3            # in % group != 0
    assert b"multiple" in lib.q4_last_error()
    assert f(FAKE, 16, 96, 96, FAKE, FAKE, None) == 3            # unsupported group
    assert f(FAKE + 2, 16, 128, 128, FAKE, FAKE, None) == 4      # W misaligned
    assert f(FAKE, 16, 128, 128, FAKE + 8, FAKE, None) == 4      # packed misaligned
    assert f(FAKE, 16, 128, 128, FAKE, FAKE + 2, None) == 4      # scales misaligned
    assert lib.q4_quantize_pack_asym(FAKE, 16, 128, 128, FAKE, FAKE, None, None) == 1
    c = lib.q4_quantize_pack_clip
    assert c(FAKE, 16, 128, 128, 0, FAKE, FAKE, None) == 5                # min_percent below 1
    assert c(FAKE, 16, 128, 128, 101, FAKE, FAKE, None) == 5              # min_percent above 100
    assert c(FAKE, 16, 512, 256, 80, FAKE, FAKE, None) == 5               # group outside 32/64/128
    assert c(None, 16, 128, 128, 80, FAKE, FAKE, None) == 1
    assert c(FAKE, 16, 96, 64, 80, FAKE, FAKE, None) == 3                 # in % group != 0
    assert c(FAKE + 2, 16, 128, 128, 80, FAKE, FAKE, None) == 4


def test_gemm_validation(lib):
    g = lib.q4_gemm
    assert g(FAKE, -1, FAKE, FAKE, 16, 128, 128, FAKE, None, 0, None) == 2
    assert g(None, 0, None, None, 16, 128, 128, None, None, 0, None) == 0      # B = 0: nothing to do
    assert g(None, 1, FAKE, FAKE, 16, 128, 128, FAKE, None, 0, None) == 1
    assert g(FAKE, 1, FAKE, FAKE, 16, 100, 32, FAKE, None, 0, None) == 3
    assert g(FAKE + 4, 1, FAKE, FAKE, 16, 128, 128, FAKE, None, 0, None) == 4
    assert g(FAKE, 1, FAKE, FAKE, 16, 128, 128, FAKE + 1, None, 0, None) == 4
    assert lib.q4_gemm_asym(FAKE, 1, FAKE, FAKE, None, 16, 128, 128, FAKE, None, 0, None) == 1
    c = lib.q4_gemm_config
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 3, 1, 1, 1, None, 0, None) == 5
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 1, 17, 1, 1, None, 0, None) == 5
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 0, 0, 0, 1, None, 0, None) == 5
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 256, 128, FAKE, 1, 8, 3, 1, None, 0, None) == 5   # k_splits > blocks
    assert c(FAKE, 16, FAKE, FAKE, None, 0, 16, 8192, 128, FAKE, 1, 8, 1, 1, None, 0, None) == 5  # x slice > LDS
    assert c(FAKE, 64, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 4, 8, 1, 4, None, 0, None) == 5   # B > 16: 4 wavefronts
    assert c(FAKE, 64, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 1, 8, 2, 4, None, 0, None) == 5   # k_splits, B > 16
    assert c(FAKE, 64, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 4, 4, 1, 8, None, 0, None) == 5   # R*CT > 16
    assert c(FAKE, 64, FAKE, FAKE, None, 0, 16, 128, 32, FAKE, 2, 4, 1, 4, None, 0, None) == 5    # R*CT*4 > 16
    assert c(FAKE, 64, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 1, 4, 1, 5, None, 0, None) == 5   # col_tiles
    assert c(FAKE, 4, FAKE, FAKE, None, 0, 16, 128, 128, FAKE, 1, 1, 1, 2, None, 0, None) == 5    # GEMV: 1 tile
    # split k needs workspace: 2 * 1 * 16 * 4 bytes here
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 256, 128, FAKE, 1, 1, 2, 1, None, 0, None) == 6
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 256, 128, FAKE, 1, 1, 2, 1, FAKE, 64, None) == 6
    assert c(FAKE, 1, FAKE, FAKE, None, 0, 16, 256, 128, FAKE, 1, 1, 2, 1, FAKE + 4, 128, None) == 4


def test_workspace_sizes(lib):
    # B = 1 on a long row: the 56 KiB activation slice fits one workgroup's LDS
    assert lib.q4_workspace_bytes(1, 4096, 4096, 128) == 0
    # B = 8 over 28672 channels cannot stage the whole row: split over workgroups
    ws = lib.q4_workspace_bytes(8, 8192, 28672, 128)
    assert ws > 0 and ws % (8 * 8192 * 4) == 0
    assert lib.q4_workspace_bytes(0, 8192, 28672, 128) == 0
    # (whether B > 16 splits depends on the device's LDS per workgroup; the size is whole partials)
    assert lib.q4_workspace_bytes(64, 8192, 8192, 128) % (64 * 8192 * 4) == 0
    assert lib.q4_gemm(FAKE, 8, FAKE, FAKE, 8192, 28672, 128, FAKE, None, 0, None) == 6


def test_layout_validation(lib):
    assert lib.q4_to_canonical(None, FAKE, None, 0, 16, 128, 128, FAKE, FAKE, None, None) == 1
    assert lib.q4_to_canonical(FAKE, FAKE, None, 1, 16, 128, 128, FAKE, FAKE, None, None) == 1
    assert lib.q4_from_canonical(FAKE, FAKE, None, 0, 16, 100, 32, FAKE, FAKE, None, None) == 3


def test_bits_per_weight_matches_pages():
    from w4a16_decode_amd import perfmodel

    gd = json.load(open(os.path.join(ROOT, "tests", "golden", "arg_bits_per_weight.json")))
    for row in gd["printed"]:
        got = perfmodel.bits_per_weight(row["g"], 4, row["b_scale"], row["b_zero"])
        digits = len(str(row["bits"]).split(".")[1])
        assert abs(got - row["bits"]) <= 0.5 * 10 ** -digits + 1e-12, row
    for row in gd["printed_bytes"]:
        digits = len(str(row["GB"]).split(".")[1])
        assert abs(row["params"] * row["bits"] / 8 / 1e9 - row["GB"]) <= 0.5 * 10 ** -digits + 1e-9, row
    # our symmetric format: float16 scale, no zero point
    assert perfmodel.weight_bytes(4096, 4096, 128) == 4096 * 4096 // 2 + 2 * 4096 * 32
    assert perfmodel.gemm_read_bytes(1, 4096, 4096, 128) == 8_658_944


def test_time_model_matches_page_numbers():
    """T_mem 16.06 GB / 3.35 TB/s ~ 4.8 ms; T_cmp(m) ~ m * 15.2 us; crossover B* ~ 79."""
    from w4a16_decode_amd import perfmodel

    t = perfmodel.time_model_s(16.06e9, 7.5e9, 1, 3.35e12, 989e12)
    assert abs(t * 1e3 - 4.8) < 0.05
    assert abs(perfmodel.time_model_s(0, 7.5e9, 1, 3.35e12, 989e12) * 1e6 - 15.2) < 0.1
    t_w4 = 4.0e9 / 3.35e12
    assert abs(t_w4 / (2 * 7.5e9 / 989e12) - 79) < 1.0


def test_w8_sizes_and_validation(lib):
    assert lib.q8_packed_bytes(4096, 4096) == 4096 * 4096
    assert lib.q8_packed_bytes(17, 96) == 32 * 128
    assert lib.q8_packed_bytes(16, 100) == 0                     # in % 8 != 0
    assert lib.q8_packed_bytes(0, 128) == 0
    assert lib.q8_scales_count(17) == 32 and lib.q8_scales_count(0) == 0
    q = lib.q8_quantize_pack
    assert q(None, 16, 128, FAKE, FAKE, None) == 1
    assert q(FAKE, 16, 100, FAKE, FAKE, None) == 2
    assert b"multiple of 8" in lib.q4_last_error()
    assert q(FAKE, 1 << 30, 128, FAKE, FAKE, None) == 2
    assert q(FAKE + 2, 16, 128, FAKE, FAKE, None) == 4
    assert q(FAKE, 16, 128, FAKE + 8, FAKE, None) == 4
    assert q(FAKE, 16, 128, FAKE, FAKE + 1, None) == 4
    g = lib.q8_gemm
    assert g(None, 0, None, None, 16, 128, None, None, 0, None) == 0       # B = 0
    assert g(FAKE, -1, FAKE, FAKE, 16, 128, FAKE, None, 0, None) == 2
    assert g(None, 1, FAKE, FAKE, 16, 128, FAKE, None, 0, None) == 1
    assert g(FAKE, 1, FAKE, FAKE, 16, 124, FAKE, None, 0, None) == 2
    assert g(FAKE + 4, 1, FAKE, FAKE, 16, 128, FAKE, None, 0, None) == 4
    assert g(FAKE, 1, FAKE, FAKE, 16, 128, FAKE + 1, None, 0, None) == 4
    c = lib.q8_gemm_config
    assert c(FAKE, 1, FAKE, FAKE, 16, 128, FAKE, 3, 1, 1, None, 0, None) == 5
    assert c(FAKE, 1, FAKE, FAKE, 16, 128, FAKE, 1, 17, 1, None, 0, None) == 5
    assert c(FAKE, 1, FAKE, FAKE, 16, 256, FAKE, 1, 8, 3, None, 0, None) == 5    # k_splits > blocks
    assert c(FAKE, 16, FAKE, FAKE, 16, 8192, FAKE, 1, 8, 1, None, 0, None) == 5  # x slice > LDS
    assert c(FAKE, 1, FAKE, FAKE, 16, 256, FAKE, 1, 1, 2, None, 0, None) == 6    # split needs workspace
    assert c(FAKE, 1, FAKE, FAKE, 16, 256, FAKE, 1, 1, 2, FAKE + 4, 128, None) == 4
    # workspace: B = 8 over 28672 channels splits; few rows at B > 16 split the channels too
    ws = lib.q8_workspace_bytes(8, 8192, 28672)
    assert ws > 0 and ws % (8 * 8192 * 4) == 0
    assert lib.q8_workspace_bytes(1, 4096, 4096) == 0
    # (B > 16 split counts depend on the device's LDS per workgroup: checked on the GPU)
    assert lib.q8_workspace_bytes(40, 1024, 8192) % (40 * 1024 * 4) == 0
    assert c(FAKE, 40, FAKE, FAKE, 16, 256, FAKE, 1, 8, 1, None, 0, None) == 5   # config is GEMV-only
    assert lib.q8_gemm(FAKE, 8, FAKE, FAKE, 8192, 28672, FAKE, None, 0, None) == 6
    assert lib.q8_to_canonical(None, FAKE, 16, 128, FAKE, FAKE, None) == 1
    assert lib.q8_from_canonical(FAKE, FAKE, 16, 100, FAKE, FAKE, None) == 2


def test_actorder_perm_host(lib):
    """q4_actorder_perm is host logic: channels of group 0 ascending, then group 1, ..."""
    import numpy as np

    from w4a16_decode_amd import ops

    r = np.random.default_rng(0)
    for K, g in ((256, 32), (1024, 128), (512, 256)):
        g_idx = r.permutation(np.arange(K) // g).astype(np.int32)
        perm = ops.actorder_perm(g_idx, g)
        assert sorted(perm.tolist()) == list(range(K))
        for j in range(K // g):
            blk = perm[j * g:(j + 1) * g]
            assert np.all(g_idx[blk] == j) and np.all(np.diff(blk) > 0)
    gi = np.zeros(64, dtype=np.int32)
    out = np.empty(64, dtype=np.int32)
    f = lib.q4_actorder_perm
    assert f(None, 64, 32, out.ctypes.data) == 1
    assert f(gi.ctypes.data, 64, 32, out.ctypes.data) == 2          # group 0 holds 64 channels
    assert b"holds 64" in lib.q4_last_error()
    gi2 = (np.arange(64) // 32).astype(np.int32)
    gi2[5] = 2
    assert f(gi2.ctypes.data, 64, 32, out.ctypes.data) == 2         # index outside [0, 2)
    gi2[5] = -1
    assert f(gi2.ctypes.data, 64, 32, out.ctypes.data) == 2
    assert f(gi.ctypes.data, 64, 48, out.ctypes.data) == 3          # unsupported group
    assert f(gi.ctypes.data, 96, 64, out.ctypes.data) == 3          # in % group != 0


def test_actorder_validation(lib):
    q = lib.q4_quantize_pack_perm
    assert q(FAKE, 16, 128, 128, None, FAKE, FAKE, None) == 1
    assert q(FAKE, 16, 128, 128, FAKE + 4, FAKE, FAKE, None) == 4    # perm misaligned
    assert q(FAKE, 16, 96, 64, FAKE, FAKE, FAKE, None) == 3
    g = lib.q4_gemm_perm
    assert g(FAKE, 1, FAKE, FAKE, None, 16, 128, 128, FAKE, None, 0, None) == 1
    assert g(FAKE, 1, FAKE, FAKE, FAKE + 8, 16, 128, 128, FAKE, None, 0, None) == 4
    assert g(None, 0, None, None, None, 16, 128, 128, None, None, 0, None) == 0   # B = 0
    # x is gathered into the workspace: B * in * 2 bytes rounded to 256, then the split partials
    for B in (1, 4, 40):
        need = lib.q4_workspace_bytes_perm(B, 64, 7168, 128)
        x_bytes = (B * 7168 * 2 + 255) // 256 * 256
        assert need == x_bytes + lib.q4_workspace_bytes(B, 64, 7168, 128)
    assert g(FAKE, 40, FAKE, FAKE, FAKE, 64, 1024, 128, FAKE, None, 0, None) == 6
    assert g(FAKE, 1, FAKE, FAKE, FAKE, 64, 1024, 128, FAKE, FAKE, 1024, None) == 6   # 2048 + partials needed


def test_kv_validation(lib):
    q = lib.q4_kv_quantize_pack
    assert q(FAKE, 4, 1, 128, 96, FAKE, FAKE, 16, 0, None) == 3            # group
    assert q(FAKE, 4, 1, 96, 64, FAKE, FAKE, 16, 0, None) == 3             # head_dim % group
    assert q(FAKE, 4, 2, 128, 128, FAKE, FAKE, 16, 15, None) == 2          # pos + n > max_seq
    assert q(FAKE, -1, 1, 128, 128, FAKE, FAKE, 16, 0, None) == 2
    assert q(None, 0, 1, 128, 128, None, None, 16, 0, None) == 0           # nothing to do
    assert q(None, 4, 1, 128, 128, FAKE, FAKE, 16, 0, None) == 1
    assert q(FAKE + 4, 4, 1, 128, 128, FAKE, FAKE, 16, 0, None) == 4
    assert q(FAKE, 4, 1, 128, 128, FAKE + 2, FAKE, 16, 0, None) == 4
    d = lib.q4_kv_dequant
    assert d(FAKE, FAKE, 4, 1, 128, 128, 16, 16, FAKE, None) == 2
    assert d(FAKE, FAKE, 4, 1, 128, 128, 16, 0, FAKE + 8, None) == 4
    assert d(None, FAKE, 4, 1, 128, 128, 16, 0, FAKE, None) == 1


def test_read_probe_validation(lib):
    assert lib.q4_read_probe(None, 8192, FAKE, None) == 1
    assert lib.q4_read_probe(FAKE, 8000, FAKE, None) == 2
    assert lib.q4_read_probe(FAKE, 0, FAKE, None) == 2
    assert lib.q4_read_probe(FAKE + 8, 8192, FAKE, None) == 4
    assert lib.q4_rtn_check(None, None) == 1
    assert lib.q4_rtn_check(FAKE + 4, None) == 4
