"""Host logic of the profile summaries (w4a16_decode_amd/profiling.py), no GPU."""

import csv
import os
import shutil

import pytest

from w4a16_decode_amd import profiling


def test_code_only_strips_comments_keeps_literals():
    src = 'int a = 1; // c\n/* x\n y */ int b;\nconst char* s = "// not /* a comment";  char q = \'"\';'
    assert profiling.code_only(src) == 'int a = 1; int b; const char* s = "// not /* a comment"; char q = \'"\';'


def test_fingerprint_follows_code_not_comments(tmp_path):
    srcs = [os.path.join(profiling.HERE, rel) for rel in profiling.KERNEL_SOURCES]
    copies = []
    for p in srcs:
        q = tmp_path / os.path.basename(p)
        shutil.copy(p, q)
        copies.append(str(q))
    base = profiling.kernel_fingerprint(copies)
    assert base == profiling.kernel_fingerprint()
    text = open(copies[0]).read()
    open(copies[0], "w").write("// a new comment\n" + text.replace(";", ";  ", 3) + "\n/* trailing */\n")
    assert profiling.kernel_fingerprint(copies) == base
    open(copies[0], "w").write(text.replace("kSuperK", "kSuperK2", 1))
    assert profiling.kernel_fingerprint(copies) != base


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_split_and_traffic(tmp_path):
    trace = tmp_path / "t.csv"
    _write(trace, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [["gemv_kernel<1>", 0, 42000], ["gemv_kernel<1>", 0, 13000], ["other", 0, 99000],
            ["gemv_kernel<1>", 100, 44100]])
    below, above = profiling.split_durations(str(trace), "gemv_kernel", 25)
    assert below == [13.0] and above == [42.0, 44.0]

    def counter_csv(name, kernel, counter, value):
        _write(tmp_path / name, ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[kernel, counter, value], [kernel, counter, value + 2], ["x", counter, 1e9]])
        return str(tmp_path / name)

    # kernel: 120000 +- 1 KiB fetched, 112 +- 1 KiB written; calibration copy of 256 MiB:
    # FETCH_SIZE reports half of it, WRITE_SIZE all of it
    t = profiling.traffic(counter_csv("f.csv", "gemv", "FETCH_SIZE", 119999),
                          counter_csv("w.csv", "gemv", "WRITE_SIZE", 111),
                          counter_csv("cf.csv", "copyBuffer", "FETCH_SIZE", 131071),
                          counter_csv("cw.csv", "copyBuffer", "WRITE_SIZE", 262143),
                          268435456, "gemv")
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["bytes"] == pytest.approx(120000 * 1024 * 2.0 + 112 * 1024)
