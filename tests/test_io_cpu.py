"""Host-side text I/O of include/gc_io.h and the galaxy_gc program's argument handling (no GPU).

The catalog reader is pinned against Python's own decimal conversion (correctly rounded to
double, then narrowed to fp32 by numpy), which shares nothing with the library's parser; the
result writer against Python's %-formatting of the same values in the page's layout.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import two_point_angular_amd as gc
from two_point_angular_amd import catalogs

OK, INVALID, UNSUPPORTED, IO = 0, 1, 2, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gc.library_path()) or not os.path.exists(gc.CLI_PATH):
        from two_point_angular_amd import build
        build.build()
    return gc.load()


def expected(tokens):
    return np.array([np.float32(float(t)) for t in tokens], dtype=np.float32)


TOKENS = ["0", "-0", "+1", "1.", ".5", "-.25", "1e3", "1E-3", "123.456e+2", "0.000001234", "5400", "-5400.0000001",
          "21599.999999999", "0.1", "0.30000000000000004", "7e22", "1e23", "9007199254740993",
          "12345678901234567890123", "1.00000000000000000000001", "3.4028235e38", "1e-50", "-1.17549435e-38",
          "000123.4500", "2.5e-0", "6.02214076e23", "1.5e+10", "-999999999.999999999"]


def test_reader_matches_python_conversion(lib, tmp_path):
    toks = TOKENS + TOKENS[::-1][: len(TOKENS) % 2]  # an even count: pairs
    n = len(toks) // 2
    seps = ["\n", "\r\n", "\t", "  ", " \t "]
    body = "".join(f"{toks[2 * i]}{seps[i % len(seps)]}{toks[2 * i + 1]}\n" for i in range(n))
    p = tmp_path / "c.txt"
    p.write_text(f"  {n}\r\n" + body.rstrip("\n"))  # leading blanks, CRLF, no final newline
    ra, dec = gc.read_catalog(str(p))
    exp = expected(toks)
    np.testing.assert_array_equal(ra.view(np.uint32), exp[0::2].view(np.uint32))
    np.testing.assert_array_equal(dec.view(np.uint32), exp[1::2].view(np.uint32))


def test_reader_round_trips_workload_text(lib, tmp_path):
    for name in ("clustered100k_720", "patch100k_1500"):
        D, R = catalogs.WORKLOADS[name].catalogs(n=20000)
        catalogs.write_text(R, str(tmp_path / "R.txt"))
        ra, dec = gc.read_catalog(str(tmp_path / "R.txt"))
        assert np.array_equal(ra.view(np.uint32), R.ra.view(np.uint32))
        assert np.array_equal(dec.view(np.uint32), R.dec.view(np.uint32))
    assert gc.catalog_count(str(tmp_path / "R.txt")) == 20000


@pytest.mark.parametrize("text,status", [
    ("", IO), ("   \n", IO), ("x\n", IO), ("1.5\n1 2\n", IO), ("-1\n", IO), ("2\n1 2\n3\n", IO),
    ("1\n1.2.3 4\n", IO), ("1\nabc 4\n", IO), ("1\n1e 4\n", IO), ("1\n--1 4\n", IO), ("1\n+ 4\n", IO),
    ("1\n. 4\n", IO), ("1\n1 2\nextra\n", IO), ("1\n1e39 2\n", IO), ("1\nnan 2\n", IO), ("1\ninf 2\n", IO),
    ("3000000000\n", UNSUPPORTED), ("0\n", OK), ("1\n1 2", OK), ("1 10 20", OK),
])
def test_reader_errors(lib, tmp_path, text, status):
    p = tmp_path / "e.txt"
    p.write_text(text)
    n = ctypes.c_int64(-7)
    ra = (ctypes.c_float * 4)()
    dec = (ctypes.c_float * 4)()
    assert lib.gc_catalog_read(os.fsencode(str(p)), ra, dec, 4, ctypes.byref(n)) == status


def test_reader_argument_checks(lib, tmp_path):
    p = tmp_path / "c.txt"
    p.write_text("3\n1 2\n3 4\n5 6\n")
    n = ctypes.c_int64(0)
    buf = (ctypes.c_float * 3)()
    assert lib.gc_catalog_read(os.fsencode(str(p)), buf, buf, 2, ctypes.byref(n)) == INVALID
    assert n.value == 3                                     # the count is reported for a retry
    assert lib.gc_catalog_read(None, buf, buf, 3, ctypes.byref(n)) == INVALID
    assert lib.gc_catalog_read(os.fsencode(str(p)), None, buf, 3, ctypes.byref(n)) == INVALID
    assert lib.gc_catalog_read(os.fsencode(str(p)), buf, buf, 3, None) == INVALID
    assert lib.gc_catalog_count(os.fsencode(str(p)), None) == INVALID
    assert lib.gc_catalog_count(os.fsencode(str(tmp_path / "missing.txt")), ctypes.byref(n)) == IO
    assert lib.gc_catalog_count(os.fsencode(str(tmp_path)), ctypes.byref(n)) == IO    # a directory
    with pytest.raises(gc.GCError, match="file input/output error"):
        gc.read_catalog(str(tmp_path / "missing.txt"))


def test_omega_writer_layout(lib, tmp_path):
    rng = np.random.default_rng(3)
    nb, w = 9, 0.25
    dd = rng.integers(0, 10**12, nb).astype(np.uint64)
    dr = rng.integers(0, 10**12, nb).astype(np.uint64)
    rr = rng.integers(1, 10**12, nb).astype(np.uint64)
    rr[[0, 4]] = 0
    om = rng.normal(0, 3, nb)
    om[[0, 4]] = np.nan
    p = tmp_path / "omega.out"
    gc.write_omega(str(p), dd, dr, rr, om, w)
    lines = p.read_text().split("\n")
    assert lines[0] == "bin start\t\tomega\t        hist_DD\t        hist_DR\t        hist_RR"
    want = ["%6.3f\t%15f\t%15d\t%15d\t%15d" % (k * w, om[k], int(dd[k]), int(dr[k]), int(rr[k]))
            for k in range(nb) if rr[k] > 0]
    assert lines[1:-1] == want and lines[-1] == ""
    # every row parses back to the same integers
    back = np.array([[int(x) for x in ln.split("\t")[2:]] for ln in lines[1:-1]], dtype=np.uint64)
    keep = rr > 0
    assert np.array_equal(back, np.stack([dd[keep], dr[keep], rr[keep]], 1))


def test_omega_writer_errors(lib, tmp_path):
    z = np.zeros(4, np.uint64)
    o = np.zeros(4)
    vp = ctypes.c_void_p
    P = [z.ctypes.data_as(vp)] * 3 + [o.ctypes.data_as(vp)]
    path = os.fsencode(str(tmp_path / "o.out"))
    assert lib.gc_omega_write(path, *P, 0, 0.25) == INVALID
    assert lib.gc_omega_write(path, *P, 4, 0.0) == INVALID
    assert lib.gc_omega_write(path, *P, 4, float("inf")) == INVALID
    assert lib.gc_omega_write(None, *P, 4, 0.25) == INVALID
    assert lib.gc_omega_write(path, None, *P[1:], 4, 0.25) == INVALID
    assert lib.gc_omega_write(os.fsencode(str(tmp_path / "no" / "o.out")), *P, 4, 0.25) == IO


def test_cli_usage_and_input_errors(lib, tmp_path):
    cli = gc.CLI_PATH
    run = lambda *a: subprocess.run([cli, *a], capture_output=True, text=True, timeout=60)  # noqa: E731
    assert run().returncode == 2
    assert run("a", "b").returncode == 2
    assert run("--bogus", "a", "b", "c").returncode == 2
    assert run("--nbins", "0", "a", "b", "c").returncode == 2
    assert run("--nbins", "9000", "a", "b", "c").returncode == 2
    assert run("--width", "-1", "a", "b", "c").returncode == 2
    r = run(str(tmp_path / "missing.txt"), str(tmp_path / "missing.txt"), str(tmp_path / "o.out"))
    assert r.returncode == 1 and "file input/output error" in r.stderr
    (tmp_path / "bad.txt").write_text("2\n1 2\n")
    r = run(str(tmp_path / "bad.txt"), str(tmp_path / "bad.txt"), str(tmp_path / "o.out"))
    assert r.returncode == 1 and "bad.txt" in r.stderr
    assert not (tmp_path / "o.out").exists()


def test_reader_matches_python_on_random_tokens(lib, tmp_path):
    """Seeded random tokens of every shape the grammar allows (sign, integer and fraction digits
    up to 30, exponent of either case and sign up to 3 digits, values up to fp32's range and
    into its subnormals): each parses to Python's correctly rounded double narrowed to fp32."""
    rng = np.random.default_rng(12)
    toks = []
    while len(toks) < 4000:
        sign = rng.choice(["", "-", "+"])
        ip = "".join(rng.choice(list("0123456789"), int(rng.integers(0, 16))))
        fp = "".join(rng.choice(list("0123456789"), int(rng.integers(0, 16))))
        if not ip and not fp:
            continue
        body = ip + ("." + fp if fp or rng.random() < 0.3 else "")
        if body == ".":
            continue
        if rng.random() < 0.5:
            body += rng.choice(["e", "E"]) + rng.choice(["", "-", "+"]) + str(int(rng.integers(0, 60)))
        t = sign + body
        v = float(t)
        if abs(v) > 3.4e38:  # the reader refuses fp32 overflow
            continue
        toks.append(t)
    p = tmp_path / "rand.txt"
    p.write_text(f"{len(toks) // 2}\n" + "\n".join(f"{a} {b}" for a, b in zip(toks[0::2], toks[1::2])) + "\n")
    ra, dec = gc.read_catalog(str(p))
    want = expected(toks)
    assert np.array_equal(ra.view(np.uint32), want[0::2].view(np.uint32))
    assert np.array_equal(dec.view(np.uint32), want[1::2].view(np.uint32))
