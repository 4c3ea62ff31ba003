"""The Python binding checks every tensor it hands to the library before the call: the library
sees only addresses, so a short, mistyped or strided buffer would otherwise become an
out-of-bounds device access.  Run on the CPU: every check that precedes the device check is
reached with host tensors, and a host tensor that passes them is refused as not on a GPU."""
import pytest
import torch

import two_point_angular_amd as gc


@pytest.fixture(scope="module", autouse=True)
def lib():
    return gc.load()


def f32(n):
    return torch.zeros(n, dtype=torch.float32)


def test_prepare_checks():
    with pytest.raises(TypeError, match="float32"):
        gc.prepare(torch.zeros(10, dtype=torch.float64), f32(10))
    with pytest.raises(TypeError, match="contiguous"):
        gc.prepare(f32(20)[::2], f32(10))
    with pytest.raises(ValueError, match="same length"):
        gc.prepare(f32(10), f32(9))
    with pytest.raises(ValueError, match="needs at least"):
        gc.prepare(f32(10), f32(10), out=torch.zeros(gc.prepared_bytes(10) - 1, dtype=torch.uint8))
    with pytest.raises(TypeError, match="uint8"):
        gc.prepare(f32(10), f32(10), out=torch.zeros(gc.prepared_bytes(10), dtype=torch.int8))
    with pytest.raises(TypeError, match="device tensor"):
        gc.prepare(f32(10), f32(10))
    with pytest.raises(TypeError, match="must be a torch tensor"):
        gc.prepare([0.0] * 10, f32(10))


def _job(**kw):
    nb = kw.pop("nbins", 720)
    a = dict(prep_d=torch.zeros(gc.prepared_bytes(100), dtype=torch.uint8), n_d=100,
             prep_r=torch.zeros(gc.prepared_bytes(50), dtype=torch.uint8), n_r=50,
             out=torch.zeros((3, nb), dtype=torch.int64),
             workspace=torch.zeros(gc.workspace_bytes(nb), dtype=torch.uint8))
    a.update(kw)
    return gc.histogram_dd_dr_rr(a["prep_d"], a["n_d"], a["prep_r"], a["n_r"], nb, 0.25, out=a["out"],
                                 workspace=a["workspace"])


def test_histogram_checks():
    with pytest.raises(ValueError, match="needs at least"):
        _job(prep_d=torch.zeros(gc.prepared_bytes(100) - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="needs at least"):
        _job(n_r=65)                                       # prep_r holds up to 64 galaxies
    with pytest.raises(TypeError, match="required"):
        _job(prep_r=None)                                  # n_r = 50 needs a catalog
    with pytest.raises(ValueError, match="shape"):
        _job(out=torch.zeros(3 * 720, dtype=torch.int64))
    with pytest.raises(ValueError, match="shape"):
        _job(out=torch.zeros((3, 719), dtype=torch.int64))
    with pytest.raises(TypeError, match="int64"):
        _job(out=torch.zeros((3, 720), dtype=torch.float64))
    with pytest.raises(TypeError, match="contiguous"):
        _job(out=torch.zeros((720, 3), dtype=torch.int64).t())
    with pytest.raises(ValueError, match="needs at least"):
        _job(workspace=torch.zeros(gc.workspace_bytes(720) - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="outside"):
        _job(n_d=-1)
    with pytest.raises(ValueError, match="outside"):
        _job(nbins=0)
    with pytest.raises(ValueError, match="outside"):
        _job(nbins=gc.MAX_BINS + 1)
    with pytest.raises(TypeError, match="device tensor"):
        _job()                                             # everything right, but on the host
    out = torch.zeros((3, 720), dtype=torch.int64)
    with pytest.raises(ValueError, match="shape"):
        gc.histogram_part(None, 0, None, 0, 720, 0.25, 0, 1, out[:2])


def test_totals_and_omega_checks():
    dd = torch.zeros(720, dtype=torch.int64)
    with pytest.raises(ValueError, match="shape"):
        gc.histogram_totals(dd, torch.zeros(719, dtype=torch.int64), dd)
    with pytest.raises(TypeError, match="int64"):
        gc.omega(dd, dd, torch.zeros(720, dtype=torch.float64), 10, 10)
    with pytest.raises(ValueError, match="needs at least"):
        gc.omega(dd, dd, dd, 10, 10, out=torch.zeros(719, dtype=torch.float64))
    with pytest.raises(ValueError, match="needs at least"):
        gc.histogram_totals(dd, dd, dd, out=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(TypeError, match="device tensor"):
        gc.histogram_totals(dd, dd, dd)


def test_ladder_and_diagnostic_checks():
    with pytest.raises(ValueError, match="same length"):
        gc.ladder_histogram(5, f32(10), f32(9), f32(10), f32(10), 720, 0.25)
    with pytest.raises(ValueError, match="needs at least"):
        gc.ladder_histogram(5, f32(10), f32(10), f32(10), f32(10), 720, 0.25,
                            workspace=torch.zeros(1, dtype=torch.uint8))
    with pytest.raises(TypeError, match="float32 or float64"):
        gc.eval_angle_core(torch.zeros(10, dtype=torch.int32), 720, 0.25)
    with pytest.raises(ValueError, match="shape"):
        gc.eval_dot_mfma(torch.zeros((3, 17)), torch.zeros((3, 17)))
    with pytest.raises(ValueError, match="shape"):
        gc.eval_dot_mfma(torch.zeros((3, 16)), torch.zeros((3, 32)))
