"""gc_histogram_part: the parts of one job sum exactly to the single call, in any order, for any
number of parts (including more parts than work units), and a checkpointed run resumed after an
interruption gives the same histograms."""
import numpy as np
import pytest

from two_point_angular_amd import catalogs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gc():
    import torch
    import two_point_angular_amd as gcm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcm.load()
    return gcm


def _prep(gc, D, R):
    import torch
    dev = "cuda"
    return (gc.prepare(torch.from_numpy(D.ra).to(dev), torch.from_numpy(D.dec).to(dev)),
            gc.prepare(torch.from_numpy(R.ra).to(dev), torch.from_numpy(R.dec).to(dev)))


def _single(gc, pd, n_d, pr, n_r, nbins, w, tuning=None):
    import torch
    out = gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w, tuning=tuning)
    torch.cuda.synchronize()
    return np.stack([o.cpu().numpy() for o in out])


def _in_parts(gc, pd, n_d, pr, n_r, nbins, w, parts, order=None, tuning=None):
    import torch
    hist = torch.zeros((3, nbins), dtype=torch.int64, device="cuda")
    for p in (order if order is not None else range(parts)):
        gc.histogram_part(pd, n_d, pr, n_r, nbins, w, p, parts, hist, tuning=tuning)
    torch.cuda.synchronize()
    return hist.cpu().numpy()


@pytest.mark.parametrize("name,nbins,w", [("clustered100k_720", 720, 0.25), ("patch100k_1500", 1500, 0.001)])
def test_parts_sum_to_the_single_call(gc, name, nbins, w):
    print(f"[gpu] parts {name}", flush=True)
    D, R = catalogs.WORKLOADS[name].catalogs(n=3000)
    R = R.subset(0, 2500)
    pd, pr = _prep(gc, D, R)
    ref = _single(gc, pd, len(D), pr, len(R), nbins, w)
    for parts in (1, 2, 3, 7, 64, 1000, 40000):
        got = _in_parts(gc, pd, len(D), pr, len(R), nbins, w, parts)
        assert np.array_equal(got, ref), parts
    rng = np.random.default_rng(0)
    got = _in_parts(gc, pd, len(D), pr, len(R), nbins, w, 13, order=rng.permutation(13))
    assert np.array_equal(got, ref)
    t = gc.Tuning(i_per_lane=4, shared_histogram=2)
    assert np.array_equal(_in_parts(gc, pd, len(D), pr, len(R), nbins, w, 9, tuning=t), ref)


def test_part_accumulates_and_empty_parts(gc):
    import torch
    print("[gpu] part accumulates", flush=True)
    D = catalogs.clustered(700, 4)
    pd, _ = _prep(gc, D, D)
    ref = _single(gc, pd, 700, pd, 700, 720, 0.25)
    hist = torch.full((3, 720), 5, dtype=torch.int64, device="cuda")
    gc.histogram_part(pd, 700, pd, 700, 720, 0.25, 0, 1, hist)
    torch.cuda.synchronize()
    assert np.array_equal(hist.cpu().numpy(), ref + 5)
    # an empty catalog: every part adds nothing to DD and DR
    E = D.subset(0, 0)
    pe, _ = _prep(gc, E, E)
    got = _in_parts(gc, pe, 0, pd, 700, 720, 0.25, 4)
    assert got[0].sum() == 0 and got[1].sum() == 0 and np.array_equal(got[2], ref[2])


def test_checkpointed_run_resumes(gc, tmp_path):
    from two_point_angular_amd import parts
    print("[gpu] checkpoint resume", flush=True)
    D, R = catalogs.WORKLOADS["clustered100k_720"].catalogs(n=4000)
    pd, pr = _prep(gc, D, R)
    ref = _single(gc, pd, 4000, pr, 4000, 720, 0.25)
    ck = str(tmp_path / "run.npz")
    key = D.sha256() + R.sha256()
    h, nxt = parts.run_in_parts(pd, 4000, pr, 4000, 720, 0.25, 7, checkpoint=ck, key=key, stop_after=3)
    assert nxt == 3
    seen = []
    h, nxt = parts.run_in_parts(pd, 4000, pr, 4000, 720, 0.25, 7, checkpoint=ck, key=key,
                                on_part=lambda p, _: seen.append(p))
    assert nxt == 7 and seen == [3, 4, 5, 6]
    assert np.array_equal(h.cpu().numpy(), ref)
    h, nxt = parts.run_in_parts(pd, 4000, pr, 4000, 720, 0.25, 7, checkpoint=ck, key=key)   # already done
    assert nxt == 7 and np.array_equal(h.cpu().numpy(), ref)
    with pytest.raises(ValueError):
        parts.run_in_parts(pd, 4000, pr, 4000, 720, 0.25, 7, checkpoint=ck, key="other catalogs")
    # a plan with another i-block height splits the job into other pairs per part: not resumed
    assert gc.launch_plan(4000, 4000, 720, 0.25, gc.Tuning(i_per_lane=4))["i_per_lane"] == 4
    with pytest.raises(ValueError):
        parts.run_in_parts(pd, 4000, pr, 4000, 720, 0.25, 7, checkpoint=ck, key=key, tuning=gc.Tuning(i_per_lane=4))


def test_million_catalogs_in_parts(gc):
    print("[gpu] clustered1m_720 in 8 parts vs one call", flush=True)
    wl = catalogs.WORKLOADS["clustered1m_720"]
    D, R = wl.catalogs()
    pd, pr = _prep(gc, D, R)
    ref = _single(gc, pd, len(D), pr, len(R), wl.nbins, wl.bin_width_deg)
    got = _in_parts(gc, pd, len(D), pr, len(R), wl.nbins, wl.bin_width_deg, 8)
    assert np.array_equal(got, ref)
    assert [int(x.sum()) for x in got] == [len(D) ** 2] * 3
