"""Checkpointable histogram runs in parts, for catalogs far beyond 10^6 galaxies.

The job (DD, DR, RR over all ordered pairs) is cut into `parts` additive pieces by
gc_histogram_part (include/gc.h, section "parts").  run_in_parts adds them one after another into
one set of device histograms and, when given a checkpoint path, saves the running histograms and
the next part index after every `save_every` parts; a later call with the same job resumes from
the saved state.  The histograms are additive over the pairs (the symmetry argument of "CUDA Deep
Dive: 10B Galaxy Pairs on an RTX 5080", section "L1: DD/RR symmetry", is the only coupling), so
the resumed result is bit-identical to an uninterrupted one.

Checkpoint file: a numpy .npz (no pickled objects) with `meta` (a JSON string describing the job),
`next_part` and `hist` (3 x nbins uint64).  It is replaced atomically (write, then rename).

Command line (a scale-out run on one GPU):

    python -m two_point_angular_amd.parts --workload clustered1m_720 --n 4000000 --parts 32 \\
        --checkpoint run.npz
"""
from __future__ import annotations

import json
import os

import numpy as np

from . import Tuning, histogram_part, launch_plan, workspace_bytes

_TUNING_FIELDS = ("dot_precision", "i_per_lane", "blocks_per_cu", "shared_histogram", "span_kernel", "fast_core",
                  "flush_interval", "hist_columns", "waves_per_group", "l1_share")


def _meta(n_d, n_r, nbins, w, parts, key, tuning, i_per_lane=0):
    """The job a checkpoint belongs to.  i_per_lane is the launch plan's galaxies per lane: part p
    of P covers the steps of an i-block of 64 of them per lane, so a part's pairs depend on it (a
    resume under another plan, or another library build that plans differently, would mix two
    decompositions); the tuning fields are kept whole."""
    t = None if tuning is None else [int(getattr(tuning, f)) for f in _TUNING_FIELDS]
    return json.dumps({"n_d": int(n_d), "n_r": int(n_r), "nbins": int(nbins), "bin_width_deg": float(w),
                       "parts": int(parts), "key": str(key), "tuning": t, "i_per_lane": int(i_per_lane)},
                      sort_keys=True)


def load_checkpoint(path: str, meta: str):
    """(next_part, hist) from a checkpoint of the same job, or None if there is no file.
    A file from a different job raises ValueError rather than being resumed."""
    if not os.path.exists(path):
        return None
    with np.load(path, allow_pickle=False) as z:
        saved = str(z["meta"])
        if saved != meta:
            raise ValueError(f"checkpoint {path} belongs to another job: {saved} != {meta}")
        return int(z["next_part"]), np.array(z["hist"], dtype=np.uint64)


def save_checkpoint(path: str, meta: str, next_part: int, hist: np.ndarray) -> None:
    tmp = f"{path}.tmp{os.getpid()}.npz"
    np.savez(tmp, meta=np.array(meta), next_part=np.int64(next_part), hist=np.asarray(hist, dtype=np.uint64))
    os.replace(tmp, path)


def run_in_parts(prep_d, n_d: int, prep_r, n_r: int, nbins: int, bin_width_deg: float, parts: int,
                 checkpoint: str | None = None, key: str = "", save_every: int = 1, tuning: Tuning | None = None,
                 stop_after: int | None = None, on_part=None, stream=None):
    """Run (or resume) the job in `parts` parts.  Returns (hist, next_part): hist is a (3, nbins)
    int64 device tensor holding parts [0, next_part); next_part == parts when the job is done.
    `key` identifies the catalogs in the checkpoint (for example their SHA-256); `stop_after`
    limits the number of parts run by this call; on_part(part, hist) is called after each part
    has completed."""
    import torch
    dev = prep_d.device if prep_d is not None else prep_r.device
    k = launch_plan(n_d, n_r, nbins, bin_width_deg, tuning)["i_per_lane"]
    meta = _meta(n_d, n_r, nbins, bin_width_deg, parts, key, tuning, k)
    hist = torch.zeros((3, nbins), dtype=torch.int64, device=dev)
    start = 0
    if checkpoint:
        got = load_checkpoint(checkpoint, meta)
        if got is not None:
            start, h = got
            hist.copy_(torch.from_numpy(h.view(np.int64)))
    ws = torch.empty(max(workspace_bytes(nbins), 1), dtype=torch.uint8, device=dev)
    end = parts if stop_after is None else min(parts, start + stop_after)
    for p in range(start, end):
        histogram_part(prep_d, n_d, prep_r, n_r, nbins, bin_width_deg, p, parts, hist, workspace=ws, tuning=tuning,
                       stream=stream)
        done = p + 1
        if on_part is not None or (checkpoint and (done % save_every == 0 or done == end)):
            torch.cuda.synchronize()
            if on_part is not None:
                on_part(p, hist)
            if checkpoint and (done % save_every == 0 or done == end):
                save_checkpoint(checkpoint, meta, done, hist.cpu().numpy().view(np.uint64))
    return hist, end


def _main(argv=None) -> int:
    import argparse
    import hashlib
    import sys
    import time

    import torch

    from . import catalogs, histogram_totals, prepare

    ap = argparse.ArgumentParser(description="Checkpointable DD/DR/RR run in parts on one GPU.")
    ap.add_argument("--workload", default="clustered1m_720", choices=sorted(catalogs.WORKLOADS))
    ap.add_argument("--n", type=int, default=None, help="galaxies per catalog (default: the workload's)")
    ap.add_argument("--parts", type=int, default=16)
    ap.add_argument("--checkpoint", default=None)
    ap.add_argument("--save-every", type=int, default=1)
    ap.add_argument("--stop-after", type=int, default=None)
    a = ap.parse_args(argv)
    wl = catalogs.WORKLOADS[a.workload]
    D, R = wl.catalogs(n=a.n)
    n_d, n_r = len(D), len(R)
    key = hashlib.sha256(D.sha256().encode() + R.sha256().encode()).hexdigest()
    dev = torch.device("cuda:0")
    pd = prepare(torch.from_numpy(D.ra).to(dev), torch.from_numpy(D.dec).to(dev))
    pr = prepare(torch.from_numpy(R.ra).to(dev), torch.from_numpy(R.dec).to(dev))
    ordered = float(n_d * n_d + n_d * n_r + n_r * n_r)
    t_last = [time.perf_counter()]

    def report(p, h):
        now = time.perf_counter()
        print(f"part {p + 1}/{a.parts} done: {now - t_last[0]:.3f} s "
              f"({ordered / a.parts / (now - t_last[0]):.3e} ordered pairs/s)", flush=True)
        t_last[0] = now

    t0 = time.perf_counter()
    hist, nxt = run_in_parts(pd, n_d, pr, n_r, wl.nbins, wl.bin_width_deg, a.parts, checkpoint=a.checkpoint,
                             key=key, save_every=a.save_every, stop_after=a.stop_after, on_part=report)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    if nxt < a.parts:
        print(f"stopped after part {nxt}/{a.parts}; run again to resume", flush=True)
        return 0
    tot = histogram_totals(hist[0], hist[1], hist[2]).cpu().numpy().view(np.uint64)
    want = [n_d * n_d, n_d * n_r, n_r * n_r]
    ok = [int(x) for x in tot] == want
    print(json.dumps({"workload": wl.name, "n_d": n_d, "n_r": n_r, "parts": a.parts, "seconds_this_call": el,
                      "totals_exact": ok, "ordered_pairs": ordered}), flush=True)
    if not ok:
        print(f"totals {list(tot)} != {want}", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    raise SystemExit(_main())
