"""Per-phase timing of the sampler kernel from the tracing build's stamps.

Runs a workload through libtsr_trace.so (build.py --trace: the same kernels
with a stamp of the device's 100 MHz real-time counter at each phase, one per
wavefront) and prints, per phase, when the workgroups reached it, measured
from the launch's first stamp: median / 90th percentile / maximum over the
rows, for all rows and for the near-flat rows of the 256 x 128256 workload
apart. A phase a row skips is left out of its statistics. Timing is what the
ordinary library does plus one store per stamp.

  python -m token_sampling_row_amd.trace [--workload 3] [--launches 20] [--out FILE]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TRACE_LIB = os.path.join(HERE, "libtsr_trace.so")
SLOTS = 16
TICK_NS = 10.0                       # s_memrealtime runs at 100 MHz
# (slot, name) in the order the sampler reaches them
PHASES = [(0, "entry"), (1, "loads issued"), (2, "pass A done"), (3, "row statistics barrier"),
          (11, "row statistics combined"), (12, "filters derived"),
          (13, "compaction: chunk rows found"), (14, "compaction: staged (last)"),
          (4, "compaction 1"), (5, "top-k bound"), (6, "compaction 2"),
          (7, "fast resolve + draw"), (8, "register search"), (9, "walk"),
          (10, "outputs written")]
HW_SLOT = 15


def run(workload: int, launches: int, run_index: int = 0):
    os.environ.setdefault("TSR_LIBRARY", TRACE_LIB)
    import torch

    import token_sampling_row_amd as tsr
    from token_sampling_row_amd import workloads as wl

    lib = tsr.load_library()
    lib.sampler_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.sampler_trace_clear.argtypes = [ctypes.c_void_p]
    w = wl.config(workload)
    prm = w.runs[run_index]
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        base = torch.from_numpy(np.ascontiguousarray(w.data).view(np.int16)).to(dev).view(
            torch.bfloat16)
    else:
        base = torch.from_numpy(np.ascontiguousarray(w.data)).to(dev)
    bufs = [base.clone() for _ in range(8)]       # rotate: every launch reads HBM
    out = torch.empty(w.rows, dtype=torch.int32, device=dev)
    waves = 8
    nwords = w.rows * waves * SLOTS
    stamps = []
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8,
                     seed=wl.philox_seed(workload)) as s:
        for i in range(8):                          # warm-up
            s.sample_rows(bufs[i % 8], prm, i, out=out)
        for i in range(launches):
            if lib.sampler_trace_clear(s._h) != 0:
                raise RuntimeError("sampler_trace_clear failed")
            s.sample_rows(bufs[i % 8], prm, 100 + i, out=out)
            host = np.zeros(nwords, dtype=np.uint64)
            if lib.sampler_trace_read(s._h, host.ctypes.data, nwords) != 0:
                raise RuntimeError("sampler_trace_read failed")
            stamps.append(host.reshape(w.rows, waves, SLOTS).astype(np.int64))
    return w, prm, stamps


def summarize(w, prm, stamps) -> str:
    flat = set(w.extra.get("flat_rows", []))
    groups = [("all rows", list(range(w.rows)))]
    if flat:
        groups += [(f"{len(flat)} near-flat rows", sorted(flat)),
                   (f"{w.rows - len(flat)} Zipf rows", [b for b in range(w.rows) if b not in flat])]
    lines = [f"workload {w.name}, params {prm}, {len(stamps)} traced launches",
             "times in microseconds from the launch's first stamp; per row the phase time is its",
             "last wavefront's stamp; median / p90 / max over rows and launches", ""]
    for gname, rows in groups:
        lines.append(f"| {gname} | rows reaching | median | p90 | max |")
        lines.append("|---|---|---|---|---|")
        for slot, name in PHASES:
            vals = []
            for st in stamps:
                t0 = st[:, :, :HW_SLOT][st[:, :, :HW_SLOT] > 0].min()
                blk = st[rows, :, slot]                    # [rows, waves]
                reached = (blk > 0).any(axis=1)
                t = np.where(blk > 0, blk, 0).max(axis=1)
                vals += [(x - t0) * TICK_NS / 1000.0 for x, r in zip(t, reached) if r]
            if not vals:
                continue
            v = np.array(vals)
            lines.append(f"| {name} | {len(v) // len(stamps)} | {np.median(v):.2f} | "
                         f"{np.percentile(v, 90):.2f} | {v.max():.2f} |")
        lines.append("")
    ends, passa = [], []
    for st in stamps:
        t = st[:, :, :HW_SLOT]
        t0 = t[t > 0].min()
        ends.append((t.max() - t0) * TICK_NS / 1000.0)
        passa.append((t[:, :, 2].max() - t0) * TICK_NS / 1000.0)
    lines.append(f"per launch, last stamp (us): median {np.median(ends):.2f}, max {max(ends):.2f}; "
                 f"last pass A: median {np.median(passa):.2f}, max {max(passa):.2f}")
    # pass A completion by accelerator complex die (XCC), over rows and launches
    hw = np.stack([st[:, 0, HW_SLOT] for st in stamps])          # [launches, rows]
    xcc = (hw >> 16) & 0xF
    pa = []
    for st in stamps:
        t = st[:, :, :HW_SLOT]
        t0 = t[t > 0].min()
        pa.append((t[:, :, 2].max(axis=1) - t0) * TICK_NS / 1000.0)
    pa = np.stack(pa)
    if (hw != 0).any():
        lines.append("")
        lines.append("| XCC | rows | pass A median | p90 | max | end median | end max |")
        lines.append("|---|---|---|---|---|---|---|")
        endr = []
        for st in stamps:
            t = st[:, :, :HW_SLOT]
            t0 = t[t > 0].min()
            endr.append((t.max(axis=(1, 2)) - t0) * TICK_NS / 1000.0)
        endr = np.stack(endr)
        for x in sorted(set(xcc.ravel().tolist())):
            m = xcc == x
            lines.append(f"| {x} | {int(m.sum()) // len(stamps)} | {np.median(pa[m]):.2f} | "
                         f"{np.percentile(pa[m], 90):.2f} | {pa[m].max():.2f} | "
                         f"{np.median(endr[m]):.2f} | {endr[m].max():.2f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--run", type=int, default=0, help="index of the workload's parameter set")
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    w, prm, stamps = run(args.workload, args.launches, args.run)
    text = summarize(w, prm, stamps)
    print(text)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    sys.exit(main())
