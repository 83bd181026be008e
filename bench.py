"""Throughput of the batched logits-to-token sampler on one MI355X.

A step is one sample_rows call over one batch: temperature, softmax, top-k,
top-p, min-p, renormalisation (eq. 39.2) and one Philox draw per row. The
headline workload is 256 rows x 128256 bf16 logits with the full chain
(T=0.9, top_k=50, top_p=0.95, min_p=0.1). Inputs are synthetic, seeded,
Zipf-like logits already resident in HBM; eight copies of the batch in eight
separate allocations are used in turn, so each call reads HBM rather than the
256 MB last-level cache.

Prints one JSON line. Also times the other workloads (greedy, pure sampling,
min-p, the verify step, the wide-nucleus batch) and, in its CPU leg, runs the
float64 oracle: on a bounded sample of the headline batch for the host
baseline, and on every row of every workload for the parity block (the GPU's
outputs of one untimed call per workload, with diagnostics, compared under the
rule of oracle/parity.py: rows in band, excused and out-of-band mismatches,
the largest relative error of p~).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extra] [--no-cpu-baseline]
                  [--no-parity]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
ROTATE = 8                     # distinct input buffers used in turn
CALIB_BYTES = 1 << 28          # size of each --copy-calibration device copy


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "token_sampling_row_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel sources (profiles/traffic_<workload>.json)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def row_kernel_label(dtype: str, vocab: int) -> str:
    """Name of the sample_kernel instance a row of this size launches: 512
    threads per row, 16-byte chunks, the smallest compiled chunk count per
    thread that covers the row."""
    epc = 8 if dtype == "bf16" else 4
    need = -(-(-(-vocab // epc)) // 512)
    nc = next((n for n in (1, 2, 4, 8, 16, 24, 32, 38) if n >= need), None)
    return f"sample_kernel<{dtype}, {nc}>" if nc else "sample_kernel_stream"


def write_traffic(fetch_csv: str, write_csv: str, workload: str, kernel_prefix: str) -> dict:
    """HBM bytes per launch of the headline kernel from two rocprofv3 --pmc runs
    of this script with --copy-calibration (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch). Each counter is scaled by what it reads for the calibration
    copies (256 MiB device-to-device, the copy dispatches after the last
    sampler dispatch) against their known size. Writes
    profiles/traffic_<workload>.json tagged with the kernel-source hash."""
    import csv

    def scaled(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        kern = [i for i, r in enumerate(rows) if r["Kernel_Name"].removeprefix("void ").startswith(kernel_prefix)]
        if not kern:
            raise SystemExit(f"no {kernel_prefix} dispatch in {path}")
        # the 256 MiB copies only (a small copy of a result may follow the kernel)
        calib = [float(r["Counter_Value"]) for r in rows[kern[-1] + 1:]
                 if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > CALIB_BYTES / 1024.0 / 100]
        if not calib:
            raise SystemExit(f"no calibration copies after the sampler dispatches in {path}")
        factor = (CALIB_BYTES / 1024.0) / (sum(calib) / len(calib))
        vals = [float(rows[i]["Counter_Value"]) for i in kern]
        kib = sum(vals) / len(vals)
        return kib, factor, len(vals), len(calib)

    fk, ff, nf, cf = scaled(fetch_csv, "FETCH_SIZE")
    wk, wf, nw, cw = scaled(write_csv, "WRITE_SIZE")
    out = {"workload": workload, "kernel": kernel_prefix, "source_hash": source_hash(),
           "fetch_kib_per_dispatch": fk, "fetch_scale": ff, "write_kib_per_dispatch": wk,
           "write_scale": wf, "dispatches": [nf, nw], "calibration_copies": [cf, cw],
           "hbm_bytes_per_launch": (fk * ff + wk * wf) * 1024.0}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    return out


def device_batch(torch, w, copies):
    import numpy as np
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(w.data).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(w.data)).to(dev)
    return [t.clone() for _ in range(copies)]


def median_call(torch, fn, calls=200):
    """Median GPU time of one call: an event pair around each call on the
    current stream (the per-call figure; the headline uses time_calls)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2]


def time_calls(torch, fn, steps, warmup):
    """Average GPU time per call with HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


BOX_CPU_SHARE = 16   # host processes a one-GPU job may run (the machine's CPU share per GPU)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, params, seed, budget_s=10.0, one_core_s=4.0):
    """The float64 oracle on the host over a bounded sample of the batch: rows/s
    with one process per core of the job's CPU share, and rows/s on one core."""
    import multiprocessing as mp
    import oracle
    cores = min(BOX_CPU_SHARE, os.cpu_count() or 1)
    values_rows = list(range(w.rows))
    ctx = mp.get_context("fork")
    done, t0 = 0, time.perf_counter()
    with ctx.Pool(cores, initializer=_pool_init, initargs=(w.data, w.dtype, params, seed)) as pool:
        while time.perf_counter() - t0 < budget_s:
            n = sum(pool.map(_oracle_rows, [values_rows[i::cores] for i in range(cores)]))
            done += n
    dt = time.perf_counter() - t0
    values = oracle.values_from_stored(w.data, w.dtype)
    one, t1 = 0, time.perf_counter()
    while time.perf_counter() - t1 < one_core_s:
        oracle.sample_row(values[one % w.rows], params, seed, one % w.rows, 0)
        one += 1
    d1 = time.perf_counter() - t1
    return {"value": done / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} rows of the {w.rows}x{w.vocab} {w.dtype} batch "
                      f"({done // w.rows} passes, {dt:.1f} s wall on {cores} processes); "
                      f"one core: {one} rows in {d1:.1f} s",
            "one_core_rows_per_s": one / d1, "os_cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
            "note": f"processes capped at {BOX_CPU_SHARE}, the host CPU share of a one-GPU job"}


_POOL = {}


def _pool_init(data, dtype, params, seed):
    import oracle
    _POOL["values"] = oracle.values_from_stored(data, dtype)
    _POOL["params"] = params
    _POOL["seed"] = seed


def _oracle_rows(rows):
    import oracle
    for b in rows:
        oracle.sample_row(_POOL["values"][b], _POOL["params"], _POOL["seed"], b, 0)
    return len(rows)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--only", default=None,
                    help="of the other workloads, run those whose name holds this text")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle comparison of every workload (CPU leg)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 256 MiB device copies (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files into profiles/traffic_*.json")
    args = ap.parse_args()
    if args.write_traffic:
        from token_sampling_row_amd import workloads as wl
        w3 = wl.config(3, rows=1)
        # the headline launches the common instance (third template argument false)
        label = row_kernel_label(w3.dtype, w3.vocab).replace('bf16', '1').replace('f32', '0')
        print(json.dumps(write_traffic(*args.write_traffic, "batch256_128256_bf16",
                                       f"tsr::{label[:-1]}, false, 0>")))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sampler shards by batch row with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import token_sampling_row_amd as tsr
    from token_sampling_row_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w3 = wl.config(3)
    params = w3.runs[0]
    seed = wl.philox_seed(3)
    bufs = device_batch(torch, w3, ROTATE)
    out = torch.empty(w3.rows, dtype=torch.int32, device="cuda:0")
    sampler = tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=seed)

    ms = time_calls(torch, lambda i: sampler.sample_rows(bufs[i % ROTATE], params, i, out=out),
                    args.steps, args.warmup)
    ms_median = median_call(torch, lambda i: sampler.sample_rows(bufs[i % ROTATE], params, i,
                                                                 out=out))
    rows_per_s = w3.rows / (ms * 1e-3)
    alg_bytes = w3.rows * w3.vocab * 2
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(w3.name)

    extra = {}
    if not args.no_extra:
        extra = run_extra(torch, tsr, wl, max(50, args.steps // 4), max(5, args.warmup // 4),
                          args.only)

    if args.copy_calibration:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w3, params, seed)
    parity = None
    if not args.no_parity:
        del bufs
        parity = parity_leg(torch, tsr, wl)

    line = {
        "metric": "sampled rows/s + achieved HBM GB/s (% peak), B=256 V=128256 full filter chain",
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "batch256_vocab128256_bf16_full_chain", "rows": w3.rows,
                   "vocab": w3.vocab, "logits": "bf16", "temperature": 0.9, "top_k": 50,
                   "top_p": 0.95, "min_p": 0.1, "tokens_per_s": rows_per_s,
                   "input_buffers": ROTATE, "median_ms_per_call": ms_median},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel": row_kernel_label(w3.dtype, w3.vocab),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
        "parity": parity,
        "extra": extra,
    }
    sampler.close()
    print(json.dumps(line))


def parity_leg(torch, tsr, wl):
    """One untimed call per workload run with every diagnostic, its outputs on
    the host, and the float64 oracle on every row (draft tokens of the verify
    workload drawn by the oracle too), compared under the rule of
    oracle/parity.py. Returns {workload run: counts}."""
    import numpy as np
    import oracle
    from oracle.parity import parity_sample_batch, parity_verify_batch

    dev = torch.device("cuda:0")
    out = {}
    t_start = time.perf_counter()

    def sample_diag(s, x, prm, step):
        rows, V = x.shape
        d = dict(status=torch.full((rows,), -7, dtype=torch.int32, device=dev),
                 kept_count=torch.full((rows,), -7, dtype=torch.int32, device=dev),
                 threshold=torch.full((rows,), float("nan"), dtype=torch.float32, device=dev),
                 kept_mass=torch.full((rows,), float("nan"), dtype=torch.float64, device=dev),
                 probs=torch.full((rows, V), float("nan"), dtype=torch.float32, device=dev))
        tok = s.sample_rows(x, prm, step, diag=d)
        torch.cuda.synchronize()
        g = {k: t.cpu().numpy() for k, t in d.items()}
        g["token"] = tok.cpu().numpy()
        return g

    for cfg in (1, 2, 3, 5):
        w = wl.config(cfg)
        seed = wl.philox_seed(cfg)
        values = oracle.values_from_stored(w.data, w.dtype)
        with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=seed) as s:
            x = device_batch(torch, w, 1)[0]
            for run, prm in enumerate(w.runs):
                g = sample_diag(s, x, prm, run)
                t = parity_sample_batch(values, prm, seed, run, g)
                key = f"{w.name}_run{run}"
                out[key] = dict(t.as_dict(), params=prm, **t.shape())
                del g
            del x
        torch.cuda.empty_cache()

    w = wl.config(4)
    K = w.extra["K"]
    seed = wl.philox_seed(4)
    tv = oracle.values_from_stored(w.data, w.dtype)
    dv = oracle.values_from_stored(w.extra["draft"], w.dtype)
    xs = np.array([[oracle.sample_row(dv[b, j], {"temperature": 1.0}, seed, b * K + j, 1000).token
                    for j in range(K)] for b in range(w.rows)], dtype=np.int32)
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=seed) as s:
        tg = torch.from_numpy(w.data).to(dev)
        df = torch.from_numpy(w.extra["draft"]).to(dev)
        xd = torch.from_numpy(xs).to(dev)
        for run, prm in enumerate(w.runs):
            st = torch.full((w.rows,), -7, dtype=torch.int32, device=dev)
            toks, acc = s.spec_verify(tg, df, xd, prm, run, out_status=st)
            torch.cuda.synchronize()
            t = parity_verify_batch(tv, dv, xs, prm, seed, run, toks.cpu().numpy(),
                                    acc.cpu().numpy(), st.cpu().numpy())
            a = acc.float().mean().item()
            out[f"{w.name}_run{run}"] = dict(t.as_dict(), params=prm, acceptance_rate=a / K,
                                             tokens_per_verify=a + 1)

    # the same verify step at 128256 bf16 logits (the wide path), the batch
    # of its bench line, at T 1 and T 0
    nseq, K, V = 64, 4, 128256
    tgt_b, dft_b = wl.verify_batch(1040, nseq, K, V, "bf16")
    tv = oracle.values_from_stored(tgt_b.reshape(-1, V), "bf16").reshape(nseq, K + 1, V)
    dv = oracle.values_from_stored(dft_b.reshape(-1, V), "bf16").reshape(nseq, K, V)
    seed = wl.philox_seed(4)
    xs = np.array([[oracle.sample_row(dv[b, j], {"temperature": 1.0}, seed, b * K + j, 1001).token
                    for j in range(K)] for b in range(nseq)], dtype=np.int32)
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=seed) as s:
        tg = torch.from_numpy(tgt_b.view(np.int16)).to(dev).view(torch.bfloat16)
        df = torch.from_numpy(dft_b.view(np.int16)).to(dev).view(torch.bfloat16)
        xd = torch.from_numpy(xs).to(dev)
        for run, prm in enumerate(({"temperature": 1.0}, {"temperature": 0.0})):
            st = torch.full((nseq,), -7, dtype=torch.int32, device=dev)
            toks, acc = s.spec_verify(tg, df, xd, prm, run, out_status=st)
            torch.cuda.synchronize()
            t = parity_verify_batch(tv, dv, xs, prm, seed, run, toks.cpu().numpy(),
                                    acc.cpu().numpy(), st.cpu().numpy())
            a = acc.float().mean().item()
            out[f"verify64_k4_128256_bf16_run{run}"] = dict(
                t.as_dict(), params=prm, acceptance_rate=a / K, tokens_per_verify=a + 1)
    total = sum(v["out_of_band"] for v in out.values())
    return {"out_of_band_total": total, "seconds": time.perf_counter() - t_start,
            "workloads": out}


def run_extra(torch, tsr, wl, steps, warmup, only=None):
    """Rows/s and GB/s of the other workloads (same timing method); `only`: a
    substring of the workload names to run (all when None)."""
    import numpy as np
    res = {}

    def want(name):
        return only is None or only in name

    dev = torch.device("cuda:0")
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=wl.philox_seed(2)) as s:
        if want("tiny64_8192_f32"):
            w = wl.config(1)
            bufs = device_batch(torch, w, ROTATE)
            out = torch.empty(w.rows, dtype=torch.int32, device="cuda:0")
            ms = time_calls(torch, lambda i: s.sample_rows(bufs[i % ROTATE], w.runs[0], i, out=out),
                            steps, warmup)
            res["tiny64_8192_f32_chain"] = _rates(w.rows, w.rows * w.vocab * 4, ms)

        if want("batch256_32000_f32"):
            w = wl.config(2)
            bufs = device_batch(torch, w, ROTATE)
            out = torch.empty(w.rows, dtype=torch.int32, device="cuda:0")
            ms = time_calls(torch, lambda i: s.greedy_argmax(bufs[i % ROTATE], out=out), steps, warmup)
            res["batch256_32000_f32_greedy"] = _rates(w.rows, w.rows * w.vocab * 4, ms)
            for name, prm in (("pure_T1", w.runs[1]), ("minp_T0.7", w.runs[2])):
                ms = time_calls(torch, lambda i: s.sample_rows(bufs[i % ROTATE], prm, i, out=out),
                                steps, warmup)
                res[f"batch256_32000_f32_{name}"] = _rates(w.rows, w.rows * w.vocab * 4, ms)
            del bufs

        if want("verify64_k4_32000_f32"):
            w = wl.config(4)
            K = w.extra["K"]
            dev = torch.device("cuda:0")
            tg = torch.from_numpy(w.data).to(dev)
            df = torch.from_numpy(w.extra["draft"]).to(dev)
            tgs = [tg.clone() for _ in range(ROTATE)]
            dfs = [df.clone() for _ in range(ROTATE)]
            # draft tokens drawn from q by the sampler itself, as a draft model would
            xs = s.sample_rows(df.view(w.rows * K, w.vocab), {"temperature": 1.0}, 777)
            xs = xs.view(w.rows, K).contiguous()
            toks = torch.empty(w.rows, K + 1, dtype=torch.int32, device=dev)
            acc = torch.empty(w.rows, dtype=torch.int32, device=dev)
            nbytes = w.rows * (2 * K + 1) * w.vocab * 4
            for name, prm in (("T1", w.runs[0]), ("greedy", w.runs[1])):
                ms = time_calls(torch, lambda i: s.spec_verify(tgs[i % ROTATE], dfs[i % ROTATE], xs, prm,
                                                               i, out_tokens=toks, out_accepted=acc),
                                steps, warmup)
                a = acc.float().mean().item()
                r = _rates(w.rows, nbytes if prm["temperature"] else w.rows * (K + 1) * w.vocab * 4, ms)
                r.update(acceptance_rate=a / K, tokens_per_verify=a + 1,
                         tokens_per_s=w.rows * (a + 1) / (ms * 1e-3))
                res[f"verify64_k4_32000_f32_{name}"] = r
            del tgs, dfs

        if want("verify64_k4_128256_bf16"):
            # the verify step at a 128,256-id bf16 vocabulary (wider than a
            # workgroup holds two rows of: one workgroup per row, then one per
            # sequence), 64 sequences, K = 4, generated as the 32000 fp32 batch is
            nseq, K, V = 64, 4, 128256
            tgt_b, dft_b = wl.verify_batch(1040, nseq, K, V, "bf16")
            tg = torch.from_numpy(tgt_b.view(np.int16)).to(dev).view(torch.bfloat16)
            df = torch.from_numpy(dft_b.view(np.int16)).to(dev).view(torch.bfloat16)
            tgs = [tg.clone() for _ in range(ROTATE)]
            dfs = [df.clone() for _ in range(ROTATE)]
            xs = s.sample_rows(df.view(nseq * K, V), {"temperature": 1.0}, 778)
            xs = xs.view(nseq, K).contiguous()
            toks = torch.empty(nseq, K + 1, dtype=torch.int32, device=dev)
            acc = torch.empty(nseq, dtype=torch.int32, device=dev)
            for name, prm in (("T1", {"temperature": 1.0}), ("greedy", {"temperature": 0.0})):
                ms = time_calls(torch, lambda i: s.spec_verify(tgs[i % ROTATE], dfs[i % ROTATE], xs, prm,
                                                               i, out_tokens=toks, out_accepted=acc),
                                steps, warmup)
                a = acc.float().mean().item()
                rows_read = (2 * K + 1) if prm["temperature"] else (K + 1)
                r = _rates(nseq, nseq * rows_read * V * 2, ms)
                r.update(acceptance_rate=a / K, tokens_per_verify=a + 1,
                         tokens_per_s=nseq * (a + 1) / (ms * 1e-3))
                res[f"verify64_k4_128256_bf16_{name}"] = r
            del tgs, dfs, tg, df

        if want("batch256_128256_bf16_chain"):
            # constrained decoding on the headline batch: allowed-token bitmask
            # (V/8 bytes per row more) and log p~ of each draw
            w = wl.config(3)
            bufs = device_batch(torch, w, ROTATE)
            out = torch.empty(w.rows, dtype=torch.int32, device="cuda:0")
            lp = torch.empty(w.rows, dtype=torch.float32, device="cuda:0")
            ms = time_calls(torch, lambda i: s.sample_rows_masked(bufs[i % ROTATE], None, w.runs[0], i,
                                                                  out=out, logprob=lp),
                            steps, warmup)
            res["batch256_128256_bf16_chain_logprob"] = _rates(w.rows, w.rows * w.vocab * 2, ms)
            for kind in ("p=0.5", "few=40"):
                words = torch.from_numpy(wl.allowed_words(31, w.rows, w.vocab, kind).view("int32"))
                words = words.to("cuda:0")
                nbytes = w.rows * w.vocab * 2 + words.numel() * 4
                ms = time_calls(torch, lambda i: s.sample_rows_masked(bufs[i % ROTATE], words,
                                                                      w.runs[0], i, out=out,
                                                                      logprob=lp),
                                steps, warmup)
                res[f"batch256_128256_bf16_chain_mask_{kind}"] = _rates(w.rows, nbytes, ms)
            # repetition penalty r = 1.1 over a 64-token window per row
            hist = torch.from_numpy(np.random.default_rng(64).integers(0, w.vocab, (w.rows, 64))
                                    .astype(np.int32)).to("cuda:0")
            ms = time_calls(torch, lambda i: s.sample_rows_ex(bufs[i % ROTATE], w.runs[0], i,
                                                              history=hist, penalty=1.1, out=out,
                                                              logprob=lp),
                            steps, warmup)
            res["batch256_128256_bf16_chain_rep64"] = _rates(
                w.rows, w.rows * w.vocab * 2 + hist.numel() * 4, ms)
            # the same rows one id shorter, contiguous: rows start 2 bytes apart
            # from a 16-byte boundary (an odd vocabulary)
            odd = [b[:, : w.vocab - 1].contiguous() for b in bufs]
            ms = time_calls(torch, lambda i: s.sample_rows(odd[i % ROTATE], w.runs[0], i, out=out),
                            steps, warmup)
            res["batch256_128255_bf16_chain_unaligned"] = _rates(w.rows, w.rows * (w.vocab - 1) * 2, ms)
            del bufs, odd

        if want("beam64x4_128256_bf16"):
            # beam-search step: 64 groups of 4 beams over the same 256 x 128256 bf16 logits
            w = wl.config(3)
            bufs = device_batch(torch, w, ROTATE)
            bsc = torch.from_numpy(np.random.default_rng(4).normal(-5.0, 2.0, w.rows)).to("cuda:0")
            ms = time_calls(torch, lambda i: s.beam_step(bufs[i % ROTATE], bsc, 4), steps, warmup)
            res["beam64x4_128256_bf16"] = _rates(w.rows, w.rows * w.vocab * 2, ms)
            del bufs

        if want("tree64_n8_32000_f32"):
            # tree verify: 64 sequences, 8-node trees (root with two children, each
            # with two, one more level on node 3), 32000 fp32 logits per node
            w = wl.config(4)
            nseq, N, V = 64, 8, w.vocab
            rng = np.random.default_rng(8)
            tgt = torch.from_numpy(rng.normal(0, 1.5, (nseq, N, V)).astype(np.float32)).to(dev)
            dft = (tgt + torch.from_numpy(rng.normal(0, 0.7, (nseq, N, V)).astype(np.float32)).to(dev))
            parent = torch.tensor([[-1, 0, 0, 1, 1, 2, 2, 3]] * nseq, dtype=torch.int32, device=dev)
            # each node's token drawn from the draft at its parent, as a draft model would
            draws = s.sample_rows(dft.view(nseq * N, V), {"temperature": 1.0}, 555).view(nseq, N)
            toks = torch.gather(draws, 1, parent.clamp(min=0).long()).to(torch.int32).contiguous()
            tgts = [tgt.clone() for _ in range(ROTATE // 2)]
            dfts = [dft.clone() for _ in range(ROTATE // 2)]
            ms = time_calls(torch, lambda i: s.tree_verify(tgts[i % (ROTATE // 2)],
                                                           dfts[i % (ROTATE // 2)], parent, toks,
                                                           {"temperature": 1.0}, i),
                            steps, warmup)
            res["tree64_n8_32000_f32_T1"] = _rates(nseq, nseq * (N + 4) * V * 4, ms)
            del tgts, dfts, tgt, dft

        if want("batch1024_151936_bf16"):
            w = wl.config(5)
            bufs = device_batch(torch, w, 2)          # 2 x 311 MB already exceeds the 256 MB cache
            out = torch.empty(w.rows, dtype=torch.int32, device="cuda:0")
            for name, prm in (("top_p0.9", w.runs[0]), ("top_k1024", w.runs[1])):
                ms = time_calls(torch, lambda i: s.sample_rows(bufs[i % 2], prm, i, out=out),
                                max(20, steps // 4), warmup)
                res[f"batch1024_151936_bf16_{name}"] = _rates(w.rows, w.rows * w.vocab * 2, ms)
    return res


def _rates(rows, nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_call": ms, "rows_per_s": rows / (ms * 1e-3), "algorithmic_GB_s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS}


if __name__ == "__main__":
    main()
