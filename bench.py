"""Benchmark: paged and sparse MLA decode on one MI355X against the HBM / bf16-MFMA roofline.

One step = one pass of the hot path over one batch: the tile-scheduler metadata, the decode
kernel (page gather, Q.K^T, online softmax, P.V, split epilogue) and the split-KV combine, on
the long-context workload (batch 16, s_q 1, 16 heads, 65536 cached tokens each, 16384 pages
permuted over the pool; 1208.6 MB of algorithmic bytes, the largest workload).  Inputs are
seeded synthetic data resident in HBM before timing.

The same JSON line also carries every workload's decode call timed on its own: median, p10 and
p90 over calls that each follow a 512 MB read evicting L2 and the Infinity Cache, with GB/s,
TFLOPS and the fraction of the roofline that bounds it (HBM for the memory-bound shapes, bf16
MFMA for the compute-bound ones).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only K]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E datasheet
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA datasheet (2.5 PFLOP/s)
D_QK, D_V = 576, 512
HEADLINE = 4                   # the long-context workload: the most bytes per call
# what bounds each workload: the tiny one is latency only
BOUND = {1: "latency", 2: "hbm", 3: "mfma", 4: "hbm", 5: "hbm", 6: "hbm", 7: "mfma", 8: "mfma", 9: "mfma",
         10: "mfma"}
PAGED_KINDS = ("paged", "paged_fp8", "paged_v4", "paged_v4_fp4")


def paged_counts(inp):
    """Algorithmic bytes and flops of one paged decode step.

    Bytes: every visible KV row once per sequence (bf16 1152 B, or 1024 B for a 512-wide latent
    row; an fp8 record's 576 codes and its fp32 scale, 580 B; an FP4 row's 256 code bytes and
    32 scale bytes, 288 B; V lies inside K), Q, O (bf16), LSE (fp32), the used block-table
    entries, the sequence lengths and the sinks.  Flops: 2 * (d + 512) per (query row, visible
    token), d = 576 or 512."""
    L = inp.seqlens.astype(np.int64)
    b, s_q, h_q = inp.batch, inp.s_q, inp.h_q
    M = s_q * h_q
    if hasattr(inp, "kv_codes"):             # FP4 pages of 512-wide rows
        d, row_bytes = D_V, 256 + 32
    else:
        d = D_QK if inp.kcache.dtype == np.uint8 else inp.kcache.shape[-1]    # 576, or 512-wide rows
        row_bytes = 580 if inp.kcache.dtype == np.uint8 else d * 2
    kv = int(L.sum()) * row_bytes
    nblk = int(((L + 63) // 64).sum())
    sinks = 0 if getattr(inp, "sinks", None) is None else h_q * 4
    byts = kv + b * M * d * 2 + b * M * D_V * 2 + b * M * 4 + nblk * 4 + b * 4 + sinks
    vis = 0
    for s in range(s_q):
        if inp.causal:
            vis += int(np.clip(L - s_q + s + 1, 0, None).sum())
        else:
            vis += int(L.sum())
    flops = 2 * (d + D_V) * h_q * vis
    return byts, flops


def fused_counts(inp):
    """The fused decode: the V4-geometry paged counts with the output as e4m3 codes (1 B per value)
    plus one fp32 scale per row instead of bf16 O, and the norm weight and angle table read."""
    byts, flops = paged_counts(inp)
    rows = inp.batch * inp.s_q * inp.h_q
    byts += rows * (D_V + 4) - rows * D_V * 2 + D_V * 4 + inp.batch * inp.s_q * 64 * 4
    return byts, flops


def sparse_counts(inp):
    """Valid index entries read 580 B each (576 fp8 codes + the fp32 scale); plus Q, O, LSE, indices."""
    valid = int((inp.indices >= 0).sum())
    b, s_q, h_q = inp.batch, inp.s_q, inp.h_q
    byts = valid * 580 + inp.indices.size * 4 + b * s_q * h_q * (D_QK * 2 + D_V * 2 + 4)
    flops = 2 * (D_QK + D_V) * h_q * valid
    return byts, flops


CSRC = os.path.join(ROOT, "head_latent_attention_paged_amd", "csrc")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_paged_longctx_b16_L65536_hbm_traffic.txt")

# sources of what the 16-row paged decode call runs (the 16-row decode kernel, the combine,
# their shared device code and the launch code); the many-row kernels are not part of it
DEFAULT_PATH_SOURCES = ("mla_device.h", "mla_internal.h", "mla_kernels.hip")


def kernel_source_hash():
    """sha256 over the sources of the 16-row paged decode call, to tell whether a stored counter
    profile still describes the kernels being run."""
    import hashlib

    h = hashlib.sha256()
    for name in DEFAULT_PATH_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_from_profile(path=TRAFFIC_PROFILE):
    """HBM bytes per decode call from the stored rocprofv3 FETCH_SIZE / WRITE_SIZE summary,
    each counter divided by what it read for a plain copy kernel of known size.  None when
    the summary is missing or was taken on other kernel sources."""
    if not os.path.exists(path):
        return None, "no counter profile"
    kv = {}
    kernels = []
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            key, val = key.strip(), val.strip()
            if key == "kernel":
                fields = dict(x.split("=") for x in val.split()[1:])
                kernels.append((val.split()[0], float(fields["fetch_kib"]), float(fields["write_kib"])))
            else:
                kv[key] = val
    if kv.get("source_sha256") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    copy_bytes = float(kv["copy_bytes_each_way"])
    f_fetch = float(kv["copy_fetch_kib"]) * 1024 / copy_bytes
    f_write = float(kv["copy_write_kib"]) * 1024 / copy_bytes
    total = sum(fk * 1024 / f_fetch + wk * 1024 / f_write for _, fk, wk in kernels)
    return int(total), "rocprofv3 FETCH_SIZE+WRITE_SIZE of %s, scaled by copy-kernel factors %.3f / %.3f" % (
        "+".join(k for k, _, _ in kernels), f_fetch, f_write)


def copy_probe(nbytes=1 << 30, reps=5):
    """A plain copy kernel of known size (reads and writes nbytes each), for counter calibration."""
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    print("copy probe: %d bytes each way x %d" % (nbytes, reps))


class Flusher:
    """Reads a 512 MB buffer to evict L2 and the 256 MB Infinity Cache between timed calls
    (a read leaves clean lines, so the timed call pays no write-back for the flush)."""

    def __init__(self, torch, dev):
        self.buf = torch.ones(128 << 20, dtype=torch.int32, device=dev)

    def __call__(self):
        self.sink = self.buf.sum()


def time_calls(torch, fn, n, flush=None):
    """Per-call device time (ms) with events on the current stream (the one the library
    launches on); optional flush before each call, outside the events."""
    s = torch.cuda.current_stream()
    times = []
    for _ in range(n):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    return np.array(times)


def setup_paged(torch, mla, inp, dev):
    """(step, decode) for a paged workload: step = metadata + decode call; decode = the call
    with the metadata computed once."""
    from tests.helpers import dev_bf16, dev_i32, dev_u8

    q = dev_bf16(inp.q, dev)
    fp4 = hasattr(inp, "kv_codes")
    if fp4:
        kc, ks = dev_u8(inp.kv_codes, dev), dev_u8(inp.kv_scales, dev)
    elif inp.kcache.dtype == np.uint8:
        kc = dev_u8(inp.kcache, dev)
    elif inp.kcache.shape[-1] == D_V:        # 512-wide latent rows (K and V)
        kc = dev_bf16(inp.kcache.reshape(inp.kcache.shape[0], 64, D_V), dev)
    else:
        kc = dev_bf16(inp.kcache, dev)
    sk = None if getattr(inp, "sinks", None) is None else torch.from_numpy(inp.sinks).to(dev)
    bt, sl = dev_i32(inp.block_table, dev), dev_i32(inp.seqlens, dev)
    P = mla.num_parts(inp.h_q, inp.s_q)
    out = torch.empty((inp.batch, inp.s_q, inp.h_q, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    ws = torch.zeros((max(mla.workspace_size(inp.batch, inp.s_q, inp.h_q, P), 256),), dtype=torch.uint8, device=dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, P)

    def call(m):
        if fp4:
            mla.decode_paged_fp4(q, kc, ks, bt, sl, m, inp.softmax_scale, inp.causal, out=out, lse=lse,
                                 workspace=ws, sinks=sk)
        else:
            mla.decode_paged(q, kc, bt, sl, m, inp.softmax_scale, inp.causal, out=out, lse=lse, workspace=ws,
                             sinks=sk)

    def decode():
        call(meta)

    def metadata():
        return mla.get_metadata(sl, inp.h_q, inp.s_q, P)

    return call, decode, metadata


def setup_sparse(torch, mla, inp, dev):
    from tests.helpers import dev_bf16, dev_i32, dev_u8

    q, kv, idx = dev_bf16(inp.q, dev), dev_u8(inp.kv, dev), dev_i32(inp.indices, dev)
    out = torch.empty((inp.batch, inp.s_q, inp.h_q, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    ws = torch.zeros((max(mla.workspace_size_sparse(inp.batch, inp.s_q, inp.h_q, inp.topk), 256),),
                     dtype=torch.uint8, device=dev)

    def decode():
        mla.decode_sparse(q, kv, idx, inp.softmax_scale, 0, out=out, lse=lse, workspace=ws)

    return decode


def setup_prefill(torch, mla, inp, dev):
    """A prompt chunk (batch 1 of the generator) through mla_sparse_prefill."""
    from tests.helpers import dev_bf16, dev_i32, dev_u8

    q, kv, idx = dev_bf16(inp.q[0], dev), dev_u8(inp.kv, dev), dev_i32(inp.indices[0], dev)
    out = torch.empty((inp.s_q, inp.h_q, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    ws = torch.zeros((max(mla.workspace_size_sparse(1, inp.s_q, inp.h_q, inp.topk), 256),),
                     dtype=torch.uint8, device=dev)

    def prefill():
        mla.sparse_prefill(q, kv, idx, inp.softmax_scale, 0, out=out, lse=lse, workspace=ws)

    return prefill


def setup_fused(torch, mla, inp, dev):
    """The fused decode (mla_decode_fused) over bf16 pages, metadata computed once."""
    from tests.helpers import dev_bf16, dev_i32

    q = dev_bf16(inp.q, dev)
    kc = dev_bf16(inp.kcache.reshape(inp.kcache.shape[0], 64, D_V), dev)
    bt, sl = dev_i32(inp.block_table, dev), dev_i32(inp.seqlens, dev)
    sk = None if inp.sinks is None else torch.from_numpy(inp.sinks).to(dev)
    w = torch.from_numpy(inp.fused.norm_weight).to(dev)
    cs = torch.from_numpy(np.ascontiguousarray(inp.fused.rope_cs)).to(dev)
    P = mla.num_parts(inp.h_q, inp.s_q)
    out = torch.empty((inp.batch, inp.s_q, inp.h_q, D_V), dtype=torch.uint8, device=dev)
    osc = torch.empty((inp.batch, inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    lse = torch.empty((inp.batch, inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    ws = torch.zeros((max(mla.workspace_size(inp.batch, inp.s_q, inp.h_q, P), 256),), dtype=torch.uint8, device=dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, P)

    def fused():
        mla.decode_fused(q, kc, bt, sl, meta, w, inp.fused.norm_eps, cs, inp.softmax_scale, inp.causal, sinks=sk,
                         out=out, out_scale=osc, lse=lse, workspace=ws)

    return fused


def setup_call(torch, mla, k, inp, dev):
    """Workload k's decode call (metadata computed once for paged workloads) and its counts."""
    from mla_inputs import CONFIGS

    kind = CONFIGS[k]["kind"]
    if kind == "fused_v4":
        return setup_fused(torch, mla, inp, dev), fused_counts(inp)
    if kind in PAGED_KINDS:
        _, fn, _ = setup_paged(torch, mla, inp, dev)
        return fn, paged_counts(inp)
    if kind == "sparse_prefill":
        return setup_prefill(torch, mla, inp, dev), sparse_counts(inp)
    return setup_sparse(torch, mla, inp, dev), sparse_counts(inp)


# the kernels each workload's call runs (kernel-trace names), for reading the profiles
KERNELS = {
    1: "mla_decode_m16_kernel + mla_combine_kernel",
    2: "mla_decode_m16_kernel + mla_combine_kernel",
    3: "mla_decode_wide_kernel<0, true, 576> + mla_combine_kernel",
    4: "mla_decode_m16_kernel + mla_combine_kernel",
    5: "mla_decode_rows_kernel<1, false, 576> (one split)",
    6: "mla_decode_m16_fp8_kernel + mla_combine_kernel",
    7: "mla_decode_wide_kernel<0, true, 512> + mla_combine_kernel",
    8: "mla_decode_wide_kernel<3, true, 512> + mla_combine_kernel",
    9: "mla_decode_rows_kernel<1, true, 576> (one split)",
    10: "mla_decode_wide_kernel<0, true, 512, true> + mla_combine_fused_kernel",
}


def workload_entry(k, name, t_ms, byts, flops):
    us = float(np.median(t_ms)) * 1e3
    gbs = byts / (us * 1e-6) / 1e9
    tfl = flops / (us * 1e-6) / 1e12
    e = {"workload": name, "kernels": KERNELS[k], "calls": int(len(t_ms)),
         "us_median": round(us, 2), "us_p10": round(float(np.percentile(t_ms, 10)) * 1e3, 2),
         "us_p90": round(float(np.percentile(t_ms, 90)) * 1e3, 2),
         "GBps": round(gbs, 1), "TFLOPS": round(tfl, 1),
         "algorithmic_bytes": byts, "algorithmic_flops": flops, "bound": BOUND[k]}
    if BOUND[k] == "hbm":
        e.update(peak=HBM_PEAK_GBS, peak_unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    elif BOUND[k] == "mfma":
        e.update(peak=BF16_PEAK_TFLOPS, peak_unit="TFLOP/s", frac=round(tfl / BF16_PEAK_TFLOPS, 4))
    return e


def cpu_baseline(inp, kind, counts_fn, min_s=10.0, max_s=30.0):
    """The float64 oracle on a bounded sample of the same workload, scaled to GB/s: whole
    sequences (paged) or query tokens (sparse) in order, repeating the workload when one pass
    takes under min_s, stopping at max_s."""
    from oracle import paged_decode, sparse_decode

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    total_bytes, _ = counts_fn(inp)
    if kind == "paged":
        units = list(range(inp.batch))
        what = "sequences"

        def run(b):
            paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, inp.causal, batches=[b])
    else:
        units = [(b, s) for b in range(inp.batch) for s in range(inp.s_q)]
        what = "query tokens"

        def run(bs):
            sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale, sets=[bs])
    per_unit = total_bytes / len(units)
    t0 = time.perf_counter()
    done = 0
    while True:
        for u in units:
            run(u)
            done += 1
            dt = time.perf_counter() - t0
            if dt > max_s:
                break
        if dt > min_s:
            break
    byts = per_unit * done
    sample = "%d %s of the %d in the workload (%.2f passes), in order" % (done, what, len(units), done / len(units))
    return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


def run_calls(k, n):
    """Workload k's decode call n times with nothing else timed around it (profiler passes)."""
    import torch

    import head_latent_attention_paged_amd as mla
    from mla_inputs import make_config

    dev = torch.device("cuda:0")
    inp = make_config(k, poison=False)
    fn, _ = setup_call(torch, mla, k, inp, dev)
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    print("ran %d decode calls of workload %d" % (n, k), flush=True)


def time_steps(torch, inp, call, metadata, steps, warmup):
    """The timed steps: metadata + decode call, K times back to back.  Wall clock around the
    whole loop (synchronised on both sides); HIP events on the launch stream around each step's
    decode call, for the per-launch time of the decode kernel and its combine."""
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        call(metadata())
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        m = metadata()
        ev[i][0].record(s)
        call(m)
        ev[i][1].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.array([a.elapsed_time(b) for a, b in ev])
    return wall, per_call


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--calls", type=int, default=30, help="flushed calls timed per workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--only", type=int, default=0, metavar="K",
                    help="time only workload K (its flushed calls; the steps too when K is the headline)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB copy kernel (HBM counter calibration) and exit")
    ap.add_argument("--calls-of", type=int, default=0, metavar="K",
                    help="only run workload K's decode call --steps times, untimed (for counter passes), and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.calls_of:
        run_calls(args.calls_of, args.steps)
        return

    import torch

    import head_latent_attention_paged_amd as mla
    from mla_inputs import CONFIGS, make_config

    dev = torch.device("cuda:0")
    res = {
        "metric": "paged MLA decode us/call, achieved HBM GB/s and TFLOPS vs MI355X roofline",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
    }
    head = None
    if args.only in (0, HEADLINE):
        print("[bench] workload %d (headline): generating" % HEADLINE, file=sys.stderr, flush=True)
        head = make_config(HEADLINE, poison=False)
        byts, flops = paged_counts(head)
        call, _, metadata = setup_paged(torch, mla, head, dev)
        wall, per_call = time_steps(torch, head, call, metadata, args.steps, args.warmup)
        ms_per_step = wall * 1e3 / args.steps
        dec_ms = float(per_call.mean())
        achieved = byts / (dec_ms * 1e-3) / 1e9
        traffic, traffic_note = traffic_from_profile()
        res.update({
            "value": round(byts / (ms_per_step * 1e-3) / 1e9, 2),
            "ms_per_step": round(ms_per_step, 5),
            "config": {"workload": CONFIGS[HEADLINE]["name"], "batch": head.batch, "s_q": head.s_q,
                       "h_q": head.h_q, "seq_len": int(head.seqlens[0]), "page": 64, "pages": head.num_pages,
                       "kv_dtype": "bf16", "parallelism": "single GPU"},
            "us_per_step": round(ms_per_step * 1e3, 2),
            "tflops_per_step": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
            "algorithmic_bytes": byts,
            "algorithmic_flops": flops,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "traffic_note": traffic_note, "algorithmic_bytes_per_launch": byts,
                         "kernel": "mla_decode_paged call (%s)" % KERNELS[HEADLINE],
                         "us_per_launch": round(dec_ms * 1e3, 2),
                         "us_per_launch_p10": round(float(np.percentile(per_call, 10)) * 1e3, 2),
                         "us_per_launch_p90": round(float(np.percentile(per_call, 90)) * 1e3, 2),
                         "timing": "HIP events on the launch stream around each timed step's decode call"},
        })

    flush = Flusher(torch, dev)
    work = {}
    for k in ([args.only] if args.only else sorted(CONFIGS)):
        print("[bench] workload %d: %s" % (k, CONFIGS[k]["name"]), file=sys.stderr, flush=True)
        ik = head if k == HEADLINE and head is not None else make_config(k, poison=False)
        fn, (b_k, f_k) = setup_call(torch, mla, k, ik, dev)
        for _ in range(3):
            fn()
        t = time_calls(torch, fn, args.calls * (4 if k == 1 else 1), flush=flush)
        work["config%d" % k] = workload_entry(k, CONFIGS[k]["name"], t, b_k, f_k)
        del fn
        if ik is not head:
            del ik
        torch.cuda.empty_cache()
    res["workloads_flushed"] = work

    if head is not None and not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(head, "paged", paged_counts)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
