#!/usr/bin/env python3
"""Throughput of quantized-KV decode attention on one MI355X.

One step = one pass of the whole path over one batch: kvq_quant_append of one new
token per sequence (quantize + pack), then kvq_decode_attn for every query head over
the whole cache.  Default workload: batch 64, 32 query / 8 KV heads, head_dim 128,
16384-token Student-t3 context, 4 BF16 sink tokens, INT2 keys, INT4 values, one appended
token per step (the largest of the five workloads; the metric is an HBM-bandwidth figure
and the smaller workloads fit in the 256 MB last-level cache).

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value           KV tokens scored per second (batch * positions attended, per step)
  roofline        decode kernel: algorithmic bytes per launch / average launch duration
                  (HIP events on the launch stream, in a pass of as many steps after the
                  timed ones, so no event sits between the timed steps' kernels), against
                  8 TB/s HBM
  clock_settle_ms decode-only calls run before the warm-up steps, whatever --warmup says,
                  until at least 40 ms of GPU work have passed (the GPU's clocks settle)
  stream_read     the practical HBM read ceiling measured in the same process, and the
                  decode kernel's rate as a fraction of it
  append          the GPU append kernel's time per call and per appended token*unit
  cpu_baseline    the CPU oracle timed on a bounded sample of the same workload (all host
                  threads and one), append+decode, quantize-pack and decode rates apart
Inputs are resident in HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..8]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
# HBM traffic records (rocprofv3 counters), per workload
TRAFFIC_FILES = {5: "decode_b64_t16k_traffic.txt", 3: "decode_b16_t32k_lloyd4_traffic.txt",
                 4: "decode_b4_t128k_pruned_traffic.txt"}
# the decode kernels' sources (kernel templates and the INT4-value instantiation the counters see)
DECODE_SRC = [os.path.join(ROOT, "bit_kv_cache_kvq_amd", "csrc", f) for f in ("kvq_decode_impl.h", "kvq_decode.hip")]


def traffic_file(wid):
    return os.path.join(ROOT, "profiles", TRAFFIC_FILES[wid]) if wid in TRAFFIC_FILES else None


def decode_source_sha256():
    h = hashlib.sha256()
    for f in DECODE_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes_unit(w, length, mask, bf16=True):
    """Algorithmic HBM bytes one decode reads for one (sequence, KV head): the code words,
    scale/zero words and channel-0 / norm halves of the kept key rows, every value word and
    value scale/zero word of the quantised positions, and (bf16=True) the BF16 rows of the
    sinks and of the recent window, which the query-prep kernel reads rather than the main
    decode kernel.  mask: kept 16-channel groups (bit p); under bucket-relative RoPE a list,
    one mask per bucket of w.rope_bucket positions."""
    d = w.head_dim
    P = d // 16

    def per_token(m):
        kept = [(m >> p) & 1 for p in range(P)]
        kbits = 2 if w.k_format == 0 else 4
        k_tok = sum(kept) * 16 * kbits // 8
        if w.k_format == 2:
            k_tok += 2
        else:
            k_tok += 4 * sum(1 for g in range(d // 32) if kept[2 * g] or kept[2 * g + 1])
            if w.k_ch0_bf16 and kept[0]:
                k_tok += 2
        v_tok = {1: d // 4 + 4, 2: d // 2 + 4}.get(w.v_format, d // 2 + 4 * (d // 32))
        return k_tok + v_tok

    ns = min(w.n_sink, length)
    nr = max(0, min(w.n_recent, length - ns))  # recent positions still in BF16
    q0, q1 = ns, length - nr  # quantised positions
    if isinstance(mask, (list, tuple)):
        bw = w.rope_bucket
        quant = sum(max(0, min(q1, (b + 1) * bw) - max(q0, b * bw)) * per_token(m) for b, m in enumerate(mask))
    else:
        quant = (q1 - q0) * per_token(mask)
    return quant + ((ns + nr) * d * 2 * 2 if bf16 else 0)


def traffic_record(wid):
    """HBM bytes per decode launch of workload wid measured with rocprofv3 counters, if the
    counters were taken on the current decode source (sha256 recorded next to the numbers)."""
    path = traffic_file(wid)
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = decode_source_sha256()
    if kv.get("decode_source_sha256") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_per_dispatch(path, want):
    """Per-dispatch totals (summed over dimensions) of the one counter in a rocprofv3
    --pmc CSV, for dispatches whose kernel name satisfies want(name)."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if want(r["Kernel_Name"]):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{path}: no matching dispatch")
    return list(per.values())


def write_traffic(dec_fetch, dec_write, copy_fetch, copy_write, out_path, wid, copy_bytes=1 << 30):
    """Reduce FETCH_SIZE / WRITE_SIZE counter runs (KiB per dispatch) of the decode kernel
    and of the --copy-probe copy (copy_bytes read and written per dispatch) to HBM bytes per
    decode launch: each counter is scaled by what it reads for the copy of known size."""
    is_dec = lambda n: "decode_kernel" in n
    is_copy = lambda n: "copy" in n.lower() and "fill" not in n.lower()
    f = _counter_per_dispatch(dec_fetch, is_dec)
    wr = _counter_per_dispatch(dec_write, is_dec)
    cf = _counter_per_dispatch(copy_fetch, is_copy)
    cw = _counter_per_dispatch(copy_write, is_copy)
    fetch_kib, write_kib = sum(f) / len(f), sum(wr) / len(wr)
    cf_kib, cw_kib = sum(cf) / len(cf), sum(cw) / len(cw)
    ff, wf = copy_bytes / (cf_kib * 1024), copy_bytes / (cw_kib * 1024)
    hbm = fetch_kib * 1024 * ff + write_kib * 1024 * wf
    sha = decode_source_sha256()
    lines = [
        "# HBM traffic of one decode_kernel launch, from rocprofv3 FETCH_SIZE and WRITE_SIZE counters",
        "# (KiB per dispatch, each counter in its own run), scaled by the same counters on a copy of",
        f"# {copy_bytes} bytes (python bench.py --copy-probe).  Valid only for the decode sources",
        "# (kvq_decode_impl.h, then kvq_decode.hip) whose sha256 is recorded below: bench.py ignores",
        "# this file once the kernel changes.",
        "# commands (from /tmp with TMPDIR=/tmp; each counter in a run of its own):",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex decode_kernel --output-format csv -d F -o decF"
        f" -- python3 <repo>/bench.py --workload {wid} --steps 4 --warmup 1 --no-cpu-baseline --no-read-probe",
        f"#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex decode_kernel --output-format csv -d W -o decW"
        f" -- python3 <repo>/bench.py --workload {wid} --steps 4 --warmup 1 --no-cpu-baseline --no-read-probe",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d CF -o cpyF -- python3 <repo>/bench.py --copy-probe",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d CW -o cpyW -- python3 <repo>/bench.py --copy-probe",
        f"#   python3 bench.py --workload {wid} --traffic-csv <decF csv> <decW csv> <cpyF csv> <cpyW csv>",
        f"decode_source_sha256: {sha}",
        f"decode_dispatches: {len(f)} fetch, {len(wr)} write",
        f"fetch_kib_per_launch: {fetch_kib:.1f}",
        f"write_kib_per_launch: {write_kib:.1f}",
        f"copy_fetch_kib: {cf_kib:.1f}",
        f"copy_write_kib: {cw_kib:.1f}",
        f"fetch_scale: {ff:.4f}",
        f"write_scale: {wf:.4f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
    ]
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, length, budget_s):
    """The oracle (plain C, fp64 attention) on a bounded sample of the same workload: a few
    sequences at the bench's context length, timed over append + decode steps with every
    host thread, the quantize-pack of the sample's prefill and its decode calls apart, then
    one thread on a smaller sample."""
    import numpy as np

    import oracle
    from bit_kv_cache_kvq_amd import synth

    oracle.lib()
    threads = oracle.num_threads()
    H = w.n_kv_heads
    nseq = max(1, math.ceil(threads / H))

    def new_cache(n):
        geo = oracle.Geometry(batch=n, n_kv_heads=H, head_dim=w.head_dim, capacity=w.capacity(1280),
                              n_sink=w.n_sink, k_format=w.k_format, k_hadamard=w.k_hadamard,
                              k_ch0_bf16=w.k_ch0_bf16, v_format=w.v_format, v_clip=w.v_clip,
                              n_recent=w.n_recent, rope_bucket=w.rope_bucket)
        return oracle.OracleCache(geo, rope_table=synth.rope_table(w, geo.capacity),
                                  qjl_signs=synth.qjl_signs(w.head_dim) if w.v_format == 2 else None)

    def run(n, prefill_len, budget, max_steps):
        oc = new_cache(n)
        k, v = synth.prefill(w, device="cpu", context=prefill_len, batch=n)
        kf = k.float().numpy().reshape(n * H, prefill_len, w.head_dim)
        vf = v.float().numpy().reshape(n * H, prefill_len, w.head_dim)
        del k, v
        t0 = time.perf_counter()
        oc.append(kf, vf)
        pack_s = time.perf_counter() - t0
        del kf, vf
        steps, tokens, t_used, dec_s, dec_tokens = 0, 0, 0.0, 0.0, 0
        while t_used < budget and steps < max_steps:
            q = synth.query(w, steps, device="cpu", batch=n).float().numpy().reshape(n * H, w.group, w.head_dim)
            if w.steps:
                kn, vn = synth.append_tokens(w, steps, device="cpu", batch=n)
                kn = kn.float().numpy().reshape(n * H, 1, w.head_dim)
                vn = vn.float().numpy().reshape(n * H, 1, w.head_dim)
            t0 = time.perf_counter()
            if w.steps:
                oc.append(kn, vn)
            t1 = time.perf_counter()
            oc.decode(q, w.sm_scale, w.keep_groups)
            t2 = time.perf_counter()
            t_used += t2 - t0
            dec_s += t2 - t1
            tokens += n * oc.len
            dec_tokens += n * oc.len
            steps += 1
        return {"tokens_per_s": tokens / t_used, "quantize_pack_token_units_per_s": n * H * prefill_len / pack_s,
                "decode_tokens_per_s": dec_tokens / dec_s, "steps": steps, "seconds": t_used + pack_s,
                "positions": oc.len, "sequences": n}

    prefill_len = length - (1 if w.steps else 0)
    full = run(nseq, prefill_len, budget_s, 1024)
    oracle.set_num_threads(1)
    try:
        one = run(1, min(prefill_len, 4096), budget_s / 4, 64)
    finally:
        oracle.set_num_threads(threads)
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"value": full["tokens_per_s"], "unit": "tokens/s", "cores": min(threads, nseq * H), "kind": "oracle",
            "sample": f"{nseq} of {w.batch} sequences x {H} KV heads at ~{full['positions']} positions, "
                      f"{full['steps']} append+decode steps, {full['seconds']:.1f} s of oracle time (prefill "
                      f"quantize-pack included)",
            "host_cpus": nproc, "cpu_model": _cpu_model(), "omp_threads": threads,
            "quantize_pack_token_units_per_s": full["quantize_pack_token_units_per_s"],
            "decode_tokens_per_s": full["decode_tokens_per_s"],
            "single_thread": {"tokens_per_s": one["tokens_per_s"],
                              "quantize_pack_token_units_per_s": one["quantize_pack_token_units_per_s"],
                              "decode_tokens_per_s": one["decode_tokens_per_s"],
                              "sample": f"1 sequence x {H} KV heads at ~{one['positions']} positions, "
                                        f"{one['steps']} steps, {one['seconds']:.1f} s"}}


def read_probe(B, torch, dev, nbytes=4 << 30):
    """Practical HBM read ceiling (GB/s): the library's streaming-read probe over nbytes, best
    of three grid sizes, 5 timed passes each after 2 untimed ones."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    props = torch.cuda.get_device_properties(dev)
    best, rows = 0.0, []
    for blocks in (props.multi_processor_count * 12, props.multi_processor_count * 24,
                   props.multi_processor_count * 48):
        o = torch.empty(blocks, dtype=torch.int32, device=dev)
        for _ in range(2):
            B.probe_stream_read(buf, o, blocks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            B.probe_stream_read(buf, o, blocks)
        e1.record()
        torch.cuda.synchronize()
        gbps = 5 * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9
        rows.append((blocks, gbps))
        best = max(best, gbps)
    del buf
    torch.cuda.empty_cache()
    return best, rows


def settle_clocks(fn, torch, min_ms=40.0, batch=16):
    """Run fn() (a decode call) in batches until at least min_ms of GPU work has passed;
    returns the milliseconds spent."""
    spent = 0.0
    while spent < min_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(batch):
            fn()
        e1.record()
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
    return spent


def trace_summary(path: str, last: int) -> None:
    """Per-kernel durations (us) of this library's kernels in a rocprofv3 kernel-trace CSV, in
    dispatch order: count, mean over all dispatches, mean over the last `last`."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if "kvq::" not in name:
            continue
        short = name.split("(anonymous namespace)::")[-1].split("(")[0]
        per.setdefault(short, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    print("| kernel | dispatches | mean us (all) | mean us (last %d) |" % last)
    print("|---|---|---|---|")
    for k, v in sorted(per.items()):
        v.sort()
        d = [(e - b) / 1e3 for b, e in v]
        tail = d[-last:]
        print(f"| `{k}` | {len(d)} | {sum(d) / len(d):.1f} | {sum(tail) / len(tail):.1f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true", help="skip the in-process HBM read-ceiling probe")
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="GPU milliseconds of decode-only calls before the warm-up steps (clock settle)")
    ap.add_argument("--replicas", type=int, default=128,
                    help="workloads 1-2: caches rotated for the cold-HBM decode time (the last-level cache "
                         "holds 256 MB)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only time the streaming-read probe over 4 GiB (practical HBM read ceiling)")
    ap.add_argument("--traffic-csv", nargs=4, metavar=("DEC_FETCH", "DEC_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="reduce rocprofv3 counter CSVs to the decode kernel's HBM bytes per launch, "
                         "write the traffic record and exit (no GPU use)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "LAST"),
                    help="average duration of this library's kernels in a rocprofv3 kernel-trace CSV, "
                         "over all dispatches and over the last LAST of each (no GPU use)")
    args = ap.parse_args()
    if args.traffic_csv:
        if traffic_file(args.workload) is None:
            raise SystemExit(f"no traffic record is kept for workload {args.workload}")
        write_traffic(*args.traffic_csv, out_path=traffic_file(args.workload), wid=args.workload)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary[0], int(args.trace_summary[1]))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs the decode path on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); multi-GPU sharding is design-only, see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_kv_cache_kvq_amd import binding as B
    from bit_kv_cache_kvq_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 5 copies of 1073741824 bytes")
        return
    if args.read_probe:
        best, rows = read_probe(B, torch, dev)
        for blocks, gbps in rows:
            log(f"read probe: {blocks} one-wave workgroups, {gbps:.0f} GB/s")
        print(json.dumps({"read_probe_GBps": best, "bytes": 4 << 30, "frac_of_8TBps": best / HBM_PEAK_GBPS}))
        return
    w = synth.WORKLOADS[args.workload]
    # appends: warm-up, the timed steps, then as many steps again for the kernel-event pass
    appends = args.warmup + 2 * args.steps if w.steps else 0
    cap = w.capacity(appends)
    c = B.Cache(w.batch, w.n_kv_heads, w.head_dim, cap, n_sink=w.n_sink, k_format=w.k_format,
                k_hadamard=w.k_hadamard, k_ch0_bf16=w.k_ch0_bf16, device=dev, v_format=w.v_format,
                v_clip=w.v_clip, n_recent=w.n_recent, rope_bucket=w.rope_bucket, rope_table=synth.rope_table(w, cap),
                qjl_signs=synth.qjl_signs(w.head_dim) if w.v_format == 2 else None)
    log(f"workload {w.name}: capacity {cap}, building cache ...")
    k, v = synth.prefill(w, device=dev)
    c.append(k, v)
    torch.cuda.synchronize()
    del k, v
    torch.cuda.empty_cache()
    nsteps = args.warmup + 2 * args.steps
    queries = [synth.query(w, i, device=dev) for i in range(nsteps)]
    news = [synth.append_tokens(w, i, device=dev) for i in range(nsteps)] if w.steps else []
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    mask = torch.zeros(w.units * c.rope_buckets, dtype=torch.uint8, device=dev)
    c.workspace(w.n_q_heads)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i, ev=None):
        if w.steps:
            if ev is not None:
                ev[4].record(stream)
            c.append(*news[i])
            if ev is not None:
                ev[5].record(stream)
        if ev is not None:
            # call events around kvq_decode_attn; kernel events (recorded by the library on
            # the same stream) around its main decode kernel alone
            B.set_decode_events(ev[2], ev[3])
            ev[0].record(stream)
        c.decode(queries[i], w.sm_scale, w.keep_groups, out=out, mask_out=mask)
        if ev is not None:
            ev[1].record(stream)

    # clock settle: decode-only calls until at least --settle-ms of GPU work (the clocks take
    # ~35 ms of load to settle), then the warm-up steps --warmup asks for
    settle_ms = settle_clocks(lambda: c.decode(queries[0], w.sm_scale, w.keep_groups, out=out, mask_out=mask),
                              torch, args.settle_ms) if args.settle_ms > 0 else 0.0
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed steps: nothing but the job on the stream (no events between its kernels)
    lens = []
    t0 = time.perf_counter()
    for j in range(args.steps):
        step(args.warmup + j)
        lens.append(c.len)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    # then as many steps again with HIP events around each decode call and (recorded by the
    # library on the same stream) around its main decode kernel alone: the kernel's duration
    # for the roofline.  Positions grow by one per step, so this pass is ~0.4 % longer.
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(6)) for _ in range(args.steps)]
    for e in evs:  # torch creates an event's handle at its first record
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    lens_ev = []
    for j in range(args.steps):
        step(args.warmup + args.steps + j, evs[j])
        lens_ev.append(c.len)
    torch.cuda.synchronize()
    B.set_decode_events()
    call_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[2].elapsed_time(e[3]) for e in evs]
    call_avg_s = sum(call_ms) / len(call_ms) / 1e3
    dec_avg_s = sum(dec_ms) / len(dec_ms) / 1e3
    app_avg_us = sum(e[4].elapsed_time(e[5]) for e in evs) / len(evs) * 1e3 if w.steps else None
    full = (1 << (w.head_dim // 16)) - 1
    if w.rope_bucket:
        masks = mask.view(w.units, -1).cpu().tolist() if w.keep_groups else [[full] * c.rope_buckets] * w.units
    else:
        masks = mask.cpu().tolist() if w.keep_groups else [full] * w.units
    bytes_per = [sum(decode_bytes_unit(w, L, m) for m in masks) for L in lens]
    # algorithmic bytes of the launches the events timed
    bytes_ev = [sum(decode_bytes_unit(w, L, m, bf16=False) for m in masks) for L in lens_ev]
    avg_bytes = sum(bytes_ev) / len(bytes_ev)
    tokens = sum(w.batch * L for L in lens)
    value = tokens / elapsed
    eff_gbps = sum(bytes_per) / elapsed / 1e9
    achieved = avg_bytes / dec_avg_s / 1e9
    traffic = traffic_record(args.workload)
    log(f"decode kernel avg {dec_avg_s * 1e6:.1f} us ({call_avg_s * 1e6:.1f} us for the whole call), "
        f"{avg_bytes / 1e9:.4f} GB/launch, {achieved:.0f} GB/s; step {elapsed / args.steps * 1e3:.3f} ms; "
        f"waves {c.splits(w.n_q_heads)}; clock settle {settle_ms:.0f} ms")

    cold = None
    if args.workload in (1, 2) and args.replicas > 1:
        # a cache of a few MB stays in the 256 MB last-level cache between calls: rotate over
        # replicas (same contents, other addresses) so every decode reads from HBM
        reps = [c]
        k1, v1 = synth.prefill(w, device=dev)
        for _ in range(args.replicas - 1):
            r = B.Cache(w.batch, w.n_kv_heads, w.head_dim, cap, n_sink=w.n_sink, k_format=w.k_format,
                        k_hadamard=w.k_hadamard, k_ch0_bf16=w.k_ch0_bf16, device=dev, v_format=w.v_format,
                        v_clip=w.v_clip, n_recent=w.n_recent)
            r.append(k1, v1)
            r.workspace(w.n_q_heads)
            reps.append(r)
        del k1, v1
        q0 = queries[0]
        for r in reps * 2:
            r.decode(q0, w.sm_scale, w.keep_groups, out=out, mask_out=mask)
        torch.cuda.synchronize()
        ce = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in reps]
        for e in ce:
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        for r, e in zip(reps, ce):
            B.set_decode_events(e[0], e[1])
            r.decode(q0, w.sm_scale, w.keep_groups, out=out, mask_out=mask)
        torch.cuda.synchronize()
        B.set_decode_events()
        cold_us = sum(e[0].elapsed_time(e[1]) for e in ce) / len(ce) * 1e3
        t2 = time.perf_counter()
        for r in reps:
            r.decode(q0, w.sm_scale, w.keep_groups, out=out, mask_out=mask)
        torch.cuda.synchronize()
        cold_call_us = (time.perf_counter() - t2) / len(reps) * 1e6
        cold_bytes = sum(decode_bytes_unit(w, c.len, m, bf16=False) for m in masks)
        cold = {"replicas": len(reps), "replica_bytes": sum(int(t.numel()) for t in c.buffers.values()),
                "decode_kernel_us": cold_us, "decode_call_us": cold_call_us,
                "hot_decode_kernel_us": dec_avg_s * 1e6, "kernel_GBps": cold_bytes / (cold_us * 1e-6) / 1e9}
        log(f"cold HBM ({len(reps)} replicas): decode kernel {cold_us:.1f} us, call {cold_call_us:.1f} us; "
            f"hot {dec_avg_s * 1e6:.1f} us")
        del reps

    stream_read = None
    if not args.no_read_probe:
        best, _ = read_probe(B, torch, dev)
        stream_read = {"GBps": best, "frac_of_8TBps": best / HBM_PEAK_GBPS,
                       "decode_kernel_frac_of_ceiling": achieved / best}
        log(f"read probe {best:.0f} GB/s: decode kernel at {achieved / best * 100:.1f} % of it")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, lens[-1], args.cpu_budget)

    res = {
        "metric": "KV tokens scored/sec and effective HBM GB/s (% of peak), 1 GPU",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8/f16/f32",
        "data": "synthetic (seeded Student-t3 keys/values, N(0,1) queries)" if w.dist == "t3"
                else "synthetic (seeded N(0,1) keys/values/queries)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "context": w.context, "positions_attended_last_step": lens[-1],
                   "key_format": ["asym_int2", "asym_int4", "wht_lloyd4"][w.k_format],
                   "value_format": {1: "asym_int2_token_clip%.2f" % w.v_clip, 2: "kqv_wht_lloyd3_qjl1"}.get(
                       w.v_format, "asym_int4_g32"),
                   "channel0_bf16": bool(w.k_ch0_bf16), "sink_tokens": w.n_sink, "recent_bf16_tokens": w.n_recent,
                   "rope_bucket": w.rope_bucket,
                   "keep_groups": w.keep_groups, "appends_per_step": 1 if w.steps else 0,
                   "parallelism": "single GPU"},
        "effective_GBps": eff_gbps,
        "effective_frac_of_hbm_peak": eff_gbps / HBM_PEAK_GBPS,
        "decode_algorithmic_bytes_per_launch": avg_bytes,
        "decode_kernel_us": dec_avg_s * 1e6,
        "decode_call_us": call_avg_s * 1e6,
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "clock_settle_ms": settle_ms,
        "stream_read": stream_read,
        # kvq_quant_append of one token per sequence, HIP events around the call (its kernels)
        "append": None if app_avg_us is None else {"us_per_call": app_avg_us, "tokens_per_unit_per_call": 1,
                                                   "units": w.units,
                                                   "ns_per_token_unit": app_avg_us * 1e3 / w.units},
        "cold_hbm": cold,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
