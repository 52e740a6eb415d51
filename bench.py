"""Benchmark of the MFA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the measured path over one batch of synthetic input
already resident in HBM:
  * attention workloads (default ``attn_bf16_4k``: batch 32, 64 query heads
    over one shared bf16 K/V head, 4096 positions): one ``mfa_decode_attn``
    call, i.e. scores, online softmax, PV and the split merge;
  * ``*_paged`` attention workloads: the same keys in a paged cache (64-row
    pages in a shuffled order), one ``mfa_decode_attn_paged`` call;
  * ``*_mtpN`` attention workloads (N = 2, 3, 4): N new query tokens per
    sequence (causal among them), one ``mfa_decode_attn_mt`` call; tokens/s
    counts all of them; ``*_paged_mtpN``: both, one
    ``mfa_decode_attn_paged_mt`` call;
  * ``layer_bf16_8k`` / ``layer_bf16_fp8kv_8k`` / ``layer_fp8_8k`` (block-fp8
    weights, e4m3 cache) / ``tiny_fp32``: the whole decode layer (q path, K/V
    append, attention, out-projection).
Prints one JSON line. ``value`` is KV-cache bytes read per second (GB/s) over
the whole step; ``tokens_per_s`` is sequences decoded per second for this one
layer. The K/V buffers rotate over several copies so that the 256 MB on-die
cache cannot serve a repeated working set. The CPU oracle is timed on a
bounded sample of the same workload on the host cores (``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MFA decode attn: KV-cache HBM GB/s (% of peak) + decode tokens/s at 4K ctx"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
# Sources the attention kernels are built from: HBM traffic measured with
# rocprofv3 counters is reported only while they are unchanged.
KERNEL_SOURCES = ["decode_attention_attn_amd/csrc/attn.hip", "decode_attention_attn_amd/csrc/attn_mt.hip",
                  "decode_attention_attn_amd/csrc/attn_core.h",
                  "decode_attention_attn_amd/csrc/mfa_common.h",
                  "decode_attention_attn_amd/csrc/mfa_internal.h", "decode_attention_attn_amd/build.py"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_traffic.json")


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per call (FETCH_SIZE + WRITE_SIZE, copy-calibrated) recorded
    for this workload, or None when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(workload)
    if ent is None or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_call")


def _kv_bytes(lengths, kv_kind):
    import numpy as np

    per = 512 * (1 if kv_kind == "fp8_e4m3" else (4 if kv_kind == "f32" else 2))
    return int(np.asarray(lengths, dtype=np.int64).sum()) * per


_SPREAD = {}  # per-call time percentiles of the last graph-timed run (ms)


def graph_plan(steps, rotate, max_calls=16):
    """How ``steps`` calls are replayed: (calls per graph, replays, remainder).

    The main graph holds a multiple of ``rotate`` calls (so consecutive calls
    always use different K/V buffer sets) and is replayed ``replays`` times;
    ``remainder`` calls (fewer than ``rotate``) follow in a second graph
    replayed once. The largest graph that still gives at least 5 replays is
    preferred; calls timed = calls * replays + remainder = steps, exactly."""
    best = None
    for c in range(rotate, max_calls + 1, rotate):
        if steps % c == 0 and steps // c >= 5:
            best = c
    if best is not None:
        return best, steps // best, 0
    c = rotate if steps >= rotate else 0
    return (c, steps // c, steps % c) if c else (0, 0, steps)


def _event_time_ms(fn, steps, warmup, stream, rotate=1):
    """Average time per step between HIP events on ``stream`` over exactly
    ``steps`` steps after ``warmup`` untimed ones.

    The steps are captured into HIP graphs (through torch's graph capture,
    which records the library's launches on the capture stream) and the graphs
    are replayed (``graph_plan``), so host-side launch latency does not show
    in the device time, as in a serving loop. An event after every replay of
    the main graph gives the per-call time of each replay; their 10th, 50th
    and 90th percentiles are kept when there are at least 5 replays.
    ``fn(i)`` must only enqueue work on the current stream; step i uses
    buffer set i % rotate.
    """
    import torch

    _SPREAD.clear()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    calls, reps, rem = graph_plan(steps, rotate)
    graphs = []
    for n, r in ((calls, reps), (rem, 1 if rem else 0)):
        if n == 0 or r == 0:
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        graphs.append((g, n, r))
    torch.cuda.synchronize()
    for g, _, _ in graphs:  # one untimed replay of each graph
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True)]
    ev[0].record(stream)
    marks = []  # calls in each timed replay, main graph first
    for g, n, r in graphs:
        for _ in range(r):
            g.replay()
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            ev.append(e)
            marks.append(n)
    torch.cuda.synchronize()
    timed = sum(marks)
    assert timed == steps, (timed, steps)
    main = [ev[k].elapsed_time(ev[k + 1]) / marks[k] for k in range(reps)] if calls else []
    if len(main) >= 5:
        per = sorted(main)
        _SPREAD.update(p10=per[int(0.1 * (len(per) - 1))], p50=per[(len(per) - 1) // 2],
                       p90=per[int(0.9 * (len(per) - 1))], replays=len(per), calls_per_replay=calls)
    return ev[0].elapsed_time(ev[-1]) / steps


def _eager_time_ms(fn, steps, warmup, stream):
    """Average time per step between HIP events on ``stream``, every step
    launched from the host (no graph)."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _attn_base(name):
    """(base workload, new tokens per sequence) of an attention workload name."""
    m = re.search(r"_mtp(\d)$", name)
    nt = int(m.group(1)) if m else 1
    return re.sub(r"_mtp\d$", "", name).replace("_paged", ""), nt


def _attn_kernels(name):
    """What one timed attention call launches."""
    _, nt = _attn_base(name)
    entry = ("mfa_decode_attn_paged_mt" if "_paged" in name and nt > 1 else "mfa_decode_attn_paged"
             if "_paged" in name else "mfa_decode_attn_mt" if nt > 1 else "mfa_decode_attn")
    if "fp32" in name or name.startswith("tiny"):
        body = "attn_f32_kernel + attn_combine_f32_kernel"
    elif nt == 1:
        body = "attn_pc_kernel + attn_combine_mfma_kernel"
    elif nt == 2:
        body = "attn_mt_kernel + attn_combine_mfma_kernel"
    else:
        body = "attn_mt_kernel (tokens 0-1) + attn_mt_kernel (the rest) + attn_combine_mfma_kernel"
    return f"{entry} call = {body} (HIP events on the call's stream)"


def bench_attn(name, steps, warmup, rotate, graph=True):
    import torch

    from decode_attention_attn_amd import inputs as gen
    from decode_attention_attn_amd import runner

    base, nt = _attn_base(name)
    w = gen.WORKLOADS[base]
    inp = gen.make_attn(w)
    if "_paged" in name:  # the same keys in 64-row pages, in a shuffled page order
        inp = gen.to_pages(inp, 64, seed=1)
    if nt > 1:  # nt new query tokens per sequence, causal among them
        inp = gen.with_tokens(inp, nt)
    dev = runner.upload_attn(inp)
    ks = [dev["k"]] + [dev["k"].clone() for _ in range(rotate - 1)]
    vs = [dev["v"]] + [dev["v"].clone() for _ in range(rotate - 1)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call = runner.AttnCall(dev, num_workgroups=0, want_lse=False, stream=None)
        ms = (_event_time_ms(lambda i: call(ks[i % rotate], vs[i % rotate]), steps, warmup, stream, rotate)
              if graph else _eager_time_ms(lambda i: call(ks[i % rotate], vs[i % rotate]), steps, warmup, stream))
    B = w.batch
    kv = _kv_bytes(inp["seq_len"], w.kv)
    qo = 2 * nt * B * 64 * 256 * (4 if w.act == "f32" else 2)
    return dict(workload=name, ms=ms, spread=dict(_SPREAD) if graph else {}, B=B, tokens=B * nt, kv_bytes=kv,
                alg_bytes=kv + qo, lengths=inp["seq_len"],
                inp=inp, w=w)


def bench_layer(name, steps, warmup, graph=True):
    import torch

    from decode_attention_attn_amd import inputs as gen
    from decode_attention_attn_amd import runner

    w = gen.WORKLOADS[name]
    inp = gen.make_layer(w)
    dev = runner.upload_layer(inp)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call = runner.LayerCall(dev, num_workgroups=0, stream=None)
        ms = (_event_time_ms(lambda i: call(), steps, warmup, stream) if graph
              else _eager_time_ms(lambda i: call(), steps, warmup, stream))
    B = w.batch
    esz = 4 if w.act == "f32" else 2
    kv = _kv_bytes(inp["seq_len"] + 1, w.kv)
    n_w = 2048 * 7168 + 16384 * 2048 + 2 * 256 * 7168 + 7168 * 16384
    # block-fp8 weights: one byte per element plus one fp32 scale per 128 x 128 block
    weights = n_w + 4 * (n_w // (128 * 128)) if w.weights == gen.FP8_BLOCK else n_w * esz
    return dict(workload=name, ms=ms, spread=dict(_SPREAD) if graph else {}, B=B, kv_bytes=kv, alg_bytes=kv + weights,
                lengths=inp["seq_len"] + 1,
                inp=inp, w=w)


def bench_probe(gib=4, reps=10):
    """Achievable HBM read rate: mfa_bw_probe over a ``gib`` GiB buffer
    (nontemporal 16-byte vector loads, one workgroup per CU), HIP events over ``reps``
    calls after two warm-up calls."""
    import torch

    from decode_attention_attn_amd import mfa

    buf = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus, dtype=torch.int32, device="cuda")
    ms = _eager_time_ms(lambda i: mfa.check(mfa.mfa_bw_probe(buf, sink), "mfa_bw_probe"), reps, 2,
                        torch.cuda.current_stream())
    out = {"GBps": round(buf.numel() / (ms * 1e-3) / 1e9, 1), "bytes": buf.numel(), "ms": round(ms, 4),
           "kernel": "mfa_bw_probe (nontemporal 16-byte vector loads, one workgroup per CU)"}
    del buf, sink
    torch.cuda.synchronize()
    return out


def cpu_baseline(res, seconds):
    """Time the float64 oracle on the host for about ``seconds`` on a sample of the workload."""
    import numpy as np

    from oracle import mfa_oracle as om

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    host_cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    inp, w = res["inp"], res["w"]
    B = len(inp["seq_len"])
    done_seqs, done_kv, t0 = 0, 0, time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < seconds:
        nt = int(inp.get("n_tokens", 1))
        if w.kind == "attn" and nt > 1:
            om.decode_attn_mt(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_off"], inp["seq_len"], nt,
                              kind_q=inp["kind_q"], kind_kv=inp["kind_kv"], k_scale=inp["k_scale"],
                              v_scale=inp["v_scale"], batch_ids=[b])
            done_kv += _kv_bytes([inp["seq_len"][b]], w.kv)
        elif w.kind == "attn":
            om.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_off"], inp["seq_len"],
                           kind_q=inp["kind_q"], kind_kv=inp["kind_kv"], k_scale=inp["k_scale"],
                           v_scale=inp["v_scale"], batch_ids=[b])
            done_kv += _kv_bytes([inp["seq_len"][b]], w.kv)
        else:
            om.decode_layer(inp, batch_ids=[b])
            done_kv += _kv_bytes([inp["seq_len"][b] + 1], w.kv)
        done_seqs += nt
        b = (b + 1) % B
    dt = time.perf_counter() - t0
    return {
        "value": round(done_kv / dt / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(done_seqs / dt, 3),
        "cores": int(threads),  # BLAS threads the oracle ran with
        "host_cores": host_cores,  # cores this process may run on
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"{done_seqs} sequences of {w.name} (cycling over the batch), {dt:.1f} s, numpy float64",
        "seconds": round(dt, 2),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="attn_bf16_4k",
                    choices=["attn_bf16_4k", "attn_fp8kv_4k", "attn_bf16_ragged", "attn_bf16_4k_paged",
                             "attn_fp8kv_4k_paged"]
                    + [f"attn_{kv}_4k{pg}_mtp{n}" for kv in ("bf16", "fp8kv") for pg in ("", "_paged")
                       for n in (2, 3, 4)]
                    + ["layer_bf16_8k", "layer_bf16_fp8kv_8k", "layer_fp8_8k", "tiny_fp32"])
    ap.add_argument("--rotate", type=int, default=4, help="K/V buffer sets cycled through (attention workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the fp8-KV 4K secondary measurement")
    ap.add_argument("--no-graph", action="store_true", help="launch every step from the host instead of replaying "
                    "a captured HIP graph")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read bandwidth probe")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first copy this many MiB device-to-device three times (a plain copy kernel of known size, "
                    "to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import decode_attention_attn_amd.mfa  # noqa: F401  (fails loudly if libmfa.so is missing)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    probe = None if args.no_probe else bench_probe()
    if args.workload.startswith("attn"):
        res = bench_attn(args.workload, args.steps, args.warmup, args.rotate, graph=not args.no_graph)
    else:
        res = bench_layer(args.workload, args.steps, args.warmup, graph=not args.no_graph)
    w = res["w"]
    ms = res["ms"]
    gbps = res["kv_bytes"] / (ms * 1e-3) / 1e9
    achieved = res["alg_bytes"] / (ms * 1e-3) / 1e9
    hbm_bytes = measured_traffic(res["workload"])
    line = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,  # calls timed, exactly
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": res["workload"],
            "batch": w.batch,
            "ctx": int(max(res["lengths"])),
            "q_heads": 64,
            "kv_heads": 1,
            "head_dim": 256,
            "kv_dtype": w.kv,
            "weights": (w.weights or w.act) if w.kind == "layer" else None,
            "kv_buffer_sets": args.rotate if w.kind == "attn" else 1,
        },
        "tokens_per_s": round(res.get("tokens", w.batch) / (ms * 1e-3), 1),
        # per-call time over each graph replay: 10th, 50th and 90th percentiles (ms), given when the
        # timed calls form at least 5 replays
        "ms_per_step_pct": {k: (round(v, 5) if isinstance(v, float) else v)
                            for k, v in res.get("spread", {}).items()} or None,
        "pct_of_peak_hbm": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            # HBM bytes per call from rocprofv3 FETCH_SIZE + WRITE_SIZE (copy-calibrated), as a rate over the
            # same call time as "achieved"; null when the kernel sources changed since the counters were taken
            "traffic": None if hbm_bytes is None else round(hbm_bytes / (ms * 1e-3) / 1e9, 2),
            "traffic_bytes_per_launch": hbm_bytes,
            "kernel": _attn_kernels(res["workload"]) if w.kind == "attn" else "whole layer (HIP events)",
            "alg_bytes_per_launch": res["alg_bytes"],
        },
    }
    if w.kind == "attn" and not args.no_secondary and args.workload == "attn_bf16_4k":
        sec = bench_attn("attn_fp8kv_4k", args.steps, args.warmup, args.rotate, graph=not args.no_graph)
        s_gbps = sec["kv_bytes"] / (sec["ms"] * 1e-3) / 1e9
        line["secondary"] = {"attn_fp8kv_4k": {
            "ms_per_step": round(sec["ms"], 5), "kv_GBps": round(s_gbps, 2),
            "pct_of_peak_hbm": round(100 * s_gbps / HBM_PEAK_GBPS, 2),
            "tokens_per_s": round(sec["B"] / (sec["ms"] * 1e-3), 1)}}
        del sec
    if probe is not None:
        # the KV rate and the roofline's achieved rate as fractions of the
        # measured streaming-read rate (the 8 TB/s peak stays the roofline)
        line["bw_probe"] = probe
        line["pct_of_probe"] = {"kv": round(100.0 * gbps / probe["GBps"], 2),
                                "achieved": round(100.0 * achieved / probe["GBps"], 2)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
