"""Benchmark of the shared compressed-KV decode path on one MI355X.

One step is the whole hot path of the Llama-3-8B-shaped workload (32 layers,
32 q heads / 8 kv heads, head_dim 128, a 4096-token shared context, 15 agents):
the pool is encoded from bf16 K/V already resident in HBM (one append of all
layers), then 128 decode steps run for all 15 agents, each agent attending to
the pool plus its own native bf16 suffix of s + 1 tokens at decode step s.
value = agent-tokens per second = 15 * 128 / (seconds per step).

The JSON line also carries the roofline of the dominant kernel (the pool
decode kernel), timed live with a HIP event pair recorded on the call's own
stream around the kernel, and the CPU oracle timed on a bounded sample of the
same work.  Only the ``cpu_baseline`` leg imports the oracle.

roofline.frac is the cold figure: the pool kernel launched right after a
plain reduction over a 1 GiB buffer (four times the 256 MB last-level cache,
so the pool comes from HBM; a read leaves only clean lines behind, whereas a
write-based flush would make the measured kernel pay for writing the flush
buffer back).  The warm figure (consecutive decode calls, the 189 MB pool
resident in the last-level cache) sits beside it, with the streaming-read
ceiling measured in the same run.  The per_layer block times the same job as
32 single-layer calls per decode step (one captured HIP graph per step), the
way a model's decoder issues them.

    python bench.py [--steps K] [--warmup W] [--kernel valu|mfma|default] [--no-cpu-baseline] [--no-per-layer]
    python bench.py --trace-summary kernel_trace.csv   (pool-kernel warm/cold averages from a rocprofv3 trace)
    python bench.py --workload qwen3_32b_comix   (8 agents, own mixed-bit pools; not the headline)
    python bench.py --comix      (the CoMixKV controller instead: its own JSON line)
    python bench.py --rotation-ablation   (plain FWHT vs randomized rotation: its own JSON line)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--kernel", default="default", choices=["default", "valu", "mfma"])
    ap.add_argument("--decode-steps", type=int, default=None, help="decode steps per job (default: workload's 128)")
    ap.add_argument("--agents", type=int, default=None,
                    help="agents sharing the pool (default: the workload's; above 16 at 4 q heads per kv head the "
                         "pool kernel runs in row blocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--private-tokens", type=int, default=0,
                    help="give every agent a private compressed segment of this many older tokens "
                         "(quantized in each job, attended with the shared pool and the native window)")
    ap.add_argument("--cold-calls", type=int, default=24,
                    help="extra pool-kernel launches outside the timed jobs, each after a streaming read of 1 GiB "
                         "(the headline roofline)")
    ap.add_argument("--no-per-layer", action="store_true", help="skip the per-layer (32 calls per step) block")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarise a rocprofv3 kernel trace of this script: pool-kernel launches after a streaming "
                         "read (cold) and after another kernel (warm)")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                            "pool_decode_traffic.json"))
    ap.add_argument("--workload", default="llama3_8b",
                    choices=["llama3_8b", "llama3_8b_long", "smollm2", "qwen3_32b_comix"],
                    help="llama3_8b (default, the headline): one shared 4096-token pool, 15 agents; "
                         "llama3_8b_long: 7194-token pool, 256-token native windows, 32 decode calls; "
                         "smollm2: 24 layers, 32 MHA heads, d 64, 1851 tokens, 3 agents; "
                         "qwen3_32b_comix: 8 agents with their own 8064-token mixed 2/3/4-bit pools")
    ap.add_argument("--comix", action="store_true",
                    help="instead of the decode job: time the CoMixKV controller (sensitivity kernel + allocation) "
                         "on the Qwen3-32B shape and measure the attention error of its bits against uniform 3 bits")
    ap.add_argument("--codec-ablation", action="store_true",
                    help="instead of the decode job: reconstruction error, attention error, bytes per token and "
                         "pool-kernel time of the codec variants (K per tensor / token / channel, corrected V norm)")
    ap.add_argument("--rotation-ablation", action="store_true",
                    help="instead of the decode job: attention error and pool-kernel time of the plain FWHT "
                         "against a randomized (signed) rotation, on Gaussian and on Hadamard-aligned V")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files into the traffic summary")
    return ap.parse_args()


def _counter_per_dispatch(path, name_part, counter):
    import csv

    vals = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} in {path}")
    return sum(vals) / len(vals), len(vals)


def pmc_summary(paths, out_path, kernel_variant, workload):
    """HBM bytes per pool-kernel launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by what it reads for a plain copy of known size
    (1 GiB read and 1 GiB written per launch, larger than the last-level cache).
    """
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = paths
    f_pool, nf = _counter_per_dispatch(fetch_csv, "k_pool_mfma", "FETCH_SIZE")
    w_pool, nw = _counter_per_dispatch(write_csv, "k_pool_mfma", "WRITE_SIZE")
    f_copy, _ = _counter_per_dispatch(cfetch_csv, "opy", "FETCH_SIZE")
    w_copy, _ = _counter_per_dispatch(cwrite_csv, "opy", "WRITE_SIZE")
    n = 1 << 30
    f_scale = n / (f_copy * 1024.0)
    w_scale = n / (w_copy * 1024.0)
    res = {"workload": workload, "kernel_variant": kernel_variant, "kernel_source_sha256": kernel_source_sha256(),
           "fetch_kib_per_dispatch": f_pool, "write_kib_per_dispatch": w_pool, "dispatches": [nf, nw],
           "copy_fetch_kib": f_copy, "copy_write_kib": w_copy, "fetch_scale": f_scale, "write_scale": w_scale,
           "bytes_per_launch": f_pool * 1024.0 * f_scale + w_pool * 1024.0 * w_scale}
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res))


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def kernel_source_sha256():
    import hashlib

    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_shared_kv_amd", "csrc")
    h = hashlib.sha256()
    # the pool kernel's sources, with the window code its split-record form runs
    for f in ("pkv_decode_mfma.h", "pkv_decode_mfma.hip", "pkv_decode_mfma_split.hip", "pkv_sfx.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        import workloads as wl

        pmc_summary(args.pmc_summary, args.traffic_json, "valu" if args.kernel == "valu" else "mfma",
                    wl.LLAMA3_8B.name)
        return
    if args.comix:
        comix_bench()
        return
    if args.rotation_ablation:
        rotation_ablation()
        return
    if args.codec_ablation:
        codec_ablation()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "qwen3_32b_comix":
        qwen_bench(args)
        return
    import torch

    import workloads as wl
    from quantized_shared_kv_amd import polykv as pk

    pk.lib()  # fails loudly if the HIP library is not built
    kernel = {"default": pk.KERNEL_DEFAULT, "valu": pk.KERNEL_VALU, "mfma": pk.KERNEL_MFMA}[args.kernel]
    w = {"llama3_8b": wl.LLAMA3_8B, "llama3_8b_long": wl.LLAMA3_8B_LONG, "smollm2": wl.SMOLLM2}[args.workload]
    if args.agents and args.agents != w.n_agents:
        w = w.replace(n_agents=args.agents, name=w.name.replace(f"_A{w.n_agents}", f"_A{args.agents}"))
    steps_per_job = args.decode_steps or w.steps

    def sfx_lens(s):  # native tokens per agent at decode step s: growing window, or a fixed one
        return [w.sfx_len(s)] * A
    dev = "cuda:0"
    L, Hkv, Hq, d, T, A, S = w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.pool_tokens, w.n_agents, w.sfx_tokens

    def dev_bf16(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)

    t0 = time.time()
    log("[bench] generating inputs")
    k_pool = torch.empty((L, Hkv, T, d), dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty_like(k_pool)
    for l in range(L):
        k_pool[l].copy_(dev_bf16(w.pool_k(0, l).raw))
        v_pool[l].copy_(dev_bf16(w.pool_v(0, l).raw))
    sfx_k = torch.empty((A, L, Hkv, S, d), dtype=torch.bfloat16, device=dev)
    sfx_v = torch.empty_like(sfx_k)
    for a in range(A):
        for l in range(L):
            sfx_k[a, l].copy_(dev_bf16(w.sfx_k(a, l).raw))
            sfx_v[a, l].copy_(dev_bf16(w.sfx_v(a, l).raw))
    q_all = torch.empty((steps_per_job, A, L, Hq, d), dtype=torch.bfloat16, device=dev)
    for s in range(steps_per_job):
        for a in range(A):
            q_all[s, a].copy_(dev_bf16(w.queries(s, a).raw))
    out = torch.empty((A, L, Hq, d), dtype=torch.float32, device=dev)
    cfg = pk.make_config(L, Hkv, d, T, w.v_bits(0))
    nbytes = pk.pool_bytes(cfg)
    pool_buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pool = pk.pool_build(cfg, pool_buf.data_ptr(), nbytes)
    pools = [pool] * A
    pk.pool_quantize_append(pool, 0, k_pool, v_pool)  # the workspace plan depends on the pool's token count
    # optional per-agent private segments: synthetic bf16 K/V of the same scale, seeded on the device
    NP = args.private_tokens
    prv_pools, prv_bufs, prv_cfg, prv_kv = None, [], None, None
    if NP > 0:
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        prv_cfg = pk.make_config(L, Hkv, d, NP, w.v_bits(0))
        pb = pk.pool_bytes(prv_cfg)
        prv_kv = [(torch.randn((L, Hkv, NP, d), generator=gen, device=dev).to(torch.bfloat16),
                   torch.randn((L, Hkv, NP, d), generator=gen, device=dev).to(torch.bfloat16)) for _ in range(A)]
        prv_pools = []
        for a in range(A):
            prv_bufs.append(torch.empty(pb, dtype=torch.uint8, device=dev))
            prv_pools.append(pk.pool_build(prv_cfg, prv_bufs[-1].data_ptr(), pb))
            pk.pool_quantize_append(prv_pools[a], 0, *prv_kv[a])
    ws_bytes = pk.agent_decode_attention(pools, q_all[0], out, 0, sfx_k, sfx_v, [S] * A, kernel=kernel,
                                         private_pools=prv_pools)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in {time.time() - t0:.1f}s; pool {nbytes / 1e6:.1f} MB, workspace "
        f"{ws_bytes / 1e6:.1f} MB")

    # The pool kernel is timed with an event pair on every EV_EVERY-th decode call of each
    # timed job (16 of 128 calls, spanning suffix lengths 1..121): an event pair recorded
    # around every call adds ~5 us per call to the job, which is instrumentation, not work.
    EV_EVERY = 8
    timed_calls = list(range(0, steps_per_job, EV_EVERY))
    n_ev = steps_per_job
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for e0, e1 in evs:  # create the underlying events
        e0.record()
        e1.record()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def one_job(timed_kernels):
        pool_fresh = pk.pool_build(cfg, pool_buf.data_ptr(), nbytes)  # host-only: n_tokens back to 0
        for f in pk.Pool._fields_:
            setattr(pool, f[0], getattr(pool_fresh, f[0]))
        if timed_kernels:
            b0.record()
        pk.pool_quantize_append(pool, 0, k_pool, v_pool)
        if prv_pools is not None:
            for a in range(A):
                fresh = pk.pool_build(prv_cfg, prv_bufs[a].data_ptr(), prv_bufs[a].numel())
                for f in pk.Pool._fields_:
                    setattr(prv_pools[a], f[0], getattr(fresh, f[0]))
                pk.pool_quantize_append(prv_pools[a], 0, *prv_kv[a])
        if timed_kernels:
            b1.record()
        for s in range(steps_per_job):
            lens = sfx_lens(s)
            pk.agent_decode_attention(pools, q_all[s], out, 0, sfx_k, sfx_v, lens, workspace=ws, kernel=kernel,
                                      pool_events=evs[s] if timed_kernels and s % EV_EVERY == 0 else None,
                                      private_pools=prv_pools)

    for i in range(args.warmup):
        one_job(False)
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pool_ms, build_ms = [], []
    start.record()
    for i in range(args.steps):
        one_job(True)
        torch.cuda.synchronize()  # event readback between jobs; inside the timed region
        pool_ms += [evs[s][0].elapsed_time(evs[s][1]) for s in timed_calls]
        build_ms.append(b0.elapsed_time(b1))
        log(f"[bench] step {i + 1}/{args.steps} done")
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    value = A * steps_per_job / (ms_per_step / 1e3)

    # Cold pass (outside the timed region): before each launch a plain reduction reads 1 GiB and
    # replaces the last-level cache's contents with clean lines, so the pool kernel reads the pool
    # from HBM.  The library's streaming read (non-temporal loads) over the same buffer, timed,
    # is the practical HBM read ceiling of this machine.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    sink = torch.empty(pk.stream_read_sink_words(), dtype=torch.int32, device=dev)
    flush_f = flush.view(torch.float32)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    read_ms = []
    for i in range(6):
        r0.record()
        pk.stream_read(flush, sink)
        r1.record()
        torch.cuda.synchronize()
        read_ms.append(r0.elapsed_time(r1))
    stream_gbps = flush.numel() * 4 / (float(np.median(read_ms[1:])) / 1e3) / 1e9
    cold_ms = []
    for i in range(args.cold_calls):
        flush_f.sum()
        pk.agent_decode_attention(pools, q_all[i % steps_per_job], out, 0, sfx_k, sfx_v, [S] * A, workspace=ws,
                                  kernel=kernel, pool_events=evs[0], private_pools=prv_pools)
        torch.cuda.synchronize()
        cold_ms.append(evs[0][0].elapsed_time(evs[0][1]))
    per_layer = None
    if not args.no_per_layer and NP == 0:
        per_layer = per_layer_block(pk, w, pools, q_all, sfx_k, sfx_v, sfx_lens, steps_per_job, kernel, flush_f)
    flush_bytes = flush.numel() * 4
    del flush

    # algorithmic bytes of one pool-kernel launch: every pool byte of the T tokens once
    # (K codes d, V codes d*b/8, norm 4 per (token, kv head); scale 4 per (token, layer)),
    # the bf16 queries read and the fp32 outputs written
    bits = 3
    pool_alg = L * Hkv * T * (d + d * bits // 8 + 4) + L * T * 4
    pool_alg += A * (L * Hkv * NP * (d + d * bits // 8 + 4) + L * NP * 4)  # private segments, if any
    q_bytes = A * L * Hq * d * 2
    out_bytes = A * L * Hq * d * 4
    alg = pool_alg + q_bytes + out_bytes
    avg_pool_ms = float(np.mean(pool_ms))
    warm_achieved = alg / (avg_pool_ms / 1e3) / 1e9
    cold_avg_ms = float(np.mean(cold_ms))
    achieved = alg / (cold_avg_ms / 1e3) / 1e9
    decode_us = (ms_per_step - float(np.mean(build_ms))) / steps_per_job * 1e3
    window_avg = sum(sum(sfx_lens(s)) * L * Hkv * d * 2 * 2 for s in range(steps_per_job)) / steps_per_job
    call_alg = alg + window_avg
    traffic = None
    variant = "valu" if kernel == pk.KERNEL_VALU else "mfma"  # the default selects MFMA at 60 rows
    if os.path.exists(args.traffic_json):
        try:
            t = json.load(open(args.traffic_json))
            if (NP == 0 and t.get("kernel_variant") == variant and t.get("workload") == w.name
                    and t.get("kernel_source_sha256") == kernel_source_sha256()):
                traffic = t.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    line = {
        "metric": "compressed-KV decode attention: achieved HBM GB/s (% peak) + agent-tokens/s",
        "value": value,
        "unit": "agent-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if kernel == pk.KERNEL_VALU else "fp16-mfma-f32-acc",
        "data": "synthetic",
        "config": {"workload": w.name, "agents": A, "decode_steps_per_step": steps_per_job, "pool_tokens": T,
                   "layers": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "v_bits": 3,
                   "suffix": (f"bf16, s+1 tokens at decode step s (max {S})" if w.sfx_mode == "grow"
                              else f"bf16, {S} tokens per agent"), "kernel": args.kernel,
                   **({"private_tokens_per_agent": NP} if NP else {})},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "pool decode" + (" (private segments + pool kernel)" if NP else ""),
                     "alg_bytes_per_launch": alg, "avg_launch_us": cold_avg_ms * 1e3, "launches": len(cold_ms),
                     "cache": "cold: a reduction over 1 GiB before each launch",
                     "frac_of_stream_read_ceiling": achieved / stream_gbps,
                     "warm": {"avg_launch_us": avg_pool_ms * 1e3, "achieved": warm_achieved,
                              "frac": warm_achieved / HBM_PEAK_GBPS, "launches": len(pool_ms),
                              "note": "every 8th decode call of the timed jobs; the pool stays in the last-level cache"}},
        "stream_read_ceiling": {"achieved": stream_gbps, "unit": "GB/s", "frac": stream_gbps / HBM_PEAK_GBPS,
                                "bytes": flush_bytes,
                                "kernel": "pkv_stream_read (16-byte non-temporal loads, grid stride)"},
        "pool_build_us": float(np.mean(build_ms)) * 1e3,
        "decode_step_us": decode_us,
        # the whole decode call: pool kernel bytes plus the agents' bf16 windows (keys and values)
        # at the job's window lengths, averaged over its decode steps, against the call's time
        "whole_call": {"alg_bytes_per_call": call_alg, "avg_call_us": decode_us,
                       "achieved": call_alg / decode_us / 1e3, "unit": "GB/s",
                       "frac": call_alg / decode_us / 1e3 / HBM_PEAK_GBPS,
                       "window_bytes_per_call": window_avg,
                       "note": "one all-layer call per decode step: native-window and pool kernels; build excluded"},
    }
    if per_layer is not None:
        line["per_layer"] = per_layer
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, steps_per_job)
    print(json.dumps(line), flush=True)


def per_layer_block(pk, w, pools, q_all, sfx_k, sfx_v, sfx_lens, steps, kernel, flush_f):
    """The decode part of the job issued the way a model's decoder issues it: per decode step,
    32 single-layer calls (layer l's queries, suffix and outputs in their own buffers), timed
    both as one captured HIP graph per step and issued call by call; the faster gives the
    agent-tokens/s.  The replay of step 0's graph is checked bit for bit against the same calls
    made eagerly, three times with eager work in between.  The pool kernel of a single-layer
    call (which also carries the call's native-window workgroups) is timed with events on sampled
    calls, warm (inside the call sequence) and cold (after a reduction over 1 GiB)."""
    import torch

    dev = q_all.device
    L, A, Hq, d, Hkv, T = w.n_layers, w.n_agents, w.n_q_heads, w.head_dim, w.n_kv_heads, w.pool_tokens
    ql = [[q_all[s, :, l:l + 1].contiguous() for l in range(L)] for s in range(steps)]
    skl = [sfx_k[:, l:l + 1].contiguous() for l in range(L)]
    svl = [sfx_v[:, l:l + 1].contiguous() for l in range(L)]
    outs = [torch.empty((A, 1, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    wsb = max(pk.agent_decode_attention(pools, ql[0][l], outs[l], l, skl[l], svl[l], sfx_lens(steps - 1),
                                        kernel=kernel) for l in range(L))
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def step_calls(s, events=None, layer=None):
        for l in range(L):
            pk.agent_decode_attention(pools, ql[s][l], outs[l], l, skl[l], svl[l], sfx_lens(s), workspace=ws,
                                      kernel=kernel, pool_events=events if l == layer else None)

    step_calls(0)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    cap = torch.cuda.Stream()  # default priority
    graphs = []
    for s in range(steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step_calls(s)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graphs[0].replay()
        torch.cuda.synchronize()
        if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
            raise RuntimeError("per-layer graph replay differs from the eager calls")
        step_calls(1 + rep)  # eager work between the replays
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for g in graphs:  # warm-up
        g.replay()
    torch.cuda.synchronize()
    job_ms = []
    for rep in range(3):
        e0.record()
        for g in graphs:
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        job_ms.append(e0.elapsed_time(e1))
    graph_ms = float(np.median(job_ms))
    eager_ms = []
    for rep in range(2):  # the same decode steps issued call by call (the host stays ahead of the GPU)
        e0.record()
        for s in range(steps):
            step_calls(s)
        e1.record()
        torch.cuda.synchronize()
        eager_ms.append(e0.elapsed_time(e1))
    eager_ms = min(eager_ms)
    # the pool kernel of one single-layer call
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    p1.record()
    # the launch of a single-layer call also carries the call's native-window work (its suffix
    # workgroups run beside the pool ones): its bf16 K and V bytes count with the pool's
    def launch_bytes(s):
        window = sum(sfx_lens(s)) * Hkv * d * 2 * 2
        return Hkv * T * (d + d * 3 // 8 + 4) + T * 4 + A * Hq * d * (2 + 4) + window

    warm, cold, warm_b, cold_b = [], [], [], []
    for s in (1, steps // 2, steps - 1):
        for l in range(0, L, 4):
            step_calls(s, (p0, p1), l)
            torch.cuda.synchronize()
            warm.append(p0.elapsed_time(p1))
            warm_b.append(launch_bytes(s))
    for i in range(16):
        l = (5 * i) % L
        flush_f.sum()
        pk.agent_decode_attention(pools, ql[i % steps][l], outs[l], l, skl[l], svl[l], sfx_lens(i % steps),
                                  workspace=ws, kernel=kernel, pool_events=(p0, p1))
        torch.cuda.synchronize()
        cold.append(p0.elapsed_time(p1))
        cold_b.append(launch_bytes(i % steps))
    alg, alg_w = float(np.mean(cold_b)), float(np.mean(warm_b))
    cold_us, warm_us = float(np.mean(cold)) * 1e3, float(np.mean(warm)) * 1e3
    best_ms = min(graph_ms, eager_ms)
    return {"calls_per_decode_step": L,
            "launch": ("one captured HIP graph per decode step (32 single-layer calls)" if graph_ms <= eager_ms else
                       "32 single-layer calls per decode step issued one by one (faster here than their captured graph)"),
            "graph_replays_checked": 3,
            "decode_agent_tokens_per_s": A * steps / (best_ms / 1e3),
            "decode_step_us": best_ms / steps * 1e3, "graph_decode_step_us": graph_ms / steps * 1e3,
            "eager_decode_step_us": eager_ms / steps * 1e3,
            "pool_kernel": {"alg_bytes_per_launch": alg, "carries_native_window": True, "avg_launch_us": cold_us,
                            "achieved": alg / (cold_us / 1e6) / 1e9, "frac": alg / (cold_us / 1e6) / 1e9 / HBM_PEAK_GBPS,
                            "cache": "cold: a reduction over 1 GiB before each launch", "launches": len(cold),
                            "warm_avg_launch_us": warm_us,
                            "warm_frac": alg_w / (warm_us / 1e6) / 1e9 / HBM_PEAK_GBPS}}


def trace_summary(path):
    """Pool-kernel launches of a rocprofv3 kernel trace of this script, split by what ran before
    each decode call: the 1 GiB reduction (cold) or another kernel (warm); with every kernel's average."""
    import csv
    import re

    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    stats = {}
    warm, cold = [], []
    for i, (t0, t1, name) in enumerate(rows):
        m = re.search(r"\b(k_[a-z0-9_]+)", name)
        short = m.group(1) if m else name[:60]
        stats.setdefault(short, []).append(t1 - t0)
        if "k_pool_mfma" in name or "k_pool_valu" in name:
            # the kernel before this decode call's own suffix / segment kernels
            j = i - 1
            while j >= 0 and re.search(r"\bk_(sfx|sfx_fast|seg)\b", rows[j][2]):
                j -= 1
            prev = rows[j][2] if j >= 0 else ""
            (cold if "reduce_kernel" in prev else warm).append(t1 - t0)
    out = {"kernels": {k: {"calls": len(v), "avg_us": float(np.mean(v)) / 1e3} for k, v in sorted(stats.items())},
           "pool_kernel_cold": {"launches": len(cold), "avg_us": float(np.mean(cold)) / 1e3 if cold else None},
           "pool_kernel_warm": {"launches": len(warm), "avg_us": float(np.mean(warm)) / 1e3 if warm else None}}
    print(json.dumps(out, indent=1))


def qwen_bench(args):
    """The Qwen3-32B CoMixKV workload: 8 agents, each with its own pool of 8064 tokens
    (64 layers, 8 kv heads, d 128, V bits per layer a seeded permutation of 21 x 2, 22 x 3,
    21 x 4) and a fixed 128-token native window; 64 query heads.  One step = one job: the
    8 pools encoded from bf16 K/V already in HBM, then 16 decode calls for the 8 agents.
    K, V = N(0, 1) * sigma with sigma ~ LogNormal(0, 0.5) per (layer, kv head, channel), drawn
    on the device (the workload's own recipe; its host slices are used by the parity tests).
    """
    import torch

    import workloads as wl
    from quantized_shared_kv_amd import polykv as pk

    pk.lib()
    w = wl.QWEN3_32B_MIXED
    dev = "cuda:0"
    L, Hkv, Hq, d, T, A, S = w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.pool_tokens, w.n_agents, w.sfx_tokens
    NS = args.decode_steps or w.steps
    t0 = time.time()
    log("[bench] generating inputs (device draws)")
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    kv = []
    for p in range(A):
        sk = torch.exp(0.5 * torch.randn((L, Hkv, 1, d), generator=g, device=dev))
        sv = torch.exp(0.5 * torch.randn((L, Hkv, 1, d), generator=g, device=dev))
        k = torch.empty((L, Hkv, T, d), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        for l in range(L):
            k[l] = (torch.randn((Hkv, T, d), generator=g, device=dev) * sk[l]).to(torch.bfloat16)
            v[l] = (torch.randn((Hkv, T, d), generator=g, device=dev) * sv[l]).to(torch.bfloat16)
        kv.append((k, v))
    sfx_k = torch.randn((A, L, Hkv, S, d), generator=g, device=dev).to(torch.bfloat16)
    sfx_v = torch.randn((A, L, Hkv, S, d), generator=g, device=dev).to(torch.bfloat16)
    q_all = torch.randn((NS, A, L, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((A, L, Hq, d), dtype=torch.float32, device=dev)
    cfgs = [pk.make_config(L, Hkv, d, T, w.v_bits(p)) for p in range(A)]
    bufs = [torch.empty(pk.pool_bytes(c), dtype=torch.uint8, device=dev) for c in cfgs]
    pools = [pk.pool_build(c, b.data_ptr(), b.numel()) for c, b in zip(cfgs, bufs)]
    for p in range(A):
        pk.pool_quantize_append(pools[p], 0, *kv[p])
    ws = torch.empty(max(pk.agent_decode_attention(pools, q_all[0], out, 0, sfx_k, sfx_v, [S] * A), 256),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in {time.time() - t0:.1f}s; pools {sum(b.numel() for b in bufs) / 1e9:.2f} GB")
    EV_EVERY = 4
    timed_calls = list(range(0, NS, EV_EVERY))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(NS)]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def one_job(timed):
        for p in range(A):
            fresh = pk.pool_build(cfgs[p], bufs[p].data_ptr(), bufs[p].numel())  # host-only: n_tokens back to 0
            for f in pk.Pool._fields_:
                setattr(pools[p], f[0], getattr(fresh, f[0]))
        if timed:
            b0.record()
        for p in range(A):
            pk.pool_quantize_append(pools[p], 0, *kv[p])
        if timed:
            b1.record()
        for s in range(NS):
            pk.agent_decode_attention(pools, q_all[s], out, 0, sfx_k, sfx_v, [S] * A, workspace=ws,
                                      pool_events=evs[s] if timed and s % EV_EVERY == 0 else None)

    for i in range(args.warmup):
        one_job(False)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pool_ms, build_ms = [], []
    start.record()
    for i in range(args.steps):
        one_job(True)
        torch.cuda.synchronize()
        pool_ms += [evs[s][0].elapsed_time(evs[s][1]) for s in timed_calls]
        build_ms.append(b0.elapsed_time(b1))
        log(f"[bench] step {i + 1}/{args.steps} done")
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    pool_alg = sum(T * (Hkv * (d + d * int(b) // 8 + 4) + 4) for p in range(A) for b in w.v_bits(p))
    alg = pool_alg + A * L * Hq * d * 2 + A * L * Hq * d * 4
    avg = float(np.mean(pool_ms))
    achieved = alg / (avg / 1e3) / 1e9
    print(json.dumps({
        "metric": "compressed-KV decode attention: achieved HBM GB/s (% peak) + agent-tokens/s",
        "value": A * NS / (ms_per_step / 1e3), "unit": "agent-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32-acc", "data": "synthetic",
        "config": {"workload": w.name, "agents": A, "pools": A, "decode_steps_per_step": NS, "pool_tokens": T,
                   "layers": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "v_bits": "per (pool, layer): seeded permutation of 21x2, 22x3, 21x4",
                   "suffix": f"bf16, {S} tokens per agent"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "pool decode",
                     "alg_bytes_per_launch": alg, "avg_launch_us": avg * 1e3, "launches_timed": len(pool_ms)},
        "pool_build_us": float(np.mean(build_ms)) * 1e3,
        "decode_step_us": (ms_per_step - float(np.mean(build_ms))) / NS * 1e3,
    }), flush=True)


def rotation_ablation():
    """Plain FWHT against a randomized rotation (signs before the FWHT), Llama-3-8B shape.

    One agent (4 query rows per kv head) over a 4096-token pool of 32 layers, 8 kv heads,
    d 128, 3 bits.  V recipes (bf16, device-seeded): "gaussian" = N(0, 1) * LogNormal(0, 0.5)
    channel scales (the workloads' recipe); "hadamard_aligned" = each token's V a Hadamard
    row of the head dimension times a LogNormal(0, 1) magnitude plus 1% Gaussian noise
    (structured V that the plain transform concentrates into one coordinate).  Error: decode
    of 8 query steps over the pool against exact attention over the same bf16 K/V (the same
    call with an empty pool and the tokens as native suffix); relative L2 per output row.
    """
    import torch

    import workloads as wl
    from quantized_shared_kv_amd import polykv as pk

    pk.lib()
    dev = "cuda:0"
    L, Hkv, Hq, d, T, R = 32, 8, 32, 128, 4096, 8
    signs = wl.rotation_signs(0, d)
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    q = torch.randn((R, 1, L, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    sk = torch.exp(0.5 * torch.randn((L, Hkv, 1, d), generator=g, device=dev))
    k = (torch.randn((L, Hkv, T, d), generator=g, device=dev) * sk).to(torch.bfloat16)
    h = torch.ones((1, 1), device=dev)
    while h.shape[0] < d:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    recipes = {
        "gaussian": (torch.randn((L, Hkv, T, d), generator=g, device=dev)
                     * torch.exp(0.5 * torch.randn((L, Hkv, 1, d), generator=g, device=dev))).to(torch.bfloat16),
        "hadamard_aligned": (h[torch.randint(0, d, (L, Hkv, T), generator=g, device=dev)]
                             * torch.exp(torch.randn((L, Hkv, T, 1), generator=g, device=dev))
                             + 0.01 * torch.randn((L, Hkv, T, d), generator=g, device=dev)).to(torch.bfloat16),
    }
    empty_cfg = pk.make_config(L, Hkv, d, 32, [3] * L)
    ebuf = torch.empty(pk.pool_bytes(empty_cfg), dtype=torch.uint8, device=dev)
    empty = pk.pool_build(empty_cfg, ebuf.data_ptr(), ebuf.numel())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()  # creates the underlying events
    e1.record()
    res = {}
    for name, v in recipes.items():
        ref = torch.empty((1, L, Hq, d), dtype=torch.float32, device=dev)
        out = torch.empty_like(ref)
        kw, vw = k.unsqueeze(0).contiguous(), v.unsqueeze(0).contiguous()
        res[name] = {}
        for variant, sg in (("plain_fwht", None), ("signed_rotation", signs)):
            cfg = pk.make_config(L, Hkv, d, T, [3] * L, v_signs=sg)
            buf = torch.empty(pk.pool_bytes(cfg), dtype=torch.uint8, device=dev)
            pool = pk.pool_build(cfg, buf.data_ptr(), buf.numel())
            pk.pool_quantize_append(pool, 0, k, v)
            ws = torch.empty(max(pk.agent_decode_attention([pool], q[0], out, 0),
                                 pk.agent_decode_attention([empty], q[0], ref, 0, kw, vw, [T])), dtype=torch.uint8,
                             device=dev)
            errs = []
            for r in range(R):
                pk.agent_decode_attention([pool], q[r], out, 0, workspace=ws)
                pk.agent_decode_attention([empty], q[r], ref, 0, kw, vw, [T], workspace=ws)
                errs.append(((out - ref).double().norm(dim=-1) / ref.double().norm(dim=-1)).flatten())
            e = torch.cat(errs)
            ts = []
            for r in range(12):
                pk.agent_decode_attention([pool], q[r % R], out, 0, workspace=ws, pool_events=(e0, e1))
                torch.cuda.synchronize()
                ts.append(1e3 * e0.elapsed_time(e1))
            res[name][variant] = {"attention_rel_error_mean": float(e.mean()),
                                  "attention_rel_error_max": float(e.max()),
                                  "pool_kernel_us": float(np.median(ts[2:]))}
            del buf
        log(f"[rotation] {name}: {json.dumps(res[name])}")
    print(json.dumps({"metric": "V codec ablation: plain FWHT vs randomized rotation (attention error, kernel time)",
                      "value": res["hadamard_aligned"]["signed_rotation"]["attention_rel_error_mean"],
                      "unit": "relative L2 error", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
                      "config": {"workload": "llama3_8b_shape_1_agent", "layers": L, "kv_heads": Hkv, "q_heads": Hq,
                                 "head_dim": d, "pool_tokens": T, "v_bits": 3, "query_steps": R},
                      "results": res}), flush=True)


def codec_ablation():
    """Codec variants on the Llama-3-8B-shaped workload (32 layers, 8 kv heads, d 128, 4096 pool
    tokens, 3 bits, K and V with LogNormal(0, 0.5) channel scales, 15 agents x 4 query steps).

    Per variant: K and V relative reconstruction error (sum of squared errors over the sum of
    squares, the pool's bytes dequantised here with torch from the documented layout and the
    library's centroid table), attention error per output row (relative L2 against fp32 torch
    attention over the same bf16 K/V), bytes per token and kv head, and the pool kernel's time
    (events; warm, and cold after a reduction over 1 GiB).
    """
    import torch

    import workloads as wl
    from quantized_shared_kv_amd import polykv as pk

    pk.lib()
    w = wl.LLAMA3_8B
    dev = "cuda:0"
    L, Hkv, Hq, d, T, A, G = w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.pool_tokens, w.n_agents, w.group
    R = 4

    def dev_bf16(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(dev)

    k = torch.stack([dev_bf16(w.pool_k(0, l).raw) for l in range(L)])
    v = torch.stack([dev_bf16(w.pool_v(0, l).raw) for l in range(L)])
    qs = [torch.stack([dev_bf16(w.queries(s, a).raw) for a in range(A)]).contiguous() for s in range(R)]
    kf, vf = k.float(), v.float()
    h = torch.ones((1, 1), device=dev)
    while h.shape[0] < d:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    cent = torch.tensor(pk.lloyd_max_table(3)[0], dtype=torch.float64, device=dev)
    sigma = 1.0 / np.sqrt(d)
    # exact attention per (step, layer): rows (agent, q head) grouped by kv head
    refs = []
    for s in range(R):
        qf = qs[s].float()  # [A][L][Hq][d]
        ref = torch.empty_like(qf)
        for l in range(L):
            qg = qf[:, l].reshape(A, Hkv, G, d).permute(1, 0, 2, 3).reshape(Hkv, A * G, d)
            sc = torch.matmul(qg, kf[l].transpose(1, 2).contiguous()) * sigma
            o = torch.matmul(torch.softmax(sc, dim=-1), vf[l])
            ref[:, l] = o.reshape(Hkv, A, G, d).permute(1, 0, 2, 3).reshape(A, Hq, d)
        refs.append(ref)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    variants = {"k_tensor (pages)": (pk.KSCALE_TENSOR, pk.VNORM_PLAIN), "k_token": (pk.KSCALE_TOKEN, pk.VNORM_PLAIN),
                "k_channel": (pk.KSCALE_CHANNEL, pk.VNORM_PLAIN),
                "v_corrected_norm": (pk.KSCALE_TENSOR, pk.VNORM_CORRECTED)}
    res = {}
    for name, (ks_mode, vn_mode) in variants.items():
        cfg = pk.make_config(L, Hkv, d, T, [3] * L, k_scale=ks_mode, v_norm=vn_mode)
        nb = pk.pool_bytes(cfg)
        buf = torch.empty(nb, dtype=torch.uint8, device=dev)
        pool = pk.pool_build(cfg, buf.data_ptr(), nb)
        pk.pool_quantize_append(pool, 0, k, v)
        torch.cuda.synchronize()
        tc = pool.tc
        # dequantise from the image: K_hat = Ks * Kq, V_hat = (Vn / d) H c[code]
        kq = buf[pool.off_kq:pool.off_kq + L * Hkv * tc * d].view(torch.int8).view(L, Hkv, tc, d)[:, :, :T].double()
        ksb = buf[pool.off_ks:pool.off_vmax]
        if ks_mode == pk.KSCALE_TENSOR:
            sc = ksb[:L * tc * 4].view(torch.float32).view(L, 1, tc, 1)[:, :, :T]
        elif ks_mode == pk.KSCALE_TOKEN:
            sc = ksb[:L * Hkv * tc * 4].view(torch.float32).view(L, Hkv, tc, 1)[:, :, :T]
        else:
            sc = ksb[:L * Hkv * d * 4].view(torch.float32).view(L, Hkv, 1, d)
        khat = kq * sc.double()
        vn = buf[pool.off_vn:pool.off_vn + L * Hkv * tc * 4].view(torch.float32).view(L, Hkv, tc)[:, :, :T].double()
        vc = buf[pool.off_vc[0]:pool.off_vc[L]].view(L, Hkv, tc // 8, d, 3).long()
        field = vc[..., 0] | (vc[..., 1] << 8) | (vc[..., 2] << 16)  # [L][Hkv][groups][d]
        codes = torch.stack([(field >> (3 * i)) & 7 for i in range(8)], dim=3).reshape(L, Hkv, tc, d)[:, :, :T]
        vhat = (vn[..., None] / d) * torch.matmul(cent[codes], h.double())
        k_err = float(((khat - kf.double()) ** 2).sum() / (kf.double() ** 2).sum())
        v_err = float(((vhat - vf.double()) ** 2).sum() / (vf.double() ** 2).sum())
        del kq, khat, vn, vc, field, codes, vhat
        out = torch.empty((A, L, Hq, d), dtype=torch.float32, device=dev)
        ws = torch.empty(max(pk.agent_decode_attention([pool] * A, qs[0], out, 0), 256), dtype=torch.uint8,
                         device=dev)
        errs = []
        for s in range(R):
            pk.agent_decode_attention([pool] * A, qs[s], out, 0, workspace=ws)
            torch.cuda.synchronize()
            errs.append(((out.double() - refs[s].double()).norm(dim=-1) / refs[s].double().norm(dim=-1)).flatten())
        e = torch.cat(errs)
        warm, cold = [], []
        for i in range(12):
            pk.agent_decode_attention([pool] * A, qs[i % R], out, 0, workspace=ws, pool_events=(e0, e1))
            torch.cuda.synchronize()
            warm.append(1e3 * e0.elapsed_time(e1))
        for i in range(8):
            flush.sum()
            pk.agent_decode_attention([pool] * A, qs[i % R], out, 0, workspace=ws, pool_events=(e0, e1))
            torch.cuda.synchronize()
            cold.append(1e3 * e0.elapsed_time(e1))
        res[name] = {"k_rel_sq_error": k_err, "v_rel_sq_error": v_err,
                     "attention_rel_error_mean": float(e.mean()), "attention_rel_error_max": float(e.max()),
                     "pool_bytes": nb, "bytes_per_token_per_kv_head": nb / (L * Hkv * T),
                     "pool_kernel_us_warm": float(np.median(warm[2:])), "pool_kernel_us_cold": float(np.mean(cold))}
        log(f"[codec] {name}: {json.dumps(res[name])}")
        del buf
    print(json.dumps({"metric": "codec variants: reconstruction and attention error, bytes, pool-kernel time",
                      "value": res["k_tensor (pages)"]["attention_rel_error_mean"], "unit": "relative L2 error",
                      "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
                      "config": {"workload": w.name, "layers": L, "kv_heads": Hkv, "q_heads": Hq, "head_dim": d,
                                 "pool_tokens": T, "agents": A, "v_bits": 3, "query_steps": R},
                      "results": res}), flush=True)


def comix_bench():
    """CoMixKV controller on the Qwen3-32B shape (8 agents, 64 layers, 64/8 heads, d 128).

    Each agent has a 128-token native window and 8 recent query steps (device-seeded
    bf16: K, V = N(0, 1) * sigma, sigma ~ LogNormal(0, 0.5) per (layer, kv head, channel);
    the second recipe also scales V by a per-(agent, layer) factor ~ LogNormal(0, 1)).
    Timed: comix_sensitivity (HIP events) and comix_allocate_bits (host).  Checked: with the
    budget of 3 bits everywhere, each agent's window is quantized into its own pool at the
    allocated per-layer widths and at uniform 3 bits, the recent queries are decoded over
    it, and the outputs are compared with exact attention over the bf16 window (the same
    decode call with an empty pool and the window as native suffix).
    """
    import torch

    from quantized_shared_kv_amd import polykv as pk

    pk.lib()
    dev = "cuda:0"
    A, L, Hq, Hkv, d, S, R = 8, 64, 64, 8, 128, 128, 8
    err = [pk.lloyd_max_distortion(b) ** 0.5 for b in (2, 3, 4)]
    cost_row = [S * (Hkv * (d + d * b // 8 + 4) + 4) for b in (2, 3, 4)]  # one layer of one agent's block
    budget = A * L * cost_row[1]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for recipe in ("channel_lognormal", "channel_and_layer_lognormal"):
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        q = torch.randn((R, A, L, Hq, d), generator=g, device=dev).to(torch.bfloat16)
        sk = torch.exp(0.5 * torch.randn((1, L, Hkv, 1, d), generator=g, device=dev))
        sv = torch.exp(0.5 * torch.randn((1, L, Hkv, 1, d), generator=g, device=dev))
        if recipe != "channel_lognormal":
            sv = sv * torch.exp(torch.randn((A, L, 1, 1, 1), generator=g, device=dev))
        wk = (torch.randn((A, L, Hkv, S, d), generator=g, device=dev) * sk).to(torch.bfloat16)
        wv = (torch.randn((A, L, Hkv, S, d), generator=g, device=dev) * sv).to(torch.bfloat16)
        sens = torch.empty((A, L), dtype=torch.float32, device=dev)
        for _ in range(2):
            pk.comix_sensitivity(q, wk, wv, [S] * A, sens)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            pk.comix_sensitivity(q, wk, wv, [S] * A, sens)
        e1.record()
        torch.cuda.synchronize()
        sens_us = 1e3 * e0.elapsed_time(e1) / 10
        s_host = sens.cpu().numpy().ravel()
        t0 = time.perf_counter()
        bits = pk.comix_allocate_bits(s_host, [cost_row] * (A * L), err, budget)
        alloc_us = 1e6 * (time.perf_counter() - t0)
        bits = np.array(bits).reshape(A, L)

        def decode_error(bits_al):
            bufs, pools = [], []
            for a in range(A):
                cfg = pk.make_config(L, Hkv, d, S, [int(b) for b in bits_al[a]])
                n = pk.pool_bytes(cfg)
                bufs.append(torch.empty(n, dtype=torch.uint8, device=dev))
                pools.append(pk.pool_build(cfg, bufs[-1].data_ptr(), n))
                pk.pool_quantize_append(pools[-1], 0, wk[a].contiguous(), wv[a].contiguous())
            empty_cfg = pk.make_config(L, Hkv, d, S, [3] * L)
            ne = pk.pool_bytes(empty_cfg)
            ebufs = [torch.empty(ne, dtype=torch.uint8, device=dev) for _ in range(A)]
            empty = [pk.pool_build(empty_cfg, b.data_ptr(), ne) for b in ebufs]
            out = torch.empty((A, L, Hq, d), dtype=torch.float32, device=dev)
            ref = torch.empty_like(out)
            wsb = max(pk.agent_decode_attention(pools, q[0], out, 0),
                      pk.agent_decode_attention(empty, q[0], ref, 0, wk, wv, [S] * A))
            ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
            rel_sum = torch.zeros((A, L), dtype=torch.float64, device=dev)
            abs_sum = torch.zeros((A, L), dtype=torch.float64, device=dev)
            for r in range(R):
                pk.agent_decode_attention(pools, q[r], out, 0, workspace=ws)
                pk.agent_decode_attention(empty, q[r], ref, 0, wk, wv, [S] * A, workspace=ws)
                diff = (out - ref).double().norm(dim=-1)
                rel_sum += (diff / ref.double().norm(dim=-1)).mean(dim=-1)
                abs_sum += diff.mean(dim=-1)
            torch.cuda.synchronize()
            return (rel_sum / R).cpu().numpy(), (abs_sum / R).cpu().numpy()

        e_alloc, a_alloc = decode_error(bits)
        e_uni, a_uni = decode_error(np.full((A, L), 3))
        s64 = s_host.astype(np.float64)
        res[recipe] = {
            "sensitivity_us": sens_us, "allocate_us": alloc_us,
            "bits_hist": {str(b): int(np.sum(bits == b)) for b in (2, 3, 4)},
            "bytes": {"budget": budget, "used": int(sum(cost_row[b - 2] for b in bits.ravel()))},
            "predicted_error_sum": {"uniform_3bit": float(np.sum(s64 * err[1])),
                                    "allocated": float(np.sum(s64 * np.array(err)[bits.ravel() - 2]))},
            "attention_abs_error_sum": {"uniform_3bit": float(a_uni.sum()), "allocated": float(a_alloc.sum())},
            "attention_rel_error_mean": {"uniform_3bit": float(e_uni.mean()), "allocated": float(e_alloc.mean())},
            "attention_rel_error_worst_item": {"uniform_3bit": float(e_uni.max()), "allocated": float(e_alloc.max())},
        }
        log(f"[comix] {recipe}: {json.dumps(res[recipe])}")
    # sensitivity kernel roofline: with bf16 operands the scores run on the matrix cores and the
    # kernel streams the windows (bf16 K and V) and the recent queries once: bound by HBM; the
    # multiply-adds (scores and ||v|| sums) are reported beside it
    flops = A * L * Hkv * (R * (Hq // Hkv) * S * d * 2 + S * d * 2)
    sens_bytes = A * L * Hkv * S * d * 2 * 2 + R * A * L * Hq * d * 2 + A * L * 4
    first = res["channel_lognormal"]
    sens_s = first["sensitivity_us"] * 1e-6
    print(json.dumps({"metric": "CoMixKV controller: sensitivity kernel time and allocation quality",
                      "value": first["sensitivity_us"], "unit": "us", "higher_is_better": False, "n_gpus": 1,
                      "dtype": "bf16 operands, fp32 accumulation", "data": "synthetic",
                      "config": {"workload": "qwen3_32b_comix_controller", "agents": A, "layers": L, "q_heads": Hq,
                                 "kv_heads": Hkv, "head_dim": d, "window": S, "recent_steps": R,
                                 "budget": "bytes of 3 bits everywhere"},
                      "roofline": {"bound": "hbm", "achieved": sens_bytes / sens_s / 1e9, "peak": HBM_PEAK_GBPS,
                                   "unit": "GB/s", "frac": sens_bytes / sens_s / 1e9 / HBM_PEAK_GBPS,
                                   "kernel": "comix sensitivity (k_comix_mfma)", "bytes_per_launch": sens_bytes,
                                   "flops_per_launch": flops, "tflops": flops / sens_s / 1e12},
                      "recipes": res}), flush=True)


def cpu_baseline(w, steps_per_job):
    """The oracle, untuned, on a bounded sample of the same job, scaled to agent-tokens/s.

    Sample: layers 0-15 of the pool build (oracle codec on the same bf16 values)
    and decode steps 0-7 over those layers for all agents (fp64 oracle attention,
    suffix of s + 1 tokens at step s).  Job time = L/16 * (build of 16 layers +
    steps_per_job * mean decode step of 16 layers).
    """
    from oracle import attention, pool_image

    threads = len(os.sched_getaffinity(0))
    L, T, A = w.n_layers, w.pool_tokens, w.n_agents
    nl, ns = 16, 8
    t0 = time.perf_counter()
    img = pool_image.PoolImage(nl, w.n_kv_heads, w.head_dim, T, w.v_bits(0)[:nl])
    img.append(0, np.stack([w.pool_k(0, l).f32 for l in range(nl)]), np.stack([w.pool_v(0, l).f32 for l in range(nl)]))
    t_build = time.perf_counter() - t0
    sk = [[w.sfx_k(a, l).f32 for l in range(nl)] for a in range(A)]
    sv = [[w.sfx_v(a, l).f32 for l in range(nl)] for a in range(A)]
    cache = {}

    def decoded(p, l, g):
        if (l, g) not in cache:
            cache[(l, g)] = img.decoded_layer(l, g)
        return cache[(l, g)]

    t_dec = 0.0
    for s in range(ns):
        q = np.stack([w.queries(s, a).f32[:nl] for a in range(A)])
        t1 = time.perf_counter()
        attention.decode_call(q, [0] * A, decoded, lambda a, l: sk[a][l], lambda a, l: sv[a][l],
                              [w.sfx_len(s)] * A, w.n_kv_heads)
        t_dec += time.perf_counter() - t1
    t_step = t_dec / ns
    job = (L / nl) * (t_build + steps_per_job * t_step)
    return {"value": A * steps_per_job / job, "unit": "agent-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"layers 0-{nl - 1}: pool build ({t_build:.2f}s) + decode steps 0-{ns - 1} for {A} agents "
                      f"({t_step:.2f}s per step), scaled x{L / nl:g} layers and x{steps_per_job} decode steps",
            "sample_seconds": t_build + t_dec}


if __name__ == "__main__":
    main()
