#!/usr/bin/env python3
"""Throughput of the Orthrus draft -> verify -> accept -> commit step on one
MI355X, on a random-init Qwen3-8B-shaped model (synthetic, seeded).

A step is one pass of the whole hot path for every sequence of the batch:
pass 1 (anchor + K mask rows through all layers, LM-head argmax), the
planted-draft copy, pass 2 (K verify rows), acceptance and commit.  Drafts
are planted from the model's own greedy trajectory so that each step
accepts a seeded number of tokens (the random model's own drafts would
almost never be accepted); the timed loop does all the work of a real step.

Prints ONE JSON line (everything else goes to stderr):
  value          verified tokens/s = sum over steps and sequences of (m+1) / time
  roofline       the dominant kernel (the draft pass's gate/up SwiGLU GEMM):
                 algorithmic bytes per launch / its average duration, timed
                 with HIP events around its launches inside the timed region
  cpu_baseline   the CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemm_gateup_draft_pmc.txt")


def tpf_from_accept(mean_accept: float) -> float:
    """Tokens per forward: a step emits m+1 tokens with two forward passes."""
    return (mean_accept + 1.0) / 2.0


MFMA_PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, published


def KV_BYTES_PER_TOKEN(sh):
    """K and V of one token, all layers, bf16."""
    return sh["L"] * 2 * sh["hkv"] * sh["hd"] * 2


def step_weight_bytes(sh):
    """Weight bytes one draft + verify step streams (bf16): pass 1 reads the
    frozen and the diffusion Q/K/V/O, the FFN and the LM head; pass 2 the
    frozen Q/K/V/O, the FFN and the LM head."""
    d, qd, kd, F, V, L = sh["d"], sh["hq"] * sh["hd"], sh["hkv"] * sh["hd"], sh["F"], sh["V"], sh["L"]
    qkvo = d * qd + 2 * d * kd + qd * d
    ffn = 3 * d * F
    return 2 * (L * (2 * qkvo + ffn) + d * V) + 2 * (L * (qkvo + ffn) + d * V)


def step_gemm_flops(sh, B, K):
    """GEMM flops of one step: pass 1 has B anchor rows on the frozen
    projections and B*K mask rows on the diffusion ones, all B*(K+1) rows
    through the FFN and LM head; pass 2 has B*K rows through the frozen
    model."""
    d, qd, kd, F, V, L = sh["d"], sh["hq"] * sh["hd"], sh["hkv"] * sh["hd"], sh["F"], sh["V"], sh["L"]
    qkvo = d * qd + 2 * d * kd + qd * d
    ffn = 3 * d * F
    draft = B * (K + 1) * (L * (qkvo + ffn) + d * V)
    verify = B * K * (L * (qkvo + ffn) + d * V)
    return 2 * (draft + verify)


def hbm_read_probe(dev, nbytes=4 << 30, reps=10):
    """The box's achievable HBM read rate: a 4 GiB buffer read once per launch
    by the library's read probe (16-byte loads, one XOR fold per workgroup),
    best over two grid sizes."""
    import torch
    from lossless_decoding_amd import _lib as C
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    out = torch.zeros(4096, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    best = (0.0, 0)
    for nwg in (1024, 2048, 4096):
        for _ in range(2):
            C.orthrus_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), nwg, st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            C.orthrus_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), nwg, st)
        e1.record()
        torch.cuda.synchronize()
        gbps = nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
        best = max(best, (gbps, nwg))
    del buf, out
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 1), "frac_of_8TBps": round(best[0] / 8000, 4), "bytes": nbytes,
            "workgroups": best[1]}


def kernel_a_bench(dev, points=((4, 16384), (16, 4096)), rows=32, hq=32, hkv=8, kb=32, reps=20):
    """Kernel (a) alone (orthrus_block_attention) at the configurations with
    at least 256 MB of cache K/V: `rows` mask rows per sequence see Lk cache
    keys and kb block keys.  Seeded N(0, 1) bf16 inputs; four independent
    buffer sets are rotated so that the 256 MB Infinity Cache does not hold
    the keys between launches.  Algorithmic bytes = cache K/V + block K/V +
    Q + output."""
    import torch

    import synth
    from lossless_decoding_amd import _lib as C
    from lossless_decoding_amd.layout import tile_v, tile_block_v
    from synth import workloads
    from synth.device import fill_normal_device

    res = []
    for B, lk in points:
        sets = []
        for i in range(4):
            st = workloads.attn_inputs_stream(B, lk) + 100 * i
            q = torch.empty(B, rows, hq, 128, dtype=torch.bfloat16, device=dev)
            fill_normal_device(q, workloads.ATTN_SEED, st, 1.0, synth.P_ATTN)
            kc = torch.empty(B, hkv, lk, 128, dtype=torch.bfloat16, device=dev)
            fill_normal_device(kc, workloads.ATTN_SEED, st + 1, 1.0, synth.P_ATTN)
            vc = torch.empty_like(kc)
            fill_normal_device(vc, workloads.ATTN_SEED, st + 2, 1.0, synth.P_ATTN)
            vt = tile_v(vc)
            del vc
            kbk = torch.empty(B, hkv, kb, 128, dtype=torch.bfloat16, device=dev)
            fill_normal_device(kbk, workloads.ATTN_SEED, st + 3, 1.0, synth.P_ATTN)
            vbk = torch.empty_like(kbk)
            fill_normal_device(vbk, workloads.ATTN_SEED, st + 4, 1.0, synth.P_ATTN)
            sets.append((q, kc, vt, kbk, tile_block_v(vbk, 32)))
        out = torch.empty(B, rows, hq, 128, dtype=torch.bfloat16, device=dev)
        wsb = C.orthrus_attention_workspace(B, rows, hq, hkv, lk)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream().cuda_stream

        def go(i):
            q, kc, vt, kbk, vbt = sets[i % 4]
            C.orthrus_block_attention(B, rows, hq, hkv, q.data_ptr(), kc.data_ptr(), vt.data_ptr(), lk,
                                      lk, kbk.data_ptr(), vbt.data_ptr(), kb, out.data_ptr(),
                                      ws.data_ptr(), wsb, stream)
        for i in range(4):
            go(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            go(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        alg = B * hkv * (lk + kb) * 128 * 2 * 2 + 2 * B * rows * hq * 128 * 2
        res.append({"batch": B, "cache_keys": lk, "block_keys": kb, "rows": rows, "us": round(us, 2),
                    "algorithmic_bytes": alg, "achieved_GBps": round(alg / us / 1e3, 1),
                    "frac_of_8TBps": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)})
        log(f"[kernel a] B={B} Lk={lk}: {us:.1f} us, {alg / us / 1e3:.0f} GB/s")
        del sets, out, ws
        torch.cuda.empty_cache()
    return res


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "lossless_decoding_amd", "csrc", "k_gemm.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def workload_desc(name, wl, sh):
    law = {"geom6": "planted accept length min(Geom(1/7), 32), mean 6",
           "uniform32": "planted accept length uniform{0..32}"}[wl["plant"]]
    return (f"{name}: Qwen3-8B-shaped random-init model (L={sh['L']}, d={sh['d']}, "
            f"{sh['hq']}q/{sh['hkv']}kv heads x {sh['hd']}, SwiGLU {sh['F']}, vocab {sh['V']}, "
            f"bf16), batch {wl['B']}, prompt {wl['P']} uniform-random tokens, K={sh['K']}, {law}")


def cpu_baseline(sh, wl, mean_tokens_per_step):
    """Oracle (plain fp64 C, as it stands) on one full draft+verify step of
    one sequence at the full model shape after a short prefill."""
    import numpy as np

    import oracle
    from synth import workloads

    t0 = time.time()
    shp = oracle.ModelShape(**sh)
    lay, total = oracle.weight_layout(shp)
    w = workloads.fill_weights(lay, total, True)
    log(f"[cpu] weights generated in {time.time() - t0:.1f}s")
    m = oracle.Model(shp, w)
    P0 = 4
    prompt = workloads.prompts(1, P0, sh["V"])[0]
    seq = m.seq(P0 + sh["K"] + 4)
    t1 = time.time()
    pending = seq.prefill(prompt)
    t2 = time.time()
    r = seq.step(pending, sh["K"])
    t3 = time.time()
    step_s = t3 - t2
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    log(f"[cpu] prefill {P0} rows {t2 - t1:.1f}s, one step {step_s:.1f}s, m={r['m']}")
    return {
        "value": mean_tokens_per_step / step_s,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"one draft+verify step (2 passes, 36 layers, K={sh['K']}, 1 sequence) of the "
                   f"fp64 oracle after a {P0}-token prefill, {step_s:.1f} s; tokens/s = the "
                   f"workload's mean tokens per step ({mean_tokens_per_step:.3f}) / step time"),
        "step_seconds": step_s,
        "host": host_info(),
    }


def gemm_class_rates(breakdown, sh, B, K):
    """Per GEMM class and pass, from the per-class times: weight bytes
    streamed (bf16, every layer; the draft pass's QKV and O read both the
    frozen and the diffusion matrices) against 8 TB/s, and GEMM flops
    (2 x rows x parameters) against the dense bf16 MFMA peak.  The class
    times come from event pairs around every launch (a few microseconds of
    record overhead each) and the QKV class includes its finish kernel when
    split, so these are lower bounds of the kernels' own rates."""
    L, d, F, V = sh["L"], sh["d"], sh["F"], sh["V"]
    qkv = d * (sh["hq"] + 2 * sh["hkv"]) * sh["hd"]
    o = sh["hq"] * sh["hd"] * d
    params = {"qkv": (qkv, L), "o_proj": (o, L), "gate_up": (2 * F * d, L), "down": (F * d, L),
              "lm_head": (V * d, 1)}
    rows = {"draft": B * (K + 1), "verify": B * K}
    out = {}
    for key, ms in breakdown.items():
        pas, _, cls = key.partition(".")
        if cls not in params or pas not in rows or ms <= 0:
            continue
        n, per = params[cls]
        sets = 2 if pas == "draft" and cls in ("qkv", "o_proj") else 1
        wbytes = sets * n * 2 * per
        flops = 2 * rows[pas] * n * per
        s_ = ms / 1e3
        out[key] = {"ms": ms, "weight_GBps": round(wbytes / s_ / 1e9, 1),
                    "hbm_frac": round(wbytes / s_ / 8e12, 4),
                    "tflops": round(flops / s_ / 1e12, 2),
                    "mfma_frac": round(flops / s_ / 2.5e15, 4)}
    return out


def host_info():
    """The host the oracle ran on: CPU model, sockets, logical CPUs visible to
    this process, memory."""
    model, sockets = "", set()
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            if k.strip() == "model name" and not model:
                model = v.strip()
            elif k.strip() == "physical id":
                sockets.add(v.strip())
    except OSError:
        pass
    mem_gib = None
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal:"):
                mem_gib = round(int(line.split()[1]) / (1 << 20), 1)
    except OSError:
        pass
    return {"cpu": model, "sockets": len(sockets) or None, "logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "mem_gib": mem_gib}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--roofline-steps", type=int, default=4,
                    help="timed steps whose gate/up launches carry HIP events for the roofline "
                         "(the first ones of the timed region; each event pair adds a few us)")
    ap.add_argument("--workload", default="qwen3_8b_b1_p512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=8)
    ap.add_argument("--no-kernel-a", action="store_true",
                    help="skip the block-attention kernel and HBM read-rate measurements")
    ap.add_argument("--attn-chunk", type=int, default=0,
                    help="attention key chunk of both contexts (default: the library's rule)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run plain 1 GiB device copies (PMC byte-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sequences shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lossless_decoding_amd import _lib as C
    from lossless_decoding_amd.engine import Engine, attn_chunk_for
    from synth import workloads
    from synth.device import fill_weights_device

    wl = workloads.WORKLOADS[args.workload]
    sh = workloads.SHAPES[wl["shape"]]
    B, P, K, V = wl["B"], wl["P"], sh["K"], sh["V"]
    W, S = args.warmup, args.steps
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    a = workloads.plant_lengths(W + S, B, K, wl["plant"])
    need = 1 + int((a + 1).sum(0).max()) + K + 2          # trajectory tokens per sequence
    max_ctx = P + (W + S) * (K + 1) + 64                  # host bound grows K+1 per step
    t0 = time.time()
    # both contexts fold attention over the same key chunks, so their rows are
    # bit-identical (the lossless check below compares them token for token)
    chunk = args.attn_chunk or attn_chunk_for(max_ctx, B, sh["hkv"])
    cfg = C.OrthrusConfig.make(sh["L"], sh["d"], sh["hq"], sh["hkv"], sh["hd"], sh["F"], V, K,
                               True, B, max_ctx, attn_chunk=chunk)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    eng = Engine(cfg, w)
    cfg0 = C.OrthrusConfig.make(sh["L"], sh["d"], sh["hq"], sh["hkv"], sh["hd"], sh["F"], V, 0,
                                True, B, P + need + 8, attn_chunk=chunk)
    ar = Engine(cfg0, w)
    del w
    torch.cuda.synchronize()
    log(f"[setup] weights + two contexts in {time.time() - t0:.1f}s "
        f"(packed {eng.sizes.packed_bytes / 1e9:.2f} GB, KV {eng.sizes.kv_bytes / 1e9:.2f} GB)")

    prompts = workloads.prompts(B, P, V)
    # greedy trajectory from the plain-decoding context (same kernels, K = 0)
    t0 = time.time()
    ar.prefill(prompts)
    traj = torch.zeros(need, B, dtype=torch.int32, device=dev)
    traj[0] = ar.pending[:B]
    # the same kernels in plain greedy decoding (K = 0): one token per
    # sequence per step, timed for the speedup figure
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for j in range(1, need):
        ar.draft(); ar.verify(); ar.commit()
        traj[j] = ar.pending[:B]
    a1.record()
    torch.cuda.synchronize()
    plain_tps = B * (need - 1) / (a0.elapsed_time(a1) / 1e3)
    traj = traj.t().contiguous().cpu().numpy()
    ar_s = time.time() - t0
    log(f"[setup] greedy trajectory of {need} tokens x {B} in {ar_s:.1f}s "
        f"(plain decoding {plain_tps:.1f} tokens/s)")
    ar.close()
    del ar
    planted = torch.from_numpy(workloads.plant_drafts(traj, 1, a, K, V)).to(dev)

    # ---------------------------------------------------------------- timed
    # prefill (the prompts through the AR view into the cache), timed on its
    # own and reported beside the step loop
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    eng.prefill(prompts)
    p1.record()
    torch.cuda.synchronize()
    prefill_ms = p0.elapsed_time(p1)
    log(f"[prefill] {B} x {P} prompt tokens in {prefill_ms:.1f} ms")
    for s in range(W):
        eng.draft(); eng.drafts[:B].copy_(planted[s]); eng.verify(); eng.commit()
    cls = C.timing_class("draft", "gate_up")
    # events around the draft gate/up launches of the first roofline-steps
    # timed steps (the library stops recording at the capacity)
    n_rs = max(1, min(args.roofline_steps, S))
    C.orthrus_timing_enable(eng.ctx, 1 << cls, n_rs * sh["L"])
    torch.cuda.synchronize()
    # one event per step boundary (the first and last bracket the timed region)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(S + 1)]
    t_wall = time.perf_counter()
    ev[0].record()
    for s in range(W, W + S):
        eng.draft()
        eng.drafts[:B].copy_(planted[s])
        eng.verify()
        eng.commit()
        ev[s - W + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev[0].elapsed_time(ev[S])
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(S)])
    tim, _ = C.orthrus_timing_read(eng.ctx)
    C.orthrus_timing_enable(eng.ctx, 0, 0)

    tokens = int((a[W:W + S] + 1).sum())
    ms_step = ms / S
    # correctness of the timed run: lengths and the emitted stream match greedy decoding
    seq_len = eng.seq_len[:B].cpu().numpy()
    want_len = P + (a + 1).sum(0)
    pend = eng.pending[:B].cpu().numpy()
    e_end = 1 + (a + 1).sum(0)
    lossless = bool((seq_len == want_len).all() and
                    all(pend[b] == traj[b, e_end[b] - 1] for b in range(B)))
    step_pct = {f"p{q}": round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)}
    log(f"[timed] {S} steps in {ms:.1f} ms ({ms_step:.3f} ms/step, wall {wall * 1e3:.1f} ms), "
        f"{tokens} tokens, lossless={lossless}, step ms {step_pct}")

    # dominant kernel: the draft pass's gate/up SwiGLU GEMM (M = B*(K+1) rows)
    gu_ms, gu_n = tim.get(("draft", "gate_up"), (0.0, 0))
    M1 = B * (K + 1)
    gu_bytes = 2 * sh["F"] * sh["d"] * 2 + M1 * sh["d"] * 2 + M1 * sh["F"] * 2
    gu_avg_s = gu_ms / max(gu_n, 1) / 1e3
    # the instantiation the library launches for it (row tiles, waves per workgroup)
    gu_mt = min(4, (M1 + 15) // 16)
    gu_wv = 6 if (2 * sh["F"] // 16) % 6 == 0 and gu_mt <= 3 else 8
    achieved = gu_bytes / gu_avg_s / 1e9 if gu_n else 0.0
    traffic = None
    if os.path.exists(PROFILE_PMC):
        pm = dict(l.split(": ", 1) for l in open(PROFILE_PMC).read().splitlines()
                  if l and not l.startswith("#"))
        if pm.get("kernel_source_hash") == kernel_source_hash() and \
                pm.get("workload") == args.workload:
            traffic = int(pm["hbm_bytes_per_launch"])

    # per-class breakdown over a few more steps (all classes timed)
    breakdown = {}
    if args.breakdown_steps > 0:
        # a few more steps with every class timed (acceptance differs: the
        # planted rows no longer line up with the trajectory; cost does not)
        C.orthrus_sync_lengths(eng.ctx, B, seq_len)
        extra = min(args.breakdown_steps, (max_ctx - int(seq_len.max()) - 64) // (K + 1))
        C.orthrus_timing_enable(eng.ctx, (1 << 24) - 1, max(extra, 1) * 800 + 64)
        for j in range(extra):
            eng.draft(); eng.drafts[:B].copy_(planted[W + j]); eng.verify(); eng.commit()
        torch.cuda.synchronize()
        tb, _ = C.orthrus_timing_read(eng.ctx)
        C.orthrus_timing_enable(eng.ctx, 0, 0)
        if extra > 0:
            breakdown = {f"{p}.{r}": round(v[0] / extra, 4) for (p, r), v in sorted(tb.items())}
        log(f"[breakdown] ms per step by class over {extra} steps: {breakdown}")
    gemm_classes = gemm_class_rates(breakdown, sh, B, K)

    if args.calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[calibrate] 3 plain copies of 1 GiB")

    # whole-step roofline: algorithmic bytes of the timed steps (weights of
    # both passes + the cache keys each pass must read) at 8 TB/s
    wb = step_weight_bytes(sh)
    n0 = P + np.concatenate([np.zeros((1, B), np.int64), np.cumsum(a + 1, axis=0)])[W:W + S]
    kv_b = float(((2 * n0 + K + 2) * KV_BYTES_PER_TOKEN(sh)).sum())
    step_bytes = S * wb + kv_b
    step_roof_ms = step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    gemm_flops = step_gemm_flops(sh, B, K) * S
    kernel_a = kernel_a_bench(dev) if not args.no_kernel_a else None
    read_probe = hbm_read_probe(dev) if not args.no_kernel_a else None

    out = {
        "metric": "verified tokens/s (and draft+verify steps/s) on 1 GPU; % of HBM roofline",
        "value": round(tokens / (ms / 1e3), 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and prompts, planted drafts)",
        "config": {"workload": workload_desc(args.workload, wl, sh), "batch": B,
                   "prompt_len": P, "block_k": K, "parallelism": "none (1 GPU)"},
        "attn_chunk": chunk,
        "steps_per_s": round(S / (ms / 1e3), 3),
        "step_ms_percentiles": step_pct,
        "tokens_per_step": round(tokens / S, 4),
        "tpf": round(tpf_from_accept(tokens / S / B - 1.0), 4),
        "prefill_ms": round(prefill_ms, 3),
        "prefill_tokens_per_s": round(B * P / (prefill_ms / 1e3), 1),
        "lossless_vs_greedy": lossless,
        "plain_decoding_tokens_per_s": round(plain_tps, 3),
        "speedup_vs_plain_decoding": round(tokens / (ms / 1e3) / plain_tps, 4),
        "step_roofline": {"bytes_per_step": round(step_bytes / S), "roofline_ms": round(step_roof_ms / S, 4),
                          "frac": round(step_roof_ms / ms, 4),
                          "gemm_tflops_per_s": round(gemm_flops / (ms / 1e3) / 1e12, 2),
                          "mfma_frac_bf16": round(gemm_flops / (ms / 1e3) / MFMA_PEAK_BF16, 4)},
        "roofline": {
            "kernel": f"k_gemm_bf16<{gu_mt}, EP_SWIGLU, {gu_wv}, false, 1> (draft-pass gate/up "
                      f"SwiGLU GEMM, M={M1}, N={2 * sh['F']}, K={sh['d']})",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_avg_s * 1e6, 3),
            "launches": gu_n,
            "timed_steps": n_rs,
        },
        "ms_per_step_by_class": breakdown,
        "gemm_classes": gemm_classes,
        "kernel_a": kernel_a,
        "hbm_read_achievable": read_probe,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(sh, wl, tokens / S / B)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
