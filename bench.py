#!/usr/bin/env python3
"""Throughput of the Orthrus draft -> verify -> accept -> commit step on one
MI355X, on random-init Qwen3-8B-shaped models (synthetic, seeded).

A step is one pass of the whole hot path for every sequence of the batch:
pass 1 (anchor + K mask rows through all layers, LM-head argmax), the
planted-draft copy, pass 2 (K verify rows), acceptance and commit.  Drafts
are planted from the model's own greedy trajectory so that each step
accepts a seeded number of tokens (a random model's own drafts would almost
never be accepted); the timed loop does all the work of a real step.

The headline workload is the largest single-GPU one: 8 sequences with a
32768-token context each (38.65 GB of KV cache), K = 32, planted accept
length uniform on {0..32}.  The batch-1 / 512-token and 16 x 8192 workloads
are run after it and reported as extra keys.

Prints ONE JSON line (everything else goes to stderr):
  value          verified tokens/s = sum over steps and sequences of (m+1) / time
  roofline       the dominant kernel of the headline workload, the draft
                 pass's block attention (kernel (a): the attention kernel and
                 its chunk merge): algorithmic bytes per launch / its average
                 duration, from HIP events on the launch stream around its
                 launches inside the timed region
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
MFMA_PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "qwen3_8b_b8_c32768"
# (steps, warmup) of each workload when it is not the headline
SECONDARY = {"qwen3_8b_b1_p512": (60, 4), "qwen3_8b_b16_c8192": (10, 2),
             "qwen3_8b_b8_c32768": (10, 2)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def tpf_from_accept(mean_accept: float) -> float:
    """Tokens per forward: a step emits m+1 tokens with two forward passes."""
    return (mean_accept + 1.0) / 2.0


def prefill_roofline(sh, B, P, rows_per_pass, prefill_ms):
    """A lower bound for the prefill of B prompts of P tokens in passes of
    rows_per_pass rows per sequence: per part, max(bytes / 8 TB/s, flops /
    2.5 PFLOP/s).  GEMMs: every pass reads the frozen view's layer weights
    once (bf16) and multiplies them with its rows, plus the LM head for the
    last row of each sequence.  Attention: a prompt row at position t sees
    t + 1 keys (Q.K and P.V, 4 flops per key and dimension per query head);
    a pass reads the cache keys and values its rows can see once and writes
    its own."""
    L, d, hq, hkv, hd, F, V = (sh[k] for k in ("L", "d", "hq", "hkv", "hd", "F", "V"))
    layer_params = d * (hq + 2 * hkv) * hd + hq * hd * d + 3 * F * d
    passes = -(-P // rows_per_pass)
    gemm_flops = 2.0 * L * layer_params * B * P + 2.0 * d * V * B
    gemm_bytes = 2.0 * (passes * L * layer_params + d * V)
    attn_flops = 4.0 * hd * hq * L * B * P * (P + 1) / 2
    seen = sum(min(P, (p + 1) * rows_per_pass) for p in range(passes))
    kv_bytes = kv_bytes_per_token(sh) * B * (seen + P)
    g = max(gemm_bytes / (HBM_PEAK_GBS * 1e9), gemm_flops / MFMA_PEAK_BF16)
    a = max(kv_bytes / (HBM_PEAK_GBS * 1e9), attn_flops / MFMA_PEAK_BF16)
    return {"method": "GEMMs and attention, each max(bytes / 8 TB/s, flops / 2.5 PFLOP/s)",
            "passes": passes, "gemm_tflop": round(gemm_flops / 1e12, 1),
            "attention_tflop": round(attn_flops / 1e12, 1),
            "roofline_ms": round((g + a) * 1e3, 3), "frac": round((g + a) * 1e3 / prefill_ms, 4)}


def kv_bytes_per_token(sh):
    """K and V of one token, all layers, bf16."""
    return sh["L"] * 2 * sh["hkv"] * sh["hd"] * 2


def gemm_classes_of(sh):
    """Per GEMM class: (parameters per layer, layers)."""
    L, d, F, V = sh["L"], sh["d"], sh["F"], sh["V"]
    qkv = d * (sh["hq"] + 2 * sh["hkv"]) * sh["hd"]
    o = sh["hq"] * sh["hd"] * d
    return {"qkv": (qkv, L), "o_proj": (o, L), "gate_up": (2 * F * d, L), "down": (F * d, L),
            "lm_head": (V * d, 1)}


def step_roofline(sh, B, K, n0):
    """Roofline time of one step whose sequences start at lengths n0 [B]:
    the sum over kernel classes of max(bytes / 8 TB/s, flops / 2.5 PFLOP/s).
    GEMM classes: weight bytes (bf16; the draft pass's QKV and O read both
    the frozen and the diffusion matrices) against 2 x rows x parameters.
    Attention: the cache K/V each pass must read (draft: slots [0, n] plus
    the block; verify: [0, n + K]), which is HBM-bound.  Returns (seconds,
    bytes, gemm flops)."""
    t = 0.0
    byts = 0.0
    flops = 0.0
    rows = {"draft": B * (K + 1), "verify": B * K}
    for cls, (n, per) in gemm_classes_of(sh).items():
        for pas, r in rows.items():
            sets = 2 if pas == "draft" and cls in ("qkv", "o_proj") else 1
            wb = sets * n * 2 * per
            fl = 2 * r * n * per
            t += max(wb / (HBM_PEAK_GBS * 1e9), fl / MFMA_PEAK_BF16)
            byts += wb
            flops += fl
    kvt = kv_bytes_per_token(sh)
    kv = float(((n0 + 1 + K) * kvt).sum() + ((n0 + 1 + K) * kvt).sum())
    t += kv / (HBM_PEAK_GBS * 1e9)
    return t, byts + kv, flops


def attn_launch_bytes(sh, B, K, n0, kind):
    """Algorithmic bytes of one layer's attention launch: every visible cache
    key's K and V once (draft: slots [0, n] incl. the staged anchor, plus the
    K block keys; verify: [0, n + K]), the queries read and the outputs
    written (bf16)."""
    hkv, hd, hq = sh["hkv"], sh["hd"], sh["hq"]
    if kind == "draft":
        keys = (n0 + 1 + K).sum()
        rows = B * (K + 1)
    else:
        keys = (n0 + 1 + K).sum()
        rows = B * K
    return float(keys * hkv * hd * 2 * 2 + 2 * rows * hq * hd * 2)


def hbm_read_probe(dev, nbytes=4 << 30, reps=10):
    """The device's achievable HBM read rate: a 4 GiB buffer read once per launch
    by the library's read probe (16-byte loads, one XOR fold per workgroup),
    best over three grid sizes."""
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


def kernel_a_bench(dev, rows=32, hq=32, hkv=8, kb=32, reps=20):
    """Kernel (a) alone (orthrus_block_attention) at all twelve points of the
    block-attention microbenchmark: `rows` mask rows per sequence see Lk cache
    keys and kb block keys, Lk in {1024, 4096, 16384, 32768} x batch
    {1, 4, 16}.  Seeded N(0, 1) bf16 inputs; enough independent buffer sets
    are rotated (at least 4, at least 1 GB in all) that the 256 MB Infinity
    Cache does not hold the keys between launches.  Algorithmic bytes = cache
    K/V + block K/V + Q + output; points under 20 us at 8 TB/s are
    launch- or latency-bound and flagged so."""
    import torch

    import synth
    from lossless_decoding_amd import _lib as C
    from lossless_decoding_amd.layout import tile_v, tile_block_v
    from synth import workloads
    from synth.device import fill_normal_device

    res = []
    for lk, B in workloads.ATTN_GRID:
        alg = B * hkv * (lk + kb) * 128 * 2 * 2 + 2 * B * rows * hq * 128 * 2
        nsets = max(4, -(-(1 << 30) // alg))
        sets = []
        for i in range(nsets):
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
            q, kc, vt, kbk, vbt = sets[i % nsets]
            C.orthrus_block_attention(B, rows, hq, hkv, q.data_ptr(), kc.data_ptr(), vt.data_ptr(), lk,
                                      lk, kbk.data_ptr(), vbt.data_ptr(), kb, out.data_ptr(),
                                      ws.data_ptr(), wsb, stream)
        for i in range(nsets):
            go(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            go(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        roof_us = alg / (HBM_PEAK_GBS * 1e3)
        res.append({"batch": B, "cache_keys": lk, "block_keys": kb, "rows": rows, "us": round(us, 2),
                    "algorithmic_bytes": alg, "achieved_GBps": round(alg / us / 1e3, 1),
                    "frac_of_8TBps": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
                    "roofline_us": round(roof_us, 2), "latency_bound": roof_us < 20.0})
        log(f"[kernel a] B={B} Lk={lk}: {us:.1f} us, {alg / us / 1e3:.0f} GB/s"
            f"{' (latency-bound point)' if roof_us < 20.0 else ''}")
        del sets, out, ws
        torch.cuda.empty_cache()
    return res


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "lossless_decoding_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_traffic(fname, workload, src_hash, key="hbm_bytes_per_launch"):
    """Bytes per launch (HBM by default) from a committed rocprofv3 PMC
    summary, if it was taken on this workload with the current kernel source."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    pm = dict(l.split(": ", 1) for l in open(path).read().splitlines()
              if l and not l.startswith("#") and ": " in l)
    if pm.get("kernel_source_hash") == src_hash and pm.get("workload") == workload and key in pm:
        return int(pm[key])
    return None


def workload_desc(name, wl, sh):
    law = {"geom6": "planted accept length min(Geom(1/7), 32), mean 6",
           "uniform32": "planted accept length uniform{0..32}"}[wl["plant"]]
    return (f"{name}: Qwen3-8B-shaped random-init model (L={sh['L']}, d={sh['d']}, "
            f"{sh['hq']}q/{sh['hkv']}kv heads x {sh['hd']}, SwiGLU {sh['F']}, vocab {sh['V']}, "
            f"bf16), batch {wl['B']}, prompt {wl['P']} uniform-random tokens, K={sh['K']}, {law}")


def gemm_class_rates(breakdown, sh, B, K):
    """Per GEMM class and pass, from the per-class times: weight bytes
    streamed (bf16, every layer; the draft pass's QKV and O read both the
    frozen and the diffusion matrices) against 8 TB/s, and GEMM flops
    (2 x rows x parameters) against the dense bf16 MFMA peak.  The class
    times come from event pairs around every launch (a few microseconds of
    record overhead each) and the QKV class includes its finish kernel when
    split, so these are lower bounds of the kernels' own rates."""
    params = gemm_classes_of(sh)
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
                    "mfma_frac": round(flops / s_ / 2.5e15, 4),
                    "bound": "mfma" if flops / MFMA_PEAK_BF16 > wbytes / (HBM_PEAK_GBS * 1e9)
                    else "hbm"}
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


def cpu_baseline(sh, wl, mean_tokens_per_step):
    """The oracle (plain fp64 C, as it stands) on a bounded sample of one
    sequence's step at the workload's context: layer 0 of the step (the
    anchor row, the K mask rows and the K verify rows) over a cache of
    P + 1 slots holding synthetic N(0, 1) keys and values, timed and scaled
    by the number of layers, plus the final norm and LM head of the 2K + 1
    rows.  Layer 0's weights, the embeddings and the LM head are the model's
    own (the weight generator draws each tensor from its own stream)."""
    import numpy as np

    import oracle
    import synth
    from synth import workloads

    P, K, L = wl["P"], sh["K"], sh["L"]
    t0 = time.time()
    shp1 = oracle.ModelShape(**dict(sh, L=1))
    lay, total = oracle.weight_layout(shp1)
    w = workloads.fill_weights(lay, total, True)
    m = oracle.Model(shp1, w)
    seq = m.seq(P + K + 2)
    kc = np.zeros((sh["hkv"], P, sh["hd"]), np.uint16)
    vc = np.zeros_like(kc)
    synth.host_fill_normal(kc, workloads.ATTN_SEED, 900, 1.0, synth.P_ATTN)
    synth.host_fill_normal(vc, workloads.ATTN_SEED, 901, 1.0, synth.P_ATTN)
    f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    seq.load_kv(0, f64(kc), f64(vc))
    del kc, vc
    seq.len = P
    log(f"[cpu] one-layer model and a {P}-slot synthetic cache in {time.time() - t0:.1f}s")
    E = f64(w[lay[0][1]:lay[0][1] + lay[0][2]]).reshape(sh["V"], sh["d"])
    toks = workloads.prompts(1, K + 1, sh["V"], seed=77)[0]
    e_mask = f64(w[lay[3][1]:lay[3][1] + lay[3][2]])
    t1 = time.time()
    ha, _ = seq.ar_layer(0, E[toks[:1]], P)                 # anchor at slot P
    hm, _ = seq.draft_layer(0, np.tile(e_mask, (K, 1)), P)  # masks over [0, P] + block
    hv, _ = seq.ar_layer(0, E[toks[1:]], P + 1)             # verify rows at P+1..P+K
    t2 = time.time()
    m.final(np.concatenate([ha, hm, hv]))
    t3 = time.time()
    layer_s, head_s = t2 - t1, t3 - t2
    step_s = L * layer_s + head_s
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    log(f"[cpu] one layer of the step {layer_s:.2f}s, final norm + LM head {head_s:.2f}s, "
        f"estimated step {step_s:.1f}s")
    return {
        "value": mean_tokens_per_step / step_s,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"one sequence's draft+verify step at the workload's {P}-token context "
                   f"(K={K}): layer 0 of both passes (anchor, {K} mask rows, {K} verify rows; "
                   f"cache of synthetic N(0,1) K/V) took {layer_s:.2f} s and the final norm + "
                   f"LM head of the {2 * K + 1} rows {head_s:.2f} s on the fp64 oracle; step "
                   f"= {L} x layer + head = {step_s:.1f} s; tokens/s = the workload's mean "
                   f"tokens per step per sequence ({mean_tokens_per_step:.3f}) / step time"),
        "step_seconds": round(step_s, 3),
        "host": host_info(),
    }


def gemm_label(plan, ep, M, N, K):
    """The kernel instantiation a GEMM launch runs (from the library's plan)."""
    sp = "true" if plan["split"] else "false"
    if plan["form"] == 0:
        name = f"k_gemm_bf16<{plan['MT']}, {ep}, {plan['WV']}, {sp}, {plan['CT']}>"
    else:
        two = "true" if plan["form"] == 2 else "false"
        name = f"k_gemm_rows<{plan['CT']}, {ep}, {sp}, {two}>"
    return f"{name} (M={M}, N={N}, K={K}, {plan['workgroups']} workgroups)"


def run_workload(name, S, W, args, headline):
    import numpy as np
    import torch

    from lossless_decoding_amd import _lib as C
    from lossless_decoding_amd.engine import Engine, attn_chunk_for
    from synth import workloads
    from synth.device import fill_weights_device

    wl = workloads.WORKLOADS[name]
    sh = workloads.SHAPES[wl["shape"]]
    B, P, K, V = wl["B"], wl["P"], sh["K"], sh["V"]
    dev = torch.device("cuda:0")
    log(f"==== {name} ({'headline' if headline else 'summary'}: {S} timed steps, {W} warmup)")

    a = workloads.plant_lengths(W + S, B, K, wl["plant"])
    need = 1 + int((a + 1).sum(0).max()) + K + 2          # trajectory tokens per sequence
    # host bound grows K+1 per step: warmup, timed steps, and the eager steps
    # after them whose launches are timed one by one
    max_ctx = P + (W + S + max(1, min(args.roofline_steps, S))) * (K + 1) + 64
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
    q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q0.record()
    ar.prefill(prompts)                    # the plain-decoding context's time to first token
    q1.record()
    traj = torch.zeros(need, B, dtype=torch.int32, device=dev)
    traj[0] = ar.pending[:B]
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for j in range(1, need):
        ar.draft(); ar.verify(); ar.commit()
        traj[j] = ar.pending[:B]
    a1.record()
    torch.cuda.synchronize()
    plain_tps = B * (need - 1) / (a0.elapsed_time(a1) / 1e3)
    plain_prefill_ms = q0.elapsed_time(q1)
    traj = traj.t().contiguous().cpu().numpy()
    log(f"[setup] greedy trajectory of {need} tokens x {B} in {time.time() - t0:.1f}s "
        f"(plain decoding {plain_tps:.1f} tokens/s)")
    ar.close()
    del ar
    torch.cuda.empty_cache()
    planted = torch.from_numpy(workloads.plant_drafts(traj, 1, a, K, V)).to(dev)

    # prefill (the prompts through the AR view into the cache), timed on its
    # own and reported beside the step loop: the time to first token
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    eng.prefill(prompts)
    p1.record()
    torch.cuda.synchronize()
    prefill_ms = p0.elapsed_time(p1)
    prefill_roof = prefill_roofline(sh, B, P, int(eng.sizes.prefill_rows), prefill_ms)
    log(f"[prefill] {B} x {P} prompt tokens in {prefill_ms:.1f} ms (roofline {prefill_roof['frac']:.3f}; "
        f"plain-decoding context {plain_prefill_ms:.1f} ms)")
    for s in range(W):
        eng.draft(); eng.drafts[:B].copy_(planted[s]); eng.verify(); eng.commit()

    # events around the dominant kernel's launches in the first roofline
    # steps of the timed region (the library stops recording at the
    # capacity).  With --graph the timed steps are replays of one captured
    # step (no events inside); the per-launch times then come from the
    # breakdown's eager steps after the timed region.
    n_rs = max(1, min(args.roofline_steps, S))
    rcls = [("draft", "attention"), ("draft", "gate_up")]
    mask = sum(1 << C.timing_class(p, r) for p, r in rcls)
    graph = None
    if args.graph:
        pbuf = torch.zeros_like(planted[0])
        try:
            graph = eng.capture_step(pbuf)
        except Exception as ex:          # fall back to eager calls, said in the output
            log(f"[graph] capture failed ({ex}); timing eager calls")
            graph = None
            torch.cuda.synchronize()
    if graph is None:
        C.orthrus_timing_enable(eng.ctx, mask, n_rs * sh["L"] * len(rcls))
    torch.cuda.synchronize()
    marker = None
    if args.markers:
        # a tiny read-probe launch before and after the timed region marks it
        # in a profiler's kernel trace
        marker = torch.zeros(4096, dtype=torch.uint8, device=dev)
        mout = torch.zeros(1, dtype=torch.int32, device=dev)
        C.orthrus_stream_read(marker.data_ptr(), 4096, mout.data_ptr(), 1, eng.s)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(S + 1)]
    t_wall = time.perf_counter()
    ev[0].record()
    for s in range(W, W + S):
        if graph is not None:
            pbuf.copy_(planted[s])
            eng.replay(graph)
        else:
            eng.draft()
            eng.drafts[:B].copy_(planted[s])
            eng.verify()
            eng.commit()
        ev[s - W + 1].record()
    if marker is not None:
        C.orthrus_stream_read(marker.data_ptr(), 4096, mout.data_ptr(), 1, eng.s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev[0].elapsed_time(ev[S])
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(S)])
    tim = {}
    if graph is None:
        tim, _ = C.orthrus_timing_read(eng.ctx)
        C.orthrus_timing_enable(eng.ctx, 0, 0)

    tokens = int((a[W:W + S] + 1).sum())
    ms_step = ms / S
    seq_len = eng.seq_len[:B].cpu().numpy()
    want_len = P + (a + 1).sum(0)
    pend = eng.pending[:B].cpu().numpy()
    e_end = 1 + (a + 1).sum(0)
    lossless = bool((seq_len == want_len).all() and
                    all(pend[b] == traj[b, e_end[b] - 1] for b in range(B)))
    step_pct = {f"p{q}": round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)}
    log(f"[timed] {S} steps in {ms:.1f} ms ({ms_step:.3f} ms/step, wall {wall * 1e3:.1f} ms), "
        f"{tokens} tokens, lossless={lossless}, step ms {step_pct}")

    # sequence lengths at the start of every step
    n_all = P + np.concatenate([np.zeros((1, B), np.int64), np.cumsum(a + 1, axis=0)])
    n_timed = n_all[W:W + S]
    n_roof = n_timed          # contexts of the steps whose launches were timed
    if graph is not None:
        # eager steps after the timed region for the per-launch times
        C.orthrus_sync_lengths(eng.ctx, B, seq_len)
        nr = max(0, min(n_rs, (max_ctx - int(seq_len.max()) - 64) // (K + 1), planted.shape[0] - W))
        C.orthrus_timing_enable(eng.ctx, mask, max(nr, 1) * sh["L"] * len(rcls))
        lens = []
        for j in range(nr):
            lens.append(eng.seq_len[:B].cpu().numpy().astype(np.int64))
            eng.draft(); eng.drafts[:B].copy_(planted[W + j]); eng.verify(); eng.commit()
        torch.cuda.synchronize()
        tim, _ = C.orthrus_timing_read(eng.ctx)
        C.orthrus_timing_enable(eng.ctx, 0, 0)
        if lens:
            n_roof = np.array(lens)
        seq_len = eng.seq_len[:B].cpu().numpy()
    roof_s, step_bytes, gemm_flops = 0.0, 0.0, 0.0
    for s in range(S):
        t_, b_, f_ = step_roofline(sh, B, K, n_timed[s])
        roof_s += t_; step_bytes += b_; gemm_flops += f_

    # the dominant kernel: the draft pass's block attention
    at_ms, at_n = tim.get(("draft", "attention"), (0.0, 0))
    at_steps = at_n // sh["L"]
    at_bytes = (sum(attn_launch_bytes(sh, B, K, n_roof[s], "draft") for s in range(at_steps))
                / max(at_steps, 1))
    at_avg_s = at_ms / max(at_n, 1) / 1e3
    # the attention kernel the draft pass launches: one query tile per wave
    # when the context's full cache at this batch gives under 512 workgroups
    G = sh["hq"] // sh["hkv"]
    nc = -(-int(eng.sizes.kv_slots) // chunk)
    rg = -(-(-(-((K + 1) * G) // 16)) // 8)
    at_kernel = "k_attn_bf16_t%d + k_attn_merge" % (1 if B * sh["hkv"] * nc * rg < 512 else 2)
    at_ach = at_bytes / at_avg_s / 1e9 if at_n else 0.0
    # the draft pass's gate/up SwiGLU GEMM, with the launch shape the library picks
    M1 = B * K + ((-(B * K)) % 16) + B if K > 0 else B
    gu_plan = C.orthrus_gemm_plan(M1, 0, 2 * sh["F"], sh["d"], C.EP_SWIGLU)
    gu_ms, gu_n = tim.get(("draft", "gate_up"), (0.0, 0))
    M1a = B * (K + 1)
    gu_bytes = 2 * sh["F"] * sh["d"] * 2 + M1a * sh["d"] * 2 + M1a * sh["F"] * 2
    gu_avg_s = gu_ms / max(gu_n, 1) / 1e3
    gu_ach = gu_bytes / gu_avg_s / 1e9 if gu_n else 0.0
    gu_flops = 2 * M1a * 2 * sh["F"] * sh["d"]

    # per-class breakdown over a few more steps (all classes timed)
    breakdown = {}
    if args.breakdown_steps > 0:
        C.orthrus_sync_lengths(eng.ctx, B, seq_len)
        extra = min(args.breakdown_steps, (max_ctx - int(seq_len.max()) - 64) // (K + 1),
                    planted.shape[0] - W)
        C.orthrus_timing_enable(eng.ctx, (1 << 24) - 1, max(extra, 1) * 800 + 64)
        for j in range(extra):
            eng.draft(); eng.drafts[:B].copy_(planted[W + j]); eng.verify(); eng.commit()
        torch.cuda.synchronize()
        tb, _ = C.orthrus_timing_read(eng.ctx)
        C.orthrus_timing_enable(eng.ctx, 0, 0)
        if extra > 0:
            breakdown = {f"{p}.{r}": round(v[0] / extra, 4) for (p, r), v in sorted(tb.items())}
        log(f"[breakdown] ms per step by class over {extra} steps: {breakdown}")
    eng.close()
    del eng, planted
    torch.cuda.empty_cache()

    res = {
        "graph": graph is not None,
        "workload": workload_desc(name, wl, sh),
        "batch": B, "prompt_len": P, "block_k": K, "attn_chunk": chunk,
        "tokens_per_s": round(tokens / (ms / 1e3), 3),
        "ms_per_step": round(ms_step, 4),
        "steps": S, "warmup": W,
        "steps_per_s": round(S / (ms / 1e3), 3),
        "step_ms_percentiles": step_pct,
        "tokens_per_step": round(tokens / S, 4),
        "tpf": round(tpf_from_accept(tokens / S / B - 1.0), 4),
        "prefill_ms": round(prefill_ms, 3),
        "prefill_tokens_per_s": round(B * P / (prefill_ms / 1e3), 1),
        # the same prompts prefilled by the plain-decoding (K = 0) context: the
        # time-to-first-token ratio of draft/verify decoding to plain decoding
        "prefill_plain_decoding_ms": round(plain_prefill_ms, 3),
        "ttft_vs_plain_decoding": round(prefill_ms / plain_prefill_ms, 4),
        "prefill_roofline": prefill_roof,
        "lossless_vs_greedy": lossless,
        "plain_decoding_tokens_per_s": round(plain_tps, 3),
        "speedup_vs_plain_decoding": round(tokens / (ms / 1e3) / plain_tps, 4),
        "step_roofline": {
            "method": "sum over kernel classes of max(bytes / 8 TB/s, flops / 2.5 PFLOP/s)",
            "bytes_per_step": round(step_bytes / S), "roofline_ms": round(roof_s * 1e3 / S, 4),
            "frac": round(roof_s * 1e3 / ms, 4),
            "gemm_tflops_per_s": round(gemm_flops / (ms / 1e3) / 1e12, 2),
            "mfma_frac_bf16": round(gemm_flops / (ms / 1e3) / MFMA_PEAK_BF16, 4)},
        "attention_draft": {
            "kernel": at_kernel,
            "bytes_per_launch": round(at_bytes), "avg_launch_us": round(at_avg_s * 1e6, 3),
            "launches": at_n, "achieved_GBps": round(at_ach, 1),
            "frac": round(at_ach / HBM_PEAK_GBS, 4)},
        "gate_up_draft": {
            "kernel": gemm_label(gu_plan, "EP_SWIGLU", M1, 2 * sh["F"], sh["d"]),
            "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_avg_s * 1e6, 3),
            "launches": gu_n, "achieved_GBps": round(gu_ach, 1),
            "hbm_frac": round(gu_ach / HBM_PEAK_GBS, 4),
            "mfma_frac": round(gu_flops / max(gu_avg_s, 1e-12) / MFMA_PEAK_BF16, 4) if gu_n else 0.0,
            "traffic": pmc_traffic("gemm_gateup_draft_%s_pmc.txt" % name, name,
                                   source_hash("k_gemm.hip")),
            "l2_read_bytes": pmc_traffic("gemm_gateup_draft_%s_pmc.txt" % name, name,
                                         source_hash("k_gemm.hip"), "l2_read_bytes_per_launch")},
        "ms_per_step_by_class": breakdown,
        "gemm_classes": gemm_class_rates(breakdown, sh, B, K),
    }
    return res, sh, wl


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--roofline-steps", type=int, default=4,
                    help="timed steps whose attention and gate/up launches carry HIP events "
                         "(the first ones of the timed region; each event pair adds a few us)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--also", default="qwen3_8b_b1_p512,qwen3_8b_b16_c8192",
                    help="comma-separated workloads summarised after the headline ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=6)
    ap.add_argument("--no-kernel-a", action="store_true",
                    help="skip the block-attention microbenchmark and HBM read-rate measurements")
    ap.add_argument("--attn-chunk", type=int, default=0,
                    help="attention key chunk of both contexts (default: the library's rule)")
    ap.add_argument("--eager", dest="graph", action="store_false",
                    help="time eager draft/verify/commit calls instead of replays of one "
                         "captured step (HIP graph; per-launch times then come from eager "
                         "steps right after the timed region)")
    ap.add_argument("--markers", action="store_true",
                    help="launch a tiny read probe before and after the headline's timed region "
                         "(marks it in a profiler's kernel trace)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run plain 1 GiB device copies (PMC byte-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode step shards by sequence with no "
              "exchange, and the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    res, sh, wl = run_workload(args.workload, args.steps, args.warmup, args, True)
    others = {}
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        S2, W2 = SECONDARY[name]
        a2 = argparse.Namespace(**vars(args))
        a2.breakdown_steps = 0
        a2.markers = False
        r2, _, _ = run_workload(name, S2, W2, a2, False)
        others[name] = r2

    if args.calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[calibrate] 3 plain copies of 1 GiB")
    kernel_a = kernel_a_bench(dev) if not args.no_kernel_a else None
    read_probe = hbm_read_probe(dev) if not args.no_kernel_a else None

    at = res["attention_draft"]
    traffic = pmc_traffic("attn_draft_%s_pmc.txt" % args.workload, args.workload,
                          source_hash("k_attn.hip"))
    out = {
        "metric": "verified tokens/s (and draft+verify steps/s) on 1 GPU; % of HBM roofline",
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and prompts, planted drafts)",
        "config": {"workload": res["workload"], "batch": res["batch"],
                   "prompt_len": res["prompt_len"], "block_k": res["block_k"],
                   "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": f"{at['kernel']} (draft-pass block attention, kernel (a), per layer)",
            "bound": "hbm",
            "achieved": at["achieved_GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": at["frac"],
            "traffic": traffic,
            "bytes_per_launch": at["bytes_per_launch"],
            "avg_launch_us": at["avg_launch_us"],
            "launches": at["launches"],
            "timed_steps": at["launches"] // sh["L"],
            "timed_on": ("eager steps right after the timed region (the timed steps are graph replays)"
                         if res["graph"] else "the first steps of the timed region"),
        },
        "step_launch": "HIP graph replay of one captured step" if res["graph"] else "eager calls",
    }
    for k, v in res.items():
        if k not in ("workload", "batch", "prompt_len", "block_k", "tokens_per_s", "ms_per_step",
                     "steps", "warmup", "graph"):
            out[k] = v
    out["other_workloads"] = others
    out["kernel_a"] = kernel_a
    out["hbm_read_achievable"] = read_probe
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(sh, wl, res["tokens_per_step"] / res["batch"])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
