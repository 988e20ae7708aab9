#!/usr/bin/env python3
"""Benchmark of the dictionary-coded KV cache on one MI355X.

Metric (two parts):
  * coded-KV decode attention, context-tokens/s at 128K: one decode step of a
    Llama-3.1-8B-shaped layer (32 query / 8 KV heads, head_dim 128, 32,768-atom
    bf16 key and value dictionaries, K=16, Klow=3, Khigh=16, top 10%) over
    131,072 coded tokens at batch 1; value = B*T / time per step.
  * KV vectors encoded/s: prefill encode of 32,768 tokens x 8 KV heads x
    {K, V} = 524,288 bf16 vectors to K=16 codes over their stream's
    32,768-atom dictionary (reported in the "encode" object).

Inputs are seeded synthetic arrays (synth), resident in HBM before timing.
Decode rotates through several copies of every input (codes, low plane,
dictionaries, query) so the 256 MB Infinity Cache cannot serve repeated
steps. The timed region holds only the steps (one event before, one after);
per-kernel times come from a second pass in which the library records HIP
events between its kernels on the call's stream.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "coded-KV decode attn context-tokens/s/GPU at 128K; KV vectors encoded/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, TFLOP/s
F16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.h.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        self.made += out
        return out

    def record(self, e, stream_handle):
        if self.h.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        t = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def close(self):
        for e in self.made:
            self.h.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


def sources_digest(paths):
    """sha256 over the concatenated contents of the given repo-relative files."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_digest(path: str):
    """The '- key: value' lines of a committed profile summary, if the
    digest it records of the kernel's sources still matches them; else None."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    srcs = [s.strip() for s in vals.get("sources", "").split(",") if s.strip()]
    if not srcs or not vals.get("sources_sha256"):
        return None
    try:
        if sources_digest(srcs) != vals["sources_sha256"]:
            return None
    except OSError:
        return None
    return vals


def read_mfma_busy(kernel: str, workload: str):
    """Share of SIMD-cycles the matrix cores were busy in the kernel
    (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE), from the
    committed summary profiles/mfma_<workload>.md while its source digest
    matches; else None. Clock-free, unlike a rate against the peak."""
    vals = read_digest(os.path.join(ROOT, "profiles", f"mfma_{workload}.md"))
    try:
        return float(vals[f"mfma_busy_{kernel}"]) if vals else None
    except (KeyError, ValueError):
        return None


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, from the
    committed summary profiles/traffic_<kernel>_<workload>.md, if the digest it
    records of the kernel's sources still matches them; else None."""
    vals = read_digest(os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md"))
    try:
        return float(vals["hbm_bytes_per_launch"]) if vals else None
    except (KeyError, ValueError):
        return None


def calibrate_copy(torch, mib: int, reps: int = 5):
    """A plain device-to-device copy of a known number of bytes: the reference
    against which the rocprofv3 FETCH_SIZE / WRITE_SIZE counters are scaled,
    and the achievable stream-copy bandwidth."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t) / reps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps + 1,
                      "copy_GBs": round(2 * n * 4 / el / 1e9, 1)}), flush=True)


def calibrate_gather(torch, rows_log2: int = 20, reps: int = 5):
    """A gather of 2**rows_log2 random 128-byte rows (32 fp32) out of a
    2**22-row table, by torch.index_select: a second reference for the
    rocprofv3 FETCH_SIZE counter, whose requests are scattered 128-byte
    lines like the row kernel's record reads (the copy reference streams).
    Bytes read: 128 per gathered row plus 8 per int64 index; bytes written:
    128 per row."""
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    table = torch.ones((1 << 22, 32), dtype=torch.float32, device="cuda")
    n = 1 << rows_log2
    idx = torch.randint(0, 1 << 22, (n,), generator=g, device="cuda")
    out = torch.index_select(table, 0, idx)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        torch.index_select(table, 0, idx, out=out)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t) / reps
    print(json.dumps({"gather_rows": n, "gather_bytes_read": n * (128 + 8),
                      "gather_bytes_written": n * 128, "reps": reps + 1,
                      "gather_GBs": round(n * (2 * 128 + 8) / el / 1e9, 1)}), flush=True)


# ---------------------------------------------------------------------------
# decode at 128K
# ---------------------------------------------------------------------------
def bench_decode(args, torch, sd, synth, ev):
    case = synth.decode_case("llama_layer_128k")
    B, Hq, Hkv, T, d, K = case.B, case.Hq, case.Hkv, case.T, case.d, case.K
    N, m = case.n_atoms, case.m
    dev = "cuda"

    def up_words(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev)

    base = dict(q=torch.from_numpy(case.q).to(dev).to(torch.bfloat16),
                dk=torch.from_numpy(case.dk).to(dev).to(torch.bfloat16),
                dv=torch.from_numpy(case.dv).to(dev).to(torch.bfloat16),
                # each token's key record, then its value record: [B, Hkv, T, 2, K]
                kv=up_words(np.stack([case.key_codes, case.val_codes], axis=3)),
                kl=up_words(case.key_low),
                # reading B's value low plane (first klow value words)
                vl=up_words(np.ascontiguousarray(case.val_codes[..., :case.klow])))
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    nsets = max(2, int(np.ceil(600e6 / set_bytes)))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    log(f"decode: {nsets} input sets of {set_bytes / 1e6:.1f} MB rotate through the timed steps")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = sd.Workspace()
    stream = torch.cuda.current_stream()
    nstage = 5  # SDKV_DECODE_STAGES + 1
    calls = [sd.DecodeCall(s["q"], s["dk"], s["dv"], s["kv"], None, klow=case.klow,
                           khigh=case.khigh, top_num=case.top_num, top_den=case.top_den,
                           scale=case.scale, key_low=s["kl"], out=out, workspace=ws)
             for s in sets]

    def step(i, stage_events=None):
        calls[i % nsets].launch(stage_events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: the steps alone, bracketed by two events
    t0, t1 = ev.create(2)
    torch.cuda.synchronize()
    ev.record(t0, stream.cuda_stream)
    for i in range(args.steps):
        step(i)
    ev.record(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / args.steps
    # per-kernel durations from a second pass with events between the kernels
    # (event records add gaps, so this pass is not the timed one)
    evs = [ev.create(nstage) for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = [float(np.mean([ev.ms(e[j], e[j + 1]) for e in evs])) for j in range(nstage - 1)]

    # the same step with each attention flag of the same call
    def time_variant(per_set=lambda s: {}, extra_bytes=0, **flags):
        vcalls = [sd.DecodeCall(s["q"], s["dk"], s["dv"], s["kv"], None, klow=case.klow,
                                khigh=case.khigh, top_num=case.top_num, top_den=case.top_den,
                                scale=case.scale, key_low=s["kl"], out=out, workspace=ws,
                                **flags, **per_set(s))
                  for s in sets]
        for i in range(args.warmup):
            vcalls[i % nsets].launch()
        torch.cuda.synchronize()
        ev.record(t0, stream.cuda_stream)
        for i in range(args.steps):
            vcalls[i % nsets].launch()
        ev.record(t1, stream.cuda_stream)
        torch.cuda.synchronize()
        vms = ev.ms(t0, t1) / args.steps
        path_b = total_b + extra_bytes
        return {"us_per_step": round(vms * 1e3, 2), "value": round(B * T / (vms * 1e-3), 1),
                "unit": "context-tokens/s", "relative_to_default_step": round(vms / ms, 3),
                "path_roofline": {"bound": "hbm", "algorithmic_bytes_per_step": path_b,
                                  "achieved_GBs": round(path_b / (vms * 1e-3) / 1e9, 1),
                                  "frac": round(path_b / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}

    # algorithmic bytes (HBM): what the method must read per step
    low_b = B * Hkv * T * case.klow * 4
    refine_b = B * Hq * m * (case.khigh - case.klow) * 4
    value_b = B * Hq * m * K * 4
    dict_b = N * d * 2
    qo_b = B * Hq * d * (2 + 4)
    stage_bytes = [dict_b + B * Hq * d * 2, low_b + refine_b + value_b, dict_b, B * Hq * d * 4]
    total_b = sum(stage_bytes)
    int_res = kv_res = b_res = None
    if not args.no_variants:
        int_res = {"metric": "decode step with the integer-only softmax",
                   **time_variant(softmax="int")}
        kv_res = {"metric": "decode step with the selection shared by each KV head's query heads",
                  **time_variant(select="kv")}
        b_res = {"metric": "decode step, reading B (every token in the softmax; Klow values "
                           "outside the selection)",
                 **time_variant(per_set=lambda s: {"val_low": s["vl"]}, reading="B",
                                # every query head reads its KV head's value low plane
                                extra_bytes=B * Hq * T * case.klow * 4)}

    dom = int(np.argmax(stage_ms))
    names = ["k_utable_bf16", "k_rows", "k_wdv_bf16", "k_reduce_out"]
    achieved = stage_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic = read_traffic(names[dom], "llama_layer_128k")
    res = dict(
        value=B * T / (ms * 1e-3), ms=ms, stage_ms=dict(zip(names, stage_ms)),
        dk=base["dk"], dv=base["dv"],
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": traffic, "kernel": names[dom],
                  "algorithmic_bytes_per_launch": stage_bytes[dom]},
        path={"algorithmic_bytes_per_step": total_b, "qo_bytes": qo_b,
              "achieved_GBs": round(total_b / (ms * 1e-3) / 1e9, 1),
              "frac": round(total_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        config=dict(B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, n_atoms=N, K=K, klow=case.klow,
                    khigh=case.khigh, top="1/10", m=m, input_sets=nsets),
        int_softmax=int_res, shared_select=kv_res, reading_b=b_res, case=case)
    return res


# ---------------------------------------------------------------------------
# the other decode workloads: 4K layer, batch 8 x 32K, Qwen-shaped 28 layers
# ---------------------------------------------------------------------------
def step_bytes(B, Hq, Hkv, T, m, d, N, K, klow, khigh, layers=1):
    """Algorithmic HBM bytes of one decode step: both dictionaries, the key
    low plane, the Khigh - Klow extra key pairs and the K value pairs of
    every selected token and query head, the queries and the outputs."""
    per = (2 * N * d * 2 + B * Hkv * T * klow * 4 + B * Hq * m * (khigh - klow) * 4
           + B * Hq * m * K * 4 + B * Hq * d * (2 + 4))
    return per * layers


def time_steps(ev, stream, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    import torch
    torch.cuda.synchronize()
    t0, t1 = ev.create(2)
    ev.record(t0, stream.cuda_stream)
    for i in range(steps):
        fn(i)
    ev.record(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    return ev.ms(t0, t1) / steps


def workload_line(name, what, B, Hq, Hkv, T, m, ms, path_b, cpu, extra=None):
    r = {"workload": what, "B": B, "Hq": Hq, "Hkv": Hkv, "T": T, "m": m,
         "us_per_step": round(ms * 1e3, 2), "value": round(B * T / (ms * 1e-3), 1),
         "unit": "context-tokens/s",
         "path_roofline": {"bound": "hbm", "algorithmic_bytes_per_step": path_b,
                           "achieved_GBs": round(path_b / (ms * 1e-3) / 1e9, 1),
                           "peak": HBM_PEAK_GBS,
                           "frac": round(path_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
         "cpu_baseline": cpu}
    if extra:
        r.update(extra)
    return r


def bench_layer_workload(args, torch, sd, synth, ev, name, what):
    """A Llama-shaped layer workload from synth (the parity-tested inputs),
    with enough copies to rotate through more than 512 MB per pass."""
    case = synth.decode_case(name)
    B, Hq, Hkv, T, d, K, N, m = case.B, case.Hq, case.Hkv, case.T, case.d, case.K, case.n_atoms, case.m
    dev = "cuda"

    def up_words(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev)

    base = dict(q=torch.from_numpy(case.q).to(dev).to(torch.bfloat16),
                dk=torch.from_numpy(case.dk).to(dev).to(torch.bfloat16),
                dv=torch.from_numpy(case.dv).to(dev).to(torch.bfloat16),
                kv=up_words(np.stack([case.key_codes, case.val_codes], axis=3)),
                kl=up_words(case.key_low))
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    nsets = max(2, int(np.ceil(600e6 / set_bytes)))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = sd.Workspace()
    calls = [sd.DecodeCall(st["q"], st["dk"], st["dv"], st["kv"], None, klow=case.klow,
                           khigh=case.khigh, top_num=case.top_num, top_den=case.top_den,
                           scale=case.scale, key_low=st["kl"], out=out, workspace=ws)
             for st in sets]
    stream = torch.cuda.current_stream()
    ms = time_steps(ev, stream, lambda i: calls[i % nsets].launch(), args.steps, args.warmup)
    calls[0].check()
    path_b = step_bytes(B, Hq, Hkv, T, m, d, N, K, case.klow, case.khigh)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_decode(case, args.cpu_budget / 3, label=what)
    del sets, calls
    torch.cuda.empty_cache()
    return workload_line(name, what, B, Hq, Hkv, T, m, ms, path_b, cpu,
                         {"input_sets": nsets, "set_bytes": set_bytes})


def gpu_dictionary(torch, gen, N, d):
    """Gaussian rows normalised to unit length (fp32), stored as bf16."""
    g = torch.randn((N, d), generator=gen, device="cuda", dtype=torch.float32)
    return (g / g.norm(dim=1, keepdim=True)).to(torch.bfloat16)


def gpu_codes(torch, gen, n, K, N):
    """Packed code words [n, K] as int32: K distinct uniform atom indices per
    row (rows with a repeat are drawn again) and binary16 coefficients
    |N(0,1)| in decreasing order, the recipe of synth.make_codes drawn on the
    device."""
    idx = torch.randint(0, N, (n, K), generator=gen, device="cuda", dtype=torch.int64)
    while True:
        srt = idx.sort(dim=1).values
        bad = (srt[:, 1:] == srt[:, :-1]).any(dim=1).nonzero().flatten()
        if bad.numel() == 0:
            break
        idx[bad] = torch.randint(0, N, (bad.numel(), K), generator=gen, device="cuda",
                                 dtype=torch.int64)
    c = torch.randn((n, K), generator=gen, device="cuda", dtype=torch.float32).abs()
    c = c.sort(dim=1, descending=True).values.to(torch.float16)
    bits = c.view(torch.int16).to(torch.int32) & 0xFFFF
    return (idx.to(torch.int32) | (bits << 16)).contiguous()


def bench_qwen_full_step(args, torch, sd, synth, ev):
    """Qwen-2.5-7B-shaped full-model decode step: 28 layers, each with its
    own 32,768-atom key and value dictionaries, 28 query / 4 KV heads,
    262,144 coded tokens at batch 1, one fresh query per layer; a step is
    the 28 per-layer calls in sequence on one stream (4.6 GB of inputs, so
    nothing is served from the 256 MB Infinity Cache between steps).
    Inputs are drawn on the device (torch's generator, seed 4000 + layer)
    with the distributions of synth.qwen_layer_case."""
    L, Hq, Hkv, T, d, K, N = 28, 28, 4, 262144, 128, 16, 32768
    klow, khigh = 3, 16
    m = max(1, min(T, -(-T * 1 // 10)))
    scale = 1.0 / np.sqrt(d)
    out = torch.empty((L, 1, Hq, d), dtype=torch.float32, device="cuda")
    layers = []
    for li in range(L):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(4000 + li)
        dk, dv = gpu_dictionary(torch, gen, N, d), gpu_dictionary(torch, gen, N, d)
        kc = gpu_codes(torch, gen, Hkv * T, K, N).view(1, Hkv, T, K)
        vc = gpu_codes(torch, gen, Hkv * T, K, N).view(1, Hkv, T, K)
        kv = torch.stack([kc, vc], dim=3).contiguous()
        del kc, vc
        kl = kv[:, :, :, 0, :klow].contiguous()
        q = torch.randn((1, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
        layers.append(dict(q=q, dk=dk, dv=dv, kv=kv, kl=kl))
    ws = sd.Workspace()
    calls = [sd.DecodeCall(ly["q"], ly["dk"], ly["dv"], ly["kv"], None, klow=klow, khigh=khigh,
                           top_num=1, top_den=10, scale=scale, key_low=ly["kl"], out=out[li],
                           workspace=ws)
             for li, ly in enumerate(layers)]
    in_bytes = sum(t.numel() * t.element_size() for ly in layers for t in ly.values())

    def step(_i):
        for c in calls:
            c.launch()
    stream = torch.cuda.current_stream()
    ms = time_steps(ev, stream, step, max(3, args.steps // 4), 2)
    calls[-1].check()
    path_b = step_bytes(1, Hq, Hkv, T, m, d, N, K, klow, khigh, layers=L)
    cpu = None
    if not args.no_cpu:
        c0 = synth.qwen_layer_case(0)
        cpu = cpu_baseline_decode(c0, args.cpu_budget / 3, label="qwen layer", scale_layers=L)
    del calls, layers
    torch.cuda.empty_cache()
    return workload_line("qwen_28_layers_256k",
                         "qwen2.5-7b-shaped full-model decode step (28 layers) at 262,144 tokens",
                         1, Hq, Hkv, T, m, ms, path_b, cpu,
                         {"layers": L, "input_bytes": in_bytes,
                          "us_per_layer": round(ms * 1e3 / L, 2),
                          "data": "drawn on the device, torch generator seeded 4000 + layer"})


# ---------------------------------------------------------------------------
# encode (prefill)
# ---------------------------------------------------------------------------
def bench_append(args, torch, sd, synth, ev, dec):
    """One decode step's append on the 128K layer shape: the new token's 8 key
    and 8 value vectors encoded (K=16 over the layer's two 32,768-atom
    dictionaries) into a slot of an interleaved code cache."""
    case = dec["case"]
    dev = "cuda"
    B, Hkv, d, K = case.B, case.Hkv, case.d, case.K
    rng = np.random.default_rng(7)
    dk = dec["dk"]
    dv = dec["dv"]
    Tc = 64
    kv = torch.zeros((B, Hkv, Tc, 2, K), dtype=torch.int32, device=dev)
    low = torch.zeros((B, Hkv, Tc, case.klow), dtype=torch.int32, device=dev)
    xs = [(torch.from_numpy(rng.standard_normal((B, Hkv, d), dtype=np.float32)).to(dev).to(torch.bfloat16),
           torch.from_numpy(rng.standard_normal((B, Hkv, d), dtype=np.float32)).to(dev).to(torch.bfloat16))
          for _ in range(4)]
    ws = sd.Workspace()
    stream = torch.cuda.current_stream()

    def step(i):
        xk, xv = xs[i % len(xs)]
        sd.sdkv_append_tokens(xk, xv, dk, dv, kv, None, i % Tc, key_low=low, workspace=ws)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    n = 20
    t0, t1 = ev.create(2)
    ev.record(t0, stream.cuda_stream)
    for i in range(n):
        step(i)
    ev.record(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / n
    dict_bytes = 2 * K * case.n_atoms * d * 2  # each pursuit step reads its dictionary once
    # the OMP comparison encoder against the pursuit on the same 16 vectors
    # (16-atom combinations of the key dictionary plus noise): time per encode
    # and mean final residual norm
    xs16 = synth.make_sparse_vectors(rng, case.dk, 2 * B * Hkv, 16, 0.05, "absdesc")[0]
    x16 = torch.from_numpy(synth.bf16_round(xs16)).to(dev).to(torch.bfloat16)
    cmp = {}
    for alg in ("pursuit", "omp"):
        wsa = sd.Workspace()
        r = sd.sdkv_encode(x16, dk, K, resid_norm=True, algorithm=alg, workspace=wsa)
        torch.cuda.synchronize()
        rn = float(r["resid_norm"].mean())
        t0, t1 = ev.create(2)
        ev.record(t0, stream.cuda_stream)
        for _ in range(n):
            sd.sdkv_encode(x16, dk, K, codes=r["codes"], resid_norm=r["resid_norm"],
                           algorithm=alg, workspace=wsa)
        ev.record(t1, stream.cuda_stream)
        torch.cuda.synchronize()
        cmp[alg] = {"us_per_encode": round(ev.ms(t0, t1) / n * 1e3, 2), "mean_resid_norm": round(rn, 5)}
    cmp["mean_x_norm"] = round(float(np.linalg.norm(xs16, axis=1).mean()), 5)
    cmp["vectors"] = 2 * B * Hkv
    return {"metric": "decode-step append encode", "us_per_step": round(ms * 1e3, 2),
            "vectors": 2 * B * Hkv, "value": round(2 * B * Hkv / (ms * 1e-3), 1),
            "unit": "vectors/s", "launches": K + 1,
            "dictionary_bytes_per_step": dict_bytes,
            "dictionary_GBs": round(dict_bytes / (ms * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(dict_bytes / (ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dict_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": "each pursuit step reads both dictionaries once"},
            "config": {"B": B, "Hkv": Hkv, "d": d, "K": K, "n_atoms": case.n_atoms,
                       "path": "small-batch fp32-accurate pursuit (n <= 64), key and value encodes sharing launches"},
            "omp_comparison": cmp}


def bench_encode(args, torch, sd, synth, ev):
    dev = "cuda"
    streams = []
    for s in (0, 1):
        e = synth.encode_case(stream=s)
        streams.append(dict(x=torch.from_numpy(e.x).to(dev).to(torch.bfloat16),
                            D=torch.from_numpy(e.dictionary).to(dev).to(torch.bfloat16),
                            codes=torch.empty((e.x.shape[0], 16), dtype=torch.int32, device=dev),
                            rn=torch.empty((e.x.shape[0],), dtype=torch.float32, device=dev),
                            case=e))
    n_total = sum(s["x"].shape[0] for s in streams)
    ws = sd.Workspace()
    stream = torch.cuda.current_stream()
    calls = [sd.EncodeCall(s["x"], s["D"], 16, codes=s["codes"], resid_norm=s["rn"],
                           workspace=ws) for s in streams]

    def step(evsets=None):
        for j, c in enumerate(calls):
            c.launch(None if evsets is None else evsets[j])

    for _ in range(args.enc_warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = ev.create(2)
    ev.record(t0, stream.cuda_stream)
    for i in range(args.enc_steps):
        step()
    ev.record(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / args.enc_steps
    evs = [[ev.create(3) for _ in streams] for _ in range(args.enc_steps)]
    for i in range(args.enc_steps):
        step(evs[i])
    torch.cuda.synchronize()
    kern_ms = float(np.mean([sum(ev.ms(e[1], e[2]) for e in es) for es in evs]))
    prep_ms = float(np.mean([sum(ev.ms(e[0], e[1]) for e in es) for es in evs]))
    flops = n_total * 2.0 * 32768 * 128 * 16
    tflops = flops / (kern_ms * 1e-3) / 1e12
    return dict(value=n_total / (ms * 1e-3), ms=ms, kernel_ms=kern_ms, prep_ms=prep_ms,
                roofline={"bound": "mfma", "achieved": round(tflops, 1), "peak": F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tflops / F16_PEAK_TFLOPS, 4),
                          "traffic": read_traffic("k_encode", "prefill_524k"),
                          "mfma_busy": read_mfma_busy("k_encode", "prefill_524k"),
                          "kernel": "k_encode<128>", "algorithmic_flops_per_step": flops},
                streams=streams)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores
# ---------------------------------------------------------------------------
def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info()]
        return int(max(n)) if n else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_decode(case, budget_s, label="128K", scale_layers=1):
    """The oracle's decode of one layer, repeated for about budget_s seconds;
    with scale_layers = L the step is L such layers (time scaled by L)."""
    import oracle
    t = time.perf_counter()
    reps = 0
    while True:
        oracle.decode_attn(case.q, case.dk, case.dv, case.key_codes, case.val_codes, case.klow,
                           case.khigh, case.top_num, case.top_den, case.scale)
        reps += 1
        el = time.perf_counter() - t
        if el >= budget_s or reps >= 20:
            break
    per = el / reps * scale_layers
    what = (f"full {label} decode step (all {case.Hq} query heads)" if scale_layers == 1 else
            f"one {label} ({case.Hq} query heads, T={case.T}), time x {scale_layers} layers")
    return {"value": case.B * case.T / per, "unit": "context-tokens/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"{what}, {reps} run(s), {el:.1f} s, fp64 NumPy"}


def cpu_baseline_encode(ecase, budget_s):
    """The oracle encoder on seeded vectors of the key stream: a 256-vector
    probe sizes a sample that takes about budget_s seconds."""
    import oracle
    rng = np.random.default_rng(5)
    n = ecase.x.shape[0]
    probe = np.sort(rng.choice(n, 256, replace=False))
    t = time.perf_counter()
    oracle.mp_encode(ecase.x[probe], ecase.dictionary, 16)
    per = (time.perf_counter() - t) / 256
    n_sample = int(min(n, max(256, budget_s / max(per, 1e-9))))
    pick = np.sort(rng.choice(n, n_sample, replace=False))
    t = time.perf_counter()
    oracle.mp_encode(ecase.x[pick], ecase.dictionary, 16)
    el = time.perf_counter() - t
    return {"value": n_sample / el, "unit": "vectors/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{n_sample} seeded vectors of the key stream, {el:.1f} s, fp64 NumPy"}


def achievable(torch, reps: int = 5):
    """What the device reaches on plain library work, as context for the
    roofline fractions (the fractions themselves use the published peaks):
    a 1 GiB device-to-device copy (bytes read + written) and an 8192^3 bf16
    matrix product (torch.matmul on contiguous 2-D operands). Medians of
    `reps` timed runs after one warm-up, timed with events on torch's stream."""
    def med(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = med(lambda: dst.copy_(src))
    del src, dst
    g = 8192
    a = torch.randn(g, g, device="cuda").to(torch.bfloat16)
    b = torch.randn(g, g, device="cuda").to(torch.bfloat16)
    t_mm = med(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBs": round(2 * n * 4 / t_copy / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2 * g ** 3 / t_mm / 1e12, 1),
            "what": "1 GiB device copy (read + write bytes); 8192^3 bf16 torch.matmul"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--enc-steps", type=int, default=3)
    ap.add_argument("--enc-warmup", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline and the achievable-rate measurements")
    ap.add_argument("--no-encode", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the attention-flag steps, the append and the OMP comparison")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 4K layer, batch-8 x 32K and 28-layer Qwen-shaped steps")
    ap.add_argument("--no-decode", action="store_true",
                    help="encode only (profiling runs); prints no benchmark line")
    ap.add_argument("--calibrate-gather", action="store_true",
                    help="only run a random 128-byte row gather (counter calibration)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this benchmark runs on one GPU only: the coded-KV path has no "
               "multi-GPU implementation here (--gpus must be 1)")
        print(msg, file=sys.stderr)
        print(json.dumps({"metric": METRIC, "error": msg, "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import decode_attention_sparse_amd as sd
    import synth
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return
    if args.calibrate_gather:
        calibrate_gather(torch)
        return
    sd.lib()
    ev = HipEvents()
    if args.no_decode:
        log("encode benchmark (524,288 vectors)")
        enc = bench_encode(args, torch, sd, synth, ev)
        log(f"  {enc['ms']:.2f} ms/step, kernel {enc['kernel_ms']:.2f} ms, "
            f"{enc['value'] / 1e6:.2f} M vectors/s, {enc['roofline']['achieved']} TFLOP/s")
        ev.close()
        return
    log("decode benchmark (128K context)")
    dec = bench_decode(args, torch, sd, synth, ev)
    log(f"  {dec['ms'] * 1e3:.1f} us/step, stages (us): "
        + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in dec["stage_ms"].items()))
    app = None
    if not args.no_variants:
        app = bench_append(args, torch, sd, synth, ev, dec)
        log(f"  decode-step append (16 vectors): {app['us_per_step']:.1f} us")
        oc = app["omp_comparison"]
        log(f"  16-vector encode: pursuit {oc['pursuit']['us_per_encode']:.1f} us, |r| "
            f"{oc['pursuit']['mean_resid_norm']:.4f}; OMP {oc['omp']['us_per_encode']:.1f} us, |r| "
            f"{oc['omp']['mean_resid_norm']:.4f} (|x| {oc['mean_x_norm']:.4f})")
        log(f"  integer-only softmax step: {dec['int_softmax']['us_per_step']:.1f} us")
        log(f"  shared-selection step: {dec['shared_select']['us_per_step']:.1f} us")
        log(f"  reading-B step: {dec['reading_b']['us_per_step']:.1f} us")
    wl = None
    if not args.no_workloads:
        wl = {}
        log("decode workloads: 4K layer, batch 8 x 32K, Qwen-shaped 28 layers at 256K")
        wl["llama_layer_4k"] = bench_layer_workload(
            args, torch, sd, synth, ev, "llama_layer_4k",
            "llama3.1-8b-shaped layer decode step at 4K context")
        wl["llama_layer_b8_32k"] = bench_layer_workload(
            args, torch, sd, synth, ev, "llama_layer_b8_32k",
            "llama3.1-8b-shaped layer decode step, batch 8 x 32K context")
        wl["qwen_28_layers_256k"] = bench_qwen_full_step(args, torch, sd, synth, ev)
        for k, v in wl.items():
            log(f"  {k}: {v['us_per_step']:.1f} us/step, {v['value']:.3e} context-tokens/s, "
                f"path {v['path_roofline']['frac']:.3f} of HBM peak")
    enc = None
    if not args.no_encode:
        log("encode benchmark (524,288 vectors)")
        enc = bench_encode(args, torch, sd, synth, ev)
        log(f"  {enc['ms']:.2f} ms/step, kernel {enc['kernel_ms']:.2f} ms, "
            f"{enc['value'] / 1e6:.2f} M vectors/s, {enc['roofline']['achieved']} TFLOP/s")
    ach = cpu = None
    if not args.no_cpu:
        ach = achievable(torch)
        log(f"achievable: device copy {ach['copy_GBs']} GB/s, bf16 GEMM "
            f"{ach['bf16_gemm_TFLOPs']} TFLOP/s")
        log("cpu baseline (fp64 oracle on host cores)")
        cpu = cpu_baseline_decode(dec["case"], args.cpu_budget)
        if enc is not None:
            enc["cpu_baseline"] = cpu_baseline_encode(enc["streams"][0]["case"], args.cpu_budget)
    ev.close()
    line = {
        "metric": METRIC, "value": round(dec["value"], 1), "unit": "context-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; unit-norm Gaussian bf16 dictionaries, random codes)",
        "config": {"workload": "llama3.1-8b-shaped layer decode step at 128K context",
                   **dec["config"], "storage": "bf16 dictionaries/query, uint16+fp16 codes",
                   "code_layout": "key and value records side by side per token"},
        "roofline": dec["roofline"],
        "path_roofline": dec["path"],
        "stage_us": {k: round(v * 1e3, 2) for k, v in dec["stage_ms"].items()},
        "cpu_baseline": cpu,
        "achievable": ach,
    }
    if wl is not None:
        line["workloads"] = wl
    if app is not None:
        line["append"] = app
        line["int_softmax"] = dec["int_softmax"]
        line["shared_select"] = dec["shared_select"]
        line["reading_b"] = dec["reading_b"]
    if enc is not None:
        line["encode"] = {
            "metric": "KV vectors encoded/s", "value": round(enc["value"], 1),
            "unit": "vectors/s", "ms_per_step": round(enc["ms"], 3),
            "steps": args.enc_steps, "warmup": args.enc_warmup,
            "config": {"workload": "prefill encode, 32768 tokens x 8 KV heads x {K,V}",
                       "vectors": 524288, "d": 128, "n_atoms": 32768, "K": 16,
                       "screen": "fp16 MFMA + exact fp32 recheck"},
            "kernel_ms": round(enc["kernel_ms"], 3), "prep_ms": round(enc["prep_ms"], 3),
            "roofline": enc["roofline"], "cpu_baseline": enc.get("cpu_baseline"),
            "dtype": "f32"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
