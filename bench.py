"""Benchmark of the DART hot path on one MI355X.

A step is one prefill pass (chunk state memories -> state passing + native
chunk output -> state-memory attention + gated add) over a batch of the
Mamba-2 ~370M layer shape: batch 4, 32 heads, groups of 8 heads sharing
B/C/Q, L = 8192, S = 256, N = 128, P = 64, bfloat16 inputs with fp32
accumulation.  `value` is prefill tokens/s (batch·L / step time).  The
decode step over a 4 GiB chunk-memory cache (batch 64, 32 heads, 128
cached chunks) is timed in the same run and reported under "decode", and
the same step over the fp8 (E4M3) cache under "decode_fp8"; the backward of the
prefill (SMA and scan) at the prefill shape is reported under "backward"; the
same prefill step at L = 4096 (8 heads) and at L = 65536 (32 heads, 256
memories per head) under "prefill_L4K" and "prefill_L64K".

Prints one JSON line.  `python bench.py --steps K --warmup W`.
"""

import argparse
import json
import os
import sys
import time

BASE = {"B": 4, "L": 8192, "H": 32, "G": 4, "N": 128, "P": 64, "S": 256, "gate": 0.5}
# the L=4K prefill (8 heads, one B/C/Q group per head) and the long-context
# prefill (one sequence of 65536 tokens, 256 chunk memories per head)
PREFILL_L4K = {"B": 1, "L": 4096, "H": 8, "G": 8, "N": 128, "P": 64, "S": 256, "gate": 0.5}
PREFILL_L64K = {"B": 1, "L": 65536, "H": 32, "G": 32, "N": 128, "P": 64, "S": 256, "gate": 0.5,
                "seed": 3}
DECODE = {"B": 64, "H": 32, "G": 32, "N": 128, "P": 64, "S": 256, "chunks": 128}
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "SMA+scan prefill tokens/s & MFMA% at L=8K; decode chunk-memory HBM GB/s"

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# benchmark (bytes read = FETCH_SIZE KiB x 2 x 1024, written = WRITE_SIZE KiB x
# 1024, as calibrated by device copies of known size; profiles/); each figure
# is valid only for the kernel source it was measured on (SHA-1 of that file).
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ssm_state_attention_amd", "csrc")
_KIB = 1024
PROFILED_TRAFFIC = {
    # dart_sma_fwd at the L=8K shape: the grouped kernel k_sma_grp
    "k_sma_grp": ("k_sma.hip", "dc9720b752190e628d3a8d436d50ca99f1838525",
                  (216334 * 2 + 131072) * _KIB),
    # the two launches of one decode call with one split per head (state
    # update, then the cache stream that also writes y and advances pos)
    "dart_sma_decode": ("k_decode.hip", "5161f28fb5c89b1dff36f1c14942a25bb2ad9145",
                        (66288 * 2 + 131584 + 2098108 * 2 + 256) * _KIB),
    "dart_sma_decode_fp8": ("k_decode.hip", "5161f28fb5c89b1dff36f1c14942a25bb2ad9145",
                            (66287 * 2 + 131584 + 1050550 * 2 + 256) * _KIB),
    # the launches of one SMA backward call (dy·o pass, gate sum, token- and
    # memory-major kernels)
    "dart_sma_bwd": ("k_sma_bwd.hip", "39e45d840efc609e8323aa62695f69393d652841",
                     (196665 * 2 + 8656 + 18 * 2 + 0 + 244766 * 2 + 520192 + 565978 * 2
                      + 133251) * _KIB),
}


def profiled_traffic(kernel):
    import hashlib
    src, sha1, nbytes = PROFILED_TRAFFIC[kernel]
    if sha1 is None:
        return None
    with open(os.path.join(CSRC, src), "rb") as f:
        if hashlib.sha1(f.read()).hexdigest() != sha1:
            return None
    return nbytes


def sma_flops(c):
    """Algorithmic SMA FLOPs: 4·N·P per visible (token, memory) pair (two
    N x P contractions per pair), S·M(M-1)/2 pairs per (batch, head)."""
    M = c["L"] // c["S"]
    return 4.0 * c["N"] * c["P"] * c["S"] * M * (M - 1) / 2 * c["B"] * c["H"]


def scan_flops(c):
    """Algorithmic chunked-scan FLOPs: chunk states 2·S·N·P per chunk;
    chunk output S(S+1)/2·P (intra) + S·N·P (inter) MACs per chunk and head,
    plus the C·Bᵀ products S(S+1)/2·N per chunk and group."""
    M = c["L"] // c["S"]
    S, N, P = c["S"], c["N"], c["P"]
    per_head = 2 * M * (S * (S + 1) / 2 * P + 2 * S * N * P)
    per_group = 2 * M * S * (S + 1) / 2 * N
    return (per_head * c["H"] + per_group * c["G"]) * c["B"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the L=4K and L=64K prefill legs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy, the reference "
                         "kernel that HBM byte counters are calibrated against")
    return ap.parse_args()


def bench_prefill(args, torch, api, synth):
    c = BASE
    inp = synth.draw_prefill(0, c["B"], c["L"], c["H"], c["G"], c["N"], c["P"],
                             io=torch.bfloat16)
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    B, L, H, N, P, S = c["B"], c["L"], c["H"], c["N"], c["P"], c["S"]
    M = L // S
    f32 = dict(dtype=torch.float32, device="cuda:0")
    out = {
        "acum": torch.empty(B, H, M, S, **f32),
        "dH": torch.empty(B, H, M, P, N, dtype=torch.bfloat16, device="cuda:0"),
        "dH_f32": torch.empty(B, H, M, P, N, **f32),
        "H_in": torch.empty(B, H, M, P, N, dtype=torch.bfloat16, device="cuda:0"),
        "h_final": torch.empty(B, H, P, N, **f32),
        "y_ssd": torch.empty(B, L, H, P, dtype=torch.bfloat16, device="cuda:0"),
        "y": torch.empty(B, L, H, P, dtype=torch.bfloat16, device="cuda:0"),
    }

    def step(ev=None):
        if ev:
            ev[0].record()
        api.dart_chunk_state(d["x"], d["dt"], d["A"], d["Bm"], out["acum"], out["dH"],
                             out["dH_f32"], S)
        if ev:
            ev[1].record()
        api.dart_state_pass(d["x"], d["dt"], d["Bm"], d["C"], out["acum"], out["dH_f32"], None,
                            out["H_in"], out["h_final"], out["y_ssd"], S)
        if ev:
            ev[2].record()
        api.dart_sma_fwd(d["Q"], d["E"], d["C"], out["dH"], out["y_ssd"], c["gate"], out["y"], S)
        if ev:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    split = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(3)]
    per_step = sorted(e[0].elapsed_time(e[3]) for e in evs)
    per_sma = sorted(e[2].elapsed_time(e[3]) for e in evs)
    flops_sma, flops_scan = sma_flops(c), scan_flops(c)
    sma_ms = split[2]
    # cold inputs: 512 MB touched between repetitions evicts them from L2 and MALL
    junk = torch.empty(128 << 20, dtype=torch.float32, device="cuda:0")
    cold = []
    for _ in range(max(3, min(args.steps, 10))):
        junk.add_(1.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[3]))
    del junk
    return {
        "ms_per_step": ms,
        "step_ms_median": per_step[len(per_step) // 2],
        "step_ms_min": per_step[0],
        "step_ms_cold_median": sorted(cold)[len(cold) // 2],
        "sma_ms_median": per_sma[len(per_sma) // 2],
        "sma_ms_min": per_sma[0],
        "tokens_per_s": B * L / (ms / 1e3),
        "kernel_ms": {"chunk_state": split[0], "state_pass+chunk_out": split[1],
                      "sma_fwd": sma_ms},
        "flops": {"sma": flops_sma, "scan": flops_scan},
        "roofline": {
            "kernel": "k_sma_grp",
            "bound": "mfma",
            "achieved": flops_sma / (sma_ms / 1e3) / 1e12,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": flops_sma / (sma_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": profiled_traffic("k_sma_grp"),
        },
        "mfma_frac_whole_prefill": (flops_sma + flops_scan) / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "inputs": inp,
    }


def bench_prefill_extra(args, torch, api, synth, c, name, steps):
    """Whole-prefill timing (same step as bench_prefill) at another
    configuration: median and min over `steps` timed steps after 2 warm-up
    steps, tokens/s and the fraction of the bf16 MFMA peak of the step's
    algorithmic FLOPs and of the SMA launch's FLOPs."""
    inp = synth.draw_prefill(c.get("seed", 0), c["B"], c["L"], c["H"], c["G"], c["N"], c["P"],
                             io=torch.bfloat16)
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    del inp
    B, L, H, N, P, S = c["B"], c["L"], c["H"], c["N"], c["P"], c["S"]
    M = L // S
    f32 = dict(dtype=torch.float32, device="cuda:0")
    bf = dict(dtype=torch.bfloat16, device="cuda:0")
    out = {"acum": torch.empty(B, H, M, S, **f32), "dH": torch.empty(B, H, M, P, N, **bf),
           "dH_f32": torch.empty(B, H, M, P, N, **f32), "H_in": torch.empty(B, H, M, P, N, **bf),
           "h_final": torch.empty(B, H, P, N, **f32), "y_ssd": torch.empty(B, L, H, P, **bf),
           "y": torch.empty(B, L, H, P, **bf)}

    def step(ev):
        ev[0].record()
        api.dart_chunk_state(d["x"], d["dt"], d["A"], d["Bm"], out["acum"], out["dH"],
                             out["dH_f32"], S)
        api.dart_state_pass(d["x"], d["dt"], d["Bm"], d["C"], out["acum"], out["dH_f32"], None,
                            out["H_in"], out["h_final"], out["y_ssd"], S)
        ev[1].record()
        api.dart_sma_fwd(d["Q"], d["E"], d["C"], out["dH"], out["y_ssd"], c["gate"], out["y"], S)
        ev[2].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps + 2)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    evs = evs[2:]
    tot = sorted(e[0].elapsed_time(e[2]) for e in evs)
    sma = sorted(e[1].elapsed_time(e[2]) for e in evs)
    f_sma, f_scan = sma_flops(c), scan_flops(c)
    med, sma_med = tot[len(tot) // 2], sma[len(sma) // 2]
    return {
        "workload": name, "batch": B, "seqlen": L, "heads": H, "groups": c["G"], "dstate": N,
        "headdim": P, "chunk": S, "steps": steps,
        "step_ms_median": med, "step_ms_min": tot[0], "sma_ms_median": sma_med,
        "tokens_per_s": B * L / (med / 1e3),
        "mfma_frac_whole_prefill": (f_sma + f_scan) / (med / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "sma_mfma_frac": f_sma / (sma_med / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "algorithmic_gflop_per_step": {"sma": f_sma / 1e9, "scan": f_scan / 1e9},
    }


def sma_bwd_flops(c):
    """Algorithmic SMA backward FLOPs per visible (token, memory) pair:
    Zq and Zc again (4·N·P, the softmax weights are not stored), dQ and dC
    (2·N·P each) and the two outer products of dDeltaH (4·N·P): 12·N·P."""
    return 3.0 * sma_flops(c)


def scan_bwd_flops(c):
    """Algorithmic scan backward FLOPs: per (batch, head, chunk) the
    N×P-sized products (the outputs' state gradient, the memory term's dx
    and dB and its dt dot, the inter term's dC and its log-decay dot:
    5 × 2·S·N·P) and the causal S×S products dy·xᵀ, dx, dB, dC (2 FLOPs per
    token pair and feature, S(S+1)/2 pairs); C·Bᵀ once per group."""
    M = c["L"] // c["S"]
    S, N, P = c["S"], c["N"], c["P"]
    pairs = S * (S + 1) / 2
    per_head = 10 * S * N * P + 2 * pairs * (P + P + N + N)
    per_group = 2 * pairs * N
    return M * c["B"] * (per_head * c["H"] + per_group * c["G"])


def bench_backward(args, torch, api, synth, inp):
    """The backward of the whole prefill at the prefill shape: the training
    forward once, then dart_sma_bwd + dart_scan_bwd timed (dy ~ N(0, 1))."""
    c = BASE
    B, L, H, G, N, P, S = c["B"], c["L"], c["H"], c["G"], c["N"], c["P"], c["S"]
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    fwd = api.prefill_train(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], c["gate"],
                            S)
    dy = synth.draw_state(60, (B, L, H, P), 1.0, torch.bfloat16, device="cuda:0")
    sm = api.dart_sma_bwd(d["Q"], d["E"], d["C"], fwd["dH"], fwd["o"], fwd["lse"], dy,
                          c["gate"], S)
    sc = api.dart_scan_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["C"], fwd["acum"], fwd["H_in"],
                           dy, S, ddH=sm["ddH"], dC_sma=sm["dC"])

    def step(ev=None):
        if ev:
            ev[0].record()
        api.dart_sma_bwd(d["Q"], d["E"], d["C"], fwd["dH"], fwd["o"], fwd["lse"], dy, c["gate"],
                         S, out=sm)
        if ev:
            ev[1].record()
        api.dart_scan_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["C"], fwd["acum"], fwd["H_in"],
                          dy, S, ddH=sm["ddH"], dC_sma=sm["dC"], out=sc)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    sma_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)[args.steps // 2]
    scan_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)[args.steps // 2]
    tot_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)[args.steps // 2]
    f_sma, f_scan = sma_bwd_flops(c), scan_bwd_flops(c)
    return {
        "metric": "prefill backward tokens/s",
        "value": B * L / (tot_ms / 1e3),
        "unit": "tokens/s",
        "ms_median": tot_ms,
        "kernel_ms_median": {"dart_sma_bwd": sma_ms, "dart_scan_bwd": scan_ms},
        "algorithmic_gflop": {"sma_bwd": f_sma / 1e9, "scan_bwd": f_scan / 1e9},
        "mfma_frac_whole_backward": (f_sma + f_scan) / (tot_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "config": {"workload": "DART prefill backward (SMA + chunked scan) at the prefill shape",
                   "batch": B, "seqlen": L, "heads": H, "groups": G, "dstate": N, "headdim": P,
                   "chunk": S, "io": "bf16", "gradients": "f32"},
        "roofline": {"kernel": "dart_sma_bwd", "bound": "mfma",
                     "achieved": f_sma / (sma_ms / 1e3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": f_sma / (sma_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic("dart_sma_bwd")},
        "scan_bwd_frac": f_scan / (scan_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
    }


def timed_steps(torch, step, steps):
    """Mean over `steps` back-to-back calls (one pair of events around all
    of them), then median and min of `steps` calls timed one by one."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in evs)
    return mean, each[len(each) // 2], each[0]


def bench_decode(args, torch, api, synth):
    c = DECODE
    B, H, G, N, P, S, k = c["B"], c["H"], c["G"], c["N"], c["P"], c["S"], c["chunks"]
    st = api.new_decode_state(B, H, G, N, P, S, k, torch.bfloat16, "cuda:0")
    st["cache"].copy_(synth.draw_state(50, (B, H, k, P, N), 0.01, torch.bfloat16,
                                       device="cuda:0"))
    st["h"].copy_(synth.draw_state(51, (B, H, P, N), 0.01, torch.float32, device="cuda:0"))
    st["n_chunks"].fill_(k)
    tok = {kk: v.to("cuda:0") for kk, v in
           synth.draw_decode_token(53, B, H, G, N, P, io=torch.bfloat16).items()}
    y = torch.empty(B, H, P, dtype=torch.bfloat16, device="cuda:0")

    def step():
        api.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["Bm"], tok["C"], tok["Q"],
                        tok["E"], 0.5, y=y)

    # stay inside one chunk (no append): timed_steps makes 2·steps calls
    steps = max(1, min(args.steps, (S - 2) // 2))
    warm = max(0, min(args.warmup, S - 2 - 2 * steps))
    for _ in range(warm):
        step()
    st["pos"].zero_()
    torch.cuda.synchronize()
    ms, med, mn = timed_steps(torch, step, steps)
    cache_bytes = B * H * k * N * P * 2
    state_bytes = 2 * 2 * B * H * N * P * 4  # h and dH_cur read + written
    gbs = cache_bytes / (ms / 1e3) / 1e9
    tot = (cache_bytes + state_bytes) / (ms / 1e3) / 1e9
    return {
        "metric": "decode chunk-memory HBM GB/s",
        "value": gbs,
        "unit": "GB/s",
        "ms_per_step": ms,
        "ms_median": med,
        "ms_min": mn,
        "steps": steps,
        "chunk_memory_bytes": cache_bytes,
        "total_bytes_incl_state": cache_bytes + state_bytes,
        "total_GBps_incl_state": (cache_bytes + state_bytes) / (ms / 1e3) / 1e9,
        "config": {"workload": "DART decode over the chunk-memory cache", "batch": B,
                   "heads": H, "dstate": N, "headdim": P, "chunk": S, "cached_chunks": k,
                   "io": "bf16"},
        # the whole decode call (state update, then the cache stream that
        # also forms y and advances the positions): its algorithmic bytes
        # over its time
        "roofline": {"kernel": "dart_sma_decode", "bound": "hbm", "achieved": tot,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": tot / PEAK_HBM_GBS,
                     "traffic": profiled_traffic("dart_sma_decode")},
    }


def bench_decode_fp8(args, torch, api, synth):
    """The decode step of bench_decode over the fp8 (E4M3 + one scale per
    memory) cache: same shape, same token; the cache is encoded from f32
    memories drawn on the device, 16 chunks at a time."""
    c = DECODE
    B, H, G, N, P, S, k = c["B"], c["H"], c["G"], c["N"], c["P"], c["S"], c["chunks"]
    st = api.new_decode_state(B, H, G, N, P, S, k, torch.bfloat16, "cuda:0", fp8_cache=True)
    for blk in range(0, k, 16):
        n = min(16, k - blk)
        mem = synth.draw_state(50 + blk, (B, H, n, P, N), 0.01, torch.float32, device="cuda:0")
        api.store_memories(st, mem, first=blk)
        del mem
    st["h"].copy_(synth.draw_state(51, (B, H, P, N), 0.01, torch.float32, device="cuda:0"))
    st["n_chunks"].fill_(k)
    tok = {kk: v.to("cuda:0") for kk, v in
           synth.draw_decode_token(53, B, H, G, N, P, io=torch.bfloat16).items()}
    y = torch.empty(B, H, P, dtype=torch.bfloat16, device="cuda:0")

    def step():
        api.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["Bm"], tok["C"], tok["Q"],
                        tok["E"], 0.5, y=y)

    steps = max(1, min(args.steps, (S - 2) // 2))
    warm = max(0, min(args.warmup, S - 2 - 2 * steps))
    for _ in range(warm):
        step()
    st["pos"].zero_()
    torch.cuda.synchronize()
    ms, med, mn = timed_steps(torch, step, steps)
    cache_bytes = B * H * k * N * P + 4 * B * H * k  # codes + scales
    state_bytes = 2 * 2 * B * H * N * P * 4
    tot = (cache_bytes + state_bytes) / (ms / 1e3) / 1e9
    return {
        "metric": "decode chunk-memory HBM GB/s, fp8 cache",
        "value": cache_bytes / (ms / 1e3) / 1e9,
        "unit": "GB/s",
        "ms_per_step": ms,
        "ms_median": med,
        "ms_min": mn,
        "steps": steps,
        "chunk_memory_bytes": cache_bytes,
        "total_bytes_incl_state": cache_bytes + state_bytes,
        "config": {"workload": "DART decode over the fp8 (E4M3) chunk-memory cache",
                   "batch": B, "heads": H, "dstate": N, "headdim": P, "chunk": S,
                   "cached_chunks": k, "io": "bf16", "cache": "e4m3 + f32 scale per memory"},
        "roofline": {"kernel": "dart_sma_decode_fp8", "bound": "hbm", "achieved": tot,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": tot / PEAK_HBM_GBS,
                     "traffic": profiled_traffic("dart_sma_decode_fp8")},
    }


def _oracle_pair_rate(inp, seconds, threads):
    """Time the unmodified fp64 oracle on whole (batch, head) pairs of the
    prefill workload for about `seconds`; returns (tokens/s of the full
    layer, pairs done, seconds)."""
    from threadpoolctl import threadpool_limits

    import oracle
    from ssm_state_attention_amd import synth

    c = BASE
    H, G, S, L = c["H"], c["G"], c["S"], c["L"]
    pairs = [(b, h) for b in range(c["B"]) for h in range(H)]
    pairs = pairs[::7] + [p for p in pairs if p not in pairs[::7]]
    done, t_total = 0, 0.0
    with threadpool_limits(limits=threads):
        for b, h in pairs:
            g = h // (H // G)
            sl = {k: synth.as_f64(inp[k][b:b + 1, :, h:h + 1]) for k in ("x", "dt", "E")}
            for k in ("Bm", "C", "Q"):
                sl[k] = synth.as_f64(inp[k][b:b + 1, :, g:g + 1])
            A = synth.as_f64(inp["A"][h:h + 1])
            t0 = time.perf_counter()
            oracle.prefill(sl["x"], sl["dt"], A, sl["Bm"], sl["C"], sl["Q"], sl["E"],
                           c["gate"], S)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= seconds:
                break
    return L / (t_total / done * H), done, t_total


def _oracle_decode_rate(seconds, threads):
    """Time the unmodified fp64 oracle's decode step on single sequences of
    the decode workload (32 heads, 128 cached memories each, drawn like the
    benchmark's cache) for about `seconds`; returns chunk-memory bytes (bf16
    cache) per second."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from ssm_state_attention_amd import synth

    c = DECODE
    H, N, P, S, k = c["H"], c["N"], c["P"], c["S"], c["chunks"]
    done, t_total = 0, 0.0
    with threadpool_limits(limits=threads):
        while t_total < seconds and done < c["B"]:
            cache = np.swapaxes(synth.as_f64(synth.draw_state(50 + done, (1, H, k, P, N), 0.01,
                                                              torch.bfloat16)), -1, -2)
            tok = {kk: synth.as_f64(v) for kk, v in
                   synth.draw_decode_token(53 + done, 1, H, H, N, P).items()}
            st = {"cache": cache, "h": np.zeros((1, H, N, P)), "dH_cur": np.zeros((1, H, N, P)),
                  "n_chunks": np.array([k]), "pos": np.array([0])}
            t0 = time.perf_counter()
            oracle.decode_step(st, tok["x"], tok["dt"], tok["A"], tok["Bm"], tok["C"], tok["Q"],
                               tok["E"], 0.5, S)
            t_total += time.perf_counter() - t0
            done += 1
    return done * H * k * N * P * 2 / t_total, done, t_total


def cpu_baseline(inp, seconds):
    """The fp64 oracle, unmodified, on whole (batch, head) pairs of the same
    workload until about `seconds` of wall time, once on one thread and once
    with BLAS/OpenMP allowed every core this process may run on; the
    full-layer rate follows from the time per pair (every pair is the same
    amount of work).  The decode step is timed the same way on single
    sequences of the decode workload."""
    cores = len(os.sched_getaffinity(0))
    v_all, n_all, t_all = _oracle_pair_rate(inp, seconds, cores)
    v_one, n_one, t_one = _oracle_pair_rate(inp, seconds, 1)
    dec_all, nd, td = _oracle_decode_rate(seconds / 3, cores)
    return {
        "value": v_all,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n_all} of 128 (batch, head) pairs of the L=8192 layer, whole sequence "
                  f"each, {t_all:.1f} s, numpy/BLAS allowed {cores} threads (the host CPUs this "
                  f"process may use; os.cpu_count() = {os.cpu_count()}); full-layer tokens/s = "
                  f"L / (time per pair x 32 heads)",
        "one_thread": {"value": v_one, "unit": "tokens/s", "cores": 1,
                       "sample": f"{n_one} pairs, {t_one:.1f} s"},
        "decode": {"value": dec_all / 1e9, "unit": "GB/s of bf16 chunk memories", "cores": cores,
                   "sample": f"{nd} sequences of 32 heads x 128 memories, {td:.1f} s"},
    }


def shader_clock_levels():
    """The shader clock's DPM levels (MHz) and the level marked current, read
    from the amdgpu sysfs table (a file read: no tool is started); None where
    the table is not readable."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                lines = f.read().splitlines()
        except OSError:
            continue
        levels, current = [], None
        for line in lines:
            m = re.search(r"(\d+)\s*Mhz", line, re.I)
            if m:
                levels.append(int(m.group(1)))
                if "*" in line:
                    current = int(m.group(1))
        if levels:
            return {"levels_mhz": levels, "current_mhz": current}
    return None


def environment(torch):
    """ROCm build and device identification."""
    prop = torch.cuda.get_device_properties(0)
    return {"hip": torch.version.hip, "torch": torch.__version__,
            "arch": getattr(prop, "gcnArchName", None), "compute_units": prop.multi_processor_count,
            "hbm_bytes": prop.total_memory, "sclk": shader_clock_levels()}


def progress(msg):
    """One line per finished leg on stderr (the JSON result stays the only
    stdout line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the DART hot path here is a single-GPU "
              "build (every (batch, head) pair is independent; no multi-GPU path exists). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    from ssm_state_attention_amd import api, synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    result = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded: x ~ N(0,1); B, C, Q ~ N(0,1)/sqrt(N); E ~ N(0,1)/sqrt(P); dt log-uniform)",
              "config": {"workload": "DART prefill at the Mamba-2 ~370M layer shape",
                         "batch": BASE["B"], "seqlen": BASE["L"], "heads": BASE["H"],
                         "groups": BASE["G"], "dstate": BASE["N"], "headdim": BASE["P"],
                         "chunk": BASE["S"], "io": "bf16", "accumulate": "fp32",
                         "parallelism": "single GPU"}}
    result["env"] = environment(torch)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    pre = None
    if not args.no_prefill:
        pre = bench_prefill(args, torch, api, synth)
        levels = shader_clock_levels()
        result["env"]["sclk_current_after_prefill_mhz"] = levels and levels["current_mhz"]
        result["value"] = pre["tokens_per_s"]
        result["ms_per_step"] = pre["ms_per_step"]
        result["roofline"] = pre["roofline"]
        result["kernel_ms"] = pre["kernel_ms"]
        result["timing_ms"] = {k: pre[k] for k in ("step_ms_median", "step_ms_min",
                                                   "step_ms_cold_median", "sma_ms_median",
                                                   "sma_ms_min")}
        result["mfma_frac_whole_prefill"] = pre["mfma_frac_whole_prefill"]
        result["algorithmic_gflop_per_step"] = {k: v / 1e9 for k, v in pre["flops"].items()}
        progress(f"prefill L=8K {pre['ms_per_step']:.3f} ms per step")
    if not args.no_extra_configs and pre is not None:
        torch.cuda.empty_cache()
        result["prefill_L4K"] = bench_prefill_extra(
            args, torch, api, synth, PREFILL_L4K, "DART prefill, L=4096, 8 heads", args.steps)
        torch.cuda.empty_cache()
        result["prefill_L64K"] = bench_prefill_extra(
            args, torch, api, synth, PREFILL_L64K,
            "DART long-context prefill, L=65536, 32 heads (256 memories per head)",
            max(3, min(args.steps, 5)))
        progress("prefill L=4K and L=64K done")
    if not args.no_backward and pre is not None:
        torch.cuda.empty_cache()
        result["backward"] = bench_backward(args, torch, api, synth, pre["inputs"])
        progress("backward done")
    if not args.no_decode:
        torch.cuda.empty_cache()
        result["decode"] = bench_decode(args, torch, api, synth)
        torch.cuda.empty_cache()
        result["decode_fp8"] = bench_decode_fp8(args, torch, api, synth)
        progress("decode done")
    if not args.no_cpu_baseline and pre is not None:
        progress("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(pre["inputs"], args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
