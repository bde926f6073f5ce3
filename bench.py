#!/usr/bin/env python3
"""Benchmark of the DFlash draft head's propose path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
ctx precompute of the new rows (fc, hidden_norm, fused ctx-K/V GEMM, RoPE,
paged scatter), the propose forward (embedding, 8 drafter layers, final norm,
LM head, argmax / confidence) and the after-verify trim. Inputs are resident
in HBM before the timed region starts.

Prints ONE JSON line. `value` is draft blocks per second over the timed
steps; `us_per_propose` times the forward alone. `roofline` is measured on
the dominant kernel (LM-head stage 1) with HIP events the library records on
its own stream during the timed steps. `cpu_baseline` times the float64 oracle
on the host on a bounded sample of the same workload.

Workloads (--workload): single_ctx1024 (default), single_ctx4096_trim,
batch32_ctx512_4096, batch64_fp8_ctx256_4096, batch64_fp8a8_ctx256_4096,
single_ctx1024_fp8w. Unless --no-extra, the batch-64 FP8 workload
(64 sequences, E4M3 LM head and KV cache, 50% grammar masks) is measured in
the same run after the headline one and reported under "batch64_fp8" with its
own µs/propose, MFMA fraction and LM-head roofline.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft blocks/sec and µs/propose (γ=16, L=8, vocab 248320); % HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of MI355X
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 matrix peak of MI355X
PREFILL_ROWS = 4096  # rows of the prompt-scale precompute timed beside the step


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(geo, ctx_rows, lm_rows_per_launch):
    """Bytes a propose must move at least: every weight once, the KV it reads,
    the embedding rows; and for one LM-head launch, the head plus its rows."""
    h, I, L = geo.hidden, geo.intermediate, geo.num_layers
    q_dim, kv_dim = geo.num_q_heads * geo.head_dim, geo.num_kv_heads * geo.head_dim
    rows = (q_dim + 2 * kv_dim) + h + 2 * I + h  # output rows of the layer matrices
    layer_w = L * ((q_dim + 2 * kv_dim) * h + h * q_dim + 2 * I * h + h * I) * 2
    if getattr(geo, "layer_dtype", "bf16") == "fp8":  # E4M3 codes + one f32 scale per row
        layer_w = layer_w // 2 + L * rows * 4
    fp8 = geo.lm_head_dtype == "fp8"
    lm = geo.vocab * h * (1 if fp8 else 2) + (geo.vocab * 4 if fp8 else 0)
    kv_elem = 1 if geo.kv_dtype == "fp8" else 2
    kv = sum(min(c, geo.ctx_window) for c in ctx_rows) * L * 2 * kv_dim * kv_elem
    n = len(ctx_rows)
    embed = n * geo.gamma * h * 2
    a8 = getattr(geo, "lm_act_dtype", "bf16") == "fp8"  # W8A8 head: E4M3 rows + one f32 scale per row
    lm_launch = lm + lm_rows_per_launch * (h + 4 if a8 else h * 2)
    return layer_w + lm + kv + embed, lm_launch


def algorithmic_flops(geo, ctx_rows):
    """Multiply-add flops (2 per MAC) of a propose: every projection and the LM
    head over n * gamma rows, and attention (QK^T and PV) of each sequence's
    gamma rows over its window plus the block; and those of the LM head."""
    h, I, L, g = geo.hidden, geo.intermediate, geo.num_layers, geo.gamma
    d, nq = geo.head_dim, geo.num_q_heads
    q_dim, kv_dim = nq * d, geo.num_kv_heads * d
    M = len(ctx_rows) * g
    proj = 2 * M * L * ((q_dim + 2 * kv_dim) * h + h * q_dim + 2 * I * h + h * I)
    attn = sum(4 * g * (min(c, geo.ctx_window) + g) * nq * d * L for c in ctx_rows)
    lm = 2 * M * geo.vocab * h
    return proj + attn + lm, lm


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_single_ctx1024_traffic.md")
KERNEL_SOURCES = {"k_gemm.hip": os.path.join(ROOT, "block_diffusion_draft_03_amd", "csrc", "k_gemm.hip"),
                  "common.hpp": os.path.join(ROOT, "block_diffusion_draft_03_amd", "csrc", "common.hpp")}


def lm_head_traffic(workload):
    """HBM bytes per LM-head dispatch from the committed rocprofv3 PMC summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    plain 1 GiB copy), or None when that summary was taken on another
    workload or on kernel sources that have changed since."""
    import hashlib
    if workload != "single_ctx1024" or not os.path.exists(TRAFFIC_FILE):
        return None
    vals, hashes = {}, {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            p = line.split()
            if len(p) == 3 and p[0] == "source_sha256":
                hashes[p[1]] = p[2]
            elif len(p) == 2 and p[0].endswith(("_dispatch", "_gib")):
                vals[p[0]] = float(p[1])
    for name, path in KERNEL_SOURCES.items():
        with open(path, "rb") as f:
            if hashes.get(name) != hashlib.sha256(f.read()).hexdigest():
                return None
    fetch = vals["fetch_kib_per_dispatch"] * 1024 * (1 << 30) / (vals["copy_fetch_kib_per_gib"] * 1024)
    write = vals["write_kib_per_dispatch"] * 1024 * (1 << 30) / (vals["copy_write_kib_per_gib"] * 1024)
    return int(round(fetch + write))


def precompute_bytes(geo, rows):
    h = geo.hidden
    fc_in = geo.num_target_layers * geo.target_hidden
    fkv = geo.num_layers * 2 * geo.num_kv_heads * geo.head_dim
    kv_elem = 1 if geo.kv_dtype == "fp8" else 2
    w = (h * fc_in + fkv * h) * 2
    if getattr(geo, "layer_dtype", "bf16") == "fp8":  # E4M3 codes + one f32 scale per row
        w = w // 2 + (h + fkv) * 4
    return w + rows * fc_in * 2 + rows * fkv * kv_elem


class Workload:
    """Head, states and inputs of one workload, plus its step. `weights`
    reuses a weight set drawn for another workload of the same matrices (the
    FP8 KV scales are added when this one needs them)."""

    def __init__(self, name, steps_planned, weights=None):
        import numpy as np
        import synth
        from block_diffusion_draft_03_amd import Head
        self.wl = synth.WORKLOADS[name]
        wl = self.wl
        geo = wl.geo
        self.geo = geo
        if weights is None:
            log(f"[bench] {name}: generating weights")
            weights = synth.make_weights(geo)
        elif geo.kv_dtype == "fp8" and "kv_scale" not in weights:
            weights = dict(weights, kv_scale=synth.make_kv_scales(geo))
        self.weights = weights
        n = wl.n_seqs
        self.lens = [wl.ctx_lo] * n if wl.ctx_lo == wl.ctx_hi else [int(x) for x in synth.make_ctx_lengths(n, wl.ctx_lo, wl.ctx_hi)]
        grow = wl.new_rows * (steps_planned + 2) if wl.trim else wl.new_rows
        blocks = sum((c + grow + 15) // 16 for c in self.lens) + 16 + PREFILL_ROWS // 16
        log(f"[bench] building head (pool {blocks} blocks)")
        self.head = Head(geo, self.weights, kv_pool_blocks=blocks, max_batch=max(1, n), max_seq_len=8192)
        self.states = []
        for i, c in enumerate(self.lens):
            budget = c + grow
            ids = None
            if wl.permute_blocks:
                nb = (budget + 15) // 16
                ids = synth.make_block_permutation(nb, blocks, tag=i)
            st = self.head.state_create(budget_tokens=budget, block_ids=ids)
            self.head.precompute([st], [c], synth.make_stack(geo, c, tag=i))
            self.head.after_verify(st, c)
            self.states.append(st)
        import torch
        dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
        self.new_stack = dev(np.concatenate([synth.make_stack(geo, wl.new_rows, tag=10000 + i) for i in range(n)]))
        self.tokens = synth.make_tokens(geo, n)
        self.masks = None
        if wl.mask_frac > 0:
            self.masks = dev(np.stack([synth.make_bitmask(geo.vocab, wl.mask_frac, tag=i) for i in range(n)]))
        self.accepted = synth.make_accepted(steps_planned + 64, wl.new_rows)
        self.k = 0
        torch.cuda.synchronize()

    def propose(self):
        wl = self.wl
        if wl.n_seqs == 1:
            st = self.states[0]
            return self.head.propose(st, int(self.tokens[0]), st.ctx_len, self.geo.gamma - 1,
                                     bitmask=None if self.masks is None else self.masks[0])
        pos = [s.ctx_len for s in self.states]
        return self.head.propose_batch(self.states, self.tokens, pos, self.geo.gamma - 1, bitmasks=self.masks)

    def step(self):
        wl = self.wl
        n = wl.n_seqs
        self.head.precompute(self.states, [wl.new_rows] * n, self.new_stack)
        if wl.trim:
            a = int(self.accepted[self.k % len(self.accepted)])
            for st in self.states:
                self.head.after_verify(st, a)
            out = self.propose()
        else:
            out = self.propose()
            for st in self.states:
                self.head.after_verify(st, 0)
        self.k += 1
        return out


def time_prefill(w, reps=3):
    """Microseconds of one prompt-scale precompute (PREFILL_ROWS rows into a
    fresh state), from the library's HIP events on its stream, and its flops."""
    import torch
    import synth
    geo = w.geo
    stack = synth.make_stack(geo, PREFILL_ROWS, tag=777)
    st = w.head.state_create(budget_tokens=PREFILL_ROWS)
    w.head.precompute([st], [PREFILL_ROWS], stack)  # warm
    st.free()
    torch.cuda.synchronize()
    w.head.timing_enable(True)
    w.head.timing_read(2)
    for _ in range(reps):
        st = w.head.state_create(budget_tokens=PREFILL_ROWS)
        w.head.precompute([st], [PREFILL_ROWS], stack)
        torch.cuda.synchronize()
        st.free()
    ms, n = w.head.timing_read(2)
    w.head.timing_enable(False)
    fkv = geo.num_layers * 2 * geo.num_kv_heads * geo.head_dim
    flops = 2 * PREFILL_ROWS * geo.hidden * (geo.num_target_layers * geo.target_hidden + fkv)
    return ms / max(1, n) * 1e3, flops


def time_loop(fn, steps):
    import torch
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def cpu_baseline(wl_obj, budget_s=12.0, max_seqs=2):
    """Time the float64 oracle on the host on a bounded sample: at most
    max_seqs sequences of the workload, whole steps (precompute of the new
    rows + propose + trim), for about budget_s seconds after one warm-up;
    with the BLAS threads numpy has (all host cores), then with one."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    out = _cpu_baseline_run(wl_obj, budget_s, max_seqs, cores)
    with threadpool_limits(limits=1):
        one = _cpu_baseline_run(wl_obj, budget_s, 1, 1)
    out["single_thread"] = one
    out["precision"] = "float64"
    return out


def _cpu_baseline_run(wl_obj, budget_s, max_seqs, cores):
    import numpy as np
    import synth
    from oracle.dflash import OracleHead
    wl = wl_obj.wl
    geo = wl_obj.geo
    log(f"[bench] cpu baseline ({cores} threads): oracle setup")
    orc = OracleHead(geo.as_dict(), wl_obj.weights)
    idx = list(range(min(max_seqs, wl.n_seqs)))
    states = []
    for i in idx:
        st = orc.new_state()
        orc.precompute(st, synth.make_stack(geo, wl_obj.lens[i], tag=i))
        orc.after_verify(st, wl_obj.lens[i])
        states.append(st)
    news = [synth.make_stack(geo, wl.new_rows, tag=10000 + i) for i in idx]
    masks = [synth.make_bitmask(geo.vocab, wl.mask_frac, tag=i) if wl.mask_frac > 0 else None for i in idx]

    def step():
        for j, st in enumerate(states):
            orc.precompute(st, news[j])
            orc.propose(st, int(wl_obj.tokens[idx[j]]), st.ctx_len, geo.gamma - 1, masks[j])
            orc.after_verify(st, 0)

    step()
    t0 = time.perf_counter()
    k = 0
    while True:
        step()
        k += 1
        if time.perf_counter() - t0 >= budget_s or k >= 400:
            break
    dt = time.perf_counter() - t0
    return {"value": round(k * len(idx) / dt, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{k} steps x {len(idx)} sequence(s) of {wl.name} (precompute {wl.new_rows} rows + "
                      f"propose + trim), float64 numpy, {dt:.1f} s"}


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for scaling PMC byte
    counters (FETCH_SIZE / WRITE_SIZE) against what they read for it."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))


def same_matrices(a, b):
    """Whether two geometries draw the same weight matrices (synth draws them
    from the shapes and the stored dtype only)."""
    key = lambda g: (g.num_layers, g.hidden, g.intermediate, g.num_q_heads, g.num_kv_heads, g.head_dim, g.vocab,
                     g.num_target_layers, g.target_hidden, g.weight_dtype)
    return key(a) == key(b)


EXTRA_WORKLOAD = "batch64_fp8_ctx256_4096"
EXTRA_KEY = "batch64_fp8"


def measure(w, steps, warmup):
    """Warm up, time `steps` whole steps (instrumented: per-phase HIP events on
    the library's stream), then the forward alone (uninstrumented) and a
    prompt-scale precompute; returns the workload's measurements."""
    import torch
    geo, wl = w.geo, w.wl
    log(f"[bench] {wl.name}: warmup {warmup}")
    for _ in range(warmup):
        w.step()
    torch.cuda.synchronize()

    log(f"[bench] {wl.name}: timing {steps} steps")
    w.head.timing_enable(True)
    w.head.timing_read(0)
    w.head.timing_read(1)
    w.head.timing_read(2)
    ms_step, wall = time_loop(w.step, steps)
    lm_ms, lm_launches = w.head.timing_read(0)
    prop_ms, prop_n = w.head.timing_read(1)
    pre_ms, pre_n = w.head.timing_read(2)
    w.head.timing_enable(False)
    # forward alone, uninstrumented
    ms_prop, _ = time_loop(w.propose, steps)
    us_prefill, prefill_flops = time_prefill(w)

    ctx_rows = [s.ctx_len + (0 if wl.trim else wl.new_rows) for s in w.states]
    rows = wl.n_seqs * geo.gamma
    lm_rows = rows  # one LM-head launch covers every row
    fwd_bytes, lm_bytes = algorithmic_bytes(geo, ctx_rows, lm_rows)
    fwd_flops, lm_flops = algorithmic_flops(geo, ctx_rows)
    lm_avg_s = lm_ms / max(1, lm_launches) / 1e3
    lm_gbs = lm_bytes / lm_avg_s / 1e9
    lm_tflops = lm_flops / lm_avg_s / 1e12
    if rows > (64 if geo.layer_dtype == "fp8" else 32) or getattr(geo, "lm_act_dtype", "bf16") == "fp8":
        # many rows (the library's switch to the tiled kernels): the LM head is an
        # MFMA-bound GEMM (bf16 MFMA, also for the E4M3 head widened to bf16; the
        # W8A8 head runs on the E4M3 matrix cores and takes their peak)
        a8 = getattr(geo, "lm_act_dtype", "bf16") == "fp8"
        peak = MFMA_FP8_PEAK_TFLOPS if a8 else MFMA_BF16_PEAK_TFLOPS
        roofline = {"kernel": "k_blm_head (tiled LM-head GEMM + argmax stage 1" + (", W8A8)" if a8 else ")"),
                    "bound": "mfma", "achieved": round(lm_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(lm_tflops / peak, 4), "traffic": None,
                    "flops_per_launch": lm_flops, "avg_launch_us": round(lm_avg_s * 1e6, 2),
                    "launches": lm_launches}
    else:
        roofline = {"kernel": "k_lm_head (LM-head GEMM + argmax stage 1)", "bound": "hbm",
                    "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": lm_head_traffic(wl.name),
                    "bytes_per_launch": lm_bytes, "avg_launch_us": round(lm_avg_s * 1e6, 2),
                    "launches": lm_launches}
    return {
        "blocks_per_s": round(wl.n_seqs / (ms_step / 1e3), 3),
        "ms_per_step": round(ms_step, 4),
        "dtype": "bf16" if geo.lm_head_dtype == "bf16" and geo.layer_dtype == "bf16" else "bf16+fp8",
        "config": {"workload": wl.name, "n_seqs": wl.n_seqs, "ctx_rows": ctx_rows if wl.n_seqs <= 4 else
                   [min(ctx_rows), max(ctx_rows)], "gamma": geo.gamma, "layers": geo.num_layers,
                   "vocab": geo.vocab, "hidden": geo.hidden, "new_rows_per_step": wl.new_rows,
                   "lm_head": geo.lm_head_dtype + ("a8" if getattr(geo, "lm_act_dtype", "bf16") == "fp8" else ""),
                   "drafter_weights": geo.layer_dtype, "kv_cache": geo.kv_dtype,
                   "grammar_mask": wl.mask_frac, "parallelism": "none"},
        "us_per_propose": round(ms_prop * 1e3, 2),
        "us_per_propose_in_step": round(prop_ms / max(1, prop_n) * 1e3, 2),
        "us_per_precompute": round(pre_ms / max(1, pre_n) * 1e3, 2),
        "propose_hbm_frac": round(fwd_bytes / (ms_prop / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "propose_algorithmic_bytes": fwd_bytes,
        "propose_mfma_frac": round(fwd_flops / (ms_prop / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "propose_algorithmic_flops": fwd_flops,
        "roofline": roofline,
        "prefill_rows": PREFILL_ROWS,
        "us_per_prefill": round(us_prefill, 2),
        "prefill_mfma_frac": round(prefill_flops / (us_prefill / 1e6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="single_ctx1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help=f"skip the {EXTRA_WORKLOAD} measurement reported under '{EXTRA_KEY}'")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--extra-warmup", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the propose path is data-parallel over sequences and each GPU "
              f"would run its own head; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    w = Workload(args.workload, args.steps + args.warmup)
    m = measure(w, args.steps, args.warmup)
    geo, wl = w.geo, w.wl
    out = {
        "metric": METRIC,
        "value": m["blocks_per_s"],
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic",
        "config": m["config"],
    }
    out.update({k: v for k, v in m.items() if k not in ("blocks_per_s", "ms_per_step", "dtype", "config")})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    import synth
    weights = w.weights if same_matrices(w.geo, synth.WORKLOADS[EXTRA_WORKLOAD].geo) else None
    for st in w.states:
        st.free()
    w.head.destroy()
    del w
    if args.extra and args.workload != EXTRA_WORKLOAD:
        # the batched FP8 workload beside the headline, in the same run
        torch.cuda.empty_cache()
        x = Workload(EXTRA_WORKLOAD, args.extra_steps + args.extra_warmup, weights=weights)
        mx = measure(x, args.extra_steps, args.extra_warmup)
        mx["steps"], mx["warmup"] = args.extra_steps, args.extra_warmup
        out[EXTRA_KEY] = mx
        for st in x.states:
            st.free()
        x.head.destroy()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
