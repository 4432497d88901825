#!/usr/bin/env python3
"""GPTQ layer-quantization benchmark on one MI355X.

One step = the whole path on one layer with its calibration set already in
HBM: clear H, H = 2·XᵀX over all tokens (one call), damping + act-order +
inverse factor, block-wise quantization with error feedback and packing.
Default workload: the 7B MLP down projection, W 4096 x 11008 bf16, X 262144
tokens x 11008 bf16, 4-bit asym, group 128, desc_act.

With the default workload it also times the 7B-shaped sweep (32 decoder
layers x {q, k, v, o, gate, up, down}, at 4-bit g128 and at 3-bit g64; X and W
regenerated per linear outside the timed calls) and reports its total seconds;
then the same sweep as a model is quantized: one calibration input per
(decoder layer, input) shared by the linears that read it (q/k/v, gate/up), its
H and inverse factor computed once and reused for both settings.

Prints ONE JSON line on stdout; progress goes to stderr.
    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-sweep]
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

METRIC = "GPTQ s/layer (4096x11008, g128); XᵀX TFLOP/s; total s for 7B-shaped sweep"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
SYRK_KERNEL_SOURCE = os.path.join(ROOT, "post_weight_quantization_14_amd", "csrc", "hessian.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "syrk_bf16_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


NEXT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "next_rows_traffic.json")


def next_rows_traffic(row: str, key: str):
    """HBM bytes per call of a next-row kernel from the committed counter runs,
    if they were taken on the current source of that row (every file it
    lists); else None."""
    try:
        with open(NEXT_TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = rec["sources"][row]
        for name, sha in src.items():
            if sha != source_hash(os.path.join(ROOT, name)):
                return None
        return rec["hbm_bytes_per_call"].get(key)
    except (OSError, ValueError, KeyError, AttributeError):
        return None


def measured_traffic(workload: str):
    """HBM bytes per SYRK launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != source_hash(SYRK_KERNEL_SOURCE):
        return None
    entry = rec.get("workloads", {}).get(workload)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


class Layer:
    """Device buffers of one layer and the three ABI calls of a step."""

    def __init__(self, pq, spec, W, X):
        import torch
        self.pq, self.spec, self.W, self.X = pq, spec, W, X
        m, n, T = spec.m, spec.n, spec.tokens
        dev = W.device
        self.cfg = pq.QuantConfig(bits=spec.bits, group_size=spec.group_size, sym=spec.sym,
                                  desc_act=spec.desc_act, damp_percent=spec.damp_percent)
        self.H = torch.empty(n, n, dtype=torch.float32, device=dev)
        self.key = torch.empty(n, dtype=torch.float64, device=dev)
        code = pq.GPTQ_BF16 if X.dtype == torch.bfloat16 else pq.GPTQ_FP32
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_h = torch.empty(max(pq.gptq_hessian_workspace_bytes(n, T, code), 1), **u8)
        self.ws_p = torch.empty(pq.gptq_prepare_workspace_bytes(n), **u8)
        self.ws_q = torch.empty(pq.gptq_quantize_workspace_bytes(m, n, self.cfg), **u8)
        self.out = pq.alloc_outputs(m, n, self.cfg, dev)
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(self):
        pq, o = self.pq, self.out
        self.H.zero_()
        self.key.zero_()
        self.ev[0].record()
        pq.gptq_hessian_accumulate(self.H, self.key, self.X, 2.0, self.ws_h)
        self.ev[1].record()
        self.lam = pq.gptq_prepare_hinv(self.H, self.key, self.cfg.damp_percent, self.cfg.desc_act,
                                        o["perm"], self.ws_p)
        self.ev[2].record()
        pq.gptq_quantize_layer(self.W, self.H, o["perm"], self.cfg, o["qweight"], o["scales"],
                               o["zeros"], o["g_idx"], o["loss"], o["status"], self.ws_q)
        self.ev[3].record()

    def stage_ms(self):
        self.ev[3].synchronize()
        return [self.ev[i].elapsed_time(self.ev[i + 1]) for i in range(3)]


def run_sweep_shared(pq, torch, bits_groups, log_every=32):
    """The 7B-shaped sweep with one calibration input per (decoder layer, input)
    and both settings in one pass: per input, H = 2·XᵀX and U once, then every
    linear reading that input quantized at every setting.  X and W are
    generated outside the timed calls; returns total and per-stage seconds."""
    import workloads
    cfgs = [pq.QuantConfig(bits=b, group_size=g, sym=False, desc_act=True, damp_percent=0.01)
            for b, g in bits_groups]
    groups = workloads.sweep_shared_groups(*bits_groups[0])
    bufs = {}

    def buf(key, make):
        if key not in bufs:
            bufs[key] = make()
        return bufs[key]

    u8 = dict(dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    stage = [0.0, 0.0, 0.0]
    total = gen_total = ideal = 0.0
    linears = 0
    outs = []
    for i, (xs, wspecs) in enumerate(groups):
        tg = time.perf_counter()
        n, T = xs.n, xs.tokens
        for k in [k for k in bufs if k[0] == "X" and k[1] != n]:
            del bufs[k]
        X = workloads.gen_x(xs, "cuda", out=buf(("X", n), lambda: torch.empty(T, n, dtype=torch.bfloat16,
                                                                              device="cuda")))
        Ws = [workloads.gen_weight(w, "cuda") for w in wspecs]
        H = buf(("H", n), lambda: torch.empty(n, n, dtype=torch.float32, device="cuda"))
        key = buf(("key", n), lambda: torch.empty(n, dtype=torch.float64, device="cuda"))
        perm = buf(("perm", n), lambda: torch.empty(n, dtype=torch.int32, device="cuda"))
        ws_h = buf(("wsh", n), lambda: torch.empty(max(pq.gptq_hessian_workspace_bytes(n, T, pq.GPTQ_BF16), 1), **u8))
        ws_p = buf(("wsp", n), lambda: torch.empty(pq.gptq_prepare_workspace_bytes(n), **u8))
        jobs = []
        for W in Ws:
            m = W.shape[0]
            for j, cfg in enumerate(cfgs):
                o = buf(("out", m, n, j), lambda: pq.alloc_outputs(m, n, cfg, "cuda"))
                wq = buf(("wsq", m, n, j), lambda: torch.empty(pq.gptq_quantize_workspace_bytes(m, n, cfg), **u8))
                jobs.append((W, cfg, o, wq))
        torch.cuda.synchronize()
        gen_total += time.perf_counter() - tg
        t0 = time.perf_counter()
        H.zero_()
        key.zero_()
        ev[0].record()
        pq.gptq_hessian_accumulate(H, key, X, 2.0, ws_h)
        ev[1].record()
        pq.gptq_prepare_hinv(H, key, 0.01, True, perm, ws_p)
        ev[2].record()
        for W, cfg, o, wq in jobs:
            pq.gptq_quantize_layer(W, H, perm, cfg, o["qweight"], o["scales"], o["zeros"], o["g_idx"],
                                   o["loss"], o["status"], wq)
        ev[3].record()
        torch.cuda.synchronize()
        total += time.perf_counter() - t0
        ideal += ideal_seconds(0, n, T, trail=False)
        for W, cfg, o, wq in jobs:
            ideal += ideal_seconds(W.shape[0], n, T, syrk=False, chol=False)
            outs.append({"status": o["status"].clone()})
        for s_ in range(3):
            stage[s_] += ev[s_].elapsed_time(ev[s_ + 1]) / 1e3
        linears += len(Ws)
        del Ws
        if (i + 1) % log_every == 0:
            log(f"sweep (shared inputs): {i + 1}/{len(groups)} inputs, {total:.2f}s so far")
    pq.check_status(outs)
    names = "+".join(f"{b}bit_g{g}" for b, g in bits_groups)
    log(f"sweep (shared inputs): {total:.3f}s, ideal {ideal:.3f}s, fraction {ideal / total:.3f}")
    return {"settings": names, "total_s": total, "ideal_s": ideal, "roofline_frac": ideal / total,
            "inputs": len(groups), "linears": linears,
            "quantizations": linears * len(cfgs), "data_gen_s": gen_total,
            "stage_s": {"hessian": stage[0], "prepare": stage[1], "quantize": stage[2]}}


def cpu_baseline(spec, W, X, log_prefix="cpu_baseline", full=False):
    """The float64 oracle on a bounded sample of the same layer, scaled to
    s/layer (full=True: the whole layer, every token and row, unscaled)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads

    cores = len(os.sched_getaffinity(0))
    # the sample: one 8192-token tile (BLAS-sized, so the Hessian rate is the
    # whole layer's) and 256 rows
    t_tok = spec.tokens if full else min(8192, spec.tokens)
    r_rows = spec.m if full else min(256, spec.m)
    if full:
        with threadpool_limits(limits=cores):
            t0 = time.perf_counter()
            H = np.zeros((spec.n, spec.n))
            key = np.zeros(spec.n)
            last = t0
            for r0 in range(0, spec.tokens, workloads.TILE_TOKENS):
                H, key = oracle.hessian_accumulate(H, key, workloads.to_numpy_f64(X[r0:r0 + workloads.TILE_TOKENS]))
                if time.perf_counter() - last > 30:
                    last = time.perf_counter()
                    log(f"{log_prefix}: full hessian {r0 + workloads.TILE_TOKENS}/{spec.tokens} tokens, "
                        f"{last - t0:.0f}s")
            t1 = time.perf_counter()
            log(f"{log_prefix}: full hessian {t1 - t0:.1f}s")
            U, perm, lam = oracle.prepare(H, key, spec.damp_percent, spec.desc_act)
            t2 = time.perf_counter()
            log(f"{log_prefix}: full prepare {t2 - t1:.1f}s")
            Wf = workloads.to_numpy_f64(W)
            # rows are independent given U: 256 at a time, with progress lines
            for r0 in range(0, spec.m, 256):
                oracle.gptq_quantize(Wf[r0:r0 + 256, perm], U, spec.bits, spec.group_size, spec.sym, block=128)
                log(f"{log_prefix}: full quantize {min(r0 + 256, spec.m)}/{spec.m} rows, "
                    f"{time.perf_counter() - t2:.0f}s")
            t3 = time.perf_counter()
        th, tp, tq = t1 - t0, t2 - t1, t3 - t2
        log(f"{log_prefix}: full layer: hessian {th:.1f}s, prepare {tp:.1f}s, quantize {tq:.1f}s")
        return {"value": th + tp + tq, "unit": "s/layer", "cores": cores, "kind": "oracle",
                "sample": "float64 NumPy oracle on the whole layer (every token; every row, 256 rows per call), not scaled",
                "stage_s": {"hessian": th, "prepare": tp, "quantize": tq}}
    Xs = workloads.to_numpy_f64(X[:t_tok])
    Ws = workloads.to_numpy_f64(W[:r_rows])
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        H, key = oracle.hessian([Xs], spec.n)
        t1 = time.perf_counter()
        U, perm, lam = oracle.prepare(H, key, spec.damp_percent, spec.desc_act)
        t2 = time.perf_counter()
        oracle.gptq_quantize(Ws[:, perm], U, spec.bits, spec.group_size, spec.sym, block=128)
        t3 = time.perf_counter()
    th, tp, tq = t1 - t0, t2 - t1, t3 - t2
    est = th * spec.tokens / t_tok + tp + tq * spec.m / r_rows
    log(f"{log_prefix}: hessian {th:.2f}s/{t_tok} tok, prepare {tp:.2f}s, quantize {tq:.2f}s/{r_rows} rows")
    return {
        "value": est, "unit": "s/layer", "cores": cores, "kind": "oracle",
        "sample": (f"float64 NumPy oracle on this layer: Hessian over the first {t_tok} of "
                   f"{spec.tokens} tokens (x{spec.tokens / t_tok:.0f}), full damping/act-order/"
                   f"inverse factor at n={spec.n}, column quantization of {r_rows} of {spec.m} rows "
                   f"(x{spec.m / r_rows:.0f}, rows are independent given U); measured "
                   f"{th + tp + tq:.1f} s, scaled to one layer"),
        "stage_s": {"hessian": th * spec.tokens / t_tok, "prepare": tp, "quantize": tq * spec.m / r_rows},
    }


def run_sweep(pq, torch, bits_groups, log_every=16):
    """The 7B-shaped sweep: 32 layers x 7 linears per setting, X regenerated
    per linear outside the timed calls; returns total seconds per setting."""
    import workloads
    res = {}
    for bits, g in bits_groups:
        specs = workloads.sweep_specs(bits, g)
        total = 0.0
        gen_total = 0.0
        ideal = 0.0
        statuses = []
        xbuf = {}
        for i, sp in enumerate(specs):
            tg = time.perf_counter()
            W = workloads.gen_weight(sp, "cuda")
            key = (sp.tokens, sp.n)
            if key not in xbuf:
                xbuf.clear()
                torch.cuda.empty_cache()
                xbuf[key] = torch.empty(sp.tokens, sp.n, dtype=torch.bfloat16, device="cuda")
            X = workloads.gen_x(sp, "cuda", out=xbuf[key])
            layer = Layer(pq, sp, W, X)
            torch.cuda.synchronize()
            gen_total += time.perf_counter() - tg
            t0 = time.perf_counter()
            layer.step()
            torch.cuda.synchronize()
            total += time.perf_counter() - t0
            statuses.append(layer.out)
            ideal += ideal_seconds(sp.m, sp.n, sp.tokens)
            del layer
            if (i + 1) % log_every == 0:
                log(f"sweep {bits}-bit g{g}: {i + 1}/{len(specs)} linears, {total:.2f}s so far")
        pq.check_status(statuses)
        res[f"{bits}bit_g{g}"] = {"total_s": total, "linears": len(specs), "data_gen_s": gen_total,
                                  "ideal_s": ideal, "roofline_frac": ideal / total}
        log(f"sweep {bits}-bit g{g}: {total:.3f}s, ideal {ideal:.3f}s, fraction {ideal / total:.3f}")
    return res


def measure_rtn(pq, torch, W, reps=20):
    """The linear round-to-nearest quantizer (the pages' LinearQuantizer) on
    this layer's weight, per setting: ms per call (HIP events on the stream
    the kernels run on, `reps` stream-ordered calls back to back; the NaN
    check is a device status word, read once after them) and the HBM
    roofline of the call's algorithmic bytes (W read once; codes, scales and
    zeros written once)."""
    m, n = W.shape
    res = {}
    for name, cfg in (("int8_sym_per_row_clip0.99", pq.RtnConfig(8, -1, True, 0.99)),
                      ("int4_asym_g128_clip1.0", pq.RtnConfig(4, 128, False, 1.0))):
        outs = pq.rtn_quantize(W, cfg)   # allocates the outputs, warms the kernels
        ws = torch.empty(max(pq.gptq_rtn_workspace_bytes(m, n, cfg), 1), dtype=torch.uint8, device=W.device)
        status = torch.zeros(1, dtype=torch.int32, device=W.device)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            pq.gptq_rtn_quantize(W, cfg, outs["qweight"], outs["scales"], outs["zeros"], outs["err"], ws,
                                 status=status, check=False)
        e1.record()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        ms = e0.elapsed_time(e1) / reps
        words = pq.gptq_qweight_words(n, cfg.bits)
        groups = pq.gptq_num_groups(n, cfg.group_size)
        nbytes = m * n * W.element_size() + m * words * 4 + m * groups * 8
        gbs = nbytes / (ms * 1e-3) / 1e9
        err = outs["err"].cpu().tolist()
        # clip ratio 1 streams (extremes only); a clipped grid needs order statistics
        kernel = ("rtn_stream_kernel + rtn_reduce_kernel" if cfg.clip_ratio >= 1.0 else
                  "rtn_row_kernel + rtn_reduce_kernel")
        res[name] = {"ms": ms, "mse": err[0], "cos": err[1],
                     "roofline": {"bound": "hbm", "kernel": kernel,
                                  "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": gbs / PEAK_HBM_GBS,
                                  "traffic": next_rows_traffic("rtn", name) if (m, n) == (4096, 11008) else None,
                                  "algorithmic_bytes_per_call": nbytes}}
        log(f"bench: rtn {name}: {ms:.3f} ms, {gbs:.0f} GB/s, mse {err[0]:.4e}, cos {err[1]:.6f}")
    return res


def measure_w4a16(pq, torch, out, m, n, bits, group_size, reps=200):
    """The product of bf16 activations with this layer's quantized weight
    (W4A16: gptq_w4a16_pack once, then gptq_w4a16_matmul per call) at 1, 16
    and 64 tokens: µs per call (HIP events on the stream the kernels run on,
    `reps` calls back to back), the HBM roofline of its algorithmic bytes
    (codes m·n/2, per-group scale and zero 8 bytes, column order 4·n, X read
    once, Y written once), and the same product through torch.matmul on the
    dequantized bf16 weight (hipBLASLt) for comparison."""
    groups = pq.gptq_num_groups(n, group_size)
    packed = pq.gptq_w4a16_pack(out["qweight"], out["scales"], out["zeros"], out["g_idx"], n, bits,
                                group_size)
    Wd = torch.randn(m, n, device="cuda").to(torch.bfloat16)   # dense weight of the same shape
    gen = torch.Generator(device="cuda").manual_seed(99)
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for tokens in (1, 16, 64):
        X = torch.randn(tokens, n, device="cuda", generator=gen).to(torch.bfloat16)
        Y = torch.empty(tokens, m, device="cuda")
        ws = torch.empty(pq.gptq_w4a16_workspace_bytes(tokens, m, n), dtype=torch.uint8, device="cuda")
        for _ in range(10):
            pq.gptq_w4a16_matmul(X, packed, m, n, group_size, Y=Y, workspace=ws)
            torch.matmul(X, Wd.t())
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            pq.gptq_w4a16_matmul(X, packed, m, n, group_size, Y=Y, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        e0.record()
        for _ in range(reps):
            torch.matmul(X, Wd.t())
        e1.record()
        torch.cuda.synchronize()
        us_bf16 = e0.elapsed_time(e1) / reps * 1e3
        nbytes = m * n // 2 + m * groups * 8 + 4 * n + tokens * n * 2 + tokens * m * 4
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"tokens_{tokens}"] = {
            "us": us, "bf16_matmul_us": us_bf16, "speedup_vs_bf16": us_bf16 / us,
            "roofline": {"bound": "hbm",
                         "kernel": ("w4_gather_kernel + w4_gemv_kernel" if tokens <= 4 else
                                    "w4_gather_kernel + w4_gemm_kernel + w4_reduce_kernel"),
                         "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                         "traffic": next_rows_traffic("w4a16", f"tokens_{tokens}") if (m, n) == (4096, 11008) else None,
                         "algorithmic_bytes_per_call": nbytes}}
        log(f"bench: w4a16 {m}x{n} tokens {tokens}: {us:.2f} us ({gbs:.0f} GB/s), "
            f"bf16 matmul {us_bf16:.2f} us, speedup {us_bf16 / us:.2f}x")
    # the same output exported to the GPTQ-checkpoint tensors (qweight
    # [n·b/32, m], qzeros [G, m·b/32], fp16 scales [G, m]): read the
    # quantizer's words, scales and zeros once, write the three tensors once
    for _ in range(10):
        pq.gptq_export_checkpoint(out["qweight"], out["scales"], out["zeros"], n, bits, group_size)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        pq.gptq_export_checkpoint(out["qweight"], out["scales"], out["zeros"], n, bits, group_size)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    words = pq.gptq_qweight_words(n, bits)
    nbytes = (m * words * 4 + m * groups * 8 + pq.gptq_checkpoint_qweight_rows(n, bits) * m * 4
              + groups * pq.gptq_checkpoint_qzeros_words(m, bits) * 4 + groups * m * 2)
    gbs = nbytes / (us * 1e-6) / 1e9
    res["checkpoint_export"] = {
        "us": us,
        "roofline": {"bound": "hbm", "kernel": "ck_qweight_kernel + ck_params_kernel", "achieved": gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes_per_call": nbytes}}
    log(f"bench: checkpoint export {m}x{n}: {us:.2f} us ({gbs:.0f} GB/s)")
    return res


def _dequant(torch, qweight, scales, zeros, gidx, n):
    """Ŵ [m, n] fp32 from the packed 4-bit output (evaluation only)."""
    shifts = torch.arange(0, 32, 4, device=qweight.device, dtype=torch.int32)
    codes = ((qweight.unsqueeze(-1) >> shifts) & 15).reshape(qweight.shape[0], -1)[:, :n].float()
    g = gidx.long()
    return (codes - zeros[:, g].float()) * scales[:, g]


def measure_awq(pq, torch, W, X, gptq_out, reps=10, eval_tokens=4096):
    """The pages' AWQ channel scaling on this layer (4-bit asym g128, s = 2):
    the channel statistics pass over the whole calibration X (HBM roofline of
    reading X once) and the scaled linear quantizer, each in ms per call (HIP
    events on the stream the kernels run on; the quantizer's NaN check is a
    device status word read once after the timed calls).  For context, the
    relative output error ‖X(W - Ŵ)ᵀ‖ / ‖X Wᵀ‖ on the first `eval_tokens`
    calibration tokens for AWQ, plain round-to-nearest and GPTQ."""
    m, n = W.shape
    T = X.shape[0]
    cfg = pq.RtnConfig(bits=4, group_size=128, sym=False, clip_ratio=1.0)
    abs_sum = torch.zeros(n, dtype=torch.float64, device="cuda")
    ws = torch.empty(pq.gptq_awq_stats_workspace_bytes(n, T), dtype=torch.uint8, device="cuda")
    pq.gptq_awq_channel_stats(X, abs_sum, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        abs_sum.zero_()
        pq.gptq_awq_channel_stats(X, abs_sum, ws)
    e1.record()
    torch.cuda.synchronize()
    stats_ms = e0.elapsed_time(e1) / reps
    xbytes = T * n * X.element_size()
    G = pq.gptq_num_groups(n, 128)
    out = dict(qweight=torch.empty(m, pq.gptq_qweight_words(n, 4), dtype=torch.int32, device="cuda"),
               scales=torch.empty(m, G, device="cuda"), zeros=torch.empty(m, G, dtype=torch.int32, device="cuda"),
               channel_scale=torch.empty(n, device="cuda"), err=torch.zeros(2, dtype=torch.float64, device="cuda"))
    qws = torch.empty(pq.gptq_awq_workspace_bytes(m, n, cfg), dtype=torch.uint8, device="cuda")
    args = (W, abs_sum, T, 2.0, cfg, out["qweight"], out["scales"], out["zeros"], out["channel_scale"],
            out["err"], qws)
    pq.gptq_awq_quantize(*args)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        pq.gptq_awq_quantize(*args, status=status, check=False)
    e1.record()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    quant_ms = e0.elapsed_time(e1) / reps
    qbytes = m * n * W.element_size() + m * (n // 8) * 4 + m * ((n + 127) // 128) * 8 + 4 * n
    # output error on a token sample
    Xs = X[:eval_tokens].float()
    Wf = W.float()
    Y = Xs @ Wf.t()
    col_g = torch.arange(n, device="cuda") // 128
    W_awq = _dequant(torch, out["qweight"], out["scales"], out["zeros"], col_g, n) / out["channel_scale"]
    rtn = pq.rtn_quantize(W, cfg)
    W_rtn = _dequant(torch, rtn["qweight"], rtn["scales"], rtn["zeros"], col_g, n)
    W_gptq = _dequant(torch, gptq_out["qweight"], gptq_out["scales"], gptq_out["zeros"], gptq_out["g_idx"], n)
    rel = {k: float(torch.linalg.norm(Xs @ (Wf - Wq).t()) / torch.linalg.norm(Y))
           for k, Wq in (("awq", W_awq), ("rtn", W_rtn), ("gptq", W_gptq))}
    err = out["err"].cpu().tolist()
    res = {
        "channel_stats": {"ms": stats_ms, "roofline": {
            "bound": "hbm", "kernel": "awq_stats_kernel + awq_stats_reduce_kernel",
            "achieved": xbytes / (stats_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": xbytes / (stats_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "traffic": next_rows_traffic("awq", "awq_channel_stats") if (m, n, T) == (4096, 11008, 262144) else None,
            "algorithmic_bytes_per_call": xbytes}},
        "quantize": {"ms": quant_ms, "weight_mse": err[0], "weight_cos": err[1], "roofline": {
            "bound": "hbm", "kernel": ("awq_scale_kernel + rtn_stream_kernel + rtn_reduce_kernel" if cfg.clip_ratio >= 1.0
                                       else "awq_scale_kernel + rtn_row_kernel + rtn_reduce_kernel"),
            "achieved": qbytes / (quant_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": qbytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "traffic": next_rows_traffic("awq", "awq_quantize") if (m, n, T) == (4096, 11008, 262144) else None,
            "algorithmic_bytes_per_call": qbytes}},
        "output_rel_error_first_%d_tokens" % eval_tokens: rel,
    }
    log(f"bench: awq stats {stats_ms:.3f} ms ({xbytes / (stats_ms * 1e-3) / 1e9:.0f} GB/s), quantize "
        f"{quant_ms:.3f} ms; output rel error awq {rel['awq']:.4f} rtn {rel['rtn']:.4f} gptq {rel['gptq']:.4f}")
    return res


def stage_rates(spec, stages_ms):
    """Per-stage rates against their bounds, counted on the algorithmic work
    (triangle only): X bytes = 2·T·n through the Hessian, Cholesky + triangular
    inverse 2n³/3 flop in the prepare stage, the trailing update m·n·(n - 128)
    flop in the quantize stage; the end-to-end fraction is the sum of the
    stages' ideal times (SYRK at the bf16 peak, the other two at the fp32
    peak) over the measured layer time."""
    n, m, T = spec.n, spec.m, spec.tokens
    h, p, q = (x * 1e-3 for x in stages_ms)
    xb = 2.0 * T * n if spec.x_dtype == "bf16" else 4.0 * T * n
    syrk = float(T) * n * (n + 1)
    chol = 2.0 * n ** 3 / 3.0
    trail = float(m) * n * max(n - 128, 0)
    ideal = syrk / (PEAK_BF16_TFLOPS * 1e12) + chol / (PEAK_FP32_TFLOPS * 1e12) + trail / (PEAK_FP32_TFLOPS * 1e12)
    return {
        "x_gbs": xb / h / 1e9, "x_frac_of_hbm": xb / h / 1e9 / PEAK_HBM_GBS,
        "prepare_tflops": chol / p / 1e12, "prepare_frac_of_fp32": chol / p / 1e12 / PEAK_FP32_TFLOPS,
        "trailing_tflops": trail / q / 1e12, "trailing_frac_of_fp32": trail / q / 1e12 / PEAK_FP32_TFLOPS,
        "end_to_end_ideal_ms": ideal * 1e3, "end_to_end_frac": ideal / (h + p + q),
    }


def ideal_seconds(m, n, T, syrk=True, chol=True, trail=True):
    """Ideal time of one layer's stages on the algorithmic work (triangle
    only): the SYRK T·n(n+1) flop at the bf16 MFMA peak, the Cholesky +
    triangular inverse 2n³/3 and the trailing update m·n·(n - 128) flop at
    the fp32 MFMA peak."""
    t = 0.0
    if syrk:
        t += float(T) * n * (n + 1) / (PEAK_BF16_TFLOPS * 1e12)
    if chol:
        t += 2.0 * n ** 3 / 3.0 / (PEAK_FP32_TFLOPS * 1e12)
    if trail:
        t += float(m) * n * max(n - 128, 0) / (PEAK_FP32_TFLOPS * 1e12)
    return t


def measure_layer(pq, torch, spec, steps, warmup):
    """Seconds per layer and per stage of another workload (same protocol as
    the headline: inputs resident, H cleared inside the step)."""
    import workloads
    W = workloads.gen_weight(spec, "cuda")
    X = workloads.gen_x(spec, "cuda")
    layer = Layer(pq, spec, W, X)
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    tot = [0.0, 0.0, 0.0]
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.step()
        for k, v in enumerate(layer.stage_ms()):
            tot[k] += v
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    st = [x / steps for x in tot]
    pq.check_status(layer.out)
    syrk = float(spec.tokens) * spec.n * (spec.n + 1)
    tf = syrk / (st[0] * 1e-3) / 1e12
    res = {"s_per_layer": ms / 1e3, "steps": steps, "stages_ms": dict(zip(("hessian", "prepare", "quantize"), st)),
           "xtx_tflops": tf, "xtx_frac_of_bf16": tf / PEAK_BF16_TFLOPS, "stage_rates": stage_rates(spec, st)}
    log(f"bench: {spec.name}: {ms:.2f} ms/layer, stages {['%.2f' % x for x in st]}, XᵀX {tf:.0f} TFLOP/s")
    del layer, W, X
    torch.cuda.empty_cache()
    return res


def gpu_clocks():
    """Current clocks as rocm-smi reports them (best effort, a child process).
    Skipped under a profiler: its preloaded library would follow the child
    into rocm-smi's interpreter start-up."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "").lower() or any(k.startswith("ROCPROF") for k in os.environ):
        return {"skipped": "under a profiler"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        rec = json.loads(r.stdout)
        card = next(iter(rec.values()))
        return {k: v for k, v in card.items() if "clock" in k.lower() or "sclk" in k.lower() or "mclk" in k.lower()}
    except Exception as e:   # the tool may be missing or print no JSON
        return {"error": repr(e)[:120]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c3_down_proj_4096x11008")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 7B-shaped sweep (224 linears at 4-bit g128 and at 3-bit g64)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-layer lines of the 4096x4096 and 8192x29568 workloads")
    ap.add_argument("--cpu-baseline-full", action="store_true",
                    help="run the oracle on the whole layer instead of a bounded sample (minutes)")
    ap.add_argument("--only-layer", action="store_true",
                    help="time the headline layer only (no next rows, sweeps, extras or CPU baseline)")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "the reference for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this path runs on one GPU "
              "(one layer per GPU; multi-GPU sharding is described in the design notes, not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_check:
        nbytes = args.copy_check << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_check_bytes": nbytes, "copies": 3}), flush=True)
        return

    import post_weight_quantization_14_amd as pq
    import workloads

    pq.lib()
    spec = workloads.CONFIGS[args.workload]
    log(f"bench: {spec.name} m={spec.m} n={spec.n} tokens={spec.tokens}; generating inputs")
    tg = time.perf_counter()
    W = workloads.gen_weight(spec, "cuda")
    X = workloads.gen_x(spec, "cuda")
    torch.cuda.synchronize()
    log(f"bench: inputs ready in {time.perf_counter() - tg:.1f}s")

    layer = Layer(pq, spec, W, X)
    for i in range(args.warmup):
        layer.step()
        torch.cuda.synchronize()
        log(f"bench: warmup {i + 1}/{args.warmup} stages ms {['%.2f' % s for s in layer.stage_ms()]}")

    stage_tot = [0.0, 0.0, 0.0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.step()
        for k, v in enumerate(layer.stage_ms()):
            stage_tot[k] += v
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / args.steps
    stages = [s / args.steps for s in stage_tot]
    log(f"bench: {args.steps} steps, {ms:.2f} ms/step; stages ms {['%.2f' % s for s in stages]}")

    n, T, m = spec.n, spec.tokens, spec.m
    syrk_flops = float(T) * n * (n + 1)
    syrk_tflops = syrk_flops / (stages[0] * 1e-3) / 1e12
    traffic = measured_traffic(spec.name)
    result = {
        "metric": METRIC,
        "value": ms / 1000.0,
        "unit": "s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "m": m, "n": n, "tokens": T, "bits": spec.bits,
                   "group_size": spec.group_size, "sym": spec.sym, "desc_act": spec.desc_act,
                   "damp_percent": spec.damp_percent, "parallelism": "single-gpu"},
        "stages_ms": {"hessian": stages[0], "prepare": stages[1], "quantize": stages[2]},
        "xtx_tflops": syrk_tflops,
        "stage_rates": stage_rates(spec, stages),
        "roofline": {
            "bound": "mfma",
            "kernel": "gptq_hessian_accumulate = syrk_bf16_ring_kernel + syrk_reduce_kernel (H += 2·XᵀX)",
            "achieved": syrk_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": syrk_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops_per_launch": syrk_flops,
        },
        "loss": layer.out["loss"].cpu().tolist(),
    }
    pq.check_status(layer.out)
    if args.only_layer:
        print(json.dumps(result), flush=True)
        return
    result["next_rows"] = {"rtn_quantize": {"workload": f"{spec.name} weight ({m} x {n})",
                                            **measure_rtn(pq, torch, W)}}
    if spec.bits <= 4 and spec.group_size in (32, 64, 128, -1):
        result["next_rows"]["w4a16_matmul"] = {
            "workload": f"bf16 activations x this layer's {spec.bits}-bit g{spec.group_size} act-order weight",
            **measure_w4a16(pq, torch, layer.out, m, n, spec.bits, spec.group_size)}
    if spec.x_dtype == "bf16" and spec.bits == 4:
        result["next_rows"]["awq"] = {
            "workload": f"{spec.name}: channel statistics over the {T}-token X, 4-bit asym g128, s = 2",
            **measure_awq(pq, torch, W, X, layer.out)}
    if not args.no_sweep and args.workload == "c3_down_proj_4096x11008":
        del layer
        torch.cuda.empty_cache()
        log("bench: 7B-shaped sweep")
        result["sweep"] = run_sweep(pq, torch, workloads.SWEEP_SETTINGS)
        log("bench: 7B-shaped sweep, one input per (decoder layer, input), both settings")
        result["next_rows"]["sweep_shared_inputs"] = run_sweep_shared(pq, torch, workloads.SWEEP_SETTINGS)
    if not args.no_extra and args.workload == "c3_down_proj_4096x11008":
        log("bench: per-layer lines of the other full-size workloads")
        result["other_workloads"] = {
            name: measure_layer(pq, torch, workloads.CONFIGS[name], steps, 1)
            for name, steps in (("c2_q_proj_4096", 5), ("c4_down_proj_8192x29568", 3))}
    result["clocks"] = gpu_clocks()
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle on " + ("the whole layer)" if args.cpu_baseline_full else "a bounded sample)"))
        result["cpu_baseline"] = cpu_baseline(spec, W, X, full=args.cpu_baseline_full)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
