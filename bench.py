#!/usr/bin/env python3
"""Benchmark of the triangle-attention forward on one MI355X.

A step is one tri_attn_fwd call (the whole forward: one kernel launch) over
the headline workload: bf16, B=1, N=768, H=4, Q=K=768, D=64, fp32 bias,
kv_lengths drawn uniformly from {384, 392, ..., 768}; inputs resident in HBM
before timing starts.  Prints one JSON line.

  value      nominal TFLOP/s, 4*B*N*H*Q*K*D per step (the metric's formula)
  roofline   the kernel against the bf16 dense MFMA peak, on ALGORITHMIC
             flops (4*H*Q*D*sum_n len_n: only the keys the mask leaves)
  cpu_baseline  the fp64 oracle timed on this host's cores over a bounded
             sample of the same workload (n rows), in the same unit
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
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CU x 2.4 GHz x 256 flop/clk)
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA (the fp32 forward's v_mfma_f32_32x32x2_f32)
METRIC = "fwd TFLOP/s + % bf16 MFMA peak, triangle attn N=Q=K=768 H=4 D=64"
PROFILES = os.path.join(ROOT, "profiles")
# the forward kernel's sources: the kernel and its tile geometry / swizzles
KERNEL_SRCS = [os.path.join(ROOT, "masked_attention_tri_amd", "csrc", f)
               for f in ("mfma_fwd.h", "mfma_common.h")]


def kernel_source_sha256():
    """SHA-256 of the forward kernel's sources, concatenated in order."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="default 100 (backward: 10)")
    # Under this load the GPU's clock first dips and then settles over a few
    # tens of milliseconds; the default warmup covers that, so the timed
    # steps see the steady clock.
    ap.add_argument("--warmup", type=int, default=None, help="default 200 (backward: 3)")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up (after --warmup steps) until this much time has "
                         "passed, so a short --warmup does not time the clock ramp")
    ap.add_argument("--backward", action="store_true",
                    help="time tri_attn_bwd (dQ, dK, dV, dBias) instead of the forward")
    ap.add_argument("--workload", default=None,
                    help="named workload (default: the headline bf16 kv_lengths N768 D64 one)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bias-dtype", choices=("fp32", "input"), default="fp32",
                    help="pass the bias as fp32 (the metric) or in the inputs' 16-bit type "
                         "(the opt-in mode of tri_attn_fwd_bias_dtype)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 10 if args.backward else 100
    if args.warmup is None:
        args.warmup = 3 if args.backward else 200
    return args


def warm_up(args, step):
    """--warmup steps, then more until --warmup-seconds have passed (the
    clock under this load dips and settles over tens of milliseconds).
    Returns the number of warmup steps run."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(args.warmup):
        step()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < args.warmup_seconds:
        for _ in range(10):
            step()
            n += 1
        torch.cuda.synchronize()
    return n


def work_counts(case, bias_elem=4):
    """Nominal and algorithmic flops, algorithmic HBM bytes of one step
    (bias_elem: bytes per bias element)."""
    import torch

    B, N, H, Q, K, D = case.shape
    esz = case.q.element_size()
    nominal = 4 * B * N * H * Q * K * D
    if case.kv_lengths is not None:
        keys = case.kv_lengths.view(B, N).clamp(0, K).to(torch.int64)  # visited keys per (b,n)
        key_rows = int(keys.sum()) * H  # sum over (b,n,h) of visited keys
        alg = 4 * Q * D * key_rows
    elif case.block is not None:
        # whole visited blocks (union of both lists, duplicates once)
        blk = case.block
        nkb = -(-K // blk.kv_block)
        visited = 0
        pairs = [(blk.kv_num_blocks, blk.kv_indices)]
        if blk.full_kv_num_blocks is not None:
            pairs.append((blk.full_kv_num_blocks, blk.full_kv_indices))
        seen = torch.zeros(*blk.kv_num_blocks.shape, nkb + 1, dtype=torch.bool)
        for num, idx in pairs:
            j = torch.arange(idx.shape[-1])
            ids = idx.long()
            ok = (j < num.unsqueeze(-1)) & (ids >= 0) & (ids < nkb)
            seen.scatter_(-1, torch.where(ok, ids, nkb), True)
        lead = blk.kv_num_blocks.shape[:3]
        reps = (B * N * H) // max(1, math.prod(lead))
        visited = int(seen[..., :nkb].sum()) * reps
        key_rows = visited * blk.kv_block * blk.q_block // Q  # key visits per query row
        alg = 4 * D * visited * blk.kv_block * blk.q_block
    else:
        key_rows = B * N * H * K
        alg = nominal
    qo = 2 * B * N * H * Q * D * esz
    kv = 2 * key_rows * D * esz
    bias = B * H * Q * K * bias_elem if case.bias is not None else 0
    aux = 2 * B * N * H * Q * 4
    mask = (B * N * 4) if case.kv_lengths is not None else (B * N * K if case.mask is not None else 0)
    return nominal, alg, qo + kv + bias + aux + mask


def traffic_entry(workload):
    """Measured HBM bytes per launch of the MFMA kernel on this workload, if
    the counters were taken on this exact kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_mfma_fwd_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return t


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, target_s):
    """Time the fp64 oracle on the first n rows of the workload."""
    import numpy as np
    import torch

    import oracle

    B, N, H, Q, K, D = case.shape
    threads = oracle.default_threads()
    blk = None
    if case.block is not None:
        # BlockMask lists with leading dims (B|1, N|1, H|1), flattened to
        # instances with strides (0 broadcasts)
        b = case.block
        lb, ln, lh = b.kv_num_blocks.shape[:3]
        sh = 1 if lh == H and H > 1 else 0
        sn = lh if ln == N and N > 1 else 0
        sb = ln * lh if lb == B and B > 1 else 0
        rows = b.kv_num_blocks.shape[3]
        flat = lambda t, *tail: None if t is None else t.reshape(-1, rows, *tail).cpu()
        blk = oracle.OracleBlockMask(
            flat(b.kv_num_blocks), flat(b.kv_indices, b.kv_indices.shape[-1]),
            flat(b.full_kv_num_blocks),
            None if b.full_kv_indices is None else flat(b.full_kv_indices,
                                                       b.full_kv_indices.shape[-1]),
            q_block=b.q_block, kv_block=b.kv_block,
            mask_mod=oracle.MOD_CAUSAL if b.mask_mod == "causal" else oracle.MOD_NONE,
            stride_b=sb, stride_n=sn, stride_h=sh)

    def run(ns):
        if blk is not None and blk.stride_n != 0:
            ns = N  # per-n lists: the instance strides assume every n
        sub_q, sub_k, sub_v = case.q[:, :ns], case.k[:, :ns], case.v[:, :ns]
        lens = case.kv_lengths[:, :ns] if case.kv_lengths is not None else None
        mask = case.mask[:, :ns] if case.mask is not None else None
        t0 = time.perf_counter()
        out = oracle.oracle_fwd(sub_q, sub_k, sub_v, case.bias, kv_lengths=lens, mask=mask,
                                block=blk, scale=case.scale, threads=threads)
        return time.perf_counter() - t0, out

    dt1, _ = run(1)
    ns = max(1, min(N, int(target_s / max(dt1, 1e-3))))
    dt, out = run(ns)
    flops = 4 * B * ns * H * Q * K * D  # nominal formula, as for `value`
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {ns} of {N} n rows (all b, h, q), fp64, {dt:.1f} s",
        "seconds": round(dt, 3),
    }, ns, out


def bench_backward(args, case, g, key, shape, dtype, desc, scale, out, lse, mx, stream, fwd):
    """One step = one tri_attn_bwd call (dQ, dK, dV, dBias) on the workload,
    after one forward for O, lse and max; inputs resident in HBM."""
    import torch

    import masked_attention_tri_amd as mat
    from masked_attention_tri_amd import _native as nat

    B, N, H, Q, K, D = case.shape
    fwd()
    gen = torch.Generator().manual_seed(4242)
    dout = torch.randn(g.q.shape, generator=gen).to(g.q.dtype).to(g.q.device)
    dq, dk, dv = torch.empty_like(g.q), torch.empty_like(g.k), torch.empty_like(g.v)
    dbias = torch.empty_like(g.bias) if g.bias is not None else None
    # the library's workspace (per-row data and dBias partial sums), allocated once
    ws = torch.empty((mat.tri_attn_bwd_workspace_size(shape, dbias is not None) + 3) // 4,
                     device=g.q.device, dtype=torch.float32)

    def step():
        st = mat.tri_attn_bwd(shape, dtype, g.q, g.k, g.v, g.bias, desc, scale, out, dout, lse,
                              mx, dq, dk, dv, dbias, stream, workspace=ws)
        if st != nat.TRIATTN_OK:
            raise RuntimeError(mat.tri_attn_status_str(st))

    warm_steps = warm_up(args, step)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] backward: {ms:.4f} ms/step", file=sys.stderr, flush=True)
    # Algorithmic work: 10 D flops per visited (query, key) pair (recomputed
    # logits, dP = dO.V, dV, dQ and dK, 2 D each), i.e. 2.5x the forward's.
    _, alg_fwd, _ = work_counts(case)
    alg = 2.5 * alg_fwd
    tflops = alg / (ms * 1e-3) / 1e12
    peak = PEAK_FP32_VALU_TFLOPS if case.dtype == torch.float32 else PEAK_BF16_TFLOPS
    res = {
        "metric": "bwd TFLOP/s (10 D flops per visited query-key pair), triangle attn",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": warm_steps, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[case.dtype],
        "data": "synthetic",
        "config": {"workload": case.name, "key": key, "B": B, "N": N, "H": H, "Q": Q, "K": K,
                   "D": D, "algorithmic_flop": alg},
        # bf16/fp16: every contraction of the backward runs on MFMA; fp32
        # inputs run them as vector FMAs
        "roofline": {"bound": "alu" if case.dtype == torch.float32 else "mfma",
                     "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 5), "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        print("[bench] timing the CPU backward oracle baseline", file=sys.stderr, flush=True)
        threads = oracle.default_threads()

        def run(ns):
            t0 = time.perf_counter()
            oracle.oracle_bwd(case.q[:, :ns], case.k[:, :ns], case.v[:, :ns], case.bias,
                              dout=dout.cpu()[:, :ns],
                              kv_lengths=None if case.kv_lengths is None else case.kv_lengths[:, :ns],
                              mask=None if case.mask is None else case.mask[:, :ns],
                              scale=case.scale, threads=threads)
            return time.perf_counter() - t0

        dt1 = run(1)
        ns = max(1, min(N, int(args.cpu_seconds / max(dt1, 1e-3))))
        dt = run(ns)
        alg_s = alg * ns / N
        res["cpu_baseline"] = {"value": round(alg_s / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": min(threads, B * H), "kind": "oracle",
                               "sample": f"first {ns} of {N} n rows, fp64, {dt:.1f} s",
                               "seconds": round(dt, 3)}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library "
              "has no multi-GPU path: rows shard over N with no exchange step)", file=sys.stderr)
        sys.exit(2)

    import torch

    import masked_attention_tri_amd as mat
    from masked_attention_tri_amd import _native as nat
    from masked_attention_tri_amd import workloads as wl

    mat.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    key = args.workload or wl.HEADLINE
    case = wl.make_workload(key)
    g = case.to(dev)
    B, N, H, Q, K, D = case.shape
    out = torch.empty_like(g.q)
    lse = torch.empty(B, N, H, Q, device=dev)
    mx = torch.empty(B, N, H, Q, device=dev)
    keep = []
    desc = None
    if g.mask is not None:
        m = g.mask.contiguous().view(torch.uint8)
        keep.append(m)
        desc = nat.TriAttnMask()
        desc.kind = nat.TRIATTN_MASK_DENSE
        desc.dense = m.data_ptr()
    elif g.kv_lengths is not None:
        desc = nat.TriAttnMask()
        desc.kind = nat.TRIATTN_MASK_KV_LENGTHS
        desc.kv_lengths = g.kv_lengths.data_ptr()
    elif g.block is not None:
        b = g.block
        bm = mat.BlockMask.from_kv_blocks(b.kv_num_blocks, b.kv_indices, b.full_kv_num_blocks,
                                          b.full_kv_indices, BLOCK_SIZE=(b.kv_block, b.q_block),
                                          mask_mod=b.mask_mod)
        desc, conv = bm._descriptor(B, N, H, Q, K, dev)
        keep.extend(conv)
    shape = nat.TriAttnShape(B, N, H, Q, K, D)
    dtype = nat.DTYPE_CODES[g.q.dtype]
    scale = math.nan if g.scale is None else g.scale
    stream = torch.cuda.current_stream(dev)

    half_bias = args.bias_dtype == "input" and g.bias is not None
    if half_bias:
        if g.q.dtype == torch.float32:
            sys.exit("--bias-dtype input needs a bf16 or fp16 workload")
        bias_arg, bias_dt = g.bias.to(g.q.dtype).contiguous(), dtype
    else:
        bias_arg, bias_dt = g.bias, nat.TRIATTN_F32

    def step():
        st = mat.tri_attn_fwd_bias_dtype(shape, dtype, g.q, g.k, g.v, bias_arg, bias_dt, desc,
                                         scale, out, lse, mx, stream)
        if st != nat.TRIATTN_OK:
            raise RuntimeError(mat.tri_attn_status_str(st))

    if args.backward:
        return bench_backward(args, case, g, key, shape, dtype, desc, scale, out, lse, mx,
                              stream, step)

    warm_steps = warm_up(args, step)
    print(f"[bench] warmup done ({warm_steps} steps)", file=sys.stderr, flush=True)

    # HIP events on the stream the kernel is launched on, around the K steps.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    # A second pass, after the timed one, with an event after every step for
    # the median and minimum step time (the extra events add gaps between
    # launches, so they stay out of the timed pass).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    print(f"[bench] timed {args.steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s)",
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        # plain copy of known size, so byte counters can be scaled
        src = torch.empty(256 * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nominal, alg, alg_bytes = work_counts(case, 2 if half_bias else 4)
    sec = ms * 1e-3
    value = nominal / sec / 1e12
    alg_tflops = alg / sec / 1e12
    fwd_peak = PEAK_FP32_MFMA_TFLOPS if case.dtype == torch.float32 else PEAK_BF16_TFLOPS
    tr = traffic_entry(key) if not half_bias else None
    traffic = None if tr is None else tr["bytes_per_launch"]
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms, 5),
        "ms_median": round(per_step[len(per_step) // 2], 5),
        "ms_min": round(per_step[0], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[
            case.dtype],
        "data": "synthetic",
        "pct_bf16_peak_nominal": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "tflops_algorithmic": round(alg_tflops, 3),
        "pct_bf16_peak_algorithmic": round(100.0 * alg_tflops / PEAK_BF16_TFLOPS, 3),
        "hbm_GBps_algorithmic": round(alg_bytes / sec / 1e9, 1),
        "config": {
            "workload": case.name + (" (bias in the input type)" if half_bias else ""),
            "key": key,
            "bias_dtype": "input" if half_bias else "fp32",
            "B": B, "N": N, "H": H, "Q": Q, "K": K, "D": D,
            "nominal_flop": nominal,
            "algorithmic_flop": alg,
            "algorithmic_bytes": alg_bytes,
        },
        # fp32 inputs run on the fp32 matrix product, the 16-bit types on
        # the bf16/fp16 one
        "roofline": {
            "bound": "mfma",
            "achieved": round(alg_tflops, 3),
            "peak": fwd_peak,
            "unit": "TFLOP/s",
            "frac": round(alg_tflops / fwd_peak, 5),
            "traffic": traffic,
            "hbm_frac_algorithmic": round(alg_bytes / sec / 1e9 / PEAK_HBM_GBPS, 5),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cb, ns, oracle_out = cpu_baseline(case, args.cpu_seconds)
        # the same rows of the GPU result against the oracle: O max-abs
        # against the unrounded fp64 oracle, lse and max against the oracle
        # rounded to fp32
        import numpy as np

        go = out[:, :ns].double().cpu().numpy()
        gl = lse[:, :ns].double().cpu().numpy()
        gm = mx[:, :ns].double().cpu().numpy()
        f32 = lambda a: np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
        err_o = float(np.abs(go - oracle_out[0]).max())
        err_l = float(np.abs(gl - f32(oracle_out[1])).max())
        err_m = float(np.abs(gm - f32(oracle_out[2])).max())
        tol = ({"o": 1e-5, "lse": 1e-5, "max": 1e-5} if case.dtype == torch.float32
               else {"o": 2e-2, "lse": 1e-3, "max": 1e-3})
        cb["max_abs_err_O_vs_gpu"] = err_o
        cb["cpu_model"] = cpu_model()
        res["cpu_baseline"] = cb
        res["parity"] = {"rows": f"first {ns} of {N} n rows (all b, h, q)", "err_O": err_o,
                         "err_lse": err_l, "err_max": err_m, "tol": tol,
                         "pass": err_o <= tol["o"] and err_l <= tol["lse"]
                         and err_m <= tol["max"]}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
