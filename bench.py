"""Benchmark of the int4-weight quantized linear layer on one MI355X.

Timed step: one W4A8 forward of the MLP up-projection workload (M=4096
tokens, K=4096, N=14336, group 128, bf16 activations): per-token int8
quantization followed by the W4A8 GEMM with its fused epilogue, inputs
resident in HBM. `value` is 2*M*N*K / step time in TOPS.

Measured in the same run and reported beside it:
  asym    the same layer with asymmetric per-token activations
          (w4a8_quantize_act_asym + w4a8_gemm_asym)
  down_proj  W4A8 per-channel down-projection (M=8192, K=14336, N=4096,
          group -1, fp16 activations with outlier channels): quantization
          and GEMM times
  decode  W4A16 decode (M=1 and M=8, K=4096, N=14336, group 64), achieved
          HBM GB/s with weights rotated through 16 distinct sets (> MALL)
  moe     W4A-FP8 routed experts (64 experts, K=7168, N=2048, 8192 tokens,
          top-8): FP8 quantization + grouped GEMM
  prefill W4A16 prefill (M=4096): dequantize to bf16 + the library's bf16
          GEMM, with the platform GEMM (hipBLASLt) timed on the same weights
  platform_refs  hipBLASLt int8 / bf16 GEMMs at 8192^3, a 1 GiB device copy
          and pure-MFMA loops (int8, fp8, bf16: the matrix core's measured
          peak, and the engine clock it implies) measured on this GPU beside
          the nominal peaks; each GEMM object also carries its fraction of
          the measured MFMA-only rate
  roofline  the dominant kernel (the W4A8 GEMM) against the int8 MFMA peak,
          its duration from HIP events on the launch stream
  cpu_baseline  the CPU oracle timed on a bounded row sample of the step

Before the first timed region the W4A8 step runs untimed for --settle-s
seconds (0.5), and each later GEMM section for half that: the clocks take a
fraction of a second of load to settle.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only w4a8|down|decode|prefill|moe|vocab]
       python bench.py --calib-copy
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only", choices=["all", "w4a8", "down", "decode", "prefill", "moe", "vocab", "shards"], default="all",
                   help="which extra measurements to add to the W4A8 step (shards: only when asked for)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle sample time")
    p.add_argument("--settle-s", type=float, default=0.5,
                   help="seconds of untimed W4A8 steps before the first timed region: the GPU's clocks take "
                        "a fraction of a second of load to settle (measured: the first ~50 ms run 10-15%% slower)")
    p.add_argument("--crossover", action="store_true",
                   help="time both paths of w4_linear over a range of row counts on the up-projection "
                        "weights and print that table instead of the benchmark line")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run three plain 1 GiB device-to-device copies: the known-size kernel that "
                        "scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    return p.parse_args()


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int4_weight_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key: str, srcs, n_launch_units: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on a different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash(*srcs):
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from int4_weight_quantized_amd import ops, workloads as W

    if not os.path.exists(ops.LIB_PATH):
        from int4_weight_quantized_amd import build as B
        B.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 3}), flush=True)
        return

    def dev_half(bits, dtype):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(dev)

    def settle(fns, seconds):
        """Run the callables untimed for about `seconds`: the engine clock
        needs a fraction of a second of load to reach its steady state."""
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(4):
                for f in fns:
                    f()
            torch.cuda.synchronize()

    def timed(fns, steps, warmup, per_call=True):
        """Run the list of launch callables per step; return mean ms per callable
        (HIP events on the launch stream; None without per_call), the mean
        step time and the wall time. With per_call the steps run twice: once
        with an event between callables (the per-callable times) and once
        without (the step time, free of the events' own cost).
        The timed launches must run back to back, without host launch gaps.
        When a step's GPU time is well above its host enqueue time (the GEMMs),
        the timed steps are simply enqueued behind a second round of warmup
        steps, which keeps the GPU busy (and its clocks up) while the host gets
        ahead. Otherwise (short kernels) a bounded spin kernel ahead of the
        timed region holds the stream while the host enqueues every launch."""
        t0 = time.perf_counter()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(max(warmup, 1)):
            for f in fns:
                f()
        e1.record(stream)
        host_per_step = (time.perf_counter() - t0) / max(warmup, 1)
        torch.cuda.synchronize()
        gpu_per_step = e0.elapsed_time(e1) * 1e-3 / max(warmup, 1)
        busy_ahead = gpu_per_step > 3.0 * host_per_step
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        if busy_ahead:
            for _ in range(max(warmup, 2)):
                for f in fns:
                    f()
        else:
            # shader-clock cycles at up to 2.4 GHz; twice the host enqueue time of
            # both timed regions, at most ~0.2 s
            rounds = 2 if per_call else 1
            torch.cuda._sleep(int(min(0.2, 2.0 * host_per_step * steps * rounds + 1e-3) * 2.4e9))
        t0 = time.perf_counter()
        if per_call:
            # the per-callable region, enqueued right ahead of the step region
            for s in range(steps):
                ev[s][0].record(stream)
                for i, f in enumerate(fns):
                    f()
                    ev[s][i + 1].record(stream)
        start.record(stream)
        for s in range(steps):
            for f in fns:
                f()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)])) if per_call else None
               for i in range(len(fns))]
        return per, start.elapsed_time(end) / steps, wall

    # ------------------------------------------------------------ W4A8 up-proj step
    d = W.named("w4a8_up_proj")
    M, K, N, g = d["M"], d["K"], d["N"], d["group"]
    x = dev_half(d["x"], "bf16")
    qw = torch.from_numpy(d["qweight"]).to(dev)
    sc = torch.from_numpy(d["scales"]).to(dev)
    wt = ops.w4_repack(qw, ops.W4_LAYOUT_GPTQ_KN, K, N)
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    s_a = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fq = lambda: ops.quantize_act_into(x, codes, s_a)
    fg = lambda: ops.w4a8_gemm(codes, s_a, wt, sc, g, N, out=y)
    # untimed steps until the clocks settle, then the W warmup steps and the K timed ones
    settle([fq, fg], args.settle_s)
    (t_q, t_g), t_step, _ = timed([fq, fg], args.steps, args.warmup)
    ops_gemm = 2.0 * M * N * K
    tops = ops_gemm / (t_step * 1e-3) / 1e12
    tops_gemm = ops_gemm / (t_g * 1e-3) / 1e12
    quant_bytes = M * K * 2 + M * K + M * 4
    w4a8 = {
        "workload": f"w4a8_up_proj M={M} K={K} N={N} group={g} bf16",
        "quant_ms": t_q, "gemm_ms": t_g, "step_ms": t_step,
        "gemm_tops": tops_gemm, "gemm_frac_int8_peak": tops_gemm / PEAK_INT8_TOPS,
        "quant_gbs": quant_bytes / (t_q * 1e-3) / 1e9,
    }

    if args.crossover:
        # both dispatch targets on the same tiled weights, rotated over copies
        # larger together than the 256 MB MALL so that weights stream from HBM
        nrot = 12
        wts = [ops.w4_repack(qw.roll(i, 1).contiguous(), ops.W4_LAYOUT_GPTQ_KN, K, N) for i in range(nrot)]
        table = []
        for Mc in (1, 2, 4, 8, 16, 24, 32, 48, 64, 80, 96, 112, 128, 192, 256, 384, 512):
            xc = x[:Mc]
            yc = torch.empty((Mc, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty((ops.w4_linear_workspace_bytes(Mc, N, K, g, 1),), dtype=torch.uint8, device=dev)
            f_wo = [(lambda w=w: ops.w4_linear(xc, w, sc, g, N, min_tokens_int8=1 << 30, out=yc)) for w in wts]
            f_i8 = [(lambda w=w: ops.w4_linear(xc, w, sc, g, N, min_tokens_int8=1, out=yc, workspace=ws))
                    for w in wts]
            reps = max(2, args.steps // 10)
            _, t_wo, _ = timed(f_wo, reps, 2, per_call=False)
            _, t_i8, _ = timed(f_i8, reps, 2, per_call=False)
            table.append({"M": Mc, "weight_only_us": t_wo / nrot * 1e3, "int8_us": t_i8 / nrot * 1e3})
            print(json.dumps(table[-1]), flush=True)
        cross = next((r["M"] for r in table if r["int8_us"] < r["weight_only_us"]), None)
        print(json.dumps({"crossover": {"workload": f"w4_linear K={K} N={N} group={g} bf16", "table": table,
                                        "first_M_int8_faster": cross}}), flush=True)
        return

    # ------------------------------------------------------------ asymmetric activations, same layer
    asym = {}
    if args.only in ("all", "w4a8"):
        z_a = torch.empty((M,), dtype=torch.float32, device=dev)
        woff = ops.w4a8_weight_offsets(wt, sc, g, K, N)
        fqa = lambda: ops.w4a8_quantize_act_asym_into(x, codes, s_a, z_a)
        fga = lambda: ops.w4a8_gemm_asym(codes, s_a, z_a, wt, sc, g, woff, N, out=y)
        settle([fqa, fga], args.settle_s / 2)
        (t_qa, t_ga), t_sa, _ = timed([fqa, fga], max(4, args.steps // 2), max(2, args.warmup // 2))
        asym = {"workload": f"w4a8_up_proj asymmetric per-token activations M={M} K={K} N={N} group={g}",
                "quant_ms": t_qa, "gemm_ms": t_ga, "step_ms": t_sa,
                "gemm_tops": ops_gemm / (t_ga * 1e-3) / 1e12}

    # ------------------------------------------------------------ W4A8 per-channel down-proj
    down = {}
    if args.only in ("all", "w4a8", "down"):
        dd = W.named("w4a8_down_proj")
        Md, Kd, Nd, gd = dd["M"], dd["K"], dd["N"], dd["group"]
        xd = dev_half(dd["x"], "f16")
        wtd = ops.w4_repack(torch.from_numpy(dd["qweight"]).to(dev), ops.W4_LAYOUT_GPTQ_KN, Kd, Nd)
        scd = torch.from_numpy(dd["scales"]).to(dev)
        codes_d = torch.empty((Md, Kd), dtype=torch.int8, device=dev)
        s_d = torch.empty((Md,), dtype=torch.float32, device=dev)
        y_d = torch.empty((Md, Nd), dtype=torch.float16, device=dev)
        fqd = lambda: ops.quantize_act_into(xd, codes_d, s_d)
        fgd = lambda: ops.w4a8_gemm(codes_d, s_d, wtd, scd, gd, Nd, out=y_d)
        settle([fqd, fgd], args.settle_s / 2)
        (t_qd, t_gd), t_sd, _ = timed([fqd, fgd], max(4, args.steps // 2), max(2, args.warmup // 2))
        ops_d = 2.0 * Md * Nd * Kd
        down = {"workload": f"w4a8_down_proj M={Md} K={Kd} N={Nd} group={gd} f16 (1% outlier channels x20)",
                "quant_ms": t_qd, "gemm_ms": t_gd, "step_ms": t_sd,
                "gemm_tops": ops_d / (t_gd * 1e-3) / 1e12,
                "gemm_frac_int8_peak": ops_d / (t_gd * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                "quant_gbs": (Md * Kd * 3 + Md * 4) / (t_qd * 1e-3) / 1e9}
        del xd, wtd, codes_d, y_d

    # ------------------------------------------------------------ one GPU's share under tensor parallelism (8)
    # column shard: N/8 output columns; row shard: K/8 input columns (its
    # partial outputs would be summed across GPUs, not done here)
    shards = {}
    if args.only == "shards":
        tp = 8
        Nc, Kr = N // tp, K // tp
        wt_c = ops.w4_repack(qw[:, :Nc].contiguous(), ops.W4_LAYOUT_GPTQ_KN, K, Nc)
        sc_c = sc[:, :Nc].contiguous()
        y_c = torch.empty((M, Nc), dtype=torch.bfloat16, device=dev)
        wt_r = ops.w4_repack(qw[: Kr // 8].contiguous(), ops.W4_LAYOUT_GPTQ_KN, Kr, N)
        sc_r = sc[: Kr // g].contiguous()
        codes_r = codes[:, :Kr].contiguous()
        f_c = lambda: ops.w4a8_gemm(codes, s_a, wt_c, sc_c, g, Nc, out=y_c)
        f_r = lambda: ops.w4a8_gemm(codes_r, s_a, wt_r, sc_r, g, N, out=y)
        (t_c, t_r), _, _ = timed([f_c, f_r], max(4, args.steps // 2), max(2, args.warmup // 2))
        for name, t, (mm, nn, kk) in (("column", t_c, (M, Nc, K)), ("row", t_r, (M, N, Kr))):
            shards[f"tp{tp}_{name}"] = {"M": mm, "N": nn, "K": kk, "gemm_us": t * 1e3,
                                        "tops": 2.0 * mm * nn * kk / (t * 1e-3) / 1e12,
                                        "frac_int8_peak": 2.0 * mm * nn * kk / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS}
        del wt_c, wt_r

    # ------------------------------------------------------------ W4A16 decode
    decode = {}
    if args.only in ("all", "decode"):
        nrot = 16
        for Md in (1, 8):
            dd = W.named("w4a16_decode", M=Md)
            Kd, Nd, gd = dd["K"], dd["N"], dd["group"]
            xd = dev_half(dd["x"], "bf16")
            base_w = torch.from_numpy(dd["w"]).to(dev)
            base_s = dev_half(dd["scale"], "bf16")
            base_z = dev_half(dd["zero"], "bf16")
            sets = [ops.w4a16_repack(base_w.roll(i, 0).contiguous(), base_s.roll(i, 0).contiguous(),
                                     base_z.roll(i, 0).contiguous(), gd) for i in range(nrot)]
            yd = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)
            calls = [(lambda st=st: ops.w4a16_gemm(xd, st[0], st[1], gd, Nd, out=yd)) for st in sets]
            reps = max(1, args.steps // 4)
            # back-to-back launches over the rotated sets: step time / launches
            _, t_rep, _ = timed(calls, reps, max(1, args.warmup // 4), per_call=False)
            t = t_rep / len(calls)
            nbytes = Nd * Kd // 2 + 2 * 2 * Nd * (Kd // gd) + 2 * Md * Kd + 2 * Md * Nd
            decode[f"M{Md}"] = {"us": t * 1e3, "bytes": nbytes, "gbs": nbytes / (t * 1e-3) / 1e9,
                                "frac_hbm": nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}
            del sets

    # ------------------------------------------------------------ W4A16 prefill: dequantize once + bf16 GEMM
    prefill = {}
    if args.only in ("all", "decode", "prefill"):
        dd = W.named("w4a16_decode", M=1)
        Kp, Np, gp, Mp = dd["K"], dd["N"], dd["group"], 4096
        wb = torch.from_numpy(dd["w"]).to(dev)
        sp, zp = dev_half(dd["scale"], "bf16"), dev_half(dd["zero"], "bf16")
        xp = torch.randn((Mp, Kp), dtype=torch.float32, device=dev).to(torch.bfloat16)
        wdq = torch.empty((Np, Kp), dtype=torch.bfloat16, device=dev)
        yp = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)
        f_dq = lambda: ops.w4a16_dequantize(wb, sp, zp, gp, out=wdq)
        f_mm = lambda: ops.w4a16_prefill_gemm(xp, wdq, out=yp)          # the library's bf16 GEMM
        f_blas = lambda: torch.matmul(xp, wdq.t(), out=yp)              # baseline: the platform GEMM (hipBLASLt)
        settle([f_dq, f_mm], args.settle_s / 2)
        (t_dq, t_mm), t_pf, _ = timed([f_dq, f_mm], max(4, args.steps // 2), max(2, args.warmup // 2))
        settle([f_blas], args.settle_s / 2)
        (t_blas,), _, _ = timed([f_blas], max(4, args.steps // 2), max(2, args.warmup // 2))
        dq_bytes = Np * Kp // 2 + 2 * 2 * Np * (Kp // gp) + 2 * Np * Kp
        fl = 2.0 * Mp * Np * Kp
        prefill = {"workload": f"w4a16 prefill M={Mp} K={Kp} N={Np} group={gp} bf16 (dequantize + bf16 GEMM)",
                   "dequantize_us": t_dq * 1e3, "dequantize_gbs": dq_bytes / (t_dq * 1e-3) / 1e9,
                   "gemm_us": t_mm * 1e3, "gemm_tflops": fl / (t_mm * 1e-3) / 1e12,
                   "gemm_frac_bf16_peak": fl / (t_mm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                   "step_us": t_pf * 1e3, "step_tflops": fl / (t_pf * 1e-3) / 1e12,
                   "baseline_hipblaslt_gemm_us": t_blas * 1e3,
                   "baseline_hipblaslt_gemm_tflops": fl / (t_blas * 1e-3) / 1e12}
        del wdq, yp

    # ------------------------------------------------------------ MoE grouped
    moe = {}
    if args.only in ("all", "moe"):
        dm = W.named("w4afp8_moe")
        Em, Km, Nm, gm, Tm = dm["E"], dm["K"], dm["N"], dm["group"], dm["T"]
        xm = dev_half(dm["x"], "bf16")
        wm = ops.w4_repack(torch.from_numpy(dm["w"]).to(dev), ops.W4_LAYOUT_CT_NK, Km, Nm, batch=Em)
        scm = torch.from_numpy(dm["scales"]).to(dev)
        rt = torch.from_numpy(dm["row_token"]).to(dev)
        off = torch.from_numpy(dm["expert_offsets"]).to(dev)
        R = rt.shape[0]
        a8 = torch.empty((Tm, Km), dtype=torch.uint8, device=dev)
        sm = torch.empty((Tm,), dtype=torch.float32, device=dev)
        gs = torch.empty((Tm, Km // gm), dtype=torch.float32, device=dev)
        ym = torch.empty((R, Nm), dtype=torch.bfloat16, device=dev)
        fq8 = lambda: ops.quantize_act_into(xm, a8, sm, gs, gm, fp8=True)
        fgg = lambda: ops.w4a8_grouped_gemm(a8, sm, gs, rt, off, wm, scm, gm, Nm, out=ym)
        settle([fq8, fgg], args.settle_s / 2)
        (t_q8, t_gg), t_moe, _ = timed([fq8, fgg], max(2, args.steps // 4), max(1, args.warmup // 2))
        flops = 2.0 * R * Nm * Km
        moe = {"workload": f"w4afp8_moe E={Em} K={Km} N={Nm} group={gm} T={Tm} top{dm['topk']} R={R}",
               "quant_ms": t_q8, "grouped_gemm_ms": t_gg, "step_ms": t_moe,
               "gemm_tflops": flops / (t_gg * 1e-3) / 1e12,
               "gemm_frac_fp8_peak": flops / (t_gg * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}
        del wm

    # ------------------------------------------------------------ int4 vocab table (tied embedding / head)
    vocab = {}
    if args.only in ("all", "vocab"):
        V, Kv, gv, Tv = 131072, 2048, 64, 8192
        rng = np.random.default_rng(1006)
        table = torch.from_numpy(rng.standard_normal((V, Kv), dtype=np.float32) * np.float32(0.02)).to(dev)
        table = table.to(torch.bfloat16)
        fqg = lambda: ops.w4_quantize_groupwise(table, gv, torch.bfloat16)
        _, t_qg, _ = timed([fqg], max(2, args.steps // 10), 2, per_call=False)
        packed, sv, zv = fqg()
        del table
        sets = []
        for i in range(3):                  # 3 x 150 MB of tiles: more than the MALL
            sets.append(ops.w4a16_repack(packed.roll(i, 0).contiguous(), sv.roll(i, 0).contiguous(),
                                         zv.roll(i, 0).contiguous(), gv))
        ids = torch.from_numpy(rng.integers(0, V, Tv).astype(np.int32)).to(dev)
        emb = torch.empty((Tv, Kv), dtype=torch.bfloat16, device=dev)
        f_emb = [(lambda st=st: ops.w4a16_embedding(ids, st[0], st[1], gv, V, Kv, out=emb)) for st in sets]
        _, t_emb, _ = timed(f_emb, max(2, args.steps // 5), 2, per_call=False)
        xh = torch.from_numpy(rng.standard_normal((1, Kv), dtype=np.float32)).to(dev).to(torch.bfloat16)
        yh = torch.empty((1, V), dtype=torch.bfloat16, device=dev)
        f_head = [(lambda st=st: ops.w4a16_gemm(xh, st[0], st[1], gv, V, out=yh)) for st in sets]
        _, t_head, _ = timed(f_head, max(2, args.steps // 5), 2, per_call=False)
        t_emb, t_head = t_emb / len(sets), t_head / len(sets)
        Gv = Kv // gv
        qg_bytes = V * Kv * 2 + V * Kv // 2 + 2 * 2 * V * Gv
        emb_bytes = Tv * (Kv // 2 + 4 * Gv + 4 + 2 * Kv)
        head_bytes = V * Kv // 2 + 4 * V * Gv + 2 * Kv + 2 * V
        vocab = {"workload": f"int4 vocab table V={V} K={Kv} group={gv}; embedding T={Tv}; tied head M=1",
                 "quantize_groupwise_us": t_qg * 1e3, "quantize_groupwise_gbs": qg_bytes / (t_qg * 1e-3) / 1e9,
                 "embedding_us": t_emb * 1e3, "embedding_gbs": emb_bytes / (t_emb * 1e-3) / 1e9,
                 "head_us": t_head * 1e3, "head_gbs": head_bytes / (t_head * 1e-3) / 1e9,
                 "head_frac_hbm": head_bytes / (t_head * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del sets, packed, sv, zv

    # ------------------------------------------------------------ platform references on this GPU
    # platform library kernels at large square sizes (hipBLASLt int8 and bf16
    # GEMMs) and a plain 1 GiB device copy, beside the nominal figures: what
    # the vendor's own kernels reach here, not an upper bound
    measured = {}
    if args.only == "all":
        mp = {}
        try:
            a8 = torch.randint(-127, 128, (8192, 8192), dtype=torch.int8, device=dev)
            b8 = torch.randint(-127, 128, (8192, 8192), dtype=torch.int8, device=dev)
            settle([lambda: torch._int_mm(a8, b8)], args.settle_s / 2)
            (t_i8,), _, _ = timed([lambda: torch._int_mm(a8, b8)], 10, 3)
            mp["int8_gemm_tops"] = 2.0 * 8192 ** 3 / (t_i8 * 1e-3) / 1e12
            del a8, b8
        except Exception as ex:                       # no int8 GEMM in this torch build
            mp["int8_gemm_error"] = type(ex).__name__
        ab = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
        bb = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
        settle([lambda: torch.matmul(ab, bb)], args.settle_s / 2)
        (t_bf,), _, _ = timed([lambda: torch.matmul(ab, bb)], 10, 3)
        mp["bf16_gemm_tflops"] = 2.0 * 8192 ** 3 / (t_bf * 1e-3) / 1e12
        del ab, bb
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        (t_cp,), _, _ = timed([lambda: dst.copy_(src)], 10, 3)
        mp["copy_gbs"] = 2.0 * (1 << 30) / (t_cp * 1e-3) / 1e9      # bytes read + written
        del src, dst
        # the matrix core's measured peak: pure MFMA loops with no memory
        # traffic (int8, fp8, bf16); the nominal peaks are quoted at 2.4 GHz,
        # so the int8 loop's rate also gives the engine clock it ran at
        sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
        for kind, key in ((0, "mfma_only_int8_tops"), (1, "mfma_only_fp8_tflops"), (2, "mfma_only_bf16_tflops")):
            n_ops = ops.w4_probe_mfma(kind, 4096, sink)
            (t_pk,), _, _ = timed([lambda kind=kind: ops.w4_probe_mfma(kind, 4096, sink)], 10, 3)
            mp[key] = n_ops / (t_pk * 1e-3) / 1e12
        mp["sclk_est_ghz"] = 2.4 * mp["mfma_only_int8_tops"] / PEAK_INT8_TOPS
        del sink
        measured = {"what": "hipBLASLt int8 and bf16 GEMMs at 8192^3, a 1 GiB device copy (read + write) and "
                            "pure-MFMA loops (the matrix core's measured peak; sclk_est_ghz = 2.4 GHz x its "
                            "int8 rate / the nominal int8 peak), measured on this GPU",
                    **mp}
        w4a8["gemm_frac_mfma_only_int8"] = tops_gemm / mp["mfma_only_int8_tops"]
        if down:
            down["gemm_frac_mfma_only_int8"] = down["gemm_tops"] / mp["mfma_only_int8_tops"]
        if moe:
            moe["gemm_frac_mfma_only_fp8"] = moe["gemm_tflops"] / mp["mfma_only_fp8_tflops"]
        if prefill:
            prefill["gemm_frac_mfma_only_bf16"] = prefill["gemm_tflops"] / mp["mfma_only_bf16_tflops"]
        if "int8_gemm_tops" in mp:
            w4a8["gemm_vs_hipblaslt_int8"] = tops_gemm / mp["int8_gemm_tops"]
            if down:
                down["gemm_vs_hipblaslt_int8"] = down["gemm_tops"] / mp["int8_gemm_tops"]
        for k in ("M1", "M8"):
            if k in decode:
                decode[k]["vs_device_copy"] = decode[k]["gbs"] / mp["copy_gbs"]
        if prefill:
            prefill["gemm_vs_hipblaslt_bf16"] = prefill["gemm_tflops"] / mp["bf16_gemm_tflops"]

    # ------------------------------------------------------------ roofline of the dominant kernel
    achieved = ops_gemm / (t_g * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": achieved / PEAK_INT8_TOPS,
                "traffic": traffic_from_profile("w4a8_gemm_up_proj", ["w4a8_gemm.hip", "w4_device.h"], 1),
                "kernel": "w4a8_gemm_kernel (int8 ops)"}

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(d, args.cpu_seconds)

    line = {
        "metric": "W4A8 GEMM TOPS & % int8 MFMA peak (M=4096); W4A16 decode GB/s & % HBM",
        "value": tops, "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": w4a8["workload"], "global_batch": M, "seq_len": 1, "parallelism": "single_gpu",
                   "step": "w4a8_quantize_act + w4a8_gemm"},
        "settle_s": args.settle_s,
        "w4a8": w4a8, "asym": asym, "down_proj": down, "shards": shards, "decode": decode, "prefill": prefill,
        "moe": moe, "vocab": vocab, "platform_refs": measured,
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(d, target_s: float):
    """The oracle as it stands on a row sample of the same layer: per-token
    quantization of the sampled rows, exact int32 group partials and the
    epilogue. Reported in the same unit (TOPS over the sampled rows)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    K, N, g = d["K"], d["N"], d["group"]
    q = O.unpack_gptq_kn(d["qweight"])
    sc = d["scales"].astype(np.float32)

    def run(rows):
        t0 = time.perf_counter()
        x32 = O.half_bits_to_f32(d["x"][:rows], d["x_dtype"])
        codes, s = O.quantize_act_int8(x32)
        P = O.group_partials(codes, q, g)
        O.w4a8_epilogue(P, s, sc)
        return time.perf_counter() - t0

    run(16)                                   # first-touch of the unpacked weights
    per_row = run(256) / 256
    want = max(256, int(target_s / per_row))
    rows, reps = (want, 1) if want <= d["M"] else (d["M"], -(-want // d["M"]))
    t = sum(run(rows) for _ in range(reps))
    total = rows * reps
    return {"value": 2.0 * total * N * K / t / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {d['M']} rows of w4a8_up_proj x{reps} (per-token quantize + exact int32 "
                      f"group partials + epilogue), {t:.1f} s", "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
