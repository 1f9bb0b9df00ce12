#!/usr/bin/env python3
"""Benchmark of the GQA block forward (Llama 3.1 8B attention block) on one MI355X.

Headline: prefill B=1, T=2048, causal, the whole block (fused QKV projection
with rotation, grouped flash attention, output projection) per step, in
TFLOP/s of algorithmic work (only unmasked query/key pairs count). Also
measured in the same run: decode (B=64, one token at position 8191 over a
bf16 KV cache of 8192 rows) in HBM GB/s, chunked prefill (B=1, 2048 new
positions after 2048 cached ones), the pre-norm + residual forms of the
headline prefill and of decode, the pre-norm SwiGLU MLP at 2048 and 64
tokens, and prefill at B=8, T=4096 and at B=1, T=131072.

Prints one JSON line. Inputs are seeded synthetic bf16 values resident in HBM
before the timed region. `roofline` describes the kernel that takes the most
time in the headline step, timed with HIP events on the stream it runs on;
`cpu_baseline` is the fp64 CPU oracle timed on this host on the full headline
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
       python bench.py --only decode|chunk|prenorm|mlp|prefill_B8_T4096|prefill_B1_T131072
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PARAMS_PER_BLOCK = 41_943_040  # W_Q + W_K + W_V + W_O

# HBM-side bytes per launch of each headline stage (B=1, T=2048), FETCH_SIZE +
# WRITE_SIZE from two rocprofv3 --pmc runs, scaled by a 1 GiB copy's counters;
# see profiles/hbm_fetch_write_prefill_B1_T2048.md. Valid for the kernel
# instantiations named here only: re-measure when they change.
PROFILED_TRAFFIC = {
    "qkv_rope": {"kernel": "gemm_nt_kernel<256, 192, 2, 4, 2, 0, 64>", "bytes": 197.3e6},
    "attention": {"kernel": "flash_fwd_kernel + flash_merge_kernel", "bytes": 102.2e6},
    "out_proj": {"kernel": "gemm_nt_kernel<128, 256, 2, 4, 2, 1, 64>", "bytes": 168.0e6},
}


def prefill_flops(B, T, start_pos=0):
    """Algorithmic flops: the four projections plus 4*32*128 per unmasked (q, k) pair."""
    pairs = T * start_pos + T * (T + 1) // 2
    return 2 * B * T * PARAMS_PER_BLOCK + 4 * B * 32 * 128 * pairs


def stage_flops(B, T):
    M = B * T
    return {"qkv_rope": 2 * M * 4096 * 6144,
            "attention": 4 * B * 32 * 128 * (T * (T + 1) // 2),
            "out_proj": 2 * M * 4096 * 4096}


def decode_bytes(B, kv_len):
    """Algorithmic HBM bytes of one decode step: weights, cached K/V rows read,
    new K/V row written, x, fp32 Δ, one rotation row."""
    return (2 * PARAMS_PER_BLOCK + B * (kv_len - 1) * 1024 * 2 * 2 + B * 1024 * 2 * 2
            + B * 4096 * 2 + B * 4096 * 4 + 64 * 2 * 4)


class Bench:
    def __init__(self, args):
        import torch
        import gqa_inputs as gi
        import grouped_query_attention_amd as gqa
        self.torch, self.gi, self.gqa = torch, gi, gqa
        self.args = args
        self.dev = torch.device("cuda:0")

    @staticmethod
    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    def up(self, bits):
        t = self.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.to(self.dev).view(self.torch.bfloat16)

    def time_steps(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return e0.elapsed_time(e1) / steps, wall

    def time_cold(self, fn, steps):
        """Median per-step time with the caches cleared before each step: a
        512 MiB buffer is read (a sum) outside the timed events, so weights and
        activations come from HBM as they would after the rest of a layer."""
        torch = self.torch
        if not hasattr(self, "_flush"):
            self._flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=self.dev)
        ts = []
        for _ in range(steps):
            self._flush.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[len(ts) // 2]

    # ---------------- headline: prefill B=1 T=2048 ----------------
    def headline(self):
        gqa, args = self.gqa, self.args
        B, T = 1, 2048
        self.log(f"[bench] prefill B={B} T={T}: generating inputs")
        inp = self.gi.make_block_inputs(2, B, T)
        x = self.up(inp.x)
        w = [self.up(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]
        rope = self.torch.from_numpy(gqa.rope_table(np.arange(T))).to(self.dev)
        out = self.torch.empty((B, T, 4096), dtype=self.torch.float32, device=self.dev)
        ws = self.torch.empty(gqa.prefill_workspace_bytes(B, T), dtype=self.torch.uint8,
                              device=self.dev)
        step = lambda: gqa.block_forward(x, *w, rope, causal=True, out=out, workspace=ws)
        ms, wall_ms = self.time_steps(step, args.steps, args.warmup)
        F = prefill_flops(B, T)
        value = F / (ms * 1e-3) / 1e12
        self.log(f"[bench] prefill C2: {ms:.4f} ms/step (wall {wall_ms:.4f}), {value:.1f} TFLOP/s")
        cold_ms = self.time_cold(step, args.steps)
        self.log(f"[bench] prefill C2 cold caches: {cold_ms:.4f} ms/step")

        # per-kernel timing (stage entries launch exactly the kernels of the step)
        q_r, k_r, v = gqa.qkv_rope(x, w[0], w[1], w[2], rope)
        aws_n = gqa.attention_workspace_bytes(B, T, T, True)
        aws = self.torch.empty(max(aws_n, 1), dtype=self.torch.uint8, device=self.dev)
        hbuf = gqa.attention(q_r, k_r, v, causal=True, workspace=aws if aws_n else None)
        stages = {
            "qkv_rope": ("gemm_nt_kernel (fused QKV GEMM + rotation epilogue)",
                         lambda: gqa.qkv_rope(x, w[0], w[1], w[2], rope, q_r=q_r, k_r=k_r, v=v)),
            "attention": ("flash_fwd_kernel + flash_merge_kernel (balanced causal launch)"
                          if aws_n else "flash_fwd_kernel",
                          lambda: gqa.attention(q_r, k_r, v, causal=True, h_out=hbuf,
                                                workspace=aws if aws_n else None)),
            "out_proj": ("gemm_nt_kernel (W_O GEMM, fp32 epilogue)",
                         lambda: gqa.output_projection(hbuf, w[3], out=out.view(B * T, 4096))),
        }
        sf = stage_flops(B, T)
        kern = {}
        for name, (kname, fn) in stages.items():
            kms, _ = self.time_steps(fn, args.steps, args.warmup)
            kern[name] = {"kernel": kname, "ms": kms, "tflops": sf[name] / (kms * 1e-3) / 1e12}
            kern[name]["frac"] = kern[name]["tflops"] / PEAK_BF16_TFLOPS
            self.log(f"[bench]   {name}: {kms:.4f} ms, {kern[name]['tflops']:.1f} TFLOP/s")
        dom = max(kern, key=lambda k: kern[k]["ms"])
        prof = PROFILED_TRAFFIC.get(dom)
        roofline = {"bound": "mfma", "kernel": kern[dom]["kernel"], "stage": dom,
                    "achieved": round(kern[dom]["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(kern[dom]["frac"], 4),
                    "traffic": prof["bytes"] if prof else None,
                    "traffic_unit": "bytes per launch (HBM-side, rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                    "traffic_kernel": prof["kernel"] if prof else None,
                    "flops_per_launch": sf[dom], "avg_launch_ms": round(kern[dom]["ms"], 5)}

        result = {
            "metric": "GQA block fwd TFLOP/s (% bf16 MFMA peak) prefill; decode HBM GB/s",
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "Llama-3.1-8B GQA attention block forward, prefill, causal",
                       "B": B, "T": T, "d": 4096, "q_heads": 32, "kv_heads": 8, "d_head": 128,
                       "rope_theta": 500000.0, "flops_per_step": F,
                       "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4)},
            "cold_cache": {"ms_per_step": round(cold_ms, 5),
                           "TFLOP/s": round(F / (cold_ms * 1e-3) / 1e12, 2),
                           "note": "median step with a 512 MiB read between steps"},
            "roofline": roofline,
            "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                            for kk, vv in d.items()} for k, d in kern.items()},
        }
        return result, inp, step, out, F

    # ---------------- decode B=64, start_pos 8191, cache 8192 rows ----------------
    def decode(self, extra):
        torch, gqa, args = self.torch, self.gqa, self.args
        Bd, S, sp = 64, 8192, 8191
        self.log("[bench] decode B=64 kv=8192: generating cache")
        dinp = self.gi.make_block_inputs(4, Bd, 1, cache_len=S)
        dx = self.up(dinp.x[:, 0])
        dw = [self.up(a) for a in (dinp.wq, dinp.wk, dinp.wv, dinp.wo)]
        kc, vc = self.up(dinp.k_cache), self.up(dinp.v_cache)
        del dinp
        drope = torch.from_numpy(gqa.rope_table([sp])[0]).to(self.dev)
        dout = torch.empty((Bd, 4096), dtype=torch.float32, device=self.dev)
        dws = torch.empty(gqa.decode_workspace_bytes(Bd, S), dtype=torch.uint8, device=self.dev)
        dstep = lambda: gqa.decode_forward(dx, *dw, drope, kc, vc, sp, out=dout, workspace=dws)
        # The step streams its K/V cache and weights past the caches (non-temporal
        # loads), so a warm loop of the same step could keep earlier data in the
        # Infinity Cache where a real layer loop would not: the figure is the median
        # step with the caches flushed (512 MiB read) before each step.
        for _ in range(args.warmup):
            dstep()
        dcold = self.time_cold(dstep, args.steps)
        dms, _ = self.time_steps(dstep, args.steps, args.warmup)
        nbytes = decode_bytes(Bd, S)
        qd = torch.zeros((Bd, 32, 128), dtype=torch.bfloat16, device=self.dev)
        hd = torch.empty_like(qd)
        ams = self.time_cold(lambda: gqa.decode_attention(qd, kc, vc, S, h_out=hd, workspace=dws),
                             args.steps)
        kv_bytes = Bd * S * 1024 * 2 * 2
        extra["decode_B64_kv8192"] = {
            "ms": round(dcold, 5), "GB/s": round(nbytes / (dcold * 1e-3) / 1e9, 1),
            "frac_of_hbm": round(nbytes / (dcold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_step": nbytes,
            "note": "median step, caches flushed (512 MiB read) before each step",
            "warm_loop": {"ms": round(dms, 5),
                          "GB/s": round(nbytes / (dms * 1e-3) / 1e9, 1)},
            "attention_kernel": {"kernel": "decode_splitkv_kernel+decode_merge_kernel",
                                 "ms": round(ams, 5),
                                 "GB/s": round(kv_bytes / (ams * 1e-3) / 1e9, 1),
                                 "frac_of_hbm": round(kv_bytes / (ams * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                      4)}}
        self.log(f"[bench] decode: {dcold:.4f} ms, {extra['decode_B64_kv8192']['GB/s']} GB/s "
                 f"(caches flushed; warm loop {dms:.4f} ms)")
        del kc, vc, dws
        torch.cuda.empty_cache()

    # ---------------- larger prefill configurations ----------------
    def prefill(self, extra, Bp, Tp, seed, steps):
        torch, gqa = self.torch, self.gqa
        self.log(f"[bench] prefill B={Bp} T={Tp}: generating inputs")
        pinp = self.gi.make_block_inputs(seed, Bp, Tp)
        px = self.up(pinp.x)
        pw = [self.up(a) for a in (pinp.wq, pinp.wk, pinp.wv, pinp.wo)]
        del pinp
        prope = torch.from_numpy(gqa.rope_table(np.arange(Tp))).to(self.dev)
        pout = torch.empty((Bp, Tp, 4096), dtype=torch.float32, device=self.dev)
        pws = torch.empty(gqa.prefill_workspace_bytes(Bp, Tp), dtype=torch.uint8, device=self.dev)
        pstep = lambda: gqa.block_forward(px, *pw, prope, causal=True, out=pout, workspace=pws)
        pms, _ = self.time_steps(pstep, steps, 1)
        Fp = prefill_flops(Bp, Tp)
        tf = Fp / (pms * 1e-3) / 1e12
        extra[f"prefill_B{Bp}_T{Tp}"] = {"ms": round(pms, 4), "TFLOP/s": round(tf, 1),
                                         "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                         "flops_per_step": Fp, "steps": steps}
        self.log(f"[bench] prefill B={Bp} T={Tp}: {pms:.3f} ms, {tf:.1f} TFLOP/s")
        del px, pw, pout, pws
        torch.cuda.empty_cache()

    # ---------------- chunked prefill into a KV cache ----------------
    def chunk(self, extra):
        """B=1: 2048 new positions at start_pos 2048 over a cache of 4096 rows."""
        torch, gqa, args = self.torch, self.gqa, self.args
        B, T, sp, S = 1, 2048, 2048, 4096
        self.log(f"[bench] chunked prefill B={B} T={T} start_pos={sp}: generating inputs")
        inp = self.gi.make_block_inputs(6, B, T, cache_len=S)
        x = self.up(inp.x)
        w = [self.up(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]
        kc, vc = self.up(inp.k_cache), self.up(inp.v_cache)
        del inp
        rope = torch.from_numpy(gqa.rope_table(np.arange(sp, sp + T))).to(self.dev)
        out = torch.empty((B, T, 4096), dtype=torch.float32, device=self.dev)
        ws = torch.empty(gqa.chunk_workspace_bytes(B, T, sp), dtype=torch.uint8, device=self.dev)
        step = lambda: gqa.chunk_forward(x, *w, rope, kc, vc, sp, out=out, workspace=ws)
        ms, _ = self.time_steps(step, args.steps, args.warmup)
        F = prefill_flops(B, T, sp)
        tf = F / (ms * 1e-3) / 1e12
        extra[f"chunk_B{B}_T{T}_start{sp}"] = {
            "ms": round(ms, 5), "TFLOP/s": round(tf, 1),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_step": F,
            "kv_len": sp + T}
        self.log(f"[bench] chunked prefill: {ms:.4f} ms, {tf:.1f} TFLOP/s")
        del kc, vc, ws
        torch.cuda.empty_cache()

    # ---------------- pre-norm + residual forms (the block's handoff) ----------------
    def prenorm(self, extra):
        """out = x + Δ(RMSNorm(x)) at the headline prefill shape and the decode shape;
        the normalisation kernel's own time and bandwidth at the prefill shape."""
        torch, gqa, args = self.torch, self.gqa, self.args
        B, T = 1, 2048
        self.log("[bench] pre-norm + residual: prefill B=1 T=2048")
        inp = self.gi.make_block_inputs(2, B, T)
        g = self.up(self.gi.make_norm_weight(2))
        x = self.up(inp.x)
        w = [self.up(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]
        rope = torch.from_numpy(gqa.rope_table(np.arange(T))).to(self.dev)
        out = torch.empty((B, T, 4096), dtype=torch.float32, device=self.dev)
        ws = torch.empty(gqa.prefill_workspace_bytes(B, T), dtype=torch.uint8, device=self.dev)
        plain = lambda: gqa.block_forward(x, *w, rope, causal=True, out=out, workspace=ws)
        pre = lambda: gqa.block_forward(x, *w, rope, causal=True, out=out, workspace=ws,
                                        norm_w=g)
        ms_plain, _ = self.time_steps(plain, args.steps, args.warmup)
        ms_pre, _ = self.time_steps(pre, args.steps, args.warmup)
        y = torch.empty_like(x)
        ms_norm, _ = self.time_steps(lambda: gqa.rmsnorm(x, g, y=y), args.steps, args.warmup)
        F = prefill_flops(B, T)
        nb = 2 * B * T * 4096 * 2
        extra["prenorm_prefill_B1_T2048"] = {
            "ms": round(ms_pre, 5), "TFLOP/s": round(F / (ms_pre * 1e-3) / 1e12, 1),
            "plain_block_ms": round(ms_plain, 5),
            "overhead_frac": round(ms_pre / ms_plain - 1.0, 4),
            "rmsnorm_kernel": {"ms": round(ms_norm, 5),
                               "GB/s": round(nb / (ms_norm * 1e-3) / 1e9, 1),
                               "bytes": nb}}
        self.log(f"[bench] pre-norm prefill: {ms_pre:.4f} ms vs plain {ms_plain:.4f} ms; "
                 f"rmsnorm {ms_norm * 1e3:.1f} us")
        del x, w, out, ws, y

        Bd, S, sp = 64, 8192, 8191
        self.log("[bench] pre-norm + residual: decode B=64 kv=8192")
        dinp = self.gi.make_block_inputs(4, Bd, 1, cache_len=S)
        dg = self.up(self.gi.make_norm_weight(4))
        dx = self.up(dinp.x[:, 0])
        dw = [self.up(a) for a in (dinp.wq, dinp.wk, dinp.wv, dinp.wo)]
        kc, vc = self.up(dinp.k_cache), self.up(dinp.v_cache)
        del dinp
        drope = torch.from_numpy(gqa.rope_table([sp])[0]).to(self.dev)
        dout = torch.empty((Bd, 4096), dtype=torch.float32, device=self.dev)
        dws = torch.empty(gqa.decode_workspace_bytes(Bd, S), dtype=torch.uint8, device=self.dev)
        dplain = lambda: gqa.decode_forward(dx, *dw, drope, kc, vc, sp, out=dout, workspace=dws)
        dpre = lambda: gqa.decode_forward(dx, *dw, drope, kc, vc, sp, out=dout, workspace=dws,
                                          norm_w=dg)
        for _ in range(args.warmup):
            dplain()
            dpre()
        # medians with the caches flushed before each step, as for the plain decode
        dms_plain = self.time_cold(dplain, args.steps)
        dms = self.time_cold(dpre, args.steps)
        nbytes = decode_bytes(Bd, S) + 4096 * 2   # plus the gain
        extra["prenorm_decode_B64_kv8192"] = {
            "ms": round(dms, 5), "GB/s": round(nbytes / (dms * 1e-3) / 1e9, 1),
            "plain_decode_ms": round(dms_plain, 5),
            "overhead_frac": round(dms / dms_plain - 1.0, 4)}
        self.log(f"[bench] pre-norm decode: {dms:.4f} ms vs plain {dms_plain:.4f} ms")
        del kc, vc, dws
        torch.cuda.empty_cache()

    # ---------------- SwiGLU MLP (the block's other half) ----------------
    def mlp(self, extra):
        """Pre-norm SwiGLU MLP with its residual: M = 2048 tokens (the headline's
        tokens) in TFLOP/s, and M = 64 (one decode step of 64 sequences) in HBM GB/s
        of weights."""
        torch, gqa, args = self.torch, self.gqa, self.args
        self.log("[bench] SwiGLU MLP: generating weights")
        m = self.gi.make_mlp_inputs(8, 2048)
        w1, w2, w3 = (self.up(a) for a in (m.w1, m.w2, m.w3))
        x = self.up(m.x)
        g = self.up(self.gi.make_norm_weight(8))
        del m
        for M in (2048, 64):
            xm = x[:M].contiguous()
            out = torch.empty((M, 4096), dtype=torch.float32, device=self.dev)
            ws = torch.empty(gqa.mlp_workspace_bytes(M), dtype=torch.uint8, device=self.dev)
            step = lambda: gqa.mlp_forward(xm, w1, w2, w3, norm_w=g, out=out, workspace=ws)
            if M <= 64:
                # a weight stream (non-temporal loads): median with flushed caches
                for _ in range(args.warmup):
                    step()
                ms = self.time_cold(step, args.steps)
            else:
                ms, _ = self.time_steps(step, args.steps, args.warmup)
            F = 3 * 2 * M * 4096 * 14336
            wbytes = 3 * 4096 * 14336 * 2
            rec = {"ms": round(ms, 5), "TFLOP/s": round(F / (ms * 1e-3) / 1e12, 1),
                   "frac_of_bf16_peak": round(F / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "flops_per_step": F}
            if M <= 64:
                nb = wbytes + M * 4096 * (2 + 4)
                rec.update({"GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                            "frac_of_hbm": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                            "bytes_per_step": nb})
            extra[f"mlp_prenorm_M{M}"] = rec
            self.log(f"[bench] MLP M={M}: {ms:.4f} ms, {rec['TFLOP/s']} TFLOP/s")
        del w1, w2, w3, x
        torch.cuda.empty_cache()

    def prefill_b8(self, extra):
        self.prefill(extra, 8, 4096, 3, max(3, self.args.steps // 4))

    def prefill_long(self, extra):
        self.prefill(extra, 1, 131072, 5, 2)

    # ---------------- CPU oracle baseline (full headline workload) ----------------
    def cpu_baseline(self, result, inp, step, out, F):
        import threadpoolctl
        from oracle import gqa_oracle as O
        cores = len(os.sched_getaffinity(0))
        with threadpoolctl.threadpool_limits(cores):
            used = max([d["num_threads"] for d in threadpoolctl.threadpool_info()] or [1])
            self.log(f"[bench] cpu oracle on {used} threads: B=1 T=2048 full forward")
            t0 = time.perf_counter()
            ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
            cpu_s = time.perf_counter() - t0
        step()
        self.torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        d = ref["delta"]
        result["cpu_baseline"] = {"value": round(F / cpu_s / 1e12, 5), "unit": "TFLOP/s",
                                  "cores": used, "kind": "oracle",
                                  "sample": "full prefill B=1 T=2048 causal, one forward, fp64 numpy",
                                  "seconds": round(cpu_s, 3)}
        result["parity_vs_oracle"] = {
            "relL2": float(np.linalg.norm(got - d) / np.linalg.norm(d)),
            "maxabs": float(np.max(np.abs(got - d)))}
        self.log(f"[bench] cpu oracle {cpu_s:.2f} s; parity {result['parity_vs_oracle']}")

    def calibrate_copy(self, mib):
        torch = self.torch
        n = mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=self.dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--only", choices=["decode", "chunk", "prenorm", "mlp", "prefill_B8_T4096",
                                       "prefill_B1_T131072"],
                    help="run just this one workload and print its figures (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB mebibytes (3 times), for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    b = Bench(args)
    if args.calibrate_copy:
        b.calibrate_copy(args.calibrate_copy)
        return
    others = {"decode": b.decode, "chunk": b.chunk, "prenorm": b.prenorm, "mlp": b.mlp,
              "prefill_B8_T4096": b.prefill_b8,
              "prefill_B1_T131072": b.prefill_long}
    if args.only:
        extra = {}
        others[args.only](extra)
        print(json.dumps({"only": args.only, **extra}), flush=True)
        return

    result, inp, step, out, F = b.headline()
    extra = {}
    if not args.quick:
        for fn in others.values():
            fn(extra)
    result["other_configs"] = extra
    if not args.no_cpu:
        b.cpu_baseline(result, inp, step, out, F)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
