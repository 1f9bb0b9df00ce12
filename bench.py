#!/usr/bin/env python3
"""Benchmark of the GQA block forward (Llama 3.1 8B attention block) on one MI355X.

Headline: the long-context prefill, B=1, T=131072, causal, the whole block
(fused QKV projection with rotation, grouped flash attention, output
projection) per step, in TFLOP/s of algorithmic work (only unmasked
query/key pairs count). The same run measures every workload of the block at
its own line under "configs":
  prefill B=1 T=128, prefill B=1 T=2048, prefill B=8 T=4096 (TFLOP/s),
  decode B=64 over a KV cache of 8192 rows at position 8191 (HBM GB/s),
  prefill B=1 T=131072 (the headline),
each with its step time (mean and median), the stages timed alone, the
roofline of its dominant kernel, the fp64 CPU oracle's wall time on the
stated scope, and the GPU/oracle parity of that run. "other_workloads" adds
chunked prefill, the pre-norm + residual forms and the SwiGLU MLP.

Prints one JSON line. Inputs are seeded synthetic bf16 values resident in HBM
before the timed region. `roofline` describes the kernel that takes the most
time in the headline step, timed with HIP events on the stream it runs on;
`cpu_baseline` is the fp64 CPU oracle timed on this host on a sample of the
headline workload (every key and value, a fixed set of query rows).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
       python bench.py --only <workload>      (one workload, for profiling)
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

# HBM-side bytes per launch of a stage on a workload, FETCH_SIZE + WRITE_SIZE
# from two rocprofv3 --pmc runs, scaled by what the counters read for a 1 GiB
# device copy (profiles/hbm_fetch_write_*.md). Valid for the kernel
# instantiation named here only: re-measure when it changes.
PROFILED_TRAFFIC = {
    ("prefill_B1_T2048", "qkv_rope"): {"kernel": "gemm_nt_kernel<256, 192, 2, 4, 2, 0, 64>",
                                       "bytes": 197.3e6},
    ("prefill_B1_T2048", "attention"): {"kernel": "flash_fwd_kernel<true, false> + flash_merge_kernel",
                                        "bytes": 102.1e6},
    ("prefill_B1_T2048", "out_proj"): {"kernel": "gemm_nt_kernel<128, 256, 2, 4, 2, 1, 64>",
                                       "bytes": 167.9e6},
    ("prefill_B1_T131072", "attention"): {"kernel": "flash_fwd_kernel<true, false> (plain causal launch)",
                                          "bytes": 19.595e9},
}

HEADLINE = "prefill_B1_T131072"
WORKLOADS = {
    # name: (kind, B, T or cache rows, seed, oracle scope)
    "prefill_B1_T128": ("prefill", 1, 128, 1, "full"),
    "prefill_B1_T2048": ("prefill", 1, 2048, 2, "full"),
    "prefill_B8_T4096": ("prefill", 8, 4096, 3, "sequence 0 of 8, every row"),
    "decode_B64_kv8192": ("decode", 64, 8192, 4, "full"),
    "prefill_B1_T131072": ("prefill", 1, 131072, 5, "sampled rows"),
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


def rows_flops(T, rows):
    """Algorithmic flops of the sampled evaluation of a causal prefill of T
    positions at the given query rows: K and V of every position, Q and Δ of
    the rows, and the attention of each row over its keys."""
    rows = np.asarray(rows, dtype=np.int64)
    R = len(rows)
    return (2 * T * 2048 * 4096 + 2 * R * 4096 * 4096 * 2
            + 4 * 32 * 128 * int(np.sum(rows + 1)))


def decode_bytes(B, kv_len):
    """Algorithmic HBM bytes of one decode step: weights, cached K/V rows read,
    new K/V row written, x, fp32 Δ, one rotation row."""
    return (2 * PARAMS_PER_BLOCK + B * (kv_len - 1) * 1024 * 2 * 2 + B * 1024 * 2 * 2
            + B * 4096 * 2 + B * 4096 * 4 + 64 * 2 * 4)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rnd(d):
    return {k: (round(v, 5) if isinstance(v, float) else rnd(v) if isinstance(v, dict) else v)
            for k, v in d.items()}


class Bench:
    def __init__(self, args):
        import torch
        import gqa_inputs as gi
        import grouped_query_attention_amd as gqa
        self.torch, self.gi, self.gqa = torch, gi, gqa
        self.args = args
        self.dev = torch.device("cuda:0")
        self.cores = len(os.sched_getaffinity(0))

    @staticmethod
    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    def up(self, bits):
        t = self.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.to(self.dev).view(self.torch.bfloat16)

    def down_f64(self, t):
        return t.detach().cpu().numpy().astype(np.float64)

    def down_bf16_f64(self, t):
        bits = t.contiguous().view(self.torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)

    def time_steps(self, fn, steps, warmup):
        """W untimed steps, then exactly K steps between synchronisations, HIP
        events around the whole run and around each step (torch's current
        stream, which the library launches on). Returns (mean ms, median ms)."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        return ev[0].elapsed_time(ev[-1]) / steps, per[len(per) // 2]

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

    def oracle(self, fn):
        """Runs an oracle call on every host core this process may use; returns
        (result, seconds, BLAS threads used)."""
        import threadpoolctl
        with threadpoolctl.threadpool_limits(self.cores):
            used = max([d["num_threads"] for d in threadpoolctl.threadpool_info()] or [1])
            t0 = time.perf_counter()
            r = fn()
            return r, time.perf_counter() - t0, used

    @staticmethod
    def parity(got, want):
        return {"relL2": float(np.linalg.norm(got - want) / np.linalg.norm(want)),
                "maxabs": float(np.max(np.abs(got - want)))}

    # ---------------- causal prefill (whole block, stages, oracle) ----------------
    def prefill(self, name, with_oracle=True):
        torch, gqa, args = self.torch, self.gqa, self.args
        _, B, T, seed, scope = WORKLOADS[name]
        self.log(f"[bench] {name}: generating inputs")
        inp = self.gi.make_block_inputs(seed, B, T)
        x = self.up(inp.x)
        w = [self.up(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]
        rope = torch.from_numpy(gqa.rope_table(np.arange(T))).to(self.dev)
        out = torch.empty((B, T, 4096), dtype=torch.float32, device=self.dev)
        ws = torch.empty(gqa.prefill_workspace_bytes(B, T), dtype=torch.uint8, device=self.dev)
        step = lambda: gqa.block_forward(x, *w, rope, causal=True, out=out, workspace=ws)
        ms, med = self.time_steps(step, args.steps, args.warmup)
        F = prefill_flops(B, T)
        tf = F / (ms * 1e-3) / 1e12
        rec = {"B": B, "T": T, "causal": True, "ms_per_step": ms, "median_ms": med,
               "steps": args.steps, "warmup": args.warmup, "TFLOP/s": tf,
               "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS, "flops_per_step": F}
        self.log(f"[bench] {name}: {ms:.4f} ms/step (median {med:.4f}), {tf:.1f} TFLOP/s")
        if B * T <= 4096:
            rec["cold_cache"] = {"median_ms": self.time_cold(step, args.steps),
                                 "note": "median step with a 512 MiB read between steps"}

        # each stage alone: with pre-scaled queries (q_scaled) and, above 256
        # tokens, the stage entries launch exactly the kernels of the step
        q_r, k_r, v = gqa.qkv_rope(x, w[0], w[1], w[2], rope, q_scaled=True)
        aws_n = gqa.attention_workspace_bytes(B, T, T, True)
        aws = torch.empty(max(aws_n, 1), dtype=torch.uint8, device=self.dev)
        hbuf = gqa.attention(q_r, k_r, v, causal=True, workspace=aws if aws_n else None,
                             q_scaled=True)
        stages = {
            "qkv_rope": ("gemm_nt_kernel (fused QKV GEMM + rotation epilogue)",
                         lambda: gqa.qkv_rope(x, w[0], w[1], w[2], rope, q_r=q_r, k_r=k_r, v=v,
                                              q_scaled=True)),
            "attention": ("flash_fwd_kernel<true, false> + flash_merge_kernel (balanced causal launch)"
                          if aws_n else "flash_fwd_kernel<true, false> (pre-scaled queries)",
                          lambda: gqa.attention(q_r, k_r, v, causal=True, h_out=hbuf,
                                                workspace=aws if aws_n else None,
                                                q_scaled=True)),
            "out_proj": ("gemm_nt_kernel (W_O GEMM, fp32 epilogue)",
                         lambda: gqa.output_projection(hbuf, w[3], out=out.view(B * T, 4096))),
        }
        sf = stage_flops(B, T)
        kern = {}
        for sname, (kname, fn) in stages.items():
            kms, _ = self.time_steps(fn, args.steps, min(args.warmup, 2))
            tfs = sf[sname] / (kms * 1e-3) / 1e12
            kern[sname] = {"kernel": kname, "ms": kms, "TFLOP/s": tfs,
                           "frac": tfs / PEAK_BF16_TFLOPS, "flops_per_launch": sf[sname]}
            self.log(f"[bench]   {sname}: {kms:.4f} ms, {tfs:.1f} TFLOP/s")
        rec["stages"] = kern
        dom = max(kern, key=lambda k: kern[k]["ms"])
        prof = PROFILED_TRAFFIC.get((name, dom))
        rec["roofline"] = {"bound": "mfma", "kernel": kern[dom]["kernel"], "stage": dom,
                           "achieved": kern[dom]["TFLOP/s"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": kern[dom]["frac"],
                           "traffic": prof["bytes"] if prof else None,
                           "traffic_kernel": prof["kernel"] if prof else None,
                           "flops_per_launch": sf[dom], "avg_launch_ms": kern[dom]["ms"]}
        del q_r, k_r, v, hbuf, aws

        if with_oracle:
            self.prefill_oracle(name, rec, inp, step, out)
        del x, w, out, ws
        torch.cuda.empty_cache()
        return rec

    def prefill_oracle(self, name, rec, inp, step, out):
        from oracle import gqa_oracle as O
        _, B, T, _, scope = WORKLOADS[name]
        step()
        self.torch.cuda.synchronize()
        if scope == "full":
            self.log(f"[bench] {name}: oracle, full forward")
            ref, sec, used = self.oracle(
                lambda: O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)["delta"])
            got = self.down_f64(out)
            flops = prefill_flops(B, T)
        elif scope.startswith("sequence 0"):
            self.log(f"[bench] {name}: oracle, sequence 0, full forward")
            ref, sec, used = self.oracle(
                lambda: O.block_forward(inp.x[:1], inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)["delta"])
            got = self.down_f64(out[:1])
            flops = prefill_flops(1, T)
        else:
            rows = self.gi.sample_positions(WORKLOADS[name][3], T)
            self.log(f"[bench] {name}: oracle, {len(rows)} sampled rows")
            ref, sec, used = self.oracle(
                lambda: O.block_forward_rows(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8,
                                             rows)["delta"])
            got = self.down_f64(out[0, self.torch.from_numpy(rows).to(self.dev)])
            flops = rows_flops(T, rows)
            scope = (f"sampled: {len(rows)} query rows (64 per KV-head group plus 0, 1, T-1 and "
                     f"tile edges), keys and values of every position")
        rec["oracle"] = {"seconds": sec, "scope": scope, "threads": used,
                         "cpu_model": cpu_model(), "TFLOP/s": flops / sec / 1e12,
                         "flops": flops, "kind": "fp64 numpy oracle"}
        rec["parity_vs_oracle"] = self.parity(got, ref)
        self.log(f"[bench] {name}: oracle {sec:.2f} s on {used} threads; "
                 f"parity {rec['parity_vs_oracle']}")

    # ---------------- decode B=64, start_pos 8191, cache 8192 rows ----------------
    def decode(self, name="decode_B64_kv8192", with_oracle=True):
        torch, gqa, args = self.torch, self.gqa, self.args
        _, Bd, S, seed, scope = WORKLOADS[name]
        sp = S - 1
        self.log(f"[bench] {name}: generating cache")
        dinp = self.gi.make_block_inputs(seed, Bd, 1, cache_len=S)
        dx = self.up(dinp.x[:, 0])
        dw = [self.up(a) for a in (dinp.wq, dinp.wk, dinp.wv, dinp.wo)]
        kc, vc = self.up(dinp.k_cache), self.up(dinp.v_cache)
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
        dms, dmed = self.time_steps(dstep, args.steps, args.warmup)
        nbytes = decode_bytes(Bd, S)
        gbs = nbytes / (dcold * 1e-3) / 1e9
        qd = torch.zeros((Bd, 32, 128), dtype=torch.bfloat16, device=self.dev)
        hd = torch.empty_like(qd)
        ams = self.time_cold(lambda: gqa.decode_attention(qd, kc, vc, S, h_out=hd, workspace=dws),
                             args.steps)
        kv_bytes = Bd * S * 1024 * 2 * 2
        rec = {"B": Bd, "start_pos": sp, "kv_len": S, "ms_per_step": dcold,
               "steps": args.steps, "warmup": args.warmup,
               "GB/s": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS, "bytes_per_step": nbytes,
               "note": "median step, caches flushed (512 MiB read) before each step",
               "warm_loop": {"ms_per_step": dms, "median_ms": dmed,
                             "GB/s": nbytes / (dms * 1e-3) / 1e9}}
        agbs = kv_bytes / (ams * 1e-3) / 1e9
        rec["roofline"] = {"bound": "hbm", "kernel": "decode_splitkv_kernel + decode_merge_kernel",
                           "achieved": agbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": agbs / PEAK_HBM_GBS, "traffic": None,
                           "bytes_per_launch": kv_bytes, "avg_launch_ms": ams}
        self.log(f"[bench] {name}: {dcold:.4f} ms, {gbs:.1f} GB/s (caches flushed; warm loop "
                 f"{dms:.4f} ms); split-KV attention {ams:.4f} ms {agbs:.1f} GB/s")
        if with_oracle:
            from oracle import gqa_oracle as O
            # the step above overwrote slot sp with the library's new row; the
            # oracle takes the cache as generated (slot sp is replaced by its own row)
            dstep()
            torch.cuda.synchronize()
            self.log(f"[bench] {name}: oracle, full step")
            ref, sec, used = self.oracle(lambda: O.decode_forward(
                dinp.x[:, 0], dinp.wq, dinp.wk, dinp.wv, dinp.wo, 32, 8, dinp.k_cache,
                dinp.v_cache, sp)["delta"])
            rec["oracle"] = {"seconds": sec, "scope": scope, "threads": used,
                             "cpu_model": cpu_model(), "GB/s": nbytes / sec / 1e9,
                             "kind": "fp64 numpy oracle"}
            rec["parity_vs_oracle"] = self.parity(self.down_f64(dout), ref)
            self.log(f"[bench] {name}: oracle {sec:.2f} s; parity {rec['parity_vs_oracle']}")
        del kc, vc, dws, dinp
        torch.cuda.empty_cache()
        return rec

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
        ms, med = self.time_steps(step, args.steps, args.warmup)
        F = prefill_flops(B, T, sp)
        tf = F / (ms * 1e-3) / 1e12
        extra[f"chunk_B{B}_T{T}_start{sp}"] = {
            "ms_per_step": ms, "median_ms": med, "TFLOP/s": tf,
            "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS, "flops_per_step": F, "kv_len": sp + T}
        self.log(f"[bench] chunked prefill: {ms:.4f} ms, {tf:.1f} TFLOP/s")
        del kc, vc, ws
        torch.cuda.empty_cache()

    # ---------------- pre-norm + residual forms (the block's handoff) ----------------
    def prenorm(self, extra):
        """out = x + Δ(RMSNorm(x)) at the B=1 T=2048 prefill shape and the decode
        shape; the normalisation kernel's own time and bandwidth at the prefill shape."""
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
            "ms_per_step": ms_pre, "TFLOP/s": F / (ms_pre * 1e-3) / 1e12,
            "plain_block_ms": ms_plain, "overhead_frac": ms_pre / ms_plain - 1.0,
            "rmsnorm_kernel": {"ms": ms_norm, "GB/s": nb / (ms_norm * 1e-3) / 1e9, "bytes": nb}}
        self.log(f"[bench] pre-norm prefill: {ms_pre:.4f} ms vs plain {ms_plain:.4f} ms; "
                 f"rmsnorm {ms_norm * 1e3:.1f} us")
        del x, w, out, ws, y
        # the normalisation kernel alone at the token counts of the larger prefills
        norm_ms = {}
        for M in (32768, 131072):
            xm = torch.randn((M, 4096), device=self.dev).to(torch.bfloat16)
            ym = torch.empty_like(xm)
            norm_ms[M], _ = self.time_steps(lambda: gqa.rmsnorm(xm, g, y=ym), args.steps,
                                            args.warmup)
            del xm, ym
        extra["rmsnorm_kernel_by_tokens"] = {
            str(M): {"ms": v, "GB/s": 2 * M * 4096 * 2 / (v * 1e-3) / 1e9}
            for M, v in norm_ms.items()}
        self.log(f"[bench] rmsnorm alone: {', '.join(f'M={M} {v:.4f} ms' for M, v in norm_ms.items())}")

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
            "ms_per_step": dms, "GB/s": nbytes / (dms * 1e-3) / 1e9,
            "plain_decode_ms": dms_plain, "overhead_frac": dms / dms_plain - 1.0}
        self.log(f"[bench] pre-norm decode: {dms:.4f} ms vs plain {dms_plain:.4f} ms")
        del kc, vc, dws
        torch.cuda.empty_cache()

    # ---------------- SwiGLU MLP (the block's other half) ----------------
    def mlp(self, extra):
        """Pre-norm SwiGLU MLP with its residual: M = 2048 tokens in TFLOP/s, and
        M = 64 (one decode step of 64 sequences) in HBM GB/s of weights."""
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
            rec = {"ms_per_step": ms, "TFLOP/s": F / (ms * 1e-3) / 1e12,
                   "frac_of_bf16_peak": F / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                   "flops_per_step": F}
            if M <= 64:
                nb = wbytes + M * 4096 * (2 + 4)
                rec.update({"GB/s": nb / (ms * 1e-3) / 1e9,
                            "frac_of_hbm": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            "bytes_per_step": nb})
            extra[f"mlp_prenorm_M{M}"] = rec
            self.log(f"[bench] MLP M={M}: {ms:.4f} ms, {rec['TFLOP/s']:.1f} TFLOP/s")
        del w1, w2, w3, x
        torch.cuda.empty_cache()

    # ---------------- one stage alone, for the profiler ----------------
    def flash_only(self, name):
        """The attention stage of a causal prefill workload, launched K times."""
        torch, gqa, args = self.torch, self.gqa, self.args
        _, B, T, _, _ = WORKLOADS[name]
        torch.manual_seed(11)
        q = torch.randn((B, T, 32, 128), dtype=torch.float32, device=self.dev).to(torch.bfloat16)
        k = torch.randn((B, T, 8, 128), dtype=torch.float32, device=self.dev).to(torch.bfloat16)
        v = torch.randn((B, T, 8, 128), dtype=torch.float32, device=self.dev).to(torch.bfloat16)
        h = gqa.attention(q, k, v, causal=True, q_scaled=True)
        ms, med = self.time_steps(lambda: gqa.attention(q, k, v, causal=True, h_out=h,
                                                        q_scaled=True),
                                  args.steps, min(args.warmup, 1))
        F = stage_flops(B, T)["attention"]
        return {"stage": "attention", "ms": ms, "median_ms": med,
                "TFLOP/s": F / (ms * 1e-3) / 1e12}

    def vendor_gemm(self, M=32768, reps=8):
        """Context only: the block's two projection stages at M tokens against
        the vendor BLAS (torch.mm, hipBLASLt on ROCm) on the same operands,
        alternated in one process so both see the same part and clock."""
        torch, gqa = self.torch, self.gqa
        g = torch.Generator(device=self.dev)
        g.manual_seed(5)
        T = 4096
        B = M // T

        def rnd_bf16(shape, std):
            return (torch.randn(shape, device=self.dev, generator=g) * std).to(torch.bfloat16)

        x = rnd_bf16((B, T, 4096), 1.0)
        wq, wk, wv, wo = (rnd_bf16((n, 4096), 0.02) for n in (4096, 1024, 1024, 4096))
        wqkv = torch.cat([wq, wk, wv], 0).contiguous()
        rope = torch.from_numpy(gqa.rope_table(np.arange(T))).to(self.dev)
        h = rnd_bf16((M, 4096), 1.0)
        x2 = x.view(M, 4096)
        legs = [("qkv_rope (this library)", lambda: gqa.qkv_rope(x, wq, wk, wv, rope, q_scaled=True)),
                ("x @ [W_Q;W_K;W_V]^T (torch.mm)", lambda: torch.mm(x2, wqkv.t())),
                ("out_proj (this library)", lambda: gqa.output_projection(h, wo)),
                ("H @ W_O^T (torch.mm)", lambda: torch.mm(h, wo.t()))]
        times = {name: [] for name, _ in legs}
        for it in range(reps + 1):
            for name, fn in legs:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                if it:
                    times[name].append(e0.elapsed_time(e1))
        for name, t in times.items():
            t.sort()
            ms = t[len(t) // 2]
            F = 2 * M * 4096 * (6144 if "W_Q" in name or "qkv" in name else 4096)
            print(json.dumps({"vendor_gemm": name, "M": M, "median_ms": round(ms, 5),
                              "TFLOP/s": round(F / (ms * 1e-3) / 1e12, 1)}), flush=True)

    def mask_timing(self, reps=8):
        """Context only: the attention stage (pre-scaled queries, B = 1) with the
        causal flag, with the same causal mask passed explicitly (through its
        64x64 tile classes, and added element by element without a workspace),
        with a sliding window of 1024 keys and with no mask; legs alternated in
        one process, each timed over back-to-back calls (so the host's launch
        work overlaps the GPU's, as inside a block step), median of `reps`."""
        torch, gqa = self.torch, self.gqa
        g = torch.Generator(device=self.dev)
        g.manual_seed(6)
        NEG = float("-inf")
        for T in (2048, 8192):
            def rnd_bf16(shape, std):
                return (torch.randn(shape, device=self.dev, generator=g) * std).to(torch.bfloat16)
            q = rnd_bf16((1, T, 32, 128), 0.16)
            k = rnd_bf16((1, T, 8, 128), 1.28)
            v = rnd_bf16((1, T, 8, 128), 1.28)
            h = torch.empty_like(q)
            i = torch.arange(T, device=self.dev)[:, None]
            j = torch.arange(T, device=self.dev)[None, :]
            causal = torch.where(j <= i, 0.0, NEG).contiguous()
            window = torch.where((j <= i) & (j > i - 1024), 0.0, NEG).contiguous()
            att = lambda **kw: gqa.attention(q, k, v, h_out=h, q_scaled=True, **kw)
            legs = [("causal flag", lambda: att(causal=True)),
                    ("causal flag, plain launch", lambda: att(causal=True, balanced=False)),
                    ("explicit causal mask (tile classes)", lambda: att(causal=False, mask=causal)),
                    ("explicit causal mask, element-wise", lambda: att(causal=False, mask=causal,
                                                                       balanced=False)),
                    ("window of 1024 keys (tile classes)", lambda: att(causal=False, mask=window)),
                    ("no mask", lambda: att(causal=False))]
            calls = 8 if T <= 2048 else 2
            times = {name: [] for name, _ in legs}
            for it in range(reps + 1):
                for name, fn in legs:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(calls):
                        fn()
                    e1.record()
                    torch.cuda.synchronize()
                    if it:
                        times[name].append(e0.elapsed_time(e1) / calls)
            att(causal=False, mask=causal)
            h_cls = h.clone()
            att(causal=False, mask=causal, balanced=False)
            same = bool(torch.equal(h_cls, h))
            for name, t in times.items():
                t.sort()
                print(json.dumps({"mask_timing": name, "B": 1, "T": T,
                                  "median_ms": round(t[len(t) // 2], 5),
                                  "classes_bitwise_equal_element_wise": same}), flush=True)
            del q, k, v, h, causal, window, h_cls

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
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs")
    ap.add_argument("--only", choices=[*WORKLOADS, "chunk", "prenorm", "mlp",
                                       *[f"flash_{n}" for n in WORKLOADS if n.startswith("prefill")]],
                    help="run just this one workload and print its figures (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB mebibytes (3 times), for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the projection stages at M = 32768 beside the vendor "
                         "BLAS on the same operands (context, not a bench line)")
    ap.add_argument("--mask-timing", action="store_true",
                    help="only time the attention stage with the causal flag against the "
                         "same mask passed explicitly, a sliding window and no mask (context)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    b = Bench(args)
    if args.calibrate_copy:
        b.calibrate_copy(args.calibrate_copy)
        return
    if args.vendor_gemm:
        b.vendor_gemm()
        return
    if args.mask_timing:
        b.mask_timing()
        return
    extras = {"chunk": b.chunk, "prenorm": b.prenorm, "mlp": b.mlp}
    if args.only:
        if args.only.startswith("flash_"):
            rec = b.flash_only(args.only[len("flash_"):])
        elif args.only in extras:
            rec = {}
            extras[args.only](rec)
        elif WORKLOADS[args.only][0] == "decode":
            rec = b.decode(args.only, with_oracle=not args.no_cpu)
        else:
            rec = b.prefill(args.only, with_oracle=not args.no_cpu)
        print(json.dumps({"only": args.only, **rnd(rec)}), flush=True)
        return

    oracle = not args.no_cpu
    head = b.prefill(HEADLINE, with_oracle=oracle)
    configs = {HEADLINE: head}
    if not args.quick:
        for name, (kind, *_rest) in WORKLOADS.items():
            if name == HEADLINE:
                continue
            configs[name] = (b.decode(name, oracle) if kind == "decode"
                             else b.prefill(name, oracle))
    _, B, T, _, _ = WORKLOADS[HEADLINE]
    result = {
        "metric": "GQA block fwd TFLOP/s (% bf16 MFMA peak) prefill; decode HBM GB/s",
        "value": round(head["TFLOP/s"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B GQA attention block forward, long-context "
                               f"prefill B={B} T={T} causal",
                   "B": B, "T": T, "d": 4096, "q_heads": 32, "kv_heads": 8, "d_head": 128,
                   "rope_theta": 500000.0, "flops_per_step": head["flops_per_step"],
                   "median_ms": round(head["median_ms"], 5),
                   "frac_of_bf16_peak": round(head["frac_of_bf16_peak"], 4)},
        "roofline": rnd(head["roofline"]),
    }
    if oracle:
        o = head["oracle"]
        result["cpu_baseline"] = {"value": round(o["TFLOP/s"], 5), "unit": "TFLOP/s",
                                  "cores": o["threads"], "kind": "oracle",
                                  "sample": o["scope"] + f" of the B={B} T={T} causal prefill, "
                                            "fp64 numpy, one evaluation",
                                  "seconds": round(o["seconds"], 3), "cpu_model": o["cpu_model"]}
    result["configs"] = {k: rnd(v) for k, v in configs.items()}
    if not args.quick:
        other = {}
        for fn in extras.values():
            fn(other)
        result["other_workloads"] = {k: rnd(v) for k, v in other.items()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
