#!/usr/bin/env python3
"""Benchmark of selected-token sparse attention with KV append on one MI355X.

A step is one pass of the whole path over one batch: reset the device error
word, append the current token(s) to the cache in place (quantizing them for
fp8 records), validate the index rows, gather + score + softmax + PV (+ split-K
combine), store Y. On the shared-latent MFMA paths this is one
sparse_attn_step call (one attention launch that also appends and resets, plus
the combine); elsewhere the three calls reset_error_async, kv_append and
forward.

Default workload (decode, bf16, shared-latent MLA rows): batch 32, one query
per sequence, 64 query heads sharing one kv head, 576-dim rows (V = first
512), past 32768 + 1 current, top-2048 uniform sorted indices. Inputs are
seeded synthetic N(0,1) values drawn on the device and stay resident in HBM.
To keep the 256 MB Infinity Cache from serving the gathers, the timed steps
rotate over R independent (query, index) sets, whose gathered rows together
exceed it several times.

Timing: W warmup steps, then K steps replayed from a captured HIP graph
between HIP events; value = selected tokens attended per second. The main
attention kernel's own duration is measured with the library's event pair
over a second, eager pass of K steps on the same stream; the roofline figure
divides the kernel's algorithmic bytes (or flops) by that duration. The CPU
baseline is the oracle on a bounded sample of the same workload.

Output: one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_FP32_PEAK_TFLOPS = 157.3
PROFILES = ROOT / "profiles"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--workload", default="decode_bf16",
                   choices=["decode_bf16", "decode_fp8", "prefill_bf16", "dense_gqa", "csa_decode",
                            "csa_index_decode", "capacity_decode", "capacity_latent_decode", "gqa_decode_b2"])
    p.add_argument("--rotate", type=int, default=8, help="independent (query, index) sets")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline duration")
    p.add_argument("--no-also", action="store_true",
                   help="default workload only: skip the decode_fp8 / prefill_bf16 figures and the concat copy")
    p.add_argument("--also-steps", type=int, default=20, help="steps timed for each extra workload")
    p.add_argument("--stats-digest", metavar="KERNEL_STATS_CSV",
                   help="turn a rocprofv3 --kernel-trace --stats CSV of this script into the committed "
                        "summary of the workload's main kernel")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--trials", type=int, default=20,
                   help="extra timed trials (>= 200 replayed steps each) whose median is reported")
    p.add_argument("--no-peaks", action="store_true", help="skip re-measuring the copy and MFMA peaks")
    p.add_argument("--pmc-run", action="store_true",
                   help="counter pass: a 256 MiB device copy (calibration), then W + K eager steps")
    p.add_argument("--digest", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc CSVs (FETCH_SIZE, WRITE_SIZE) of a --pmc-run "
                        "into the committed counters summary of the main kernel")
    return p.parse_args()


# sources whose text decides each main kernel's code (the counters summary is
# only used while their hash is unchanged)
KERNEL_SOURCES = {
    "latent_forward_kernel": ["k_forward_latent.hip", "sa_internal.h", "sa_validate_dev.h", "sa_mfma_dev.h"],
    "latent_decode_kernel": ["k_forward_latent_decode.hip", "sa_internal.h", "sa_validate_dev.h",
                             "sa_mfma_dev.h"],
    "pair_forward_kernel": ["k_forward_pair.hip", "sa_internal.h", "sa_validate_dev.h", "sa_mfma_dev.h",
                            "sa_quant_dev.h"],
    "mla_forward_kernel": ["k_forward_mla.hip", "sa_internal.h"],
    "generic_forward_kernel": ["k_forward_generic.hip", "sa_internal.h"],
    "gqa_forward_kernel": ["k_forward_gqa.hip", "sa_internal.h", "sa_mfma_dev.h"],
    "csa_attention_kernel": ["k_csa_attention.hip", "sa_internal.h", "sa_mfma_dev.h", "sa_quant_dev.h"],
    "csa_index_score_kernel": ["k_csa_index.hip", "sa_internal.h", "sa_mfma_dev.h"],
}
CALIB_BYTES = 256 << 20


def cpu_threads():
    """Threads of the CPU baseline: the host's CPUs, capped by the CPU share the
    environment grants (OMP_NUM_THREADS, set on shared GPU hosts)."""
    n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return n


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        h.update((ROOT / "sparse_attention_kv_append_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


class Setup:
    """Device-resident inputs and the step closure for one workload."""

    def __init__(self, name, rotate):
        import numpy as np
        import torch

        import sa_workloads as W
        import sparse_attention_kv_append_amd as sa
        self.np, self.torch, self.W, self.sa = np, torch, W, sa
        self.w = w = W.WORKLOADS[name]
        self.name = name
        self.R = rotate
        dev = "cuda"
        B, Hq, Sq, Dk, Dv = w.batch, w.hq, w.q_seq, w.dk, w.dv
        cap = w.cap
        fp8 = w.cache_format == W.CACHE_FP8
        self.ctx = sa.Context(num_heads=Hq, kv_num_heads=w.hkv, head_dim_qk=Dk, head_dim_v=Dv,
                              dtype=w.dtype, kv_layout=w.layout,
                              cache_format=sa.SA_CACHE_FP8_E4M3_BLOCK64 if fp8 else sa.SA_CACHE_DENSE,
                              rope_dim=w.rope, scale=w.scale, softcap=w.softcap, max_batch=B,
                              max_q_seq=Sq, max_index_width=w.width, max_cache_len=cap)
        seed = w.seed
        gen = lambda shape, s: W.torch_normal_bf16(shape, s, dev)
        self.gen = gen
        self.chunk = 4096                      # fp8 past rows are drawn and quantized per chunk
        self.chunk_seed = lambda c: seed * 1000 + c
        # caches
        if w.layout == W.LAYOUT_SHARED_LATENT:
            if fp8:
                rec = (Dk - w.rope) // 64 * 65 + 2 * w.rope
                self.k = torch.empty((B, 1, cap, rec), dtype=torch.uint8, device=dev)
                # the latent rows are quantized into records by the library's
                # own quantize-on-append (the oracle's block-quantizer rule)
                chunk = self.chunk
                for t0 in range(0, w.past, chunk):
                    n = min(chunk, w.past - t0)
                    rows = gen((B, 1, n, Dk), self.chunk_seed(t0 // chunk))
                    plen = torch.full((B,), t0, dtype=torch.int32, device=dev)
                    self.ctx.kv_append(B, self.k, None, cap, plen, rows, None, n, self.k, None, cap,
                                       cur_is_unquantized_bf16=True)
                torch.cuda.synchronize()
            else:
                self.k = gen((B, 1, cap, Dk), seed * 1000)
            self.v = None
            self.cur_k = gen((B, 1, w.cur, Dk), seed * 1000 + 999)
            self.cur_v = None
        else:
            self.k = gen((B, w.hkv, cap, Dk), seed * 1000)
            self.v = gen((B, w.hkv, cap, Dv), seed * 1000 + 1)
            self.cur_k = gen((B, w.hkv, w.cur, Dk), seed * 1000 + 998)
            self.cur_v = gen((B, w.hkv, w.cur, Dv), seed * 1000 + 999)
        self.fp8 = fp8
        self.plen = torch.full((B,), w.past, dtype=torch.int32, device=dev)
        self.vlen = torch.zeros((B,), dtype=torch.int32, device=dev)
        # rotating query / index sets
        self.qs, self.idx_host, self.idxs = [], [], []
        for r in range(self.R):
            self.qs.append(gen((B, Hq, Sq, Dk), seed * 1000 + 500 + r))
            rng = np.random.default_rng(seed * 100 + r)
            ih = W.index_rows(w, rng)
            self.idx_host.append(ih)
            self.idxs.append(torch.from_numpy(ih).to(dev))
            if w.pattern != "uniform":
                break  # the causal patterns are deterministic: one set
        ydt = {W.DT_F32: torch.float32, W.DT_F16: torch.float16, W.DT_BF16: torch.bfloat16}[w.dtype]
        self.y = torch.empty((B, Hq, Sq, Dv), dtype=ydt, device=dev)
        self.selected = [int((ih >= 0).sum()) // 1 for ih in self.idx_host]
        self.path, self.splits = self.ctx.query_plan(B, Sq, 1, w.width)

    def fused_step(self):
        """True when the step is one library call that the library runs as one
        forward launch (plus its combine): sparse_attn_step on the
        shared-latent MFMA paths (at most 8 current rows), sparse_attn_step_kv
        on the grouped-query path."""
        return (self.path in (2, 3) and self.w.cur <= 8) or self.path == 4

    def step(self, i):
        w, c = self.w, self.ctx
        r = i % len(self.idxs)
        if self.path == 4:
            c.step_kv(self.qs[r % len(self.qs)], w.batch, w.q_seq, self.k, self.v, w.cap, self.plen, self.cur_k,
                      self.cur_v, w.cur, self.vlen, self.idxs[r], 1, w.width, self.y, reset_error=True)
            return
        if self.fused_step():
            c.step(self.qs[r % len(self.qs)], w.batch, w.q_seq, self.k, w.cap, self.plen, self.cur_k, w.cur,
                   self.vlen, self.idxs[r], 1, w.width, self.y, reset_error=True,
                   cur_is_unquantized_bf16=self.fp8)
            return
        c.reset_error_async()
        c.kv_append(w.batch, self.k, self.v, w.cap, self.plen, self.cur_k, self.cur_v, w.cur, self.k,
                    self.v, w.cap, cur_is_unquantized_bf16=self.fp8, present_len=self.vlen)
        c.forward(self.qs[r % len(self.qs)], w.batch, w.q_seq, self.k, self.v, w.cap, self.vlen,
                  self.idxs[r], 1, w.width, self.y, fused_validate=True)

    # ---- work accounting (per step, averaged over the rotation sets)
    def tokens_per_step(self):
        """Selected (row, key) pairs attended per step, all heads of a row counted once."""
        return sum(self.selected) / len(self.selected)

    def kernel_work(self):
        """Algorithmic bytes and flops of ONE launch of the main attention kernel."""
        w = self.w
        sel = self.tokens_per_step()
        if w.layout == self.W.LAYOUT_SHARED_LATENT:
            row_bytes = ((w.dk - w.rope) // 64 * 65 + 2 * w.rope) if self.fp8 else w.dk * 2
            gather = sel * row_bytes
            heads_per_key = w.hq
        else:
            # separate K/V: each (row, kv head) selects K and V rows of 2*D bytes
            # (the grouped-query kernel gathers a shared tile once for all its rows)
            gather = sel * w.hkv * (w.dk + w.dv) * 2
            heads_per_key = w.hq
        qbytes = w.batch * w.hq * w.q_seq * w.dk * 2
        ibytes = sum(ih.size for ih in self.idx_host) / len(self.idx_host) * 4
        flops = sel * heads_per_key * 2 * (w.dk + w.dv)
        return dict(bytes=gather + qbytes + ibytes, gather_bytes=gather, flops=flops)

    def step_bytes(self):
        w = self.w
        kw = self.kernel_work()
        ybytes = w.batch * w.hq * w.q_seq * w.dv * 2
        row_bytes = ((w.dk - w.rope) // 64 * 65 + 2 * w.rope) if self.fp8 else w.dk * 2
        append = w.batch * w.hkv * w.cur * (row_bytes + (w.dv * 2 if self.v is not None else 0))
        return kw["bytes"] + ybytes + 2 * append

    # ---- reporting
    def roofline(self, kw, k_avg_s):
        w = self.w
        if w.pattern == "causal_prefill" or (self.path == 4 and w.q_seq > 1):
            return "mfma", MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", kw["flops"] / k_avg_s / 1e12
        if self.path == 4:  # grouped-query decode: the gathers bound it
            return "hbm", HBM_PEAK_GBS, "GB/s", kw["bytes"] / k_avg_s / 1e9
        if w.layout == self.W.LAYOUT_SEPARATE:
            return "alu", VALU_FP32_PEAK_TFLOPS, "TFLOP/s", kw["flops"] / k_avg_s / 1e12
        return "hbm", HBM_PEAK_GBS, "GB/s", kw["bytes"] / k_avg_s / 1e9

    def dtype_name(self):
        return "fp8" if self.fp8 else {0: "f32", 1: "f16", 2: "bf16"}[self.w.dtype]

    def config(self, use_graph, nset, tokens, ms_per_step):
        w = self.w
        return {"workload": f"{w.name}: batch {w.batch}, q_seq {w.q_seq}, {w.hq} q heads / "
                            f"{w.hkv} kv heads, Dk {w.dk} / Dv {w.dv}, past {w.past} + {w.cur}, "
                            f"index width {w.width}, {'graph replay' if use_graph else 'eager'}, "
                            f"{nset} rotating index sets",
                "selected_tokens_per_step": tokens, "splits": self.splits,
                "step_calls": ("sparse_attn_step_kv (reset + append + validation + forward in one launch)"
                               if self.path == 4 else
                               "sparse_attn_step (reset + append + forward in one launch)" if self.fused_step()
                               else "reset_error_async + kv_append + forward"),
                "step_hbm_GBps": self.step_bytes() / (ms_per_step / 1e3) / 1e9}

    def cpu_baseline(self, target_s, threads=None):
        return cpu_baseline(self, target_s, threads)


class CapacitySetup(Setup):
    """Capacity-mode decode with the optional attention bias (IndexShare's
    fixed-capacity present): bf16 K and V caches (or one shared-latent cache)
    of `capacity` rows drawn on the device, per-batch live lengths carried
    only by the bias's -inf frontier, and a step of capacity_lengths (valid
    length and write position from the bias) -> in-place kv_append at the
    write position -> forward_bias with fused validation against the
    recovered lengths (one sparse_attn_capacity_step call)."""

    def __init__(self, name, rotate):
        import numpy as np
        import torch

        import sa_workloads as W
        import sparse_attention_kv_append_amd as sa
        self.np, self.torch, self.W, self.sa = np, torch, W, sa
        self.w = w = W.CAPACITY_WORKLOADS[name]
        self.name = name
        self.R = rotate
        dev = "cuda"
        B, Hq, Hkv, Sq, Dk, Dv, cap = w.batch, w.hq, w.hkv, w.q_seq, w.dk, w.dv, w.cap
        assert w.dtype == W.DT_BF16 and w.cache_format == W.CACHE_DENSE
        self.latent = latent = w.layout == W.LAYOUT_SHARED_LATENT
        self.ctx = sa.Context(num_heads=Hq, kv_num_heads=Hkv, head_dim_qk=Dk, head_dim_v=Dv, dtype=w.dtype,
                              kv_layout=sa.SA_KV_SHARED_LATENT if latent else sa.SA_KV_SEPARATE,
                              scale=w.scale, softcap=w.softcap, max_batch=B,
                              max_q_seq=Sq, max_index_width=w.width, max_cache_len=cap)
        seed = w.seed
        gen = lambda shape, s: W.torch_normal_bf16(shape, s, dev)
        self.k = gen((B, Hkv, cap, Dk), seed * 1000)
        self.v = None if latent else gen((B, Hkv, cap, Dv), seed * 1000 + 1)
        self.cur_k = gen((B, Hkv, w.cur, Dk), seed * 1000 + 998)
        self.cur_v = None if latent else gen((B, Hkv, w.cur, Dv), seed * 1000 + 999)
        # the caches as drawn, before any step writes the current rows (oracle inputs)
        self.k0, self.v0 = self.k.clone(), None if latent else self.v.clone()
        rng = np.random.default_rng(seed)
        self.valid, bias32 = W.capacity_frontier(w, rng)
        self.bias_host = W.store_elems(bias32, w.dtype)
        self.bias = torch.from_numpy(self.bias_host.view(np.int16)).to(dev)
        self.qs, self.idx_host, self.idxs = [], [], []
        for r in range(self.R):
            self.qs.append(gen((B, Hq, Sq, Dk), seed * 1000 + 500 + r))
            ih = W.index_rows(w, np.random.default_rng(seed * 100 + r), bound=self.valid)
            self.idx_host.append(ih)
            self.idxs.append(torch.from_numpy(ih).to(dev))
        self.y = torch.empty((B, Hq, Sq, Dv), dtype=torch.bfloat16, device=dev)
        self.vl = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.wp = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.fp8 = False
        self.selected = [int((ih >= 0).sum()) for ih in self.idx_host]
        # a biased forward runs on the grouped-query or shared-latent MFMA
        # kernel where the plan takes one (the general latent kernel on a bf16
        # shared-latent cache, never the decode kernel), else generic
        plan, nsplit = self.ctx.query_plan(B, Sq, 1, w.width)
        self.path, self.splits = (plan, nsplit) if plan in (2, 3, 4) else (0, 1)

    def fused_step(self):
        return False

    def step(self, i):
        w, c = self.w, self.ctx
        r = i % len(self.idxs)
        c.capacity_step(self.qs[r], w.batch, w.q_seq, self.k, self.v, w.cap, self.cur_k, self.cur_v, w.cur,
                        self.idxs[r], 1, w.width, self.bias, self.y, self.vl, self.wp, reset_error=True)

    def kernel_work(self):
        kw = Setup.kernel_work(self)
        kw["bytes"] += self.tokens_per_step() * 2    # the bias at each selected (row, key)
        return kw

    def step_bytes(self):
        w = self.w
        return Setup.step_bytes(self) + w.batch * w.q_seq * w.cap * 2   # the frontier scan

    def roofline(self, kw, k_avg_s):
        return "hbm", HBM_PEAK_GBS, "GB/s", kw["bytes"] / k_avg_s / 1e9

    def config(self, use_graph, nset, tokens, ms_per_step):
        w = self.w
        layout = (f"one shared-latent row of {w.dk} dims (V = its first {w.dv})" if self.latent
                  else f"{w.hkv} kv heads, head dim {w.dk}")
        return {"workload": f"{w.name}: capacity mode, batch {w.batch}, q_seq {w.q_seq}, {w.hq} q heads / "
                            f"{layout}, capacity {w.cap}, live lengths "
                            f"{int(self.valid.min())}..{int(self.valid.max())} from a [B, 1, {w.q_seq}, {w.cap}] "
                            f"bf16 bias, {w.cur} current row, top-{w.topk}, "
                            f"{'graph replay' if use_graph else 'eager'}, {nset} rotating index sets",
                "selected_tokens_per_step": tokens, "splits": self.splits,
                "step_calls": "sparse_attn_capacity_step (reset, lengths + in-place append in one launch, "
                              "validation, biased forward)",
                "step_hbm_GBps": self.step_bytes() / (ms_per_step / 1e3) / 1e9}

    def oracle_inputs(self, b, r=0):
        """Host copies of batch entry b's inputs (storage bits): q, past_k,
        past_v (as drawn; None for a shared-latent cache), cur_k, cur_v,
        indices, bias."""
        np = self.np
        bits = lambda t: None if t is None else t.contiguous().view(self.torch.int16).cpu().numpy().view(np.uint16)
        one = lambda t: None if t is None else t[b:b + 1]
        return dict(q=bits(self.qs[r][b:b + 1]), past_k=bits(self.k0[b:b + 1]), past_v=bits(one(self.v0)),
                    cur_k=bits(self.cur_k[b:b + 1]), cur_v=bits(one(self.cur_v)),
                    indices=self.idx_host[r][b:b + 1], bias=self.bias_host[b:b + 1])

    def oracle_y(self, inp, threads):
        """The oracle's capacity step for one batch entry: lengths from the
        bias, in-place append at the write position, biased forward."""
        import oracle
        w = self.w
        valid, wpos = oracle.capacity_lengths(inp["bias"], w.cap, w.cur, batch=1, heads=w.hq, q_seq=w.q_seq,
                                              bias_dtype=w.dtype)
        pk = oracle.kv_append(inp["past_k"].copy(), wpos, inp["cur_k"])
        pv = None if inp["past_v"] is None else oracle.kv_append(inp["past_v"].copy(), wpos, inp["cur_v"])
        y = oracle.forward(inp["q"], pk, pv, inp["indices"], q_dtype=w.dtype, cache_fmt=w.dtype,
                           kv_layout=w.layout, hkv=w.hkv, dv=w.dv, scale=w.scale, softcap=w.softcap,
                           bias=inp["bias"], threads=threads)
        return y, valid, wpos

    def cpu_baseline(self, target_s):
        """The oracle's whole capacity step (lengths, append, biased forward)
        on batch entries taken in order until about target_s seconds of oracle
        time; only the oracle calls are timed."""
        w = self.w
        threads = cpu_threads()
        n, t, done = 0, 0.0, 0
        while t < target_s and done < 4 * w.batch:
            b = done % w.batch
            inp = self.oracle_inputs(b)
            t0 = time.perf_counter()
            self.oracle_y(inp, threads)
            t += time.perf_counter() - t0
            n += int((inp["indices"] >= 0).sum())
            done += 1
        return {"value": n / t, "unit": "selected tokens/s", "cores": threads, "host_cpus": os.cpu_count(),
                "kind": "oracle",
                "sample": f"{done} batch entries (in order, cycling over {w.batch}) of the same workload, "
                          f"all {w.hq} heads, {n} selected keys, {t:.1f} s of oracle time"}


class CsaSetup:
    """Device-resident inputs and the step closure of CSA ratio-4 selected sink
    attention: fp32 query and current_kv, 583-byte fp8 records made from bf16
    rows by the library's quantize-on-append, a random-order top-k selection of
    complete records per query, a head sink. The timed steps rotate over R
    (query, current_kv, selection) sets so the gathered bytes of one rotation
    exceed the Infinity Cache."""

    path = 5
    splits = 1

    def __init__(self, name, rotate):
        import numpy as np
        import torch

        import sa_workloads as W
        import sparse_attention_kv_append_amd as sa
        self.np, self.torch, self.W, self.sa = np, torch, W, sa
        self.w = w = W.CSA_WORKLOADS[name]
        self.name = name
        self.R = rotate
        dev = "cuda"
        B, S, H, T = w.batch, w.seq, w.heads, w.cur_len
        self.ctx = sa.Context(num_heads=16, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_F32)
        seed = w.seed
        self.chunk = 4096
        self.chunk_seed = lambda c: seed * 1000 + c
        qctx = sa.Context(num_heads=1, kv_num_heads=1, head_dim_qk=512, head_dim_v=512, dtype=sa.SA_BF16,
                          kv_layout=sa.SA_KV_SHARED_LATENT, cache_format=sa.SA_CACHE_FP8_E4M3_BLOCK64,
                          rope_dim=64, max_batch=B, max_q_seq=1, max_index_width=1, max_cache_len=w.cap)
        rec = torch.zeros((B, 1, w.cap, 583), dtype=torch.uint8, device=dev)
        for t0 in range(0, w.records, self.chunk):
            n = min(self.chunk, w.records - t0)
            rows = W.torch_normal_bf16((B, 1, n, 512), self.chunk_seed(t0 // self.chunk), dev)
            plen = torch.full((B,), t0, dtype=torch.int32, device=dev)
            qctx.kv_append(B, rec, None, w.cap, plen, rows, None, n, rec, None, w.cap,
                           cur_is_unquantized_bf16=True)
        torch.cuda.synchronize()
        word, _, msg = qctx.read_error()
        assert word == 0, msg
        qctx.destroy()
        self.rec = rec.view(B, w.cap, 583)
        self.qs, self.ckvs, self.idx_host, self.idxs = [], [], [], []
        for r in range(self.R):
            self.qs.append(W.torch_normal_f32((B, S, H, 512), seed * 1000 + 500 + r, dev))
            self.ckvs.append(W.torch_normal_f32((B, T, 512), seed * 1000 + 700 + r, dev))
            sel = W.csa_selection(w, np.random.default_rng(seed * 100 + r))
            self.idx_host.append(sel)
            self.idxs.append(torch.from_numpy(sel).to(dev))
        self.sink_host = np.random.default_rng(seed).standard_normal(H).astype(np.float32)
        self.sink = torch.from_numpy(self.sink_host).to(dev)
        self.total = torch.tensor([w.total], dtype=torch.int64, device=dev)
        self.y = torch.empty((B, S, H, 512), dtype=torch.float32, device=dev)
        self.fp8 = True

    def fused_step(self):
        return False

    def step(self, i):
        r = i % len(self.idxs)
        self.ctx.reset_error_async()
        self.ctx.csa_forward(self.qs[r], self.ckvs[r], self.rec, self.idxs[r], self.sink, self.total, self.y,
                             scale=self.w.scale)

    def _dense(self):
        """Dense candidates per query (the window rows at or before it)."""
        w = self.w
        start, base = w.total - w.seq, w.total - w.cur_len
        dn = min(w.cur_len, 128) if start == 0 else 128
        out = []
        for s in range(w.seq):
            pos = start + s
            ws = max(base, pos + 1 - 128)
            out.append(min(dn, pos - ws + 1))
        return out

    def tokens_per_step(self):
        """Candidates attended per step (dense window rows + valid selected
        records), all heads of a (batch, query) counted once."""
        w = self.w
        sel = sum(int(((ih[:, 0] >= 0) & (ih[:, 0] < w.records)).sum()) for ih in self.idx_host) / len(self.idx_host)
        return w.batch * sum(self._dense()) + sel

    def kernel_work(self):
        w = self.w
        nsel = sum(int((ih[:, 0] >= 0).sum()) for ih in self.idx_host) / len(self.idx_host)
        ndense = w.batch * sum(self._dense())
        qy = 2 * w.batch * w.seq * w.heads * 512 * 4
        # current_kv rows: a (batch) reads the union of its queries' windows once
        rows = w.batch * min(w.cur_len, sum(self._dense()) if w.seq == 1 else w.cur_len)
        gather = nsel * 583 + rows * 512 * 4
        ibytes = w.batch * w.seq * w.topk * 4
        flops = (nsel + ndense) * w.heads * 2 * 2 * 512
        return dict(bytes=qy + gather + ibytes, gather_bytes=gather, flops=flops)

    def step_bytes(self):
        return self.kernel_work()["bytes"]

    def roofline(self, kw, k_avg_s):
        return "hbm", HBM_PEAK_GBS, "GB/s", kw["bytes"] / k_avg_s / 1e9

    def dtype_name(self):
        return "f32"

    def config(self, use_graph, nset, tokens, ms_per_step):
        w = self.w
        return {"workload": f"{w.name}: CSA ratio-4 selected sink attention, batch {w.batch}, q_seq {w.seq}, "
                            f"{w.heads} heads, dim 512, current_kv {w.cur_len} fp32 rows (window 128), "
                            f"total {w.total} ({w.records} fp8_e4m3_block64 583-byte records), top-{w.topk} "
                            f"selected, {'graph replay' if use_graph else 'eager'}, {nset} rotating sets",
                "candidates_per_step": tokens, "splits": 1,
                "step_calls": "reset_error_async + csa_forward",
                "step_hbm_GBps": self.step_bytes() / (ms_per_step / 1e3) / 1e9}

    def oracle_inputs(self, bs):
        """The oracle's inputs for batch entries bs (rotation set 0), from the
        seeded generators: query and current_kv as drawn, the selected records
        packed by the oracle's own quantizer from the generator's bf16 rows (the
        other records are zeros, never read)."""
        import oracle
        np, torch, w = self.np, self.torch, self.w
        sels = [self.idx_host[0][b:b + 1] for b in bs]
        needs = [np.unique(sel[sel >= 0]) for sel in sels]
        recs = [np.zeros((1, w.cap, 583), np.uint8) for _ in bs]
        chunks = np.unique(np.concatenate([n // self.chunk for n in needs]))
        for c in chunks:
            t0 = int(c) * self.chunk
            n = min(self.chunk, w.records - t0)
            rows = self.W.torch_normal_bf16((w.batch, 1, n, 512), self.chunk_seed(int(c)), "cuda")
            for j, b in enumerate(bs):
                keys = needs[j][(needs[j] >= t0) & (needs[j] < t0 + n)]
                if len(keys):
                    v = rows[b, 0].index_select(0, torch.from_numpy(keys - t0).cuda()).float().cpu().numpy()
                    recs[j][0, keys] = oracle.fp8_pack_rows(v, 64)
            del rows
        return [dict(query=self.qs[0][b:b + 1].cpu().numpy(), current_kv=self.ckvs[0][b:b + 1].cpu().numpy(),
                     records=recs[j], selected=sels[j], sink=self.sink_host) for j, b in enumerate(bs)]

    def oracle_y(self, inp):
        import oracle
        y, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], inp["records"], inp["selected"],
                                             inp["sink"], self.w.total, scale=self.w.scale)
        assert flags == 0, flags
        return y

    def cpu_baseline(self, target_s):
        """The oracle (unchanged) on a bounded sample: the first batch entries of
        the same workload, one per thread (each C call releases the GIL),
        repeated until the target time is reached."""
        import threading
        w = self.w
        threads = cpu_threads()
        nb = min(w.batch, threads)
        inputs = self.oracle_inputs(list(range(nb)))
        ndense = sum(self._dense())
        cands = sum(ndense + int((inp["selected"][0, 0] >= 0).sum()) for inp in inputs)

        def run():
            t0 = time.perf_counter()
            ts = [threading.Thread(target=self.oracle_y, args=(inp,)) for inp in inputs]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
            return time.perf_counter() - t0

        reps, total_t = 0, 0.0
        while total_t < target_s and reps < 200:
            total_t += run()
            reps += 1
        return {"value": cands * reps / total_t, "unit": "candidates/s", "cores": nb,
                "host_cpus": os.cpu_count(), "kind": "oracle",
                "sample": f"the first {nb} (batch, query) rows of the same workload x {reps}, one thread each, "
                          f"all {w.heads} heads, {cands * reps} candidates, {total_t:.1f} s of oracle time"}


class CsaIndexSetup:
    """Device-resident inputs and the step of the CSA selection producer:
    index queries and weights fp32, FP4 index keys drawn as random bytes on the
    device, the caller-owned workspace, R rotating (query, weight) sets."""

    path = 6
    splits = 1
    # among 16384 fp32 scores per row, exactly equal scores (which the CPU page
    # rejects) occur by chance in synthetic data; the device reports them
    tolerated_bits = 0x2000  # SA_ERR_INDEX_TIE

    def __init__(self, name, rotate):
        import torch

        import sa_workloads as W
        import sparse_attention_kv_append_amd as sa
        self.torch, self.W, self.sa = torch, W, sa
        self.w = w = W.CSA_INDEX_WORKLOADS[name]
        self.name = name
        self.R = rotate
        dev = "cuda"
        B, S, H = w.batch, w.seq, w.heads
        self.ctx = sa.Context(num_heads=16, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_F32)
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed * 1000 + 77)
        keys = torch.randint(0, 256, (B, w.key_cap, 68), generator=g, device=dev, dtype=torch.uint8)
        keys[:, :, 0::17] = torch.randint(122, 127, (B, w.key_cap, 4), generator=g, device=dev,
                                          dtype=torch.uint8)
        self.keys = keys
        self.iqs = [W.torch_normal_f32((B, S, H, 128), w.seed * 1000 + 500 + r, dev) for r in range(self.R)]
        self.iws = [W.torch_normal_f32((B, S, H), w.seed * 1000 + 600 + r, dev) for r in range(self.R)]
        self.idxs = self.iqs  # rotation sets
        self.total = torch.tensor([w.total], dtype=torch.int64, device=dev)
        self.sel = torch.empty((B, w.out_heads, S, w.topk), dtype=torch.int32, device=dev)
        self.ws = torch.empty(self.ctx.csa_index_workspace_bytes(B, S, H, w.key_cap), dtype=torch.uint8,
                              device=dev)
        self.fp8 = False

    def fused_step(self):
        return False

    def step(self, i):
        r = i % len(self.iqs)
        self.ctx.reset_error_async()
        self.ctx.csa_index_select(self.iqs[r], self.iws[r], self.keys, self.total, self.sel, self.ws)

    def _n(self):
        w = self.w
        return [min((w.total - w.seq + s + 1) // 4, w.key_cap) for s in range(w.seq)]

    def tokens_per_step(self):
        """Records scored per step (all index heads of a (batch, query) counted once)."""
        return self.w.batch * sum(self._n())

    def kernel_work(self):
        """Algorithmic bytes and flops of one score launch."""
        w = self.w
        n = self.tokens_per_step()
        keys = n * 68
        q = w.batch * w.seq * w.heads * (128 * 2 + 4)   # the finalized query (bf16) and the weights
        scores = n * 4
        flops = n * w.heads * 2 * 128
        return dict(bytes=keys + q + scores, gather_bytes=keys, flops=flops)

    def step_bytes(self):
        w = self.w
        n = self.tokens_per_step()
        return (n * 68 + n * 4 * 2 + w.batch * w.seq * w.heads * (128 * 4 * 2 + 128 * 2 + 4)
                + w.batch * w.out_heads * w.seq * w.topk * 4)

    def roofline(self, kw, k_avg_s):
        return "hbm", HBM_PEAK_GBS, "GB/s", kw["bytes"] / k_avg_s / 1e9

    def dtype_name(self):
        return "fp4"

    def config(self, use_graph, nset, tokens, ms_per_step):
        w = self.w
        return {"workload": f"{w.name}: CSA ratio-4 selection producer, batch {w.batch}, q_seq {w.seq}, "
                            f"{w.heads} index heads of 128 dims, {w.key_cap} FP4 E2M1 block-32 index keys "
                            f"(68 B), total {w.total}, top-{w.topk}, {'graph replay' if use_graph else 'eager'}, "
                            f"{nset} rotating query sets",
                "records_scored_per_step": tokens, "splits": 1,
                "step_calls": "reset_error_async + csa_index_select (finalize, score, select launches)",
                "step_hbm_GBps": self.step_bytes() / (ms_per_step / 1e3) / 1e9}

    def oracle_inputs(self, b):
        """Batch entry b of rotation set 0 as host arrays (generator outputs)."""
        return {"index_query": self.iqs[0][b:b + 1].cpu().numpy(),
                "index_weight": self.iws[0][b:b + 1].cpu().numpy(),
                "index_keys": self.keys[b:b + 1].cpu().numpy()}

    def cpu_baseline(self, target_s):
        """The oracle (unchanged) on the first batch entries, one per thread,
        repeated until the target time is reached."""
        import threading

        import oracle
        w = self.w
        threads = cpu_threads()
        nb = min(w.batch, threads)
        inputs = [self.oracle_inputs(b) for b in range(nb)]

        def one(inp):
            oracle.csa_index_select(inp["index_query"], inp["index_weight"], inp["index_keys"], w.total, w.topk)

        reps, total_t = 0, 0.0
        while total_t < target_s and reps < 200:
            t0 = time.perf_counter()
            ts = [threading.Thread(target=one, args=(inp,)) for inp in inputs]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
            total_t += time.perf_counter() - t0
            reps += 1
        recs = nb * sum(self._n()) * reps
        return {"value": recs / total_t, "unit": "records scored/s", "cores": nb,
                "host_cpus": os.cpu_count(), "kind": "oracle",
                "sample": f"the first {nb} (batch, query) rows of the same workload x {reps}, one thread each, "
                          f"all {w.heads} index heads, {recs} records scored and ranked, {total_t:.1f} s"}


def make_setup(name, rotate):
    import sa_workloads as W
    if name in W.CAPACITY_WORKLOADS:
        return CapacitySetup(name, rotate)
    if name in W.CSA_INDEX_WORKLOADS:
        return CsaIndexSetup(name, rotate)
    return CsaSetup(name, rotate) if name in W.CSA_WORKLOADS else Setup(name, rotate)


def kernel_name(setup):
    if setup.path == 2 and not isinstance(setup, CapacitySetup):
        return "latent_decode_kernel"
    return {0: "generic_forward_kernel", 1: "mla_forward_kernel", 2: "latent_forward_kernel",
            3: "pair_forward_kernel", 4: "gqa_forward_kernel", 5: "csa_attention_kernel",
            6: "csa_index_score_kernel"}[setup.path]


def counters_for(setup):
    """HBM traffic of the main kernel from a committed rocprofv3 --pmc summary,
    if it was taken on the current kernel source; else None."""
    f = PROFILES / f"{kernel_name(setup)}_{setup.name}_counters.json"
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except Exception:
        return None
    if d.get("source_hash") != source_hash(*KERNEL_SOURCES[kernel_name(setup)]):
        return None
    return d.get("traffic_bytes_per_launch")


def pmc_run(args):
    """Short eager pass for rocprofv3 --pmc: first a plain device-to-device copy
    of CALIB_BYTES (its counter reading calibrates KiB -> bytes), then the steps."""
    import torch
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    s = make_setup(args.workload, args.rotate)
    print(f"pmc-run: {args.workload} kernel {kernel_name(s)}", file=sys.stderr, flush=True)
    for i in range(args.warmup + args.steps):
        s.step(i)
    torch.cuda.synchronize()
    word, _, msg = s.ctx.read_error()
    assert word & ~getattr(s, "tolerated_bits", 0) == 0, msg
    print(json.dumps({"pmc_run": args.workload, "kernel": kernel_name(s),
                      "steps": args.warmup + args.steps}), flush=True)


def digest(args):
    """Per-launch HBM traffic of the main kernel from two rocprofv3 counter CSVs."""
    import csv
    import statistics

    def read(path, counter):
        per_kernel, calib = {}, []
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                per_kernel.setdefault(r["Kernel_Name"], []).append(v)
                if "copyBuffer" in r["Kernel_Name"]:
                    calib.append(v)
        # the calibration copy is the run's first device copy (pmc_run makes
        # it before building any input; later copies may be larger)
        return per_kernel, calib[0]

    fetch, f_copy = read(args.digest[0], "FETCH_SIZE")
    write, w_copy = read(args.digest[1], "WRITE_SIZE")
    f_scale = f_copy * 1024 / CALIB_BYTES
    w_scale = w_copy * 1024 / CALIB_BYTES
    mains = [k for k in fetch if any(n in k for n in KERNEL_SOURCES)]
    assert len(mains) == 1, f"main kernel not unique: {mains}"
    main = mains[0]
    name = next(n for n in KERNEL_SOURCES if n in main)
    fb = statistics.mean(fetch[main]) * 1024 / f_scale
    wb = statistics.mean(write[main]) * 1024 / w_scale
    srcs = KERNEL_SOURCES[name]
    out = {
        "kernel": name, "workload": args.workload, "dispatches": len(fetch[main]),
        "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
        "traffic_bytes_per_launch": fb + wb,
        "calibration": {"copy_bytes": CALIB_BYTES, "fetch_scale": f_scale, "write_scale": w_scale},
        "sources": srcs, "source_hash": source_hash(*srcs),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o run -- python3 bench.py "
            f"--pmc-run --workload {args.workload} --steps 4 --warmup 2",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o run -- python3 bench.py "
            f"--pmc-run --workload {args.workload} --steps 4 --warmup 2",
            f"python3 bench.py --workload {args.workload} --digest <dir_f>/run_counter_collection.csv "
            f"<dir_w>/run_counter_collection.csv"],
    }
    PROFILES.mkdir(exist_ok=True)
    f = PROFILES / f"{name}_{args.workload}_counters.json"
    f.write_text(json.dumps(out, indent=1) + "\n")
    print(json.dumps(out))


def oracle_row_inputs(setup, rows):
    """Host inputs of the oracle for (batch, query) rows of a bench workload,
    taken from the seeded generators, never from anything the library wrote:
    for each row, its query rows (all heads) as storage bits, a compact cache
    of its selected keys in order (the device cache's rows below past_len are
    the generator's; the appended rows are the current rows the step was
    given; fp8 records are made by the oracle's own quantizer from the bf16
    source rows) and the number of selected keys. An order-preserving
    relabelling of the selected keys leaves the forward's result unchanged,
    so the compact cache is indexed 0..n-1.
    Returns a list of dicts with q [Hq, Dk], k, v (None for shared latent)
    and n."""
    import numpy as np
    import torch

    import oracle
    w, W = setup.w, setup.W
    ih = setup.idx_host[0]

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    sels = []
    for (b, qi) in rows:
        sel = ih[b, 0, qi]
        sels.append(sel[sel >= 0].astype(np.int64))
    # source rows of the shared-latent cache / K and V, per requested row
    srcs_k, srcs_v = [], []
    if setup.fp8:
        # the past was drawn chunk by chunk; draw each needed chunk again
        need = {}
        for j, ((b, qi), sel) in enumerate(zip(rows, sels)):
            for c in np.unique(sel[sel < w.past] // setup.chunk):
                need.setdefault(int(c), []).append(j)
        parts = [dict() for _ in rows]
        for c, js in sorted(need.items()):
            t0 = c * setup.chunk
            n = min(setup.chunk, w.past - t0)
            chunk = setup.gen((w.batch, 1, n, w.dk), setup.chunk_seed(c))
            for j in js:
                b = rows[j][0]
                keys = sels[j]
                m = (keys >= t0) & (keys < t0 + n)
                parts[j][c] = (np.nonzero(m)[0],
                               bits(chunk[b, 0].index_select(0, torch.from_numpy(keys[m] - t0).cuda())))
            del chunk
        for j, ((b, qi), sel) in enumerate(zip(rows, sels)):
            out = np.empty((len(sel), w.dk), np.uint16)
            for pos, vals in parts[j].values():
                out[pos] = vals
            cur = sel >= w.past
            if cur.any():
                out[cur] = bits(setup.cur_k[b, 0].index_select(
                    0, torch.from_numpy(sel[cur] - w.past).cuda()))
            f32 = (out.astype(np.uint32) << 16).view(np.float32)
            srcs_k.append(oracle.fp8_pack_rows(f32, w.rope))
            srcs_v.append(None)
    else:
        for (b, qi), sel in zip(rows, sels):
            t = torch.from_numpy(sel).cuda()
            past = t < w.past
            tp = t.clamp(max=max(w.past - 1, 0))
            tc = (t - w.past).clamp(min=0)
            if w.layout == W.LAYOUT_SHARED_LATENT:
                r = setup.cur_k[b, 0].index_select(0, tc)
                if w.past > 0:
                    r = torch.where(past[:, None], setup.k[b, 0].index_select(0, tp), r)
                srcs_k.append(bits(r))
                srcs_v.append(None)
            else:
                k = torch.where(past[None, :, None], setup.k[b].index_select(1, tp),
                                setup.cur_k[b].index_select(1, tc))
                v = torch.where(past[None, :, None], setup.v[b].index_select(1, tp),
                                setup.cur_v[b].index_select(1, tc))
                srcs_k.append(bits(k))
                srcs_v.append(bits(v))
    out = []
    for j, ((b, qi), sel) in enumerate(zip(rows, sels)):
        out.append(dict(q=bits(setup.qs[0][b, :, qi]), k=srcs_k[j], v=srcs_v[j], n=len(sel)))
    return out


def oracle_row(setup, inp, threads):
    """The oracle's Y [Hq, Dv] (fp32) for one row built by oracle_row_inputs."""
    import numpy as np

    import oracle
    w, W = setup.w, setup.W
    q = inp["q"][None, :, None, :]
    if w.layout == W.LAYOUT_SHARED_LATENT:
        kc, vc = inp["k"][None, None], None
    else:
        kc, vc = inp["k"][None], inp["v"][None]
    ix = np.arange(inp["n"], dtype=np.int32)[None, None, None, :]
    fmt = oracle.FP8_BLOCK64 if setup.fp8 else w.dtype
    y = oracle.forward(q, kc, vc, ix, q_dtype=w.dtype, cache_fmt=fmt, kv_layout=w.layout,
                       hkv=w.hkv, dv=w.dv, rope=w.rope, scale=w.scale, softcap=w.softcap,
                       threads=threads)
    return y[0, :, 0, :]


def cpu_baseline(setup, target_s, threads=None):
    """The oracle (unchanged) on a bounded sample: the first rows of the same
    workload, each over a compact cache of its selected keys. Only the oracle
    calls are timed, not the input preparation."""
    w = setup.w
    threads = threads or cpu_threads()

    def run(nrows_b):
        rows = [(rb // w.q_seq, rb % w.q_seq) for rb in range(nrows_b)]
        inputs = oracle_row_inputs(setup, rows)
        n_total, t = 0, 0.0
        for inp in inputs:
            t0 = time.perf_counter()
            oracle_row(setup, inp, threads)
            t += time.perf_counter() - t0
            n_total += inp["n"]
        return n_total, t

    n1, t1 = run(1)
    total_rows = w.batch * w.q_seq
    nb = max(1, min(total_rows, int(target_s / max(t1, 1e-3))))
    n, t = run(nb) if nb > 1 else (n1, t1)
    reps = 1
    if nb == total_rows and t < target_s / 2:
        # the whole workload is shorter than the target: repeat it
        reps = max(1, int(target_s / max(t, 1e-3)))
        n, t = 0, 0.0
        for _ in range(reps):
            dn, dt = run(nb)
            n, t = n + dn, t + dt
    what = f"all {total_rows}" if nb == total_rows else f"first {nb} of {total_rows}"
    return {"value": n / t, "unit": "selected tokens/s", "cores": threads, "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{what} (batch, query) rows of the same workload x {reps}, all {w.hq} heads, "
                      f"{n} selected keys, {t:.1f} s of oracle time"}


def stats_file(setup):
    return PROFILES / f"{kernel_name(setup)}_{setup.name}_stats.md"


def stats_for(setup):
    """The main kernel's average duration in the committed rocprofv3 summary of
    this workload, if that summary was taken on the current kernel source."""
    f = stats_file(setup)
    if not f.exists():
        return None
    text = f.read_text()
    name = kernel_name(setup)
    if f"source hash: {source_hash(*KERNEL_SOURCES[name])}" not in text:
        return None
    best = None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 4 and name in cells[1]:
            calls, avg = int(cells[2]), float(cells[3])
            if best is None or calls > best[0]:
                best = (calls, avg)
    if best is None:
        return None
    return {"file": str(f.relative_to(ROOT)), "avg_us": best[1]}


def stats_digest(args):
    """A committed summary of a rocprofv3 --kernel-trace --stats run of this
    script (its kernel_stats.csv), with the source hash of the main kernel."""
    import csv
    s_name = args.workload
    rows = list(csv.DictReader(open(args.stats_digest)))
    mains = [r["Name"] for r in rows if any(n in r["Name"] for n in KERNEL_SOURCES)]
    assert mains, "no main kernel in the CSV"
    main = max((r for r in rows if r["Name"] in mains), key=lambda r: int(r["Calls"]))["Name"]
    name = next(n for n in KERNEL_SOURCES if n in main)
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py "
           f"--workload {s_name} --steps {args.steps} --warmup {args.warmup} --no-cpu-baseline --no-also")
    out = [f"# rocprofv3 kernel statistics: {s_name}", "",
           "Command (run from the repository root on one MI355X), then "
           f"`python3 bench.py --workload {s_name} --stats-digest <dir>/run_kernel_stats.csv`:", "",
           "```", cmd, "```", "",
           f"main kernel: `{name}`; sources {', '.join(KERNEL_SOURCES[name])}; "
           f"source hash: {source_hash(*KERNEL_SOURCES[name])}", "",
           "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        short = n.split("(")[0] if ("sa::" in n or "__amd" in n) else n.split("<")[0] + "<...>"
        out.append(f"| `{short[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    PROFILES.mkdir(exist_ok=True)
    f = PROFILES / f"{name}_{s_name}_stats.md"
    f.write_text("\n".join(out) + "\n")
    print(f"wrote {f}")


def measure(s, steps, warmup, use_graph, n_trials=0):
    """W warmup steps, then exactly `steps` steps between events: graph replays
    of one captured pass over the rotation sets (and one more graph of the
    remaining sets when `steps` is not a multiple of their number), then an
    eager pass of the same steps with the main kernel's dispatch-stamped
    events, then `n_trials` more timed trials of at least 200 replayed steps
    each. Returns (ms per step, main kernel seconds per launch, trials)."""
    torch = s.torch
    ok = getattr(s, "tolerated_bits", 0)
    for i in range(warmup):
        s.step(i)
    torch.cuda.synchronize()
    word, _, msg = s.ctx.read_error()
    assert word & ~ok == 0, msg
    nset = len(s.idxs)
    full, rem = divmod(steps, nset)
    graphs = {}
    if use_graph:
        for n in {nset if full else 0, rem} - {0}:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    s.step(i)
            graphs[n] = g
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if use_graph:
        for _ in range(full):
            graphs[nset].replay()
        if rem:
            graphs[rem].replay()
    else:
        for i in range(steps):
            s.step(i)
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / steps
    word, _, msg = s.ctx.read_error()
    assert word & ~ok == 0, msg
    s.ctx.profile_enable(steps)
    for i in range(steps):
        s.step(i)
    k_ms, k_n = s.ctx.profile_read()
    s.ctx.profile_enable(0)
    trials = None
    if use_graph and n_trials > 0:
        import statistics
        per = nset if nset in graphs else rem
        g = graphs[per]
        reps = max(1, -(-200 // per))
        ts = []
        for _ in range(n_trials):
            start.record()
            for _ in range(reps):
                g.replay()
            stop.record()
            torch.cuda.synchronize()
            ts.append(start.elapsed_time(stop) / (reps * per))
        word, _, msg = s.ctx.read_error()
        assert word & ~ok == 0, msg
        ts.sort()
        trials = {"n": n_trials, "steps_each": reps * per, "median_ms_per_step": statistics.median(ts),
                  "min_ms_per_step": ts[0], "max_ms_per_step": ts[-1]}
    return ms_per_step, k_ms / max(k_n, 1) / 1e3, trials


def measured_peaks(torch, sa, copy_bytes=1 << 30, reps=8):
    """The device's attainable HBM rate (a streaming copy, read + write bytes)
    and bf16 matrix-core rate (independent 16x16x32 products on every SIMD),
    each the best of `reps` timed launches after a warmup."""
    ctx = sa.Context(num_heads=16, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_F32)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(call):
        call()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) / 1e3)
        return min(t)

    src = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    t_copy = best(lambda: ctx.measure_copy(dst, src, copy_bytes))
    sink = torch.empty(sa.SA_PEAK_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    t_read = best(lambda: ctx.measure_read(sink, src, copy_bytes))
    del src, dst, sink
    wgs, iters = 256 * 8, 2048
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    t_mfma = best(lambda: ctx.measure_mfma(out, wgs, iters))
    ctx.destroy()
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": 2 * copy_bytes / t_copy / 1e9, "hbm_read_GBps": copy_bytes / t_read / 1e9,
            "mfma_bf16_TFLOPs": wgs * 4 * iters * 8 * 16384 / t_mfma / 1e12,
            "how": f"best of {reps}: streaming copy of {copy_bytes >> 20} MiB (read + write bytes), streaming "
                   f"read of the same; {wgs} workgroups x 4 waves x {iters} x 8 independent bf16 16x16x32 "
                   f"matrix-core products"}


def kernel_record(s, k_avg_s, peaks=None):
    kw = s.kernel_work()
    bound, peak, unit, achieved = s.roofline(kw, k_avg_s)
    rec = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
           "traffic": counters_for(s), "kernel": kernel_name(s), "kernel_avg_us": k_avg_s * 1e6,
           "algorithmic_bytes_per_launch": kw["bytes"], "algorithmic_flops_per_launch": kw["flops"]}
    if peaks:
        # the attention kernels' HBM bytes are almost all reads: the read rate is their ceiling
        mp = peaks["hbm_read_GBps"] if unit == "GB/s" else peaks["mfma_bf16_TFLOPs"] if unit == "TFLOP/s" else None
        if mp:
            rec["measured_peak"] = mp
            rec["frac_measured"] = achieved / mp
    prof = stats_for(s)
    if prof:
        _, _, _, a_prof = s.roofline(kw, prof["avg_us"] / 1e6)
        prof["frac"] = a_prof / peak
        rec["profile"] = prof
    return rec


def concat_append_figure(s, reps=5):
    """kv_append in concat mode over the workload's whole cache: the past copied
    into a fresh present plus the current rows, timed with events."""
    torch, w = s.torch, s.w
    if s.fp8 or w.layout != s.W.LAYOUT_SHARED_LATENT:
        return None
    B, cap = w.batch, w.cap
    past = s.k[:, :, :w.past]
    present = torch.empty_like(s.k)
    plen = torch.full((B,), w.past, dtype=torch.int32, device="cuda")
    vlen = torch.zeros((B,), dtype=torch.int32, device="cuda")
    call = lambda: s.ctx.kv_append(B, past, None, w.past, plen, s.cur_k, None, w.cur, present, None, cap,
                                   present_len=vlen)
    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    row = w.dk * 2
    nbytes = B * (w.past * row * 2 + w.cur * row * 2)   # past read + written, current read + written
    del present
    return {"what": f"kv_append concat: {B} x {w.past} past rows of {row} B copied into a fresh present "
                    f"+ {w.cur} current row", "bytes": nbytes, "us": us,
            "GBps": nbytes / (us / 1e6) / 1e9, "frac": nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS}


def c0_single_thread(target_s=1.0):
    """The oracle on the tiny fp32 workload (append + validation + forward), one
    thread, repeated until about target_s seconds."""
    import oracle
    import sa_workloads as W
    w = W.WORKLOADS["tiny_f32"]
    inp = W.make_numpy(w)
    n, t, reps = 0, 0.0, 0
    while t < target_s and reps < 100000:
        t0 = time.perf_counter()
        pk = oracle.kv_append(inp["past_k"].copy(), inp["past_len"], inp["cur_k"])
        pv = oracle.kv_append(inp["past_v"].copy(), inp["past_len"], inp["cur_v"])
        oracle.forward(inp["q"], pk, pv, inp["indices"], q_dtype=w.dtype, cache_fmt=w.dtype,
                       kv_layout=w.layout, hkv=w.hkv, dv=w.dv, scale=w.scale, softcap=w.softcap, threads=1)
        t += time.perf_counter() - t0
        n += int((inp["indices"] >= 0).sum())
        reps += 1
    return {"value": n / t, "unit": "selected tokens/s", "cores": 1, "workload": "tiny_f32",
            "sample": f"the whole tiny_f32 workload (append, forward) x {reps}, {n} selected keys, {t:.2f} s"}


def also_record(name, args, peaks=None):
    """Step time, main-kernel time, roofline and traffic of another workload, for
    the default line."""
    import torch
    s = make_setup(name, args.rotate)
    ms, k_avg, trials = measure(s, args.also_steps, 4, not args.no_graph, args.trials)
    rec = {"workload": name, "ms_per_step": ms, "steps": args.also_steps, "splits": s.splits,
           "trials": trials, "roofline": kernel_record(s, k_avg, peaks)}
    s.ctx.destroy()
    del s
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.digest:
        digest(args)
        return
    if args.stats_digest:
        stats_digest(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by batch with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.pmc_run:
        pmc_run(args)
        return
    print(f"bench: workload {args.workload}, building inputs", file=sys.stderr, flush=True)
    s = make_setup(args.workload, args.rotate)
    print(f"bench: path {kernel_name(s)} splits {s.splits}", file=sys.stderr, flush=True)
    use_graph = not args.no_graph
    steps = args.steps
    ms_per_step, k_avg_s, trials = measure(s, steps, args.warmup, use_graph, args.trials)
    peaks = None
    if not args.no_peaks:
        print("bench: measuring the copy and matrix-core peaks", file=sys.stderr, flush=True)
        peaks = measured_peaks(torch, s.sa)
    nset = len(s.idxs)
    tokens = s.tokens_per_step()
    result = {
        "metric": "selected KV tokens attended/sec (decode) + achieved HBM GB/s % of peak",
        "value": tokens / (ms_per_step / 1e3),
        "unit": {5: "candidates/s", 6: "records scored/s"}.get(s.path, "selected tokens/s"),
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype_name(),
        "data": "synthetic",
        "config": s.config(use_graph, nset, tokens, ms_per_step),
        "roofline": kernel_record(s, k_avg_s, peaks),
        "trials": trials,
        "peaks_measured": peaks,
    }
    if args.workload == "decode_bf16" and not args.no_also:
        print("bench: concat-append copy figure", file=sys.stderr, flush=True)
        result["concat_append"] = concat_append_figure(s)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cb = s.cpu_baseline(args.cpu_seconds)
        if isinstance(s, Setup) and not isinstance(s, CapacitySetup):
            one = s.cpu_baseline(max(2.0, args.cpu_seconds / 4), threads=1)
            cb["single_thread"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}
            cb["c0_single_thread"] = c0_single_thread()
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    s.ctx.destroy()
    del s
    torch.cuda.empty_cache()
    if args.workload == "decode_bf16" and not args.no_also:
        also = []
        for name in ("decode_fp8", "prefill_bf16"):
            print(f"bench: also {name}", file=sys.stderr, flush=True)
            also.append(also_record(name, args, peaks))
        result["also"] = also
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
