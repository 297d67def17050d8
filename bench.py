"""Benchmark of the HCA + MLA-DSA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one prefill pass of the hybrid layer pair over T = 32768 tokens:
  HCA layer (64 heads, d = 512, bf16):  hca_compress(K), hca_compress(V),
                                        hca_attention_fwd(PREFILL)
  MLA-DSA layer (64 query heads sharing one 256-wide KV head):
                                        dsa_indexer_topk(2048)
                                        -> dsa_sparse_attention_fwd
(dsa_indexer_topk writes the same indices as dsa_indexer_scores followed by
dsa_topk; the line also times that pair and checks the two agree.)
`value` is prefill tokens/s of that step (inputs resident in HBM).  The same
JSON line carries decode microseconds per step for the 128K context
(batch 64) and the 1M context (batch 4, HCA layer + MLA-DSA layer, whose
indices come from dsa_indexer_topk; the separate pair is timed beside it), per-kernel
times, the roofline of the dominant kernel, and the float64 CPU oracle timed
on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

T_PREFILL, H, D_HCA, BLK, WIN = 32768, 64, 512, 128, 128
HQ, D_DSA, HI, DI, TOPK = 64, 256, 4, 128, 2048
D_QK_WIDE = 576  # query/key width of the wider HCA head shape (value width stays D_HCA)
CSA_RATIO = 4  # CSA variant: indexer keys, K and V averaged over 4 tokens


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of parts: prefill,variants,decode128k,decode1m (default all; variants = the CSA layer "
                         "and the qk 576 / v 512 HCA head, run with prefill); "
                         "'copy' runs a plain 1 GiB device copy used to calibrate counter byte totals")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move / compute)
# ---------------------------------------------------------------------------


def hca_pairs_per_head(T, blk=BLK, window=WIN):
    """Sum over queries of (visible compressed entries + window tokens)."""
    tot = 0
    for t in range(T):
        tot += max(0, (t - window + 1) // blk) + min(window, t + 1)
    return tot


def dsa_pairs(T, k=TOPK):
    return sum(min(t + 1, k) for t in range(T))


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters):
        torch = self.torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        evs[0].record()
        for i in range(iters):
            fn()
            evs[i + 1].record()
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(iters)]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        print("bench.py: only --gpus 1 is supported (single-GPU build).", file=sys.stderr)
        return 2

    # The CPU baseline runs first, in a pool of forked single-threaded workers,
    # before anything initialises the GPU (a process that has touched the GPU is
    # not forked).
    parts0 = set(args.only.split(",")) if args.only else {"prefill"}
    cpu = None
    if not args.no_cpu_baseline and "prefill" in parts0:
        print("[bench] cpu baseline (float64 oracle, process pool)", file=sys.stderr, flush=True)
        cpu = cpu_baseline()

    import torch

    import sparse_attention_long_hca_amd as sa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    sa.lib()
    dev = "cuda:0"
    timer = Timer(torch)
    parts = set(args.only.split(",")) if args.only else {"prefill", "variants", "backward", "decode128k", "decode1m",
                                                          "tiny", "hbm"}
    result = {}
    kernels = {}
    if "copy" in parts:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return 0

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # -------------------------------------------------------------------
    # Measured HBM rate beside the 8 TB/s figure: a 2 GiB device copy
    # -------------------------------------------------------------------
    if "hbm" in parts:
        progress("HBM copy")
        n = 1 << 29  # 2 GiB of fp32
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        t_c = sorted(timer.time(lambda: b_.copy_(a), 10))[5]
        result["hbm_measured"] = {"copy_GBs": 2 * 4 * n / (t_c * 1e-3) / 1e9, "peak_GBs": HBM_PEAK_GBS,
                                  "note": "median of 10 device copies of 2 GiB (read + write bytes)"}
        del a, b_
        torch.cuda.empty_cache()

    # -------------------------------------------------------------------
    # Tiny HCA, fp32: T = 1024, 4 heads, d = 64, block 128, window 128
    # (compression of K and V, then attention), with a 512 MB scrub write
    # between runs so that no input is served from the caches
    # -------------------------------------------------------------------
    if "tiny" in parts:
        progress("tiny fp32 HCA")
        qt = synth.torch_normal((1, 4, 1024, 64), 1.0, torch.float32, 101, dev)
        kt = synth.torch_normal((1, 4, 1024, 64), 1.0, torch.float32, 102, dev)
        vt = synth.torch_normal((1, 4, 1024, 64), 1.0, torch.float32, 103, dev)
        kct = torch.empty((1, 4, 8, 64), dtype=torch.float32, device=dev)
        vct = torch.empty_like(kct)
        scrub = torch.empty(1 << 27, dtype=torch.float32, device=dev)  # 512 MB

        def tiny():
            sa.hca_compress(kt, BLK, out=kct)
            sa.hca_compress(vt, BLK, out=vct)
            return sa.hca_attention_fwd(sa.HCA_PREFILL, qt, kt, vt, kct, vct, BLK, WIN)

        tiny()
        times = []
        for _ in range(max(20, args.steps)):
            scrub.fill_(1.0)
            times += timer.time(tiny, 1)
        us = sorted(times)[len(times) // 2] * 1e3
        result["tiny_hca_f32"] = {"us": us, "workload": "HCA f32 T=1024, 4 heads, d=64, block 128, window 128: "
                                  "hca_compress(K), hca_compress(V), hca_attention_fwd(PREFILL); median of "
                                  f"{len(times)} runs, 512 MB scrub write between runs"}
        del qt, kt, vt, kct, vct, scrub
        torch.cuda.empty_cache()

    # -------------------------------------------------------------------
    # Prefill: HCA layer + MLA-DSA layer over T = 32768 tokens
    # -------------------------------------------------------------------
    if "prefill" in parts:
        progress("generating prefill inputs")
        sig = 1.0 / math.sqrt(D_HCA)
        q = synth.torch_normal((1, H, T_PREFILL, D_HCA), sig, torch.bfloat16, 201, dev)
        k = synth.torch_normal((1, H, T_PREFILL, D_HCA), sig, torch.bfloat16, 202, dev)
        v = synth.torch_normal((1, H, T_PREFILL, D_HCA), sig, torch.bfloat16, 203, dev)
        kc = torch.empty((1, H, T_PREFILL // BLK, D_HCA), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        qi = synth.torch_normal((1, T_PREFILL, HI, DI), DI ** -0.5, torch.bfloat16, 401, dev)
        ki = synth.torch_normal((1, T_PREFILL, DI), DI ** -0.5, torch.bfloat16, 402, dev)
        wi = synth.torch_uniform((1, T_PREFILL, HI), 403, dev)
        qd = synth.torch_normal((1, T_PREFILL, HQ, D_DSA), 1.0 / 16, torch.bfloat16, 404, dev)
        kd = synth.torch_normal((1, T_PREFILL, D_DSA), 1.0 / 16, torch.bfloat16, 405, dev)
        vd = synth.torch_normal((1, T_PREFILL, D_DSA), 1.0 / 16, torch.bfloat16, 406, dev)
        scores = torch.empty((1, T_PREFILL, T_PREFILL), dtype=torch.float32, device=dev)
        idx = torch.empty((1, T_PREFILL, TOPK), dtype=torch.int32, device=dev)
        idx_sep = torch.empty_like(idx)
        wsf = torch.empty(sa.dsa_indexer_topk_workspace_size(1, T_PREFILL, T_PREFILL, TOPK), dtype=torch.uint8,
                          device=dev)
        torch.cuda.synchronize()

        def k_compress():
            sa.hca_compress(k, BLK, out=kc)
            sa.hca_compress(v, BLK, out=vc)

        def k_hca():
            return sa.hca_attention_fwd(sa.HCA_PREFILL, q, k, v, kc, vc, BLK, WIN)

        def k_indexer():
            sa.dsa_indexer_scores(qi, ki, wi, out=scores)

        def k_topk():
            sa.dsa_topk(scores, TOPK, out=idx_sep)

        def k_indexer_topk():
            sa.dsa_indexer_topk(qi, ki, wi, TOPK, out=idx, workspace=wsf)

        def k_sparse():
            return sa.dsa_sparse_attention_fwd(qd, kd, vd, idx)

        def step():
            k_compress()
            k_hca()
            k_indexer_topk()
            k_sparse()

        progress("prefill warmup")
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        progress("prefill timed steps")
        t0 = time.perf_counter()
        ms = timer.time(step, args.steps)
        wall = time.perf_counter() - t0
        step_ms = sum(ms) / len(ms)
        result["prefill"] = {"ms_per_step": step_ms, "tokens_per_s": T_PREFILL / (step_ms * 1e-3), "wall_s": wall}

        progress("prefill per-kernel timing")
        n_it = max(3, args.steps)
        per = {
            "hca_compress_kv": (k_compress, None),
            "hca_attention_prefill": (k_hca, None),
            "dsa_indexer_topk": (k_indexer_topk, None),
            "dsa_sparse_attention": (k_sparse, None),
            "dsa_indexer_scores": (k_indexer, None),
            "dsa_topk": (k_topk, None),
        }
        for name, (fn, _) in per.items():
            fn()
            torch.cuda.synchronize()
            t = timer.time(fn, n_it)
            kernels[name] = {"ms": sum(t) / len(t)}
        kernels["dsa_indexer_topk"]["equals_separate"] = bool(torch.equal(idx, idx_sep))

        if "backward" in parts:
            # Backward of the DSA sparse attention over the step's selection (an extra
            # figure, not part of the step): upstream gradient N(0,1) bf16.
            progress("DSA backward")
            do_ = synth.torch_normal((1, T_PREFILL, HQ, D_DSA), 1.0, torch.bfloat16, 407, dev)
            o_f, lse_f = sa.dsa_sparse_attention_fwd(qd, kd, vd, idx, return_lse=True)
            wsb = torch.empty(sa.dsa_sparse_attention_bwd_workspace_size(1, T_PREFILL, T_PREFILL, TOPK),
                              dtype=torch.uint8, device=dev)

            def k_bwd():
                return sa.dsa_sparse_attention_bwd(qd, kd, vd, idx, o_f, lse_f, do_, workspace=wsb)

            k_bwd()
            torch.cuda.synchronize()
            t = timer.time(k_bwd, 2)
            ms_b = sum(t) / len(t)
            flop_b = 10 * D_DSA * dsa_pairs(T_PREFILL) * HQ
            result["dsa_sparse_attention_bwd"] = {
                "ms": ms_b, "alg_flop": flop_b, "TFLOPs": flop_b / (ms_b * 1e-3) / 1e12,
                "mfma_frac": flop_b / (ms_b * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                "workload": "dq, dk, dv of the MLA-DSA sparse attention, T=32768, top-2048, 64 heads x 256"}
            del do_, o_f, lse_f, wsb
            torch.cuda.empty_cache()

            # Backward of the HCA layer over the step's inputs (an extra figure, not part
            # of the step): dq, dk, dv through the window and the block mean, dk_c, dv_c.
            progress("HCA backward")
            k_compress()
            o_h, lse_h = sa.hca_attention_fwd(sa.HCA_PREFILL, q, k, v, kc, vc, BLK, WIN, return_lse=True)
            do_h = synth.torch_normal((1, H, T_PREFILL, D_HCA), 1.0, torch.bfloat16, 208, dev)
            wsh = torch.empty(sa.hca_attention_bwd_workspace_size(1, H, T_PREFILL, T_PREFILL // BLK, WIN),
                              dtype=torch.uint8, device=dev)

            def k_hbwd():
                return sa.hca_attention_bwd(q, k, v, kc, vc, o_h, lse_h, do_h, BLK, WIN, workspace=wsh)

            k_hbwd()
            torch.cuda.synchronize()
            t = timer.time(k_hbwd, max(3, args.steps))
            ms_h = sum(t) / len(t)
            flop_h = 10 * D_HCA * hca_pairs_per_head(T_PREFILL) * H
            bytes_h = T_PREFILL * H * D_HCA * (5 * 2 + 3 * 4) + 2 * (T_PREFILL // BLK) * H * D_HCA * (2 + 4)
            result["hca_attention_bwd"] = {
                "ms": ms_h, "alg_flop": flop_h, "TFLOPs": flop_h / (ms_h * 1e-3) / 1e12,
                "mfma_frac": flop_h / (ms_h * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, "alg_bytes": bytes_h,
                "hbm_frac": bytes_h / (ms_h * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "workload": "dq, dk, dv (window and block-mean paths), dk_c, dv_c of the HCA layer, T=32768, "
                            "64 heads x 512, block 128, window 128"}
            del o_h, lse_h, do_h, wsh
            torch.cuda.empty_cache()

        if "variants" in parts:
            # The CSA variant of the MLA layer over the same token-level inputs (an
            # extra figure, not part of the step): block-4 means of k_I, K and V,
            # then indexer, top-2048 and sparse attention over the 8192 entries.
            progress("CSA variant")
            S_c = T_PREFILL // CSA_RATIO
            kci = torch.empty((1, 1, S_c, DI), dtype=torch.bfloat16, device=dev)
            kcd = torch.empty((1, 1, S_c, D_DSA), dtype=torch.bfloat16, device=dev)
            vcd = torch.empty_like(kcd)
            sc_c = torch.empty((1, T_PREFILL, S_c), dtype=torch.float32, device=dev)
            idx_c = torch.empty((1, T_PREFILL, TOPK), dtype=torch.int32, device=dev)

            def csa_step():
                sa.hca_compress(ki[:, None], CSA_RATIO, out=kci)
                sa.hca_compress(kd[:, None], CSA_RATIO, out=kcd)
                sa.hca_compress(vd[:, None], CSA_RATIO, out=vcd)
                sa.csa_indexer_scores(qi, kci[:, 0], wi, CSA_RATIO, out=sc_c)
                sa.csa_topk(sc_c, TOPK, CSA_RATIO, out=idx_c)
                return sa.dsa_sparse_attention_fwd(qd, kcd[:, 0], vcd[:, 0], idx_c)

            for _ in range(args.warmup):
                csa_step()
            torch.cuda.synchronize()
            t_c = timer.time(csa_step, max(3, args.steps))
            ms_c = sum(t_c) / len(t_c)
            result["csa_prefill"] = {"ms_per_layer": ms_c, "tokens_per_s": T_PREFILL / (ms_c * 1e-3), "ratio": CSA_RATIO,
                                     "entries": S_c, "top_k": TOPK}
            del kci, kcd, vcd, sc_c, idx_c

            # HCA attention with the wider query/key head (qk 576, v 512) over the
            # same T = 32768, 64 heads (an extra figure, not part of the step).
            progress("HCA qk576/v512 variant")
            q6 = synth.torch_normal((1, H, T_PREFILL, D_QK_WIDE), sig, torch.bfloat16, 211, dev)
            k6 = synth.torch_normal((1, H, T_PREFILL, D_QK_WIDE), sig, torch.bfloat16, 212, dev)
            kc6 = sa.hca_compress(k6, BLK)

            def k_hca_wide():
                return sa.hca_attention_fwd(sa.HCA_PREFILL, q6, k6, v, kc6, vc, BLK, WIN)

            for _ in range(args.warmup):
                k_hca_wide()
            torch.cuda.synchronize()
            t_w = timer.time(k_hca_wide, max(3, args.steps))
            ms_w = sum(t_w) / len(t_w)
            pairs_w = hca_pairs_per_head(T_PREFILL) * H
            bytes_w = T_PREFILL * H * (2 * D_QK_WIDE + 2 * D_HCA) * 2
            flops_w = 2 * (D_QK_WIDE + D_HCA) * pairs_w
            result["hca_prefill_qk576_v512"] = {
                "ms": ms_w, "tokens_per_s": T_PREFILL / (ms_w * 1e-3), "alg_bytes": bytes_w, "alg_flops": flops_w,
                "hbm_frac": bytes_w / (ms_w * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "mfma_frac": flops_w / (ms_w * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
            del q6, k6, kc6

        pairs_hca = hca_pairs_per_head(T_PREFILL) * H
        pairs_dsa = dsa_pairs(T_PREFILL) * HQ
        tensor_bytes = T_PREFILL * H * D_HCA * 2
        kernels["hca_compress_kv"]["alg_bytes"] = 2 * tensor_bytes + 2 * (tensor_bytes // BLK)
        kernels["hca_attention_prefill"]["alg_bytes"] = 4 * tensor_bytes + 2 * (tensor_bytes // BLK)
        kernels["hca_attention_prefill"]["alg_flop"] = 4 * D_HCA * pairs_hca
        causal = T_PREFILL * (T_PREFILL + 1) // 2
        kernels["dsa_indexer_scores"]["alg_flop"] = 2 * HI * DI * causal
        kernels["dsa_indexer_scores"]["alg_bytes"] = 4 * causal + T_PREFILL * (HI * DI * 2 + DI * 2 + HI * 4)
        kernels["dsa_topk"]["alg_bytes"] = 4 * causal + 4 * T_PREFILL * TOPK
        kernels["dsa_indexer_topk"]["alg_flop"] = 2 * HI * DI * causal
        kernels["dsa_indexer_topk"]["alg_bytes"] = T_PREFILL * (HI * DI * 2 + DI * 2 + HI * 4) + 4 * T_PREFILL * TOPK
        kernels["dsa_sparse_attention"]["alg_flop"] = 4 * D_DSA * pairs_dsa
        kernels["dsa_sparse_attention"]["alg_bytes"] = 2 * T_PREFILL * HQ * D_DSA * 2 + 4 * T_PREFILL * TOPK + 2 * T_PREFILL * D_DSA * 2
        kernels["dsa_sparse_attention"]["gathered_bytes"] = pairs_dsa // HQ * D_DSA * 2 * 2
        for name, kd_ in kernels.items():
            s_ = kd_["ms"] * 1e-3
            if "alg_bytes" in kd_:
                kd_["hbm_GBs"] = kd_["alg_bytes"] / s_ / 1e9
                kd_["hbm_frac"] = kd_["hbm_GBs"] / HBM_PEAK_GBS
            if "alg_flop" in kd_:
                kd_["TFLOPs"] = kd_["alg_flop"] / s_ / 1e12
                kd_["mfma_frac"] = kd_["TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
        del q, k, v, kc, vc, qi, ki, wi, qd, kd, vd, scores, idx, idx_sep, wsf
        torch.cuda.empty_cache()

    # -------------------------------------------------------------------
    # Decode at 128K context, batch 64 (HCA layer)
    # -------------------------------------------------------------------
    if "decode128k" in parts:
        progress("generating 128K decode inputs")
        B3, NC3 = 64, 1024
        sig = 1.0 / math.sqrt(D_HCA)
        q3 = synth.torch_normal((B3, H, D_HCA), sig, torch.bfloat16, 301, dev)
        kc3 = synth.torch_normal((B3, H, NC3, D_HCA), sig, torch.bfloat16, 302, dev)
        vc3 = synth.torch_normal((B3, H, NC3, D_HCA), sig, torch.bfloat16, 303, dev)
        rk3 = synth.torch_normal((B3, H, WIN, D_HCA), sig, torch.bfloat16, 304, dev)
        rv3 = synth.torch_normal((B3, H, WIN, D_HCA), sig, torch.bfloat16, 305, dev)
        pos3 = torch.full((B3,), 131071, dtype=torch.int64, device=dev)
        ws3 = torch.empty(max(1, sa.hca_attention_workspace_size(sa.HCA_DECODE, q3, kc3, BLK, WIN)),
                          dtype=torch.uint8, device=dev)

        def dec3():
            return sa.hca_attention_fwd(sa.HCA_DECODE, q3, rk3, rv3, kc3, vc3, BLK, WIN, pos=pos3, workspace=ws3)

        for _ in range(args.warmup):
            dec3()
        torch.cuda.synchronize()
        t = timer.time(dec3, max(20, args.steps * 5))
        us = sorted(t)[len(t) // 2] * 1e3
        keys3 = (NC3 - 1) + WIN
        bytes3 = B3 * H * keys3 * 2 * D_HCA * 2 + 2 * B3 * H * D_HCA * 2
        result["decode_128k_b64"] = {"us_per_step": us, "alg_bytes": bytes3, "hbm_GBs": bytes3 / (us * 1e-6) / 1e9,
                                     "hbm_frac": bytes3 / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        kernels["hca_attention_decode_128k"] = {"ms": us * 1e-3, "alg_bytes": bytes3,
                                                "hbm_GBs": result["decode_128k_b64"]["hbm_GBs"],
                                                "hbm_frac": result["decode_128k_b64"]["hbm_frac"]}
        # The same step over an FP8 (E4M3) copy of the cache: an extra figure
        # beside the bf16 headline (one byte per element plus a 4-byte scale per row).
        enc3 = {n: sa.hca_quantize_fp8(t) for n, t in (("rk", rk3), ("rv", rv3), ("kc", kc3), ("vc", vc3))}
        ws3f = torch.empty(max(1, sa.hca_decode_fp8_workspace_size(q3, kc3, BLK, WIN)), dtype=torch.uint8, device=dev)

        def dec3f():
            return sa.hca_decode_fp8(q3, *enc3["rk"], *enc3["rv"], *enc3["kc"], *enc3["vc"], BLK, WIN, pos3,
                                     workspace=ws3f)

        for _ in range(args.warmup):
            dec3f()
        torch.cuda.synchronize()
        t = timer.time(dec3f, max(20, args.steps * 5))
        us_f = sorted(t)[len(t) // 2] * 1e3
        bytes3f = B3 * H * keys3 * 2 * (D_HCA + 4) + 2 * B3 * H * D_HCA * 2
        result["decode_128k_b64_fp8_cache"] = {"us_per_step": us_f, "alg_bytes": bytes3f,
                                               "hbm_GBs": bytes3f / (us_f * 1e-6) / 1e9,
                                               "hbm_frac": bytes3f / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del q3, kc3, vc3, rk3, rv3, ws3, enc3, ws3f
        torch.cuda.empty_cache()

    # -------------------------------------------------------------------
    # Decode at 1M context, batch 4: HCA layer + MLA-DSA layer
    # -------------------------------------------------------------------
    if "decode1m" in parts:
        progress("generating 1M decode inputs")
        B5, L5 = 4, 1 << 20
        NC5 = L5 // BLK
        sig = 1.0 / math.sqrt(D_HCA)
        q5 = synth.torch_normal((B5, H, D_HCA), sig, torch.bfloat16, 501, dev)
        kc5 = synth.torch_normal((B5, H, NC5, D_HCA), sig, torch.bfloat16, 502, dev)
        vc5 = synth.torch_normal((B5, H, NC5, D_HCA), sig, torch.bfloat16, 503, dev)
        rk5 = synth.torch_normal((B5, H, WIN, D_HCA), sig, torch.bfloat16, 504, dev)
        rv5 = synth.torch_normal((B5, H, WIN, D_HCA), sig, torch.bfloat16, 505, dev)
        pos5 = torch.full((B5,), L5 - 1, dtype=torch.int64, device=dev)
        ws5 = torch.empty(max(1, sa.hca_attention_workspace_size(sa.HCA_DECODE, q5, kc5, BLK, WIN)),
                          dtype=torch.uint8, device=dev)
        qi5 = synth.torch_normal((B5, 1, HI, DI), DI ** -0.5, torch.bfloat16, 506, dev)
        ki5 = synth.torch_normal((B5, L5, DI), DI ** -0.5, torch.bfloat16, 507, dev)
        wi5 = synth.torch_uniform((B5, 1, HI), 508, dev)
        qd5 = synth.torch_normal((B5, 1, HQ, D_DSA), 1.0 / 16, torch.bfloat16, 509, dev)
        kd5 = synth.torch_normal((B5, L5, D_DSA), 1.0 / 16, torch.bfloat16, 510, dev)
        vd5 = synth.torch_normal((B5, L5, D_DSA), 1.0 / 16, torch.bfloat16, 511, dev)
        qpos5 = torch.full((B5,), L5 - 1, dtype=torch.int64, device=dev)
        sc5 = torch.empty((B5, 1, L5), dtype=torch.float32, device=dev)
        idx5 = torch.empty((B5, 1, TOPK), dtype=torch.int32, device=dev)
        idx5s = torch.empty_like(idx5)
        wst5 = torch.empty(max(1, sa.dsa_topk_workspace_size(B5, 1, L5, TOPK)), dtype=torch.uint8, device=dev)
        wsf5 = torch.empty(sa.dsa_indexer_topk_workspace_size(B5, 1, L5, TOPK), dtype=torch.uint8, device=dev)
        wss5 = torch.empty(max(1, sa.dsa_sparse_attention_fwd_workspace_size(B5, 1, HQ, D_DSA, TOPK)),
                           dtype=torch.uint8, device=dev)

        def hca5():
            return sa.hca_attention_fwd(sa.HCA_DECODE, q5, rk5, rv5, kc5, vc5, BLK, WIN, pos=pos5, workspace=ws5)

        def dsa5():
            sa.dsa_indexer_topk(qi5, ki5, wi5, TOPK, q_pos=qpos5, out=idx5, workspace=wsf5)
            return sa.dsa_sparse_attention_fwd(qd5, kd5, vd5, idx5, workspace=wss5)

        def dsa5_separate():
            sa.dsa_indexer_scores(qi5, ki5, wi5, q_pos=qpos5, out=sc5)
            sa.dsa_topk(sc5, TOPK, q_pos=qpos5, out=idx5s, workspace=wst5)
            return sa.dsa_sparse_attention_fwd(qd5, kd5, vd5, idx5s, workspace=wss5)

        for _ in range(args.warmup):
            hca5()
            dsa5()
            dsa5_separate()
        torch.cuda.synchronize()
        n_it = max(20, args.steps * 5)
        t_h = sorted(timer.time(hca5, n_it))[n_it // 2] * 1e3
        t_d = sorted(timer.time(dsa5, n_it))[n_it // 2] * 1e3
        t_ds = sorted(timer.time(dsa5_separate, n_it))[n_it // 2] * 1e3
        keys5 = (NC5 - 1) + WIN
        b_h = B5 * H * keys5 * 2 * D_HCA * 2
        # indexer keys read once, the selected K and V rows gathered (the fused call
        # writes no score row)
        b_d = B5 * L5 * DI * 2 + B5 * TOPK * 2 * D_DSA * 2
        result["decode_1m_b4"] = {
            "us_per_step": t_h + t_d,
            "hca_us": t_h,
            "dsa_us": t_d,
            "hca_hbm_frac": b_h / (t_h * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "dsa_hbm_frac": b_d / (t_d * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "dsa_separate_us": t_ds,
            "indices_equal_separate": bool(torch.equal(idx5, idx5s)),
        }
        del q5, kc5, vc5, rk5, rv5, ws5, qi5, ki5, wi5, qd5, kd5, vd5, sc5, idx5, idx5s, wst5, wsf5, wss5
        torch.cuda.empty_cache()

    # -------------------------------------------------------------------
    # Roofline of the dominant prefill kernel
    # -------------------------------------------------------------------
    roofline = None
    if "prefill" in result:
        pk = {n: kernels[n] for n in ("hca_compress_kv", "hca_attention_prefill", "dsa_indexer_topk",
                                      "dsa_sparse_attention")}
        dom = max(pk, key=lambda n: pk[n]["ms"])
        kd_ = pk[dom]
        if "alg_flop" in kd_ and dom in ("dsa_sparse_attention",):
            roofline = {"kernel": dom, "bound": "mfma", "achieved": kd_["TFLOPs"], "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": kd_["mfma_frac"]}
        else:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": kd_["hbm_GBs"], "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": kd_["hbm_frac"]}
        roofline["traffic"] = traffic_for(dom)

    step_ms = result.get("prefill", {}).get("ms_per_step")
    line = {
        "metric": "HCA/DSA prefill tokens/s + decode us/step at 128K; % of MFMA/HBM peak",
        "value": result.get("prefill", {}).get("tokens_per_s"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(d) bf16 inputs; indexer weights U(0,1) fp32)",
        "config": {
            "workload": "hybrid prefill: HCA layer (T=32768, 64 heads, d=512, block 128, window 128) + "
                        "MLA-DSA layer (T=32768, indexer 4x128, top-2048, 64 query heads x d=256 MQA)",
            "global_batch": 1,
            "seq_len": T_PREFILL,
            "parallelism": "single GPU",
        },
        "decode": {k_: v_ for k_, v_ in result.items() if k_.startswith("decode")},
        "tiny_hca_f32": result.get("tiny_hca_f32"),
        "hbm_measured": result.get("hbm_measured"),
        "variants": {k_: v_ for k_, v_ in result.items() if k_.startswith(("csa", "hca_prefill_qk576"))},
        "backward": {k_: v_ for k_, v_ in result.items() if k_.endswith("_bwd")},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line, default=float))
    return 0


def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel)
    if not ent:
        return None
    if ent.get("source_hash") != source_hash(ent.get("sources", [])):
        return None
    return ent.get("bytes_per_launch")


_CPU = {}


def _cpu_hca_rows(rows):
    import oracle

    c = _CPU
    t0 = time.perf_counter()
    oracle.hca_attention_prefill(c["q"], c["k"], c["v"], c["kc"], c["vc"], BLK, WIN, rows=rows)
    return time.perf_counter() - t0


def _cpu_dsa_rows(rs):
    import oracle

    c = _CPU
    t0 = time.perf_counter()
    for r in rs:
        p = c["pos"][r]
        sc = oracle.dsa_indexer_scores(c["qi"][:, r:r + 1], c["ki"], c["w"][:, r:r + 1], q_pos=[p])
        idx = oracle.dsa_topk(sc, TOPK, q_pos=[p])
        oracle.dsa_sparse_attention(c["qd"][:, r:r + 1], c["kd"], c["vd"], idx)
    return time.perf_counter() - t0


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)  # one thread per worker: the pool size is the core count used


def cpu_baseline():
    """Time the float64 oracle on a bounded sample of the prefill workload on the host's cores: a pool of
    forked single-threaded workers, one per core (at most 16, the machine's CPU share), splits the query rows.
    Must run before anything initialises the GPU (the workers are forked)."""
    import multiprocessing as mp

    import numpy as np

    import oracle
    import synth

    cores = min(16, len(os.sched_getaffinity(0)))
    g = np.random.default_rng(7)
    # HCA: 4 heads of the 32768 x 512 prefill.  Compression is a per-token cost
    # over all T tokens; attention is timed on query rows spread over T.
    hs, rows = 4, list(np.linspace(0, T_PREFILL - 1, 1024 * cores).astype(int))
    sig = 1.0 / math.sqrt(D_HCA)
    c = _CPU
    c["q"] = synth.np_normal((1, hs, T_PREFILL, D_HCA), sig, "bf16", 901, 0)
    c["k"] = synth.np_normal((1, hs, T_PREFILL, D_HCA), sig, "bf16", 901, 1)
    c["v"] = synth.np_normal((1, hs, T_PREFILL, D_HCA), sig, "bf16", 901, 2)
    t0 = time.perf_counter()
    c["kc"], c["vc"] = oracle.hca_compress(c["k"], BLK), oracle.hca_compress(c["v"], BLK)
    t_comp = time.perf_counter() - t0
    # MLA-DSA: query rows at positions >= 2048 (indexer over the prefix, top-2048, 64-head attention).
    S, nq = T_PREFILL, 48 * cores
    c["qi"] = synth.np_normal((1, nq, HI, DI), DI ** -0.5, "bf16", 902, 0)
    c["ki"] = synth.np_normal((1, S, DI), DI ** -0.5, "bf16", 902, 1)
    c["w"] = synth.np_uniform((1, nq, HI), 902, 2)
    c["qd"] = synth.np_normal((1, nq, HQ, D_DSA), 1.0 / 16, "bf16", 902, 3)
    c["kd"] = synth.np_normal((1, S, D_DSA), 1.0 / 16, "bf16", 902, 4)
    c["vd"] = synth.np_normal((1, S, D_DSA), 1.0 / 16, "bf16", 902, 5)
    c["pos"] = [int(x) for x in g.integers(TOPK, S, size=nq)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        t0 = time.perf_counter()
        busy_h = sum(pool.map(_cpu_hca_rows, [rows[i::cores] for i in range(cores)]))
        t_att = time.perf_counter() - t0
        t0 = time.perf_counter()
        busy_d = sum(pool.map(_cpu_dsa_rows, [list(range(i, nq, cores)) for i in range(cores)]))
        t_dsa = time.perf_counter() - t0
    hca_s_per_token = (t_comp / T_PREFILL + t_att / len(rows)) * (H / hs)
    dsa_s_per_token = t_dsa / nq
    per_token = hca_s_per_token + dsa_s_per_token
    _CPU.clear()
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{cores} single-threaded worker processes. HCA: {hs} of 64 heads of the T=32768 d=512 prefill: "
                  f"block-mean compression of all 32768 tokens (one process, {t_comp:.1f} s) + attention for "
                  f"{len(rows)} query rows ({t_att:.1f} s wall, {busy_h:.1f} s of worker time), per-token cost "
                  f"scaled x{H // hs} to 64 heads; MLA-DSA: {nq} query rows at positions >= 2048 (indexer over the "
                  f"causal prefix, top-2048, 64-head attention; {t_dsa:.1f} s wall, {busy_d:.1f} s of worker time)",
        "seconds": t_comp + t_att + t_dsa,
    }


if __name__ == "__main__":
    sys.exit(main())
