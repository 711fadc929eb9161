"""Benchmark of the block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config hunyuan720]

One step = the whole hot path on one batch of synthetic input already resident
in HBM: block mean pooling of Q and K, reduced attention + CDF selection (the
mask stage), then the block-sparse attention forward. Prints ONE JSON line.
The headline workload is the 118,800-token 720p layer at ~90 % block sparsity
(24 heads, d 128, thr 0.1); the 32,760-token 480p layer follows under "also"
with the same step and warm-up counts and its own roofline.

  value      effective TFLOP/s of the whole step: F_eff / step time, where
             F_eff = 4 * d * sum over kept (query block I, key block J) of
             len_I * len_J (QK^T and PV of kept tiles only, padding excluded)
  roofline   the attention kernel (the dominant one) against the bf16 dense
             MFMA peak of MI355X (2516.6 TFLOP/s), timed with HIP events on
             the stream the library launches on; traffic = calibrated HBM
             bytes per launch from the committed counter summary of that
             kernel (null once its source changed)
  cpu_baseline  the float64 CPU reference timed on a bounded sample of the
             same workload and extrapolated to one step (the 480p layer under
             "also": the whole step, not extrapolated)

Beside the step, on the same inputs (each switchable off):
  backward   forward with row normalisers + dQ/dK/dV over the step's lists
  paths      the reorder-based layouts on the 480p layer (fractal patches +
             window with its backward, per-head box tilings, semantic
             clusters), mask reuse and warm-started k-means at a drifted next
             step, and the mask's recall against the full attention
  cold_cache the step with Q, K, V flushed from the caches
  mfma_probe / dense_gemm_ref  what the MFMA pipe and the vendor GEMM reach
             on the same box (context for the roofline fraction)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_attention_avg_amd as bsa  # noqa: E402
from gen import WORKLOADS, generate  # noqa: E402

METRIC = "block-sparse attn effective TFLOP/s & % bf16 MFMA peak at ~90% sparsity"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def describe(w) -> str:
    return (f"{w.key}: B{w.B} H{w.H} d{w.d} N{w.N} ({w.T}x{w.Hl}x{w.Wl} latent, "
            f"{w.n_valid} tokens), block {w.block}, thr {w.thr}")


def block_lengths(w):
    nb = -(-w.n_valid // w.block)
    ln = np.full(nb, w.block, dtype=np.int64)
    ln[-1] = w.n_valid - w.block * (nb - 1)
    return ln


def effective_flops(w, cnt: np.ndarray, idx: np.ndarray):
    """F_eff and block / token-pair sparsity from the kept lists."""
    ln = block_lengths(w)
    nb = len(ln)
    rows_c = cnt.reshape(-1, nb)
    rows_i = idx.reshape(-1, nb, idx.shape[-1])
    stride = idx.shape[-1]
    col = np.arange(stride)[None, None, :]
    valid = col < rows_c[:, :, None]
    klen = np.where(valid, ln[np.clip(rows_i, 0, nb - 1)], 0).sum(-1)     # [BH, nqb]
    flops = 4.0 * w.d * float((klen * ln[None, :]).sum())
    kept = float(rows_c.sum())
    total = rows_c.shape[0] * nb * nb
    pair_total = rows_c.shape[0] * float(ln.sum()) ** 2
    return flops, 1.0 - kept / total, 1.0 - float((klen * ln[None, :]).sum()) / pair_total


class Runner:
    """Holds device inputs and preallocated outputs for one workload."""

    def __init__(self, w, dev):
        self.w = w
        q, k, v = generate(w)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.q_cpu, self.k_cpu, self.v_cpu = q, k, v
        nb = -(-w.n_valid // w.block)
        self.nb = nb
        self.cnt = torch.empty((w.B, w.H, nb), dtype=torch.int32, device=dev)
        self.idx = torch.empty((w.B, w.H, nb, nb), dtype=torch.int32, device=dev)
        self.o = torch.empty_like(self.q)
        lib = bsa.load()
        self.ws = torch.empty(lib.bsa_build_block_mask_workspace(w.B, w.H, nb, nb, w.d),
                              dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(lib.bsa_block_sparse_attn_fwd_workspace(w.B, w.H, nb, None),
                                   dtype=torch.uint8, device=dev)

    def mask(self):
        bsa.build_block_mask(self.q, self.k, self.w.thr, n_valid=self.w.n_valid,
                             out=(self.cnt, self.idx), workspace=self.ws)

    def attn(self):
        bsa.block_sparse_attn_fwd(self.q, self.k, self.v, self.cnt, self.idx,
                                  n_valid=self.w.n_valid, out=self.o, workspace=self.ws_attn)

    def step(self):
        self.mask()
        self.attn()

    def timed(self, steps: int, warmup: int, min_warm_s: float = 1.0):
        # at least `warmup` steps and at least min_warm_s of GPU work, so the
        # clocks have left their idle state before the timed steps
        t0 = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t0 < min_warm_s:
            self.step()
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for e in evs:
            e[0].record()
            self.mask()
            e[1].record()
            self.attn()
            e[2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.attn_each = [e[1].elapsed_time(e[2]) for e in evs]
        t_mask = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        t_attn = sum(self.attn_each) / steps
        return wall / steps * 1e3, t_mask, t_attn

    def backward(self, steps: int, warmup: int = 3):
        """Mean times of the forward-with-lse and the backward on this step's
        lists (upstream gradient: seeded Gaussian)."""
        g = torch.randn(self.q.shape, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
        g = g.to(self.q.device)
        self.mask()
        o, lse = bsa.block_sparse_attn_fwd_lse(self.q, self.k, self.v, self.cnt, self.idx, n_valid=self.w.n_valid)
        grads = tuple(torch.empty_like(self.q) for _ in range(3))
        lib = bsa.load()
        ws = torch.empty(lib.bsa_block_sparse_attn_bwd_workspace(self.w.B, self.w.H, self.w.N, None, None),
                         dtype=torch.uint8, device=self.q.device)

        def fwd():
            bsa.block_sparse_attn_fwd_lse(self.q, self.k, self.v, self.cnt, self.idx, n_valid=self.w.n_valid,
                                          out=o, lse=lse, workspace=self.ws_attn)

        def bwd():
            bsa.block_sparse_attn_bwd(self.q, self.k, self.v, o, g, lse, self.cnt, self.idx,
                                      n_valid=self.w.n_valid, out=grads, workspace=ws)

        for _ in range(warmup):
            fwd()
            bwd()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in evs:
            e[0].record()
            fwd()
            e[1].record()
            bwd()
            e[2].record()
        torch.cuda.synchronize()
        t_f = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        t_b = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        return t_f, t_b

    def cold(self, reps: int, scratch_mib: int = 512):
        """Median mask / attention times with the caches flushed before each step.

        A scratch buffer larger than the 256 MB Infinity Cache is overwritten
        before every step (outside the timed events), so Q, K, V come from HBM.
        """
        scratch = torch.empty(scratch_mib << 20, dtype=torch.uint8, device=self.q.device)
        tm, ta = [], []
        for _ in range(reps):
            scratch.fill_(1)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            self.mask()
            e[1].record()
            self.attn()
            e[2].record()
            torch.cuda.synchronize()
            tm.append(e[0].elapsed_time(e[1]))
            ta.append(e[1].elapsed_time(e[2]))
        del scratch
        return float(np.median(tm)), float(np.median(ta))

    def summary(self, ms_step, t_mask, t_attn):
        w = self.w
        cnt = self.cnt.cpu().numpy()
        idx = self.idx.cpu().numpy()
        flops, sp_block, sp_pair = effective_flops(w, cnt, idx)
        attn_tflops = flops / (t_attn * 1e-3) / 1e12
        qk_bytes = 2.0 * w.B * w.H * w.N * w.d * 2
        mask_bytes = qk_bytes + cnt.nbytes + 4.0 * float(cnt.sum())
        return {
            "flops_eff": flops,
            "step_tflops": flops / (ms_step * 1e-3) / 1e12,
            "attn_tflops": attn_tflops,
            "attn_frac_of_peak": attn_tflops / PEAK_BF16_TFLOPS,
            "t_mask_ms": t_mask,
            "t_attn_ms": t_attn,
            "mask_over_attn": t_mask / t_attn,
            "mask_gbs": mask_bytes / (t_mask * 1e-3) / 1e9,
            "mask_frac_of_hbm": mask_bytes / (t_mask * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "sparsity_blocks": sp_block,
            "sparsity_token_pairs": sp_pair,
            "kept_per_row_mean": float(cnt.mean()),
            "kept_per_row_max": int(cnt.max()),
        }


def _var_flops(d, cnt, idx, lq, lk):
    """F_eff over variable blocks: 4 d sum_I len_I sum_{J kept} len_J (device tensors)."""
    valid = torch.arange(idx.shape[-1], device=idx.device) < cnt[..., None].long()
    lk = lk.long().expand(*cnt.shape[:2], lk.shape[-1]) if lk.dim() == 1 else lk.long()
    lq = lq.long().expand(*cnt.shape) if lq.dim() == 1 else lq.long()
    kl = torch.gather(lk, 2, idx.long().clamp(0, lk.shape[-1] - 1).flatten(2)).view(idx.shape)
    kl = torch.where(valid, kl, torch.zeros_like(kl)).sum(-1)
    return 4.0 * d * float((kl * lq).sum())


def paths_bench(r: Runner, steps: int = 10, warmup: int = 3):
    """Stage times (HIP events, means over `steps`) of the reorder-based paths on
    the 480p layer: fractal + window, per-head box tilings, semantic clusters."""
    import block_sparse_attention_avg_amd.pipelines as pl
    from gen import kmeans_uniforms
    w = r.w
    dev = r.q.device
    q, k, v = r.q, r.k, r.v
    out = {}

    def run(stages):
        for _ in range(warmup):
            for _, f in stages:
                f()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
        for e in ev:
            e[0].record()
            for i, (_, f) in enumerate(stages):
                f()
                e[i + 1].record()
        torch.cuda.synchronize()
        t = {name: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / steps for i, (name, _) in enumerate(stages)}
        t["total"] = sum(e[0].elapsed_time(e[-1]) for e in ev) / steps
        return {k2: round(v2, 4) for k2, v2 in t.items()}

    def reorder_path(key, perm, blocks, window):
        st = {}
        buf = [torch.empty_like(q) for _ in range(4)]
        nb = blocks.nblocks
        cnt = torch.empty((w.B, w.H, nb), dtype=torch.int32, device=dev)
        idx = torch.empty((w.B, w.H, nb, nb), dtype=torch.int32, device=dev)

        def permute():
            bsa.permute_tokens(q, perm, out=buf[0])
            bsa.permute_tokens(k, perm, out=buf[1])
            bsa.permute_tokens(v, perm, out=buf[2])

        def mask():
            bsa.build_block_mask(buf[0], buf[1], w.thr, window=window, n_valid=w.n_valid, qb=blocks, kb=blocks,
                                 out=(cnt, idx))

        def attn():
            bsa.block_sparse_attn_fwd(buf[0], buf[1], buf[2], cnt, idx, n_valid=w.n_valid, qb=blocks, kb=blocks,
                                      out=buf[3])

        def unpermute():
            bsa.unpermute_tokens(buf[3], perm, out=r.o)
        st = run([("permute_qkv", permute), ("mask", mask), ("attention", attn), ("unpermute_o", unpermute)])
        f = _var_flops(w.d, cnt, idx, blocks.length, blocks.length)
        st["attn_tflops"] = round(f / (st["attention"] * 1e-3) / 1e12, 3)
        st["step_tflops"] = round(f / (st["total"] * 1e-3) / 1e12, 3)
        st["kept_blocks"] = int(cnt.sum())
        if blocks.max_len:
            # the backward over the same lists and blocks (seeded upstream gradient)
            g = torch.randn(q.shape, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(dev)
            o_l = [None, None]

            def fwd_lse():
                o_l[0], o_l[1] = bsa.block_sparse_attn_fwd_lse(buf[0], buf[1], buf[2], cnt, idx, n_valid=w.n_valid,
                                                               qb=blocks, kb=blocks)

            def bwd():
                bsa.block_sparse_attn_bwd(buf[0], buf[1], buf[2], o_l[0], g, o_l[1], cnt, idx, n_valid=w.n_valid,
                                          qb=blocks, kb=blocks)
            tb = run([("fwd_lse", fwd_lse), ("backward", bwd)])
            st["backward_ms"] = tb["backward"]
            st["backward_tflops_eff"] = round(2.5 * f / (tb["backward"] * 1e-3) / 1e12, 3)
        out[key] = st

    wf = WORKLOADS["wan480_fractal_sta"]
    lay = pl.fractal_layout(wf.T, wf.Hl, wf.Wl, wf.patch, wf.N, dev)
    reorder_path("fractal_sta", lay.perm, lay.blocks, (*lay.grid, *wf.window))
    wh = WORKLOADS["wan480_head_tiling"]
    factors = [wh.tilings[h % len(wh.tilings)] for h in range(wh.H)]
    ht = pl.head_tiling_layout(wh.T, wh.Hl, wh.Wl, factors, wh.N, wh.B, dev)
    reorder_path("head_tiling", ht.perm, ht.blocks, None)
    out["head_tiling"]["factors"] = sorted(set(factors))

    ws = WORKLOADS["wan480_semantic"]
    uq = torch.from_numpy(kmeans_uniforms(ws.B, ws.H, ws.Cq, stream=0)).to(dev)
    uk = torch.from_numpy(kmeans_uniforms(ws.B, ws.H, ws.Ck, stream=1)).to(dev)
    S = {}

    def km():
        S["cq"], S["aq"], S["nq"] = bsa.kmeans(q, ws.Cq, ws.kmeans_iters, uq, ws.n_valid)
        S["ck"], S["ak"], S["nk"] = bsa.kmeans(k, ws.Ck, ws.kmeans_iters, uk, ws.n_valid)

    def order():
        S["pq"], S["sq"], S["lq"] = bsa.cluster_order(S["aq"], ws.Cq, ws.n_valid)
        S["pk"], S["sk"], S["lk"] = bsa.cluster_order(S["ak"], ws.Ck, ws.n_valid)

    def permute():
        S["qp"] = bsa.permute_tokens(q, S["pq"])
        S["kp"] = bsa.permute_tokens(k, S["pk"])
        S["vp"] = bsa.permute_tokens(v, S["pk"])

    def mask():
        S["cnt"], S["idx"] = bsa.build_centroid_mask(S["cq"], S["nq"], S["ck"], S["nk"], ws.top_p)

    def attn():
        S["op"] = bsa.block_sparse_attn_fwd(S["qp"], S["kp"], S["vp"], S["cnt"], S["idx"], n_valid=ws.n_valid,
                                            qb=bsa.Blocks(S["sq"], S["lq"]), kb=bsa.Blocks(S["sk"], S["lk"]))

    def unpermute():
        bsa.unpermute_tokens(S["op"], S["pq"], out=r.o)
    st = run([("kmeans_qk", km), ("cluster_order", order), ("permute_qkv", permute), ("mask", mask),
              ("attention", attn), ("unpermute_o", unpermute)])
    f = _var_flops(ws.d, S["cnt"], S["idx"], S["lq"], S["lk"])
    st["attn_tflops"] = round(f / (st["attention"] * 1e-3) / 1e12, 3)
    st["step_tflops"] = round(f / (st["total"] * 1e-3) / 1e12, 3)
    st["kept_blocks"] = int(S["cnt"].sum())
    st["clusters"] = [ws.Cq, ws.Ck]
    st["kmeans_iters"] = ws.kmeans_iters
    out["semantic"] = st

    # the next denoising step: k-means warm-started from this step's centroids
    from gen import next_step
    q1 = next_step(r.q_cpu, 1, stream=0).to(dev)
    k1 = next_step(r.k_cpu, 1, stream=1).to(dev)
    cq0, ck0 = S["cq"], S["ck"]
    cap = 100
    tol = ws.n_valid // 100                     # stop once a round moves <= 1 % of the tokens

    def rounds(ch):
        c = ch.reshape(-1, ch.shape[-1]).cpu().numpy()
        rr = [int(np.argmax(x <= tol)) + 1 if (x <= tol).any() else ch.shape[-1] for x in c]
        return {"mean": round(float(np.mean(rr)), 2), "max": int(np.max(rr))}

    def warm():
        S["wq"] = bsa.kmeans_warm(q1, cq0, cap, ws.n_valid, tol)
        S["wk"] = bsa.kmeans_warm(k1, ck0, cap, ws.n_valid, tol)
    tw = run([("kmeans_qk_warm", warm)])
    # cold start on the same step, run to convergence: seeding, then Lloyd
    # rounds from the seeds until no token moves
    sq0, _, _ = bsa.kmeans(q1, ws.Cq, 0, uq, ws.n_valid)
    sk0, _, _ = bsa.kmeans(k1, ws.Ck, 0, uk, ws.n_valid)

    def cold():
        bsa.kmeans(q1, ws.Cq, 0, uq, ws.n_valid)
        bsa.kmeans(k1, ws.Ck, 0, uk, ws.n_valid)
        S["cq1"] = bsa.kmeans_warm(q1, sq0, cap, ws.n_valid, tol)
        S["ck1"] = bsa.kmeans_warm(k1, sk0, cap, ws.n_valid, tol)
    tc = run([("kmeans_qk_cold", cold)])
    # reuse of the raster mask across that step: the lists built at step 0
    # applied at step 1, against the lists built at step 1
    v1 = next_step(r.v_cpu, 1, stream=2).to(dev)
    c0m, i0m = bsa.build_block_mask(q, k, w.thr, n_valid=w.n_valid)
    c1m, i1m = bsa.build_block_mask(q1, k1, w.thr, n_valid=w.n_valid)
    nb = c0m.shape[-1]

    def dense(c, i):
        # entries past each row's count go to a spare last column
        m = torch.zeros((*c.shape, nb + 1), dtype=torch.bool, device=dev)
        valid = torch.arange(i.shape[-1], device=dev) < c[..., None].long()
        m.scatter_(3, torch.where(valid, i.long(), nb), True)
        return m[..., :nb]
    m0, m1 = dense(c0m, i0m), dense(c1m, i1m)
    o_re = bsa.block_sparse_attn_fwd(q1, k1, v1, c0m, i0m, n_valid=w.n_valid).float()
    o_fr = bsa.block_sparse_attn_fwd(q1, k1, v1, c1m, i1m, n_valid=w.n_valid).float()
    dlt = (o_re - o_fr).abs()
    out["mask_reuse_next_step"] = {
        "what": "raster CDF mask of step 0 reused at the next step (5 % RMS drift of Q, K, V) vs the mask "
                "rebuilt there: kept-tile overlap and the attention output difference",
        "kept_step0": int(m0.sum()), "kept_step1": int(m1.sum()),
        "jaccard": round(float((m0 & m1).sum()) / float((m0 | m1).sum()), 4),
        "out_max_abs_diff": round(float(dlt.max()), 4), "out_mean_abs_diff": round(float(dlt.mean()), 5),
        "out_rms": round(float(o_fr.pow(2).mean().sqrt()), 4),
    }
    # mask quality of this step's raster mask against the full attention
    import block_sparse_attention_avg_amd.pipelines as pl2
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    mq = pl2.mask_quality(q, k, c0m, i0m, n_valid=w.n_valid)
    ev[1].record()
    torch.cuda.synchronize()
    out["mask_quality"] = {
        "what": "CDF mask of the 480p layer against the full attention's tile map (two passes: full forward "
                "with row normalisers, then max/sum/min per 64x64 tile): recall of the equal-budget max-pooled "
                "oracle mask and share of the attention mass kept, means over query blocks",
        "oracle_recall": round(float(mq.oracle_recall.mean()), 4),
        "mass_recall": round(float(mq.mass_recall.mean()), 4),
        "mass_recall_p10": round(float(torch.quantile(mq.mass_recall.flatten(), 0.1)), 4),
        "ms": round(ev[0].elapsed_time(ev[1]), 3),
    }
    out["semantic_next_step"] = {
        "what": "k-means of Q and K at the next denoising step (inputs drifted by 5 % RMS noise): warm start "
                "from the previous step's centroids vs k-means++ seeding + Lloyd rounds, both run until a "
                f"round moves at most {tol} tokens (1 %; at most {cap} rounds)",
        "warm_ms": tw["kmeans_qk_warm"], "cold_ms": tc["kmeans_qk_cold"],
        "speedup": round(tc["kmeans_qk_cold"] / tw["kmeans_qk_warm"], 2),
        "warm_rounds_q": rounds(S["wq"][3]), "warm_rounds_k": rounds(S["wk"][3]),
        "cold_rounds_q": rounds(S["cq1"][3]), "cold_rounds_k": rounds(S["ck1"][3]),
    }
    return out


def mfma_probe():
    """Sustained bf16 MFMA rate from the measurement program built beside the
    library (a child process; None when it is missing or fails)."""
    import subprocess
    exe = os.path.join(ROOT, "block_sparse_attention_avg_amd", "mfma_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except Exception:
        return None


def attn_kernel_name(w) -> str:
    # with the full workspace the library splits uniform d = 128 rows over at
    # least 1024 key blocks into key segments (plan, then two item launches,
    # the second merging each query block's partials); two waves per 64-row
    # tile otherwise
    nb = -(-w.n_valid // w.block)
    if w.d == 128 and nb >= 1024:
        return "attn_fwd_kernel (items over key segments, two launches) + split_rows/plan/prefix kernels"
    return "attn_fwd_kernel"


# Kernels launched by one attention-forward call (summed against its events).
ATTN_CALL_KERNELS = ("bsa::attn_fwd", "bsa::split_", "bsa::qorder_kernel", "bsa::zero_rows_kernel",
                     "bsa::tile_base_kernel")


def dense_gemm_ref(dev, n: int = 8192, reps: int = 20):
    """bf16 dense GEMM throughput of the vendor library on this machine (TFLOP/s)."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    return 2.0 * n ** 3 / t / 1e12


def cpu_baseline(r: Runner, flops_total: float, mask_heads=None, attn_blocks=None):
    """Times the float64 CPU reference (untuned) on the host.

    mask_heads / attn_blocks None: the whole step (every head's mask stage and
    every query block's attention). Otherwise a bounded sample -- the mask
    stage of ``mask_heads`` heads and the attention of ``attn_blocks`` seeded
    query blocks of head 0 on head 0's own mask -- extrapolated to one step by
    the share of heads and query blocks it covers.
    """
    from oracle import attention as oa, layout as ol, mask as om  # CPU reference (baseline leg only)
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    w = r.w
    st, ln = ol.raster_blocks(w.n_valid, w.block)
    full = mask_heads is None
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    mheads = heads if full else heads[:mask_heads]
    t0 = time.perf_counter()
    keeps = {}
    for b, h in mheads:
        keeps[(b, h)], _ = om.block_mask(r.q_cpu[b, h].double().numpy(), r.k_cpu[b, h].double().numpy(),
                                         st, ln, st, ln, w.thr)
    t_mask = (time.perf_counter() - t0) * len(heads) / len(mheads)
    if full:
        blocks = None
        aheads = heads
    else:
        rng = np.random.default_rng(0)
        blocks = sorted(rng.choice(len(st), size=min(attn_blocks, len(st)), replace=False).tolist())
        aheads = heads[:1]
    t0 = time.perf_counter()
    for b, h in aheads:
        qh, kh, vh = (t[b, h].double().numpy() for t in (r.q_cpu, r.k_cpu, r.v_cpu))
        oa.masked_attention(qh, kh, vh, st, ln, st, ln, keeps[(b, h)], blocks=blocks)
    t_att = time.perf_counter() - t0
    if not full:
        t_att *= len(st) / len(blocks) * len(heads)
    t_step = t_mask + t_att
    if full:
        sample = (f"float64 numpy reference, the whole step: mask stage of all {len(heads)} heads and "
                  f"attention of all {len(st)} query blocks of every head ({t_step:.1f} s/step, measured)")
    else:
        sample = (f"float64 numpy reference on a bounded sample, extrapolated: mask stage of {len(mheads)} of "
                  f"{len(heads)} heads and attention of {len(blocks)} of {len(st)} query blocks of head 0 "
                  f"(est. {t_step:.1f} s/step)")
    return {
        "value": flops_total / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": sample,
        "extrapolated": not full,
        "host_cpus": os.cpu_count(),
        "blas_threads": int(cores),
    }


# ---------------------------------------------------------------- profiles
# Summaries of rocprofv3 CSV output (kernel trace statistics, counter runs),
# written as the text files kept under profiles/.

CSRC = os.path.join(ROOT, "block_sparse_attention_avg_amd", "csrc")
# Sources of the attention forward kernels; the counter summary of a kernel
# stays valid while their combined hash is unchanged.
ATTN_SOURCES = ("attn.h", "attn_fwd.hip", "attn_fwd_1w.hip", "lds_tile.h", "common.h")


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.txt")


def _sha256(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        if os.path.exists(p):
            with open(p, "rb") as f:
                h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def attn_sources_sha() -> str:
    return _sha256([os.path.join(CSRC, n) for n in ATTN_SOURCES])


def _csv_rows(path: str):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    name = name.replace("void ", "")
    return name.split("(")[0]


def rocprof_stats(run_dir: str):
    """[(kernel, calls, avg_us, min_us, max_us, pct)] from run_kernel_stats.csv."""
    out = []
    for r in _csv_rows(os.path.join(run_dir, "run_kernel_stats.csv")):
        out.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return out


def rocprof_counter(run_dir: str, counter: str, kernel: str):
    """Mean per dispatch of one counter over the dispatches of `kernel`."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(os.path.join(run_dir, "run_counter_collection.csv"))
            if r["Counter_Name"] == counter and _short(r["Kernel_Name"]) == kernel]
    if not vals:
        raise SystemExit(f"no {counter} samples for {kernel} in {run_dir}")
    return sum(vals) / len(vals), len(vals)


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary of
    that workload, or None when the attention sources changed after the
    counters were taken."""
    try:
        with open(traffic_file(workload)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
        if kv.get("source_sha256", "").strip() != attn_sources_sha():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def rocprof_summary(kind: str, dirs, bench_log=None, command="", kernel="", workload=""):
    lines = []
    if kind == "stats":
        lines.append(f"command: {command}")
        lines.append("kernel                                   calls    avg_us      min_us      max_us    pct")
        for name, calls, avg, mn, mx, pct in rocprof_stats(dirs[0]):
            lines.append(f"{name[:40]:40s} {calls:6d} {avg:10.2f} {mn:10.2f} {mx:10.2f} {pct:6.2f}")
        if bench_log:
            with open(bench_log) as f:
                js = [json.loads(l) for l in f if l.startswith("{")]
            if js:
                b = js[-1]
                st = rocprof_stats(dirs[0])
                att = [x for x in st if x[0].startswith("bsa::attn_fwd")]
                call = [x for x in st if x[0].startswith(ATTN_CALL_KERNELS)]
                ev = b['stages_ms']['attention'] * 1e3
                lines.append(f"bench (same run): attention stage {ev:.1f} us per call (HIP events around the "
                             f"C-ABI call), roofline.achieved {b['roofline']['achieved']} TFLOP/s")
                # calls = the fewest launches of any kernel of the call (the
                # split path launches the attention kernel twice per call; the
                # backward launches the order kernel too)
                n_calls = min((x[1] for x in call), default=1)
                paths = bool(b.get("paths")) or any(isinstance(v, dict) and v.get("paths")
                                                     for v in b.get("also", {}).values())
                if paths:
                    # the variant paths launch the same kernels: no per-call
                    # comparison with the attention stage's events
                    att, call = [], []
                    lines.append("rocprof: the variant paths of this run launch the attention kernels too, so "
                                 "launch counts are not per attention call; see the paths' own timings in the "
                                 "bench line")
                if att:
                    a_us = att[0][1] * att[0][2] / n_calls
                    lines.append(f"rocprof {att[0][0]}: {att[0][1] / n_calls:g} launch(es) per call, "
                                 f"average {att[0][2]:.1f} us, {a_us:.1f} us per call "
                                 f"(ratio events / kernel {ev / a_us:.3f})")
                if len(call) > 1:
                    tot = sum(x[1] * x[2] for x in call) / n_calls
                    lines.append(f"rocprof kernels of one attention call ({', '.join(x[0] for x in call)}): "
                                 f"{tot:.1f} us over {n_calls} calls (ratio events / kernels {ev / tot:.3f})")
                if "backward" in b:
                    bw = [x for x in rocprof_stats(dirs[0]) if x[0].startswith("bsa::bwd_") or
                          x[0].startswith("bsa::csc_")]
                    per_call = sum(x[2] * x[1] for x in bw) / max(1, max((x[1] for x in bw), default=1))
                    lines.append(f"bench (same run): backward {b['backward']['ms'] * 1e3:.1f} us per call "
                                 f"(HIP events), {b['backward']['tflops_eff']} TFLOP/s effective; rocprof "
                                 f"backward kernels {per_call:.1f} us per call")
    elif kind == "counters":
        lines.append(f"command: {command}")
        rows = _csv_rows(os.path.join(dirs[0], "run_counter_collection.csv"))
        kernels = sorted({_short(r["Kernel_Name"]) for r in rows if _short(r["Kernel_Name"]).startswith("bsa::")})
        for k in kernels:
            counters = sorted({r["Counter_Name"] for r in rows if _short(r["Kernel_Name"]) == k})
            vals = []
            for c in counters:
                v, n = rocprof_counter(dirs[0], c, k)
                vals.append(f"{c}={v:.5g}")
            lines.append(f"{k} (mean per dispatch): " + " ".join(vals))
    elif kind == "traffic":
        fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
        # `kernel`: comma-separated name prefixes; the per-dispatch means of
        # every matching kernel are summed (the kernels of one attention call)
        prefixes = tuple(p for p in kernel.split(",") if p)

        def summed(d, counter):
            # per attention call: every matching dispatch summed, over the
            # dispatch count of the kernels launched once per call (the split
            # path launches the attention kernel twice per call)
            names = sorted({_short(r["Kernel_Name"]) for r in _csv_rows(os.path.join(d, "run_counter_collection.csv"))
                            if _short(r["Kernel_Name"]).startswith(prefixes)})
            vals = {nm: rocprof_counter(d, counter, nm) for nm in names}
            once = [n for nm, (_, n) in vals.items() if not nm.startswith("bsa::attn_fwd")]
            n_calls = min(once) if once else min((n for _, n in vals.values()), default=1)
            return sum(v * n for v, n in vals.values()) / n_calls, n_calls, names
        kern = kernel
        copy = "bsa::permute_kernel<16>"
        f_att, n1, names = summed(fetch_dir, "FETCH_SIZE")
        w_att, n2, _ = summed(write_dir, "WRITE_SIZE")
        kern = " + ".join(names)
        f_cp, n3 = rocprof_counter(cfetch_dir, "FETCH_SIZE", copy)
        w_cp, n4 = rocprof_counter(cwrite_dir, "WRITE_SIZE", copy)
        gib = 1024.0 ** 3
        f_scale = gib / (f_cp * 1024.0)          # bytes the copy really read per counted byte
        w_scale = gib / (w_cp * 1024.0)
        fetch_b = f_att * 1024.0 * f_scale
        write_b = w_att * 1024.0 * w_scale
        lines += [
            f"command: {command}",
            f"kernel: {kern} ({workload} workload)",
            f"FETCH_SIZE per call: {f_att:.1f} KiB over {n1} calls",
            f"WRITE_SIZE per call: {w_att:.1f} KiB over {n2} calls",
            f"copy calibration ({copy}, identity permutation reading and writing 1 GiB): "
            f"FETCH_SIZE {f_cp:.1f} KiB (x{f_scale:.3f}), WRITE_SIZE {w_cp:.1f} KiB (x{w_scale:.3f}) over {n3}/{n4}",
            f"fetch_bytes_per_launch: {fetch_b:.6g}",
            f"write_bytes_per_launch: {write_b:.6g}",
            f"traffic_bytes_per_launch: {fetch_b + write_b:.6g}",
            f"sources: {' '.join(ATTN_SOURCES)}",
            f"source_sha256: {attn_sources_sha()}",
        ]
    print("\n".join(lines))


def copy_calibration(dev, steps: int):
    """Identity permutation: reads and writes exactly 1 GiB per launch."""
    B, H, N, d = 1, 16, 262144, 128        # 16 * 262144 * 128 * 2 bytes = 1 GiB
    x = torch.randn((B, H, N, d), device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    perm = torch.arange(N, dtype=torch.int32, device=dev)
    for _ in range(steps):
        bsa.permute_tokens(x, perm, out=y)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    print(json.dumps({"copy_calibration": {"bytes_read": x.numel() * 2, "bytes_written": y.numel() * 2,
                                           "launches": steps}}), flush=True)


def measure(w, a, dev):
    """Times one raster workload: the step, its roofline, and (per flags) the
    backward, the cold-cache step, the reorder-based paths (480p layer only)
    and the CPU reference. Returns (entry dict, step summary)."""
    r = Runner(w, dev)
    ms_step, t_mask, t_attn = r.timed(a.steps, a.warmup)
    s = r.summary(ms_step, t_mask, t_attn)
    e = {
        "workload": describe(w),
        "ms_per_step": round(ms_step, 4),
        "step_tflops": round(s["step_tflops"], 3),
        "roofline": {
            "bound": "mfma",
            "kernel": attn_kernel_name(w),
            "achieved": round(s["attn_tflops"], 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(s["attn_frac_of_peak"], 4),
            "traffic": measured_traffic(w.key),
        },
        "pct_bf16_peak_attn": round(100 * s["attn_frac_of_peak"], 2),
        "sparsity": {"blocks": round(s["sparsity_blocks"], 4),
                     "token_pairs": round(s["sparsity_token_pairs"], 4),
                     "kept_per_row_mean": round(s["kept_per_row_mean"], 2),
                     "kept_per_row_max": s["kept_per_row_max"]},
        "stages_ms": {"mask": round(t_mask, 4), "attention": round(t_attn, 4),
                      "attention_median": round(float(np.median(r.attn_each)), 4),
                      "attention_min": round(float(np.min(r.attn_each)), 4),
                      "mask_over_attention": round(s["mask_over_attn"], 4),
                      "mask_gbs": round(s["mask_gbs"], 1),
                      "mask_frac_of_hbm": round(s["mask_frac_of_hbm"], 4)},
        "flops_eff_per_step": s["flops_eff"],
    }
    if a.bwd_steps > 0:
        tf, tb = r.backward(a.bwd_steps)
        fb = 2.5 * s["flops_eff"]                  # five products per kept tile
        e["backward"] = {"ms": round(tb, 4), "tflops_eff": round(fb / (tb * 1e-3) / 1e12, 3),
                         "frac_of_peak": round(fb / (tb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "fwd_with_lse_ms": round(tf, 4), "steps": a.bwd_steps,
                         "flops": "2.5 x the forward's effective FLOP (S, dP, dV, dK, dQ products of "
                                  "kept tiles; the dQ pass also recomputes S and dP, not counted)"}
    if a.path_steps > 0 and w.key == "wan480":
        e["paths"] = paths_bench(r, a.path_steps)
    if a.cold_reps > 0:
        cm, ca = r.cold(a.cold_reps)
        e["cold_cache"] = {"mask_ms": round(cm, 4), "attention_ms": round(ca, 4),
                           "attn_tflops": round(s["flops_eff"] / (ca * 1e-3) / 1e12, 3),
                           "reps": a.cold_reps,
                           "how": "median; 512 MiB written before each step (outside the events)"}
    return r, e, s


# Bounded CPU-reference samples per workload (mask heads, attention query
# blocks), sized to about 10-30 s on 16 host cores; None = the whole step.
CPU_SAMPLE = {"hunyuan720": (2, 128), "wan480": (None, None), "tiny": (None, None)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="hunyuan720", choices=sorted(WORKLOADS))
    ap.add_argument("--also", default="wan480", help="second workload to report, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="extra steps timed with flushed caches (reported under cold_cache; 0 = skip)")
    ap.add_argument("--bwd-steps", type=int, default=20,
                    help="steps timing the backward on the same lists (reported under backward; 0 = skip)")
    ap.add_argument("--path-steps", type=int, default=10,
                    help="steps timing the reorder-based paths on the 480p layer (fractal + window, "
                         "per-head box tilings, semantic clusters; reported under paths; 0 = skip)")
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the MFMA-rate probe and the dense bf16 GEMM reference")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (identity token permutation of "
                         "1 GiB of bf16 rows) to calibrate hardware byte counters")
    ap.add_argument("--rocprof-summary", nargs="+", metavar=("KIND", "DIR"),
                    help="summarise rocprofv3 CSV output: 'stats DIR' (kernel trace), "
                         "'counters DIR' (counter means) or "
                         "'traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR' "
                         "(with --kernel and --workload)")
    ap.add_argument("--kernel", default="", help="kernel name of a traffic summary")
    ap.add_argument("--workload", default="", help="workload of a traffic summary")
    ap.add_argument("--bench-log", help="bench output of the profiled run (stats summary)")
    ap.add_argument("--command", default="", help="profiling command recorded in the summary")
    a = ap.parse_args()
    if a.rocprof_summary:
        rocprof_summary(a.rocprof_summary[0], a.rocprof_summary[1:], a.bench_log, a.command, a.kernel,
                        a.workload)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the hot path shards by head with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    bsa.load()
    if a.copy_calibration:
        copy_calibration(dev, a.steps)
        return

    w = WORKLOADS[a.config]
    if w.order != "raster":
        print("bench.py times the raster-order workloads (tiny, wan480, hunyuan720)", file=sys.stderr)
        sys.exit(1)
    r, e, s = measure(w, a, dev)
    line = {
        "metric": METRIC,
        "value": e["step_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": e["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Fourier-feature Q/K, Gaussian V)",
        "config": {"workload": describe(w), "global_batch": w.B, "seq_len": w.N,
                   "heads": w.H, "head_dim": w.d, "block": w.block, "thr": w.thr,
                   "parallelism": "single GPU"},
    }
    line.update({k: v for k, v in e.items() if k not in ("workload", "ms_per_step", "step_tflops")})
    if not a.no_gemm_ref:
        mp = mfma_probe()
        if mp:
            mp["attn_over_probe"] = round(s["attn_tflops"] / mp["tflops"], 4)
            line["mfma_probe"] = mp
        g = dense_gemm_ref(dev)
        line["dense_gemm_ref"] = {"tflops": round(g, 1), "frac_of_peak": round(g / PEAK_BF16_TFLOPS, 4),
                                  "attn_over_gemm": round(s["attn_tflops"] / g, 4),
                                  "how": "torch.matmul bf16 8192x8192x8192 (vendor GEMM) on this box"}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(r, s["flops_eff"], *CPU_SAMPLE.get(w.key, (1, 24)))
    if a.also and a.also != "none" and a.also != a.config:
        del r
        torch.cuda.empty_cache()
        w2 = WORKLOADS[a.also]
        r2, e2, s2 = measure(w2, a, dev)
        if not a.no_cpu_baseline:
            e2["cpu_baseline"] = cpu_baseline(r2, s2["flops_eff"], *CPU_SAMPLE.get(w2.key, (1, 24)))
        line["also"] = {w2.key: e2}
        del r2
    print(json.dumps(line), flush=True)
    # leave no device work or allocation to interpreter teardown (where a
    # profiler's own finaliser may already have run)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
