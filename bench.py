#!/usr/bin/env python3
"""Benchmark of the sparse gated-FFN forward on one MI355X.

A step is one forward of a Llama-7B-shaped FFN layer (d_model 4096, d_ff
11008, bf16 weights, fp32 accumulate) for one decode token: gate GEMV +
shifted-ReLU select, sparse up projection, split down projection. The headline
point is tau = 1.2816 (about 90% of channels inactive). Weights come from the
seeded synthetic recipe (random init, no trained checkpoint).

To measure HBM rather than the 256 MB Infinity Cache, steps rotate over
several device copies of the layer, so more than 512 MB of other weights are
read between two uses of a copy.

Prints one JSON line. Besides the contract fields it carries:
  roofline      the gate kernel (the dominant one): algorithmic bytes per launch
                (gate rows, the selected W_up rows, x) over its mean duration,
                from HIP events that take the kernel's own begin/end timestamps
                on the forward's stream, in a second timed region of the same
                steps (the events serialise the stream, so `value` comes from
                the uninstrumented region), against 8 TB/s;
  step_roofline the whole step: touched bytes (x, gate weights, active W_up and
                W_down rows, y) over the step time, against 8 TB/s;
  sweep         every tau of the workload: sparsity, step time, tokens/s, HBM
                fraction, and the speedup over this library's dense forward;
  points        the other workloads (tiny fp32 layer, LoPA ranks, Mixture-of-Channels
                Top-K, 2:8 and top-p at 1/16/64 tokens, 70B-shaped prefill at 256/2048
                tokens, and a 2048-token training step with masked activation storage):
                tokens/s, HBM fraction on touched bytes or MFMA fraction on the
                path's FLOPs, and the speedup over this library's dense forward;
  cpu_baseline  the CPU oracle (plain C, fp64) on a bounded sample: sparse skip and
                masked dense, one thread and every core (OpenMP build), host CPU;
                each sweep point also carries its parity against the oracle
                (band, flips, out-of-band mismatches, y error) and the oracle's time.
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

PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15  # MI355X dense bf16 MFMA, FLOP/s
MALL_BYTES = 256 << 20  # Infinity Cache
WORKLOAD = "llama7b_ffn_bf16_d4096_f11008"
HEADLINE_TAU = 1.2816
METRIC = "sparse FFN layer tokens/s + % HBM roofline at batch 1, 50–99% sparsity"
# sources of the gate kernel: its counters stay valid while these are unchanged
GATE_SRC = [os.path.join(ROOT, "activation_sparse_gated_gate_amd", "csrc", f)
            for f in ("gate.hip", "rowdot.h", "device_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gate_llama7b_bf16_pmc.md")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--copies", type=int, default=8, help="layer copies rotated to defeat the Infinity Cache")
    p.add_argument("--no-sweep", action="store_true", help="headline point only (no tau sweep, no other workloads)")
    p.add_argument("--no-points", action="store_true", help="skip the other workloads' points")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample length (0 = skip)")
    p.add_argument("--only", default="",
                   help="comma list of point families to measure (tiny, lopa, moc, prefill, train); runs them even "
                        "with --no-sweep")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="after timing, run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def sha256(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per gate launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.strip().startswith(("traffic_bytes_per_launch", "source_sha256")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != sha256(GATE_SRC):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(ffn, xt, wlist, mode, y, steps, warmup, tau=0.0, k=0):
    """Seconds per forward, rotating over the weight copies in wlist."""
    import torch

    L = len(wlist)
    for s in range(warmup):
        ffn.forward(xt, wlist[s % L], mode, y, tau=tau, k=k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ffn.forward(xt, wlist[s % L], mode, y, tau=tau, k=k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def copies_for(layer_bytes, touched_bytes):
    """Layer copies so that > 2x the Infinity Cache is read between reuses."""
    return max(2, min(32, int(math.ceil(2 * MALL_BYTES / max(1, touched_bytes))) + 1))


def measure_points(args, dev, S, inputs, np, torch):
    """The other workloads' points, by family (all, or those named by --only)."""
    W = inputs.WORKLOADS
    out = []
    fams = {f.strip() for f in args.only.split(",") if f.strip()}

    def want(fam):
        return not fams or fam in fams

    def replicate(tensors, L):
        return [tensors] + [{k: (v.clone() if v is not None else None) for k, v in tensors.items()}
                            for _ in range(L - 1)]

    # dense denominators on the Llama-7B-shaped layer (also the LoPA shape)
    dense2 = {}
    if want("lopa"):
        wl2 = W["llama7b_ffn_bf16_d4096_f11008"]
        d2, f2 = wl2.d_model, wl2.d_ff
        lay2 = inputs.make_layer(0, d2, f2, "bf16")
        t2 = {"w_gate": dev(lay2.w_gate), "w_up": dev(lay2.w_up), "w_down": dev(lay2.w_down)}
        c2 = replicate(t2, 4)
        w2 = [S.SparseFFN.weights(**c) for c in c2]
        for n in (1, 4):
            ffn = S.SparseFFN(d2, f2, n, "bf16")
            xt = dev(inputs.make_x(0, n, d2, "bf16"))
            y = torch.empty(n, d2, dtype=torch.float32, device="cuda")
            dense2[n] = timed(ffn, xt, w2, "dense_relu", y, 100, 10)
        del c2, w2, t2
    if want("tiny"):
        out += points_tiny(W, S, inputs, torch, timed_union(torch))
    if want("lopa"):
        out += points_lopa(W, S, inputs, torch, dev, dense2, timed_union(torch), replicate)
    if want("moc"):
        out += points_moc(W, S, inputs, torch, dev, timed_union(torch), replicate)
    if want("prefill"):
        out += points_prefill(W, S, inputs, torch, dev, timed_union(torch), replicate)
    if want("train"):
        out += points_train(W, S, inputs, torch, dev, timed_union(torch))
    return out


def timed_union(torch):
    def union(ffn, xt, w, mode, y, tau=0.0, k=0):
        u = torch.zeros(1, dtype=torch.int32, device="cuda")
        ffn.forward(xt, w, mode, y, tau=tau, k=k, union_cnt=u)
        torch.cuda.synchronize()
        return int(u.item())
    return union


def points_tiny(W, S, inputs, torch, union):
    """Tiny fp32 layer: cache-resident, latency and tokens/s only."""
    out = []
    wl = W["tiny_swiglu_fp32_d256_f1024"]
    lay = inputs.make_layer(0, wl.d_model, wl.d_ff, "f32")
    tt = {"w_gate": torch.from_numpy(lay.w_gate).cuda(), "w_up": torch.from_numpy(lay.w_up).cuda(),
          "w_down": torch.from_numpy(lay.w_down).cuda()}
    w = [S.SparseFFN.weights(**tt)]
    for n in wl.tokens:
        ffn = S.SparseFFN(wl.d_model, wl.d_ff, n, "f32")
        xt = torch.from_numpy(inputs.make_x(0, n, wl.d_model, "f32")).cuda()
        y = torch.empty(n, wl.d_model, dtype=torch.float32, device="cuda")
        na = union(ffn, xt, w[0], "threshold", y, tau=1.2816)
        sp = timed(ffn, xt, w, "threshold", y, 300, 30, tau=1.2816)
        de = timed(ffn, xt, w, "dense_relu", y, 300, 30)
        out.append({"workload": wl.name, "tokens": n, "mode": "threshold", "tau": 1.2816, "union": na,
                    "us_per_step": round(sp * 1e6, 2), "tokens_per_s": round(n / sp, 1),
                    "speedup_vs_dense": round(de / sp, 3), "note": "cache-resident (3 MB): no HBM fraction"})
    return out


def points_lopa(W, S, inputs, torch, dev, dense2, union, replicate):
    """LoPA low-rank gate, speedup against the dense Llama-7B-shaped layer."""
    out = []
    es = 2
    wl = W["lopa_gate_bf16_d4096_f11008"]
    d, f = wl.d_model, wl.d_ff
    for r in wl.ranks:
        lay = inputs.make_layer(0, d, f, "bf16", rank=r, with_gate=False)
        base = {"lopa_a": dev(lay.lopa_a), "lopa_b": dev(lay.lopa_b), "w_up": dev(lay.w_up),
                "w_down": dev(lay.w_down)}
        for n in wl.tokens:
            ffn = S.SparseFFN(d, f, n, "bf16", rank=r)
            xt = dev(inputs.make_x(0, n, d, "bf16"))
            y = torch.empty(n, d, dtype=torch.float32, device="cuda")
            na = union(ffn, xt, S.SparseFFN.weights(**base), "lopa", y, tau=1.2816)
            touched = n * d * es + r * d * es + f * r * es + 2 * na * d * es + n * d * 4
            cl = replicate(base, copies_for(0, touched))
            wlist = [S.SparseFFN.weights(**c) for c in cl]
            sp = timed(ffn, xt, wlist, "lopa", y, 200, 20, tau=1.2816)
            out.append({"workload": wl.name, "tokens": n, "mode": "lopa", "rank": r, "tau": 1.2816, "union": na,
                        "us_per_step": round(sp * 1e6, 2), "tokens_per_s": round(n / sp, 1),
                        "touched_bytes": touched, "hbm_frac": round(touched / sp / PEAK_HBM, 4),
                        "speedup_vs_dense": round(dense2[n] / sp, 3), "layer_copies": len(wlist)})
            del cl, wlist
        del base
        torch.cuda.empty_cache()
    return out


TOPP_PS = (0.3, 0.5)


def points_moc(W, S, inputs, torch, dev, union, replicate):
    """Mixture-of-Channels Top-K, its 2:8 structured option and top-p, decode and batched."""
    out = []
    es = 2
    wl = W["moc_topk_bf16_d2048_f5632"]
    d, f = wl.d_model, wl.d_ff
    lay = inputs.make_layer(0, d, f, "bf16")
    base = {"w_gate": dev(lay.w_gate), "w_up": dev(lay.w_up), "w_down": dev(lay.w_down)}
    cl = replicate(base, copies_for(0, 3 * f * d * es // 2))
    wlist = [S.SparseFFN.weights(**c) for c in cl]
    for n in wl.tokens:
        ffn = S.SparseFFN(d, f, n, "bf16")
        xt = dev(inputs.make_x(0, n, d, "bf16"))
        y = torch.empty(n, d, dtype=torch.float32, device="cuda")
        de = timed(ffn, xt, wlist, "dense_silu", y, 100, 10)
        for k in wl.ks:
            na = union(ffn, xt, wlist[0], "topk", y, k=k)
            touched = n * d * es + f * d * es + 2 * na * d * es + n * d * 4
            sp = timed(ffn, xt, wlist, "topk", y, 200, 20, k=k)
            out.append({"workload": wl.name, "tokens": n, "mode": "topk", "k": k, "union": na,
                        "union_frac": round(na / f, 4), "us_per_step": round(sp * 1e6, 2),
                        "tokens_per_s": round(n / sp, 1), "touched_bytes": touched,
                        "hbm_frac": round(touched / sp / PEAK_HBM, 4), "speedup_vs_dense": round(de / sp, 3),
                        "layer_copies": len(wlist)})
        # the 2:8 structured option: 2 of every 8 channels per token (d_ff / 4)
        na = union(ffn, xt, wlist[0], "topk_2_8", y)
        touched = n * d * es + f * d * es + 2 * na * d * es + n * d * 4
        sp = timed(ffn, xt, wlist, "topk_2_8", y, 200, 20)
        out.append({"workload": wl.name, "tokens": n, "mode": "topk_2_8", "k": f // 4, "union": na,
                    "union_frac": round(na / f, 4), "us_per_step": round(sp * 1e6, 2),
                    "tokens_per_s": round(n / sp, 1), "touched_bytes": touched,
                    "hbm_frac": round(touched / sp / PEAK_HBM, 4), "speedup_vs_dense": round(de / sp, 3),
                    "layer_copies": len(wlist)})
        # top-p: the shortest Top-K-order prefix holding a p share of the
        # softmax mass of the SiLU keys (p = 0.3 / 0.5 keep ~8.5 % / ~22.5 %)
        for pp in TOPP_PS:
            na = union(ffn, xt, wlist[0], "topp", y, tau=pp)
            touched = n * d * es + f * d * es + 2 * na * d * es + n * d * 4
            sp = timed(ffn, xt, wlist, "topp", y, 200, 20, tau=pp)
            out.append({"workload": wl.name, "tokens": n, "mode": "topp", "p": pp, "union": na,
                        "union_frac": round(na / f, 4), "us_per_step": round(sp * 1e6, 2),
                        "tokens_per_s": round(n / sp, 1), "touched_bytes": touched,
                        "hbm_frac": round(touched / sp / PEAK_HBM, 4), "speedup_vs_dense": round(de / sp, 3),
                        "layer_copies": len(wlist)})
    del cl, wlist, base
    torch.cuda.empty_cache()
    return out


def points_prefill(W, S, inputs, torch, dev, union, replicate):
    """70B-shaped prefill layer on the MFMA union path."""
    out = []
    wl = W["prefill70b_ffn_bf16_d8192_f28672"]
    d, f = wl.d_model, wl.d_ff
    lay = inputs.make_layer(0, d, f, "bf16")
    base = {"w_gate": dev(lay.w_gate), "w_up": dev(lay.w_up), "w_down": dev(lay.w_down)}
    del lay
    wlist = [S.SparseFFN.weights(**c) for c in replicate(base, 2)]
    tau = wl.taus[0]
    for n in wl.tokens:
        ffn = S.SparseFFN(d, f, n, "bf16")
        xt = dev(inputs.make_x(0, n, d, "bf16", correlated=True))
        y = torch.empty(n, d, dtype=torch.float32, device="cuda")
        na = union(ffn, xt, wlist[0], "threshold", y, tau=tau)
        steps = 20 if n >= 1024 else 50
        sp = timed(ffn, xt, wlist, "threshold", y, steps, 5, tau=tau)
        de = timed(ffn, xt, wlist, "dense_relu", y, max(5, steps // 2), 3)
        flops = 2 * n * d * (f + 2 * na)
        out.append({"workload": wl.name, "tokens": n, "mode": "threshold", "tau": tau, "union": na,
                    "union_frac": round(na / f, 4), "us_per_step": round(sp * 1e6, 2),
                    "tokens_per_s": round(n / sp, 1), "flops": flops,
                    "tflops": round(flops / sp / 1e12, 1), "mfma_frac": round(flops / sp / PEAK_BF16, 4),
                    "dense_us_per_step": round(de * 1e6, 2), "speedup_vs_dense": round(de / sp, 3),
                    "flop_ratio_vs_dense": round(3 * f / (f + 2 * na), 3)})
        # token groups (opt-in): each group's up and down products over its own union
        for groups in (2, 4, 8):
            if n < 64 * groups:
                continue
            ffn.set_token_groups(groups)
            sg = timed(ffn, xt, wlist, "threshold", y, steps, 3, tau=tau)
            ffn.set_token_groups(1)
            out.append({"workload": wl.name, "tokens": n, "mode": "threshold", "tau": tau, "token_groups": groups,
                        "us_per_step": round(sg * 1e6, 2), "tokens_per_s": round(n / sg, 1),
                        "speedup_vs_one_union": round(sp / sg, 3), "speedup_vs_dense": round(de / sg, 3)})
    del wlist, base
    torch.cuda.empty_cache()
    return out


TRAIN_TOKENS = 2048


def points_train(W, S, inputs, torch, dev, union):
    """Training step on the MoC layer: the forward with masked activation
    storage plus the backward, for a micro-batch of 2048 tokens, against the
    same step in the dense SwiGLU mode (every channel stored)."""
    out = []
    wl = W["moc_topk_bf16_d2048_f5632"]
    d, f, n = wl.d_model, wl.d_ff, TRAIN_TOKENS
    lay = inputs.make_layer(0, d, f, "bf16")
    w = S.SparseFFN.weights(w_gate=dev(lay.w_gate), w_up=dev(lay.w_up), w_down=dev(lay.w_down))
    ffn = S.SparseFFN(d, f, n, "bf16")
    xt = dev(inputs.make_x(0, n, d, "bf16"))
    dyt = dev(inputs.make_x(1, n, d, "bf16"))
    y = torch.empty(n, d, dtype=torch.float32, device="cuda")
    dx = torch.empty(n, d, dtype=torch.float32, device="cuda")
    dws = [torch.zeros(f, d, dtype=torch.float32, device="cuda") for _ in range(3)]

    def step_time(mode, cap, k, steps=10, warmup=2):
        cnt = torch.empty(n, dtype=torch.int32, device="cuda")
        idx = torch.empty(n, cap, dtype=torch.int32, device="cuda")
        z = torch.empty(n, cap, dtype=torch.float32, device="cuda")
        u = torch.empty(n, cap, dtype=torch.float32, device="cuda")
        sv = S.SparseFFN.saved(cap, cnt, idx, z, u)

        def one():
            ffn.forward_train(xt, w, mode, y, sv, k=k)
            ffn.backward(xt, dyt, w, mode, sv, dx, *dws, k=k)

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            one()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    de = step_time("dense_silu", f, 0)
    cases = [("topk", 704, 704), ("topk", 1408, 1408), ("topk_2_8", (f // 8) * 2 + min(f % 8, 2), 0)]
    for mode, cap, k in cases:
        na = union(ffn, xt, w, mode, y, k=k)
        sp = step_time(mode, cap, k)
        flops = 2 * n * d * (f + 8 * na)  # forward gate, up, down; backward dH, dx (2), dW (3)
        out.append({"workload": wl.name, "tokens": n, "mode": "train_" + mode, "k": cap, "union": na,
                    "union_frac": round(na / f, 4), "us_per_step": round(sp * 1e6, 2),
                    "tokens_per_s": round(n / sp, 1), "flops": flops, "tflops": round(flops / sp / 1e12, 1),
                    "mfma_frac": round(flops / sp / PEAK_BF16, 4), "dense_us_per_step": round(de * 1e6, 2),
                    "speedup_vs_dense": round(de / sp, 3),
                    "stored_bytes_per_token": 4 + 12 * cap, "dense_stored_bytes_per_token": 4 + 12 * f,
                    "stored_ratio_vs_dense": round((4 + 12 * f) / (4 + 12 * cap), 2)})
    del w, dws
    torch.cuda.empty_cache()
    return out


class OracleLeg:
    """The CPU oracle (plain C, fp64; its OpenMP build, where the pragmas only
    share out independent outputs) for the CPU baseline and the per-point
    parity: timing at one thread and at every core the process may use."""

    def __init__(self):
        import ctypes

        import oracle

        oracle.use_openmp()
        oracle.lib()
        self.oracle = oracle
        self.gomp = ctypes.CDLL("libgomp.so.1")
        self.cores = int(self.gomp.omp_get_max_threads())

    def threads(self, k):
        self.gomp.omp_set_num_threads(int(k))

    def forward(self, x_h, lay, tau, skip):
        t0 = time.perf_counter()
        r = self.oracle.forward("threshold", x_h, lay.w_up, lay.w_down, w_gate=lay.w_gate, tau=tau, skip=skip)
        return r, time.perf_counter() - t0

    def parity(self, ref, idx, cnt, y, x_h, lay):
        """Band channels, out-of-band set mismatches and y error (max-abs over
        max-abs, against the oracle on the GPU's own set) of one token."""
        import numpy as np

        f = ref.mask.shape[1]
        got = np.zeros(f, dtype=bool)
        got[idx[:cnt]] = True
        oset = ref.mask[0].astype(bool)
        diff = got ^ oset
        y_ref = ref.y[0]
        if diff.any():
            y_ref = self.oracle.forward_with_mask(x_h, lay.w_up, lay.w_down, ref.g, got[None].astype(np.uint8))[0]
        return {"band": int(ref.band.sum()), "band_flips": int(diff.sum()),
                "out_of_band_mismatches": int((diff & ~ref.band[0]).sum()),
                "y_rel_err": float(np.abs(y - y_ref).max() / np.abs(y_ref).max())}


def host_cpu():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable": len(os.sched_getaffinity(0)), "model": model}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library's forward is a single-GPU kernel path and "
              "no multi-GPU path is built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from activation_sparse_gated_gate_amd import inputs
    from activation_sparse_gated_gate_amd import sffn as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = inputs.WORKLOADS[WORKLOAD]
    d, f, n = wl.d_model, wl.d_ff, 1
    es = 2

    # ---- inputs resident in HBM before timing ----
    lay = inputs.make_layer(0, d, f, wl.dtype)
    x_h = inputs.make_x(0, n, d, wl.dtype)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")

    base = [dev(lay.w_gate), dev(lay.w_up), dev(lay.w_down)]
    copies = [base] + [[t.clone() for t in base] for _ in range(max(1, args.copies) - 1)]
    weights = [S.SparseFFN.weights(w_gate=g, w_up=u, w_down=dn) for g, u, dn in copies]
    x = dev(x_h)
    y = torch.empty(n, d, dtype=torch.float32, device="cuda")
    ucnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    ffn = S.SparseFFN(d, f, n, wl.dtype)
    stream = torch.cuda.current_stream()

    def run(mode, tau, steps, warmup, rotate=True, events=None):
        L = len(weights) if rotate else 1
        for s in range(warmup):
            ffn.forward(x, weights[s % L], mode, y, tau=tau)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            if events is not None:
                ffn.set_profile_events(*events[s])
            ffn.forward(x, weights[s % L], mode, y, tau=tau)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if events is not None:
            ffn.set_profile_events(None, None)
        return (t1 - t0) / steps

    def active_count(mode, tau):
        ffn.forward(x, weights[0], mode, y, tau=tau, union_cnt=ucnt)
        torch.cuda.synchronize()
        return int(ucnt.item())

    # ---- headline: timed region (no instrumentation) ----
    sec = run("threshold", HEADLINE_TAU, args.steps, args.warmup)
    n_act = active_count("threshold", HEADLINE_TAU)
    # ---- the same steps again with HIP events that take the gate kernel's own
    # begin/end timestamps (they serialise the stream, so they get their own
    # timed region and do not enter `value`) ----
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:  # torch creates the underlying hipEvent_t on first record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    ev_sec = run("threshold", HEADLINE_TAU, args.steps, 5, events=ev)
    gate_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    # k_gate reads every gate row, the W_up rows of the selected channels and x
    gate_bytes = f * d * es + n_act * d * es + n * d * es
    touched = lambda na: n * d * es + f * d * es + 2 * na * d * es + n * d * 4  # noqa: E731
    roofline = {
        "bound": "hbm",
        "kernel": "k_gate (gate GEMV + threshold select + selected W_up rows)",
        "achieved": round(gate_bytes / (gate_ms * 1e-3) / 1e9, 1),
        "peak": PEAK_HBM / 1e9,
        "unit": "GB/s",
        "frac": round(gate_bytes / (gate_ms * 1e-3) / PEAK_HBM, 4),
        "traffic": read_traffic(),
        "algorithmic_bytes_per_launch": gate_bytes,
        "mean_launch_us": round(gate_ms * 1e3, 2),
    }
    step_roofline = {
        "touched_bytes": touched(n_act),
        "achieved_GBps": round(touched(n_act) / sec / 1e9, 1),
        "frac": round(touched(n_act) / sec / PEAK_HBM, 4),
    }
    hot_sec = run("threshold", HEADLINE_TAU, args.steps, 5, rotate=False)

    # ---- the same forwards replayed from a HIP graph (one capture of a
    # forward per layer copy); each replay's y is checked against the eager
    # forward of that copy, bit for bit ----
    graph_sec = None
    try:
        y_eager = torch.empty_like(y)
        ffn.forward(x, weights[-1], "threshold", y_eager, tau=HEADLINE_TAU)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for w in weights:
                ffn.forward(x, w, "threshold", y, tau=HEADLINE_TAU)
        reps = max(1, args.steps // len(weights))
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_eager), "graph replay differs from the eager forward"
            ffn.forward(x, weights[0], "threshold", y_eager, tau=HEADLINE_TAU)  # eager work in between
            ffn.forward(x, weights[-1], "threshold", y_eager, tau=HEADLINE_TAU)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_sec = (time.perf_counter() - t0) / (reps * len(weights))
        del graph
    except Exception as exc:  # reported, never hidden: the eager number stands
        print(f"graph replay not measured: {exc}", file=sys.stderr)

    # ---- sweep over tau, with the dense forward as denominator ----
    sweep = []
    gpu_out = {}
    dense_sec = run("dense_relu", 0.0, max(50, args.steps // 4), 10)
    if not args.no_sweep:
        idx_t = torch.empty(n, f, dtype=torch.int32, device="cuda")
        cnt_t = torch.empty(n, dtype=torch.int32, device="cuda")
        for tau in wl.taus:
            na = active_count("threshold", tau)
            s = run("threshold", tau, max(50, args.steps // 2), 10)
            # this point's GPU outputs, checked against the oracle in the CPU leg below
            ffn.forward(x, weights[0], "threshold", y, tau=tau, active_idx=idx_t, active_cnt=cnt_t)
            torch.cuda.synchronize()
            gpu_out[tau] = (idx_t[0].cpu().numpy(), int(cnt_t[0].item()), y[0].cpu().numpy())
            sweep.append({
                "tau": tau, "sparsity": round(1 - na / f, 4), "active": na,
                "us_per_step": round(s * 1e6, 2), "tokens_per_s": round(n / s, 1),
                "hbm_frac": round(touched(na) / s / PEAK_HBM, 4),
                "speedup_vs_dense": round(dense_sec / s, 3),
                "byte_bound_speedup": round(3 * f * d * es / touched(na), 3),
            })

    # ---- optional plain copy for counter calibration ----
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb * (1 << 20), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---- the other workloads ----
    pts = []
    n_copies = len(weights)
    if not args.no_points and (args.only or not args.no_sweep):
        del weights, copies, base
        torch.cuda.empty_cache()
        pts = measure_points(args, dev, S, inputs, np, torch)

    # ---- CPU oracle baseline (bounded sample): sparse skip and masked dense,
    # at one thread and at every core ----
    cpu = None
    if args.cpu_seconds > 0:
        leg = OracleLeg()
        # each sweep point: the oracle's time (both forms, every core) and the
        # GPU result's parity against it
        for pt in sweep:
            tau = pt["tau"]
            ref, t_skip = leg.forward(x_h, lay, tau, True)
            _, t_mask = leg.forward(x_h, lay, tau, False)
            pt["oracle"] = {"sparse_skip_ms": round(t_skip * 1e3, 2), "masked_dense_ms": round(t_mask * 1e3, 2),
                            "threads": leg.cores}
            pt["parity"] = leg.parity(ref, *gpu_out[tau], x_h, lay)
        legs = []
        per = args.cpu_seconds / 4
        for variant, skip in (("sparse_skip", True), ("masked_dense", False)):
            for k in (1, leg.cores):
                leg.threads(k)
                reps, el = 0, 0.0
                while el < per or reps == 0:
                    el += leg.forward(x_h, lay, HEADLINE_TAU, skip)[1]
                    reps += 1
                legs.append({"variant": variant, "threads": k, "forwards": reps, "seconds": round(el, 2),
                             "tokens_per_s": round(reps * n / el, 3)})
        leg.threads(leg.cores)
        best = [g for g in legs if g["variant"] == "sparse_skip" and g["threads"] == leg.cores][0]
        cpu = {"value": best["tokens_per_s"], "unit": "tokens/s", "cores": leg.cores, "kind": "oracle",
               "sample": f"{best['forwards']} single-token forwards of the same layer (tau={HEADLINE_TAU}, sparse "
                         f"skip, fp64, OpenMP over channels and columns), {best['seconds']} s on {leg.cores} "
                         f"threads; 'legs' has the masked-dense form and one thread",
               "legs": legs, "host": host_cpu()}

    out = {
        "metric": METRIC,
        "value": round(n / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) token, N(0,1/d_in) weights, random init)",
        "config": {"workload": WORKLOAD, "d_model": d, "d_ff": f, "tokens": n, "mode": "threshold",
                   "tau": HEADLINE_TAU, "sparsity": round(1 - n_act / f, 4), "layer_copies": n_copies},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "ms_per_step_with_kernel_events": round(ev_sec * 1e3, 5),
        "hot_cache_ms_per_step": round(hot_sec * 1e3, 5),
        "graph_replay_ms_per_step": round(graph_sec * 1e3, 5) if graph_sec else None,
        "dense_ms_per_step": round(dense_sec * 1e3, 5),
        "speedup_vs_dense": round(dense_sec / sec, 3),
        "sweep": sweep,
        "points": pts,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
