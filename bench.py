"""Forward-pass throughput of the HIP GPT-2 library on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload small|medium|xl] [--no-cpu-baseline] [--no-loss] [--no-decode] [--no-train] [--no-kernels] [--configs all|attention|none]

One step = one gpt2_forward over a batch of synthetic token ids already resident in HBM:
embedding, every block, ln_f, the tied lm_head (fp32 logits) and the fused argmax. Weights are the
seeded synthetic init (no checkpoint exists). Prints one JSON line. After the timed region it also
times gpt2_forward_loss (the same forward with the shifted next-token cross-entropy fused into the
vocabulary projection, logits not stored) under "forward_loss", and cached greedy decode steps
(gpt2_decode_step after a gpt2_prefill of half the context) under "decode", and the same steps with
sampling (gpt2_sample at temperature 0.7, top-k 50, top-p 0.95, repetition penalty 1.2) under
"decode_sampled", and the training gradients (gpt2_backward: forward keeping activations, the loss,
the backward pass) under "train".

The roofline object is for the lm_head GEMM, the largest single launch: its duration is taken
from HIP events the library records on its own stream around that launch in every timed step.
"kernels" gives the same for every launch kind of the forward (mean duration per launch from one
launch of that kind repeated 100 times back to back inside a forward, between two events;
algorithmic work, roofline fraction, share of the forward's kernel time), and "cold_cache" the
LayerNorm and the embedding right after a write that evicts the caches. With --configs all it
also times the isolated attention (B=8 H=12 T=1024) and the GPT-2 medium (B=8) and XL (B=4)
forwards.
The CPU baseline times the fp64 oracle on a bounded sample (one full sequence) on the host.
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

from decoder_only_transformer_gpt2_amd import synth  # noqa: E402

METRIC = "forward tokens/s, GPT-2 small B=4 T=1024 bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "small": (synth.GPT2_SMALL, 4, 1024),
    "medium": (synth.GPT2_MEDIUM, 8, 1024),
    "xl": (synth.GPT2_XL, 4, 1024),
}


def forward_flops(s: synth.ModelShape, B: int, T: int) -> float:
    """Algorithmic FLOPs: block GEMMs + causal half of attention + lm_head (no padded columns)."""
    M = B * T
    return 24.0 * M * s.n_layer * s.d_model ** 2 + 2.0 * B * s.n_layer * s.d_model * T * (T + 1) \
        + 2.0 * M * s.d_model * s.n_vocab


def train_flops(s: synth.ModelShape, B: int, T: int) -> float:
    """Algorithmic FLOPs of forward + backward: each GEMM once forward and twice backward (input and
    weight gradients), the causal attention products once forward and twice backward."""
    M = B * T
    gemm = 24.0 * M * s.n_layer * s.d_model ** 2 + 2.0 * M * s.d_model * s.n_vocab
    attn = 2.0 * B * s.n_layer * s.d_model * T * (T + 1)
    return 3.0 * gemm + 3.0 * attn


def kernel_work(kind: str, s: synth.ModelShape, B: int, T: int, embed_ln1: bool = False):
    """(bound, algorithmic work per launch) of one launch kind of the forward: FLOPs for the matrix
    products (attention: its causal half, diagonal included), HBM bytes for the row-wise kernels
    (each operand read once, each result written once). embed_ln1: the embedding launch also
    computes the first block's ln_1."""
    M, d, V = B * T, s.d_model, s.n_vocab
    if kind == "qkv":
        return "mfma", 2.0 * M * 3 * d * d
    if kind == "attn_proj":
        return "mfma", 2.0 * M * d * d
    if kind in ("fc", "mlp_proj"):
        return "mfma", 2.0 * M * s.d_mlp * d
    if kind == "attn":
        return "mfma", 2.0 * B * d * T * (T + 1)
    if kind == "lm_head":
        return "mfma", 2.0 * M * d * V
    if kind in ("ln", "ln_f"):  # fp32 rows in, bf16 rows out, gamma and beta
        return "hbm", M * d * 4.0 + M * d * 2.0 + 2 * d * 4.0
    if kind == "embed":  # token ids, wte and wpe rows (bf16), fp32 residual out
        work = M * 4.0 + M * d * 2.0 + T * d * 2.0 + M * d * 4.0
        if embed_ln1:  # and the first block's ln_1: gamma, beta in, bf16 rows out
            work += M * d * 2.0 + 2 * d * 4.0
        return "hbm", work
    if kind == "argmax":  # (value, column) partials per 256-column tile, int32 result
        return "hbm", M * ((V + 255) // 256) * 8.0 + M * 4.0
    return None, None


GEMM_SOURCES = ("gemm_bf16_impl.h", "gemm_bf16.hip", "common.h")  # the kernel, its launch / tile choice, helpers


def gemm_source_sha() -> str:
    """sha256 (first 16 hex digits) of the GEMM kernel sources, in GEMM_SOURCES order."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "decoder_only_transformer_gpt2_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record():
    """HBM bytes per lm_head launch from the stored rocprofv3 counter summary, or None when the
    summary is missing or was taken on a different version of the GEMM sources."""
    path = os.path.join(ROOT, "profiles", "forward_traffic_gpt2_small_b4_t1024.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != gemm_source_sha() or "lm_head_traffic_bytes" not in kv:
        return None
    return float(kv["lm_head_traffic_bytes"])


def host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS library numpy calls (threadpoolctl)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api')} {p.get('version')}"
                threads = p.get("num_threads", threads)
                break
    except Exception:  # pragma: no cover
        pass
    return model, blas, int(threads)


def cpu_baseline(weights: dict, tokens: np.ndarray, s: synth.ModelShape):
    """Oracle (fp64 numpy) forward of one full sequence of the workload on the host cores."""
    from oracle import gpt2_oracle as O
    model, blas, cores = host_info()
    sample = tokens[:1]
    O.forward(weights, tokens[:1, :4], s.n_head, s.n_layer)  # warm-up on a tiny input
    t0 = time.perf_counter()
    O.forward(weights, sample, s.n_head, s.n_layer)
    dt = time.perf_counter() - t0
    return {"value": sample.size / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"one sequence (B=1, T={sample.shape[1]}) of the workload, full forward incl. logits, "
                      f"fp64 numpy, {dt:.1f} s"}


def decode_step_bytes(s: synth.ModelShape, B: int, keys: float) -> float:
    """HBM bytes one cached decode step reads at least: every block matrix and wte (the tied head)
    once in bf16, row-major and unpadded (the few-row products stream them; the k-blocked copies
    are not touched), the fp32 vectors, one wpe row, and the cached K and V of
    `keys` positions for every layer and sequence (bf16)."""
    d, f, L = s.d_model, s.d_mlp, s.n_layer
    mats = L * (3 * d * d + d * d + f * d + d * f) + s.n_vocab * d
    vecs = L * (2 * d + 3 * d + d + 2 * d + f + d) + 2 * d
    return mats * 2.0 + vecs * 4.0 + d * 2.0 + 2.0 * L * B * d * keys * 2.0


def random_model(gpt2, shape: synth.ModelShape, seed: int):
    """A bf16 model of the given shape with weights of the synthetic init's distribution drawn on the
    GPU (throughput only: the larger models' parity tests use the seeded host generator)."""
    import torch
    m = gpt2.GPT2(gpt2.ModelConfig(n_vocab=shape.n_vocab, n_ctx=shape.n_ctx, d_model=shape.d_model,
                                   n_head=shape.n_head, n_layer=shape.n_layer, d_mlp=shape.d_mlp, dtype="bf16"))
    gen = torch.Generator(device="cuda").manual_seed(seed)
    ts = []
    for _, shp, kind in synth.tensor_specs(shape):
        if kind in ("emb", "w", "w_res"):
            std = 0.02 if kind != "w_res" else 0.02 / (2.0 * shape.n_layer) ** 0.5
            t = torch.randn(shp, generator=gen, device="cuda") * std
        elif kind == "gamma":
            t = torch.ones(shp, device="cuda")
        else:
            t = torch.zeros(shp, device="cuda")
        ts.append(t.to(torch.bfloat16))
    m.load_weights(ts)
    del ts
    return m


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="small")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-loss", action="store_true", help="skip the fused forward+loss measurement")
    ap.add_argument("--no-decode", action="store_true", help="skip the cached decode measurement")
    ap.add_argument("--no-train", action="store_true", help="skip the forward+backward (gradients) measurement")
    ap.add_argument("--no-kernels", action="store_true",
                    help="skip the per-kernel breakdown and the cold-cache LayerNorm / embedding figures")
    ap.add_argument("--configs", choices=("all", "attention", "none"), default="all",
                    help="the other workloads measured after the headline: the isolated attention (B=8 H=12 "
                         "T=1024) and the GPT-2 medium / XL forwards (all), the attention alone, or none")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed region, run a plain device-to-device copy of this many bytes three "
                         "times (a known-size reference for hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the forward is not sharded "
              "across GPUs in this build", file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_only_transformer_gpt2_amd import gpt2

    shape, B, T = WORKLOADS[args.workload]
    M = B * T
    w = synth.make_weights(shape, bf16=True)
    m = gpt2.GPT2(gpt2.ModelConfig(n_vocab=shape.n_vocab, n_ctx=shape.n_ctx, d_model=shape.d_model,
                                   n_head=shape.n_head, n_layer=shape.n_layer, d_mlp=shape.d_mlp, dtype="bf16"))
    m.load_numpy(w)
    tok_np = synth.make_tokens(B, T, shape.n_vocab)
    tokens = torch.from_numpy(tok_np).cuda()
    logits = torch.empty((B, T, shape.n_vocab), dtype=torch.float32, device="cuda")
    am = torch.empty((B, T), dtype=torch.int32, device="cuda")
    ws = m.workspace(B, T)
    kinds = m.launches(B, T, with_argmax=True)
    embed_ln1 = kinds[1] != "ln"  # the embedding launch computes the first ln_1
    lm_idx = kinds.index("lm_head")
    stream = torch.cuda.current_stream()

    def raw_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    for _ in range(args.warmup):
        m.forward(tokens, logits, am, ws)
    ev = [(raw_event(), raw_event()) for _ in range(args.steps)]
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        before = [None] * (lm_idx + 1)
        after = [None] * (lm_idx + 1)
        before[lm_idx] = ev[i][0].cuda_event
        after[lm_idx] = ev[i][1].cuda_event
        m.forward_timed(tokens, logits, am, before, after, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if m.check(B, T, ws) != gpt2.OK:
        raise RuntimeError("token check failed")

    ms = (t1 - t0) * 1e3 / args.steps
    lm_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    lm_flops = 2.0 * M * shape.d_model * shape.n_vocab
    achieved = lm_flops / (lm_ms * 1e-3) / 1e12
    flops = forward_flops(shape, B, T)
    traffic = traffic_record()

    out = {
        "metric": METRIC, "value": M / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random-init weights and token ids)",
        "config": {"workload": f"GPT-2 {args.workload} forward, bf16 operands / fp32 accumulation, fp32 logits",
                   "batch": B, "seq_len": T, "d_model": shape.d_model, "n_layer": shape.n_layer,
                   "n_head": shape.n_head, "n_vocab": shape.n_vocab, "parallelism": "none (1 GPU)"},
        "forward_tflops": flops / (ms * 1e-3) / 1e12,
        "forward_mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"kernel": "lm_head GEMM (tied wte, fp32 logits + argmax partials)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "avg_launch_ms": lm_ms,
                     "flops_per_launch": lm_flops},
    }

    if not args.no_loss:
        # The forward followed by the shifted cross-entropy, with the logits never stored (timed
        # separately, after the headline region).
        nll = torch.empty((B, T), dtype=torch.float32, device="cuda")
        loss = torch.empty((1,), dtype=torch.float32, device="cuda")
        for _ in range(3):
            m.forward_loss(tokens, None, nll, loss, ws)
        n_loss = max(5, args.steps // 5)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(n_loss):
            m.forward_loss(tokens, None, nll, loss, ws)
        torch.cuda.synchronize()
        lms = (time.perf_counter() - t2) * 1e3 / n_loss
        out["forward_loss"] = {"ms_per_step": lms, "tokens_per_s": M / (lms * 1e-3), "steps": n_loss,
                               "loss": float(loss.item()),
                               "what": "forward + shifted next-token cross-entropy, logits not stored"}

    if not args.no_decode:
        # Cached greedy decoding at the same batch: prefill half the context, then timed steps.
        # Each step reads every weight once plus the cache up to its position, so HBM bounds it.
        T0, n_dec = T // 2, 64
        cache = m.kv_cache(B)
        nxt = torch.empty((B,), dtype=torch.int32, device="cuda")
        cur = torch.empty((B,), dtype=torch.int32, device="cuda")
        prompt = tokens[:, :T0].contiguous()
        m.prefill(prompt, cache, logits=False, nxt=cur)
        wsd = m.workspace(B, 1)
        for i in range(4):  # warm-up steps (their cache rows are rewritten below)
            m.decode_step(cur, T0 + i, cache, logits=False, nxt=nxt, ws=wsd)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        for i in range(n_dec):
            m.decode_step(cur, T0 + i, cache, logits=False, nxt=nxt, ws=wsd)
            cur, nxt = nxt, cur
        torch.cuda.synchronize()
        dms = (time.perf_counter() - t3) * 1e3 / n_dec
        step_bytes = decode_step_bytes(shape, B, T0 + (n_dec + 1) / 2)  # mean keys over the steps
        out["decode"] = {"ms_per_step": dms, "tokens_per_s": B / (dms * 1e-3), "batch": B, "prefill_len": T0,
                         "steps": n_dec, "hbm_bytes_per_step": step_bytes,
                         "hbm_frac": step_bytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "what": "greedy cached decode step (next-token argmax); hbm_bytes_per_step = the row-major bf16 "
                                 "weights (block matrices and wte), vectors and the cached K/V one step reads"}

        # Sampled decoding with the knobs of the pages' generation example (temperature 0.7, top-k 50,
        # top-p 0.95, repetition penalty 1.2 over the whole sequence so far): each step writes the
        # next-token logits, gpt2_sample draws from them, and the token is appended to the sequence.
        knobs = dict(temperature=0.7, top_k=50, top_p=0.95, repetition_penalty=1.2)
        seq = torch.zeros((B, T0 + n_dec + 8), dtype=torch.int32, device="cuda")
        seq[:, :T0] = prompt
        lg = torch.empty((B, shape.n_vocab), dtype=torch.float32, device="cuda")
        u = torch.rand((n_dec + 8, B), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
        sws = gpt2._aligned_empty(gpt2.sample_workspace_bytes(B, shape.n_vocab), "cuda")
        m.prefill(prompt, cache, logits=lg, nxt=False)
        gpt2.sample(lg, u[0], history=seq[:, :T0], out=cur, ws=sws, **knobs)

        def sampled_step(i, cur, nxt):
            m.decode_step(cur, T0 + i, cache, logits=lg, nxt=False, ws=wsd)
            gpt2.sample(lg, u[i + 1], history=seq[:, :T0 + i + 1], out=nxt, ws=sws, **knobs)
            seq[:, T0 + i + 1] = nxt

        for i in range(4):
            sampled_step(i, cur, nxt)
        torch.cuda.synchronize()
        t4 = time.perf_counter()
        for i in range(n_dec):
            sampled_step(i, cur, nxt)
            cur, nxt = nxt, cur
        torch.cuda.synchronize()
        sms = (time.perf_counter() - t4) * 1e3 / n_dec
        # the sampler alone, timed with events on the stream it runs on
        n_s = 50
        e0, e1 = raw_event(), raw_event()
        e0.record()
        for i in range(n_s):
            gpt2.sample(lg, u[i % n_dec], history=seq[:, :T0 + n_dec], out=nxt, ws=sws, **knobs)
        e1.record()
        torch.cuda.synchronize()
        out["decode_sampled"] = {"ms_per_step": sms, "tokens_per_s": B / (sms * 1e-3), "batch": B,
                                 "prefill_len": T0, "steps": n_dec, "knobs": knobs,
                                 "sample_call_us": e0.elapsed_time(e1) * 1e3 / n_s,
                                 "what": "cached decode step + gpt2_sample + append to the sequence; sample_call_us is "
                                         "one gpt2_sample call through the Python binding (host-bound at this batch)"}

    if not args.no_train:
        # Training gradients at the same shape: gpt2_backward = forward keeping activations, the
        # shifted cross-entropy, and the backward pass writing fp32 gradients of every weight.
        tws = m.train_workspace(B, T)
        gbuf = m.grad_buffer()
        tloss = torch.empty((1,), dtype=torch.float32, device="cuda")
        n_train = 5
        for _ in range(2):
            m.backward(tokens, grads=gbuf, loss=tloss, ws=tws)
        torch.cuda.synchronize()
        t5 = time.perf_counter()
        for _ in range(n_train):
            m.backward(tokens, grads=gbuf, loss=tloss, ws=tws)
        torch.cuda.synchronize()
        tms = (time.perf_counter() - t5) * 1e3 / n_train
        tfl = train_flops(shape, B, T)
        out["train"] = {"ms_per_step": tms, "tokens_per_s": M / (tms * 1e-3), "steps": n_train,
                        "tflops": tfl / (tms * 1e-3) / 1e12, "mfma_frac": tfl / (tms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "loss": float(tloss.item()), "workspace_gb": tws.numel() / 1e9,
                        "what": "forward keeping activations + shifted cross-entropy + backward (fp32 gradients "
                                "of every weight, tied wte summed); no optimizer step"}
        del tws, gbuf

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_bytes"] = args.copy_bytes

    # Every launch kind of the forward: one launch of each kind (its first in the forward) enqueued
    # REPS times back to back inside an otherwise ordinary forward, with HIP events around the
    # group only, so the mean per launch carries no event gaps. Algorithmic work and its roofline
    # per launch; share = launches x mean / sum over kinds.
    REPS = 100
    kernels = {}
    if not args.no_kernels:
        first = {}
        for i, k in enumerate(kinds):
            first.setdefault(k, i)
        per = {}
        for k, i in first.items():
            e0, e1 = raw_event(), raw_event()  # recorded once so that their handles exist
            m.forward_repeat(tokens, logits, am, i, REPS, e0.cuda_event, e1.cuda_event, ws)
            torch.cuda.synchronize()
            per[k] = e0.elapsed_time(e1) * 1e3 / REPS
        all_us = sum(per[k] * kinds.count(k) for k in per)
        for k, us in per.items():
            n = kinds.count(k)
            bound, work = kernel_work(k, shape, B, T, embed_ln1)
            e = {"launches": n, "avg_us": us, "share": us * n / all_us, "timing": f"{REPS} back-to-back launches"}
            if bound == "mfma":
                e.update(bound="mfma", unit="TFLOP/s", work_per_launch=work, achieved=work / (us * 1e-6) / 1e12,
                         peak=PEAK_BF16_TFLOPS)
            elif bound == "hbm":
                e.update(bound="hbm", unit="GB/s", work_per_launch=work, achieved=work / (us * 1e-6) / 1e9,
                         peak=PEAK_HBM_GBS)
            if bound:
                e["frac"] = e["achieved"] / e["peak"]
            kernels[k] = e
        out["kernels"] = kernels

        # Cold caches: the LayerNorm (gpt2_layernorm, [B*T, d] fp32 -> bf16) and the embedding (the
        # forward's first launch) each right after a 512 MiB write that evicts the 256 MB memory-side
        # cache and the L2s; median of 10.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        xs = torch.randn((M, shape.d_model), device="cuda")
        gam, bet = torch.ones(shape.d_model, device="cuda"), torch.zeros(shape.d_model, device="cuda")
        yb = torch.empty((M, shape.d_model), dtype=torch.bfloat16, device="cuda")
        cold = {"ln": [], "embed": []}
        for _ in range(10):
            flush.fill_(1)
            e0, e1 = raw_event(), raw_event()
            e0.record()
            gpt2.layernorm(xs, gam, bet, 1e-5, torch.bfloat16, out=yb)
            e1.record()
            torch.cuda.synchronize()
            cold["ln"].append(e0.elapsed_time(e1) * 1e3)
            flush.fill_(2)
            e0, e1 = raw_event(), raw_event()
            m.forward_repeat(tokens, logits, am, 0, 1, e0.cuda_event, e1.cuda_event, ws)
            torch.cuda.synchronize()
            cold["embed"].append(e0.elapsed_time(e1) * 1e3)
        out["cold_cache"] = {}
        embed_what = "the forward's embedding launch" + (" (with the first ln_1)" if embed_ln1 else "")
        for k, what in (("ln", "gpt2_layernorm on [B*T, d] fp32 -> bf16 (row-major output)"), ("embed", embed_what)):
            us = float(np.median(cold[k]))
            work = kernel_work(k, shape, B, T, embed_ln1)[1]
            out["cold_cache"][k] = {"avg_us": us, "achieved": work / (us * 1e-6) / 1e9, "unit": "GB/s",
                                    "frac": work / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "work_per_launch": work,
                                    "what": what + ", after a 512 MiB write; median of 10 (one launch between events)"}
        del flush, xs, yb

    if args.configs != "none":
        # The isolated-attention workload (B=8, H=12, T=1024, dh=64, bf16 Q/K/V ~ N(0,1)): 100
        # back-to-back gpt2_attention calls between two events.
        Bq, Hq, Tq = 8, 12, 1024
        q, k_, v = (torch.randn((Bq, Hq, Tq, 64), device="cuda").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        for _ in range(5):
            gpt2.attention(q, k_, v, o)
        e0, e1 = raw_event(), raw_event()
        e0.record()
        for _ in range(REPS):
            gpt2.attention(q, k_, v, o)
        e1.record()
        torch.cuda.synchronize()
        aus = e0.elapsed_time(e1) * 1e3 / REPS
        afl = 2.0 * 2.0 * Bq * Hq * 64 * Tq * (Tq + 1) / 2.0
        out["attention_config"] = {
            "workload": "causal MHA alone, B=8 H=12 T=1024 dh=64, bf16", "avg_us": aus,
            "tokens_per_s": Bq * Tq / (aus * 1e-6),
            "roofline": {"bound": "mfma", "achieved": afl / (aus * 1e-6) / 1e12, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": afl / (aus * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                         "flops_per_launch": afl},
            "timing": f"{REPS} back-to-back calls"}
        del q, k_, v, o
        # GPT-2 medium (B=8) and XL (B=4) forwards at T=1024
        for name in (("medium", "xl") if args.configs == "all" else ()):
            if name == args.workload:
                continue
            sh, Bm, Tm = WORKLOADS[name]
            mm = random_model(gpt2, sh, 11)
            tk = torch.from_numpy(synth.make_tokens(Bm, Tm, sh.n_vocab)).cuda()
            lg = torch.empty((Bm, Tm, sh.n_vocab), dtype=torch.float32, device="cuda")
            amx = torch.empty((Bm, Tm), dtype=torch.int32, device="cuda")
            wsm = mm.workspace(Bm, Tm)
            for _ in range(3):
                mm.forward(tk, lg, amx, wsm)
            n_m = 10
            torch.cuda.synchronize()
            t6 = time.perf_counter()
            for _ in range(n_m):
                mm.forward(tk, lg, amx, wsm)
            torch.cuda.synchronize()
            mms = (time.perf_counter() - t6) * 1e3 / n_m
            fl = forward_flops(sh, Bm, Tm)
            out[f"forward_{name}"] = {
                "workload": f"GPT-2 {name} forward, B={Bm} T={Tm}, bf16 operands / fp32 accumulation, fp32 logits",
                "ms_per_step": mms, "tokens_per_s": Bm * Tm / (mms * 1e-3), "steps": n_m,
                "roofline": {"bound": "mfma", "achieved": fl / (mms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": fl / (mms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                             "flops_per_step": fl, "what": "whole forward"}}
            del mm, lg, amx, wsm
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, tok_np, shape)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
