#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verification step on one MI355X.

A step is one spec_verify call: the whole target pass (every MLP block and
the LM head, each weight byte streamed once for all gamma+1 positions) and
the acceptance rule over the vocabulary, for one batch of synthetic inputs
already resident in HBM.  Inputs cycle through a pool of 8 sets and the
verify seed changes every step.

Prints one JSON line: verify passes/s (value), accepted tokens/s
(sum of n_accepted + 1 per second), whole-step HBM GB/s, the roofline of the
GEMM kernels (algorithmic weight bytes / their event-timed duration vs
8 TB/s), and the float64 CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload mid]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify passes/sec & accepted tokens/sec at B=1, γ=4; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
MFMA_BOUND_ROWS = 112            # above this many rows the three-term MFMA work exceeds the weight stream
POOL = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="mid")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the timed oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def source_hash():
    """Hash of the kernel sources, to tie stored counter readings to them."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verification_06_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, or
    None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))


# ---------------------------------------------------------------- workload (harness side)

def build_inputs(torch, sv, synth, wl, w, key):
    """Pool of (hidden, draft, q) on the device.  The synthetic draft is
    q = softmax(target logits + N(0, sigma)); its logits come from the
    target pass itself (spec_verify_debug), sigma is bisected so the mean
    acceptance sum(min(p', q')) meets the workload's target."""
    B, gamma, V, T = wl.B, wl.gamma, wl.V, wl.temperature
    G1 = gamma + 1
    hid = [synth.normal_torch((*key, synth.T_HIDDEN, i), (B, G1, wl.d), 1.0, "cuda")
           for i in range(POOL)]
    zero_d = torch.zeros((B, gamma), dtype=torch.int32, device="cuda")
    flat_q = torch.full((B, gamma, V), 1.0 / V, device="cuda")
    logits = []
    for h in hid:
        _, _, lg, _, _ = sv.verify_debug(w, h, zero_d, flat_q, 1.0, 1.0, 0, want_probs=False)
        if not bool(torch.isfinite(lg).all()):
            raise RuntimeError("target logits are not finite: the GEMM path is broken")
        logits.append(lg)
    z = [synth.normal_torch((*key, synth.T_NOISE, i), (B, gamma, V), 1.0, "cuda") for i in range(POOL)]
    Tq = T if T > 0 else 1.0

    def q_of(lg, zz, sig):
        return torch.softmax(lg[:, :gamma].double() + sig * zz.double(), dim=-1).float()

    def alpha(sig):
        a = []
        for lg, zz in zip(logits, z):
            p = torch.softmax(lg[:, :gamma].double() / Tq, dim=-1)
            qq = torch.softmax(torch.log(q_of(lg, zz, sig).double()) / Tq, dim=-1)
            a.append(torch.minimum(p, qq).sum(-1).mean().item())
        return sum(a) / len(a)

    if wl.name == "topp":
        gen = synth.generator(*key, synth.T_MISC)
        sig = torch.tensor(gen.uniform(0.2, 1.5, size=B), dtype=torch.float64,
                           device="cuda").view(B, 1, 1)
    elif wl.alpha_target and T > 0:
        lo, hi = 0.01, 4.0
        for _ in range(16):
            mid = 0.5 * (lo + hi)
            lo, hi = (mid, hi) if alpha(mid) > wl.alpha_target else (lo, mid)
        sig = 0.5 * (lo + hi)
    else:
        sig = 0.5
    qs = [q_of(lg, zz, sig) for lg, zz in zip(logits, z)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.torch_seed(*key, synth.T_DRAFT))
    drafts = []
    for lg, qq in zip(logits, qs):
        if T == 0:
            am = lg[:, :gamma].argmax(-1)
            other = torch.randint(0, V - 1, am.shape, generator=gen, device="cuda")
            other = other + (other >= am).long()
            keep = torch.rand(am.shape, generator=gen, device="cuda") < 0.75
            drafts.append(torch.where(keep, am, other).to(torch.int32).contiguous())
            continue
        w_ = torch.softmax(torch.log(qq.double()) / T, dim=-1)
        if wl.top_p < 1.0:
            srt, idx = torch.sort(w_, dim=-1, descending=True, stable=True)
            c = torch.cumsum(srt, -1)
            keep = (c - srt) < wl.top_p
            w_ = torch.zeros_like(w_).scatter(-1, idx, srt * keep)
        d = torch.multinomial(w_.reshape(-1, V).float(), 1, generator=gen).view(B, gamma)
        drafts.append(d.to(torch.int32).contiguous())
    return hid, drafts, qs, sig


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(torch, synth, wl, host_weights, hidden0, sig, key, seconds):
    """The float64 oracle, as it stands, on this host's cores: a bounded
    sample of the same workload (inputs built by the oracle itself)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    B, gamma, V, T = wl.B, wl.gamma, wl.V, wl.temperature
    h = hidden0.cpu().numpy()
    ell = oracle.forward(h, host_weights["blocks"], host_weights["lm_head"], 1e-6)
    zz = synth.noise_np(key, B, gamma, V, 1.0)
    s = sig.cpu().numpy().reshape(-1, 1, 1) if hasattr(sig, "cpu") else sig
    qlog = ell[:, :gamma] + s * zz
    q = np.exp(qlog - qlog.max(-1, keepdims=True))
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    rng = synth.generator(*key, synth.T_DRAFT, 1)
    if T == 0:
        draft = ell[:, :gamma].argmax(-1).astype(np.int32)
    else:
        draft = np.array([[rng.choice(V, p=oracle.warp_probs(q[b, i], T, wl.top_p)[0])
                           for i in range(gamma)] for b in range(B)], dtype=np.int32)
    passes, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        r = oracle.spec_verify(h, host_weights, draft, q, T, wl.top_p, passes)
        passes += 1
        tokens += int((r.n_accepted + 1).sum())
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": passes / el, "unit": "verify passes/s", "cores": int(cores),
            "kind": "oracle", "accepted_tokens_per_s": tokens / el,
            "sample": f"{passes} oracle spec_verify passes of the {wl.name} workload "
                      f"(B={B}, one input set, float64 weights resident) in {el:.1f} s"}


# ---------------------------------------------------------------- main

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    progress("importing torch")
    import torch
    import synth
    import speculative_decoding_verification_06_amd as sv

    wl = synth.WORKLOADS[args.workload]
    key = (300 + list(synth.WORKLOADS).index(wl.name),)
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    model = synth.model_torch(key, wl.d, wl.ffn, wl.n_blocks, wl.V, wl.wdtype, "cuda")
    w = sv.Weights(model["blocks"], model["lm_head"])
    progress(f"weights registered {time.perf_counter() - t_setup:.1f}s")
    host = None
    if not args.no_cpu_baseline:
        f64 = lambda t: t.detach().to("cpu").to(torch.float64).numpy()
        host = {"blocks": [{"w_up": f64(b["w_up"]), "w_down": f64(b["w_down"]), "gain": None}
                           for b in model["blocks"]], "lm_head": f64(model["lm_head"])}
    del model
    torch.cuda.empty_cache()
    hid, drafts, qs, sig = build_inputs(torch, sv, synth, wl, w, key)
    B, gamma, T, top_p = wl.B, wl.gamma, wl.temperature, wl.top_p
    G1 = gamma + 1
    ws = w.workspace(B, gamma)
    K, W = args.steps, args.warmup
    n_out = torch.empty((K, B), dtype=torch.int32, device="cuda")
    e_out = torch.empty((K, B, G1), dtype=torch.int32, device="cuda")
    qarg = [q if T > 0 else None for q in qs]
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f}s workload={wl.name} "
          f"steps={K} warmup={W}", file=sys.stderr, flush=True)

    for k in range(W):
        sv.verify(w, hid[k % POOL], drafts[k % POOL], qarg[k % POOL], T, top_p, 10 ** 6 + k,
                  workspace=ws, n_accepted=n_out[k % K], emitted=e_out[k % K])
    torch.cuda.synchronize()
    progress("warmup done")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(K):
        sv.verify(w, hid[k % POOL], drafts[k % POOL], qarg[k % POOL], T, top_p, k,
                  workspace=ws, n_accepted=n_out[k], emitted=e_out[k])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    progress(f"timed {K} steps: {ms / K:.4f} ms/step")
    n_acc = n_out.cpu()
    tokens = int((n_acc + 1).sum())
    passes_s = K / (ms / 1e3)

    # Kernel timing: the same steps again with every GEMM launch bracketed by
    # HIP events on its stream.
    w.profile(True)
    kp = min(K, 200)
    for k in range(kp):
        sv.verify(w, hid[k % POOL], drafts[k % POOL], qarg[k % POOL], T, top_p, k,
                  workspace=ws, n_accepted=n_out[k], emitted=e_out[k])
    gemm_ms, launches, wbytes = w.profile_read()
    w.profile(False)
    progress("kernel timing done")
    per_launch_bytes = wbytes / launches
    per_launch_s = gemm_ms / 1e3 / launches
    achieved = per_launch_bytes / per_launch_s / 1e9
    # executed bf16 MFMA flops: every fp32 x bf16 product is three bf16
    # products (hi, mid, lo terms), 2 flops each, for M = B (gamma + 1) rows
    M = B * G1
    mfma_tflops = 6.0 * M * (per_launch_bytes / 2) / per_launch_s / 1e12

    weight_bytes = wbytes / kp
    other = 4 * (B * G1 * wl.d + (B * gamma * wl.V if T > 0 else 0) + B * gamma)
    step_gbs = (weight_bytes + other) / (ms / K / 1e3) / 1e9
    traffic = stored_traffic(wl.name)

    out = {
        "metric": METRIC, "value": passes_s, "unit": "verify passes/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": ms / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={B} gamma={gamma} d={wl.d} ffn={wl.ffn} "
                               f"blocks={wl.n_blocks} V={wl.V} {wl.wdtype} weights, "
                               f"T={T} top_p={top_p}",
                   "B": B, "gamma": gamma, "d": wl.d, "ffn": wl.ffn, "blocks": wl.n_blocks,
                   "V": wl.V, "temperature": T, "top_p": top_p},
        "accepted_tokens_per_s": tokens / (ms / 1e3),
        "mean_tokens_per_pass": tokens / (K * B),
        "hbm_gbs_whole_step": step_gbs,
        "hbm_frac_whole_step": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": weight_bytes + other,
        "roofline": ({"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
                     if wl.wdtype == "f32" or M <= MFMA_BOUND_ROWS else
                     {"bound": "mfma", "achieved": mfma_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": mfma_tflops / MFMA_BF16_PEAK_TFLOPS,
                      "traffic": traffic, "hbm_gbs": achieved}),
        "gemm": {"kernel": "weight-streaming GEMMs (MLP up/down, LM head)",
                 "bytes_per_launch": per_launch_bytes, "launches": launches,
                 "avg_launch_us": per_launch_s * 1e6, "hbm_gbs": achieved,
                 "hbm_frac": achieved / HBM_PEAK_GBS, "mfma_tflops": mfma_tflops,
                 "mfma_frac": mfma_tflops / MFMA_BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if host is not None:
        out["cpu_baseline"] = cpu_baseline(torch, synth, wl, host, hid[0], sig, key,
                                           args.cpu_seconds)
    w.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
