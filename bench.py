#!/usr/bin/env python3
"""Benchmark of fused linear cross-entropy forward + backward on one MI355X.

Workload: the large-vocabulary case -- h bf16 [2, 4096, 4096] ~ N(0, 1),
W bf16 [131072, 4096] ~ N(0, 0.02), Zipf(1.1) labels, the first quarter of
each sequence ignored, reduction 'mean' (N = 8192 tokens, H = 4096,
V = 131072). Synthetic, seeded, generated on the host and copied to HBM
before the timed region. One step = one call of flce_forward_backward
(label scan, forward GEMM + log-sum-exp, merge + loss, and per vocabulary
chunk the logit-gradient GEMM, the dW GEMM and the dH GEMM).

Prints one JSON line (the last line of stdout). `value` is tokens/s of the
whole step, timed over a loop of steps with nothing else in it; `roofline`
covers the kernel with the largest share of the step time, timed with HIP
events around each launch on the stream it runs on, in a separate pass after
the timed loop; `configs` times the same step on the small, softcapped and
long configurations; `cpu_baseline` times the float64 oracle on all tokens of
the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/sec @ H=4096,V=131072 bf16; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0
GEMM_KINDS = ("lse_fwd_gemm", "grad_logits_gemm", "dW_gemm", "dH_gemm", "dH_dW_gemm")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_large_vocab.txt")
# Every source of the library: the committed counters are used only while all
# of them are unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "lm_head_linear_amd", "csrc", f)
                  for f in ("kernels_bf16.hip", "kernels_common.hip", "kernels_f32.hip",
                            "flce_api.hip", "flce_check.cpp", "flce_plan.h", "flce_internal.h",
                            "gemm_index.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_tokens(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one
    space: what the compiler sees, so that editing a comment does not count as
    a change of the kernels. String and character literals are kept whole."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """sha256 (first 16 hex digits) over the library sources' code, comments
    and layout left out."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]


def read_traffic(kernel: str):
    """Per-launch HBM bytes of `kernel` from the committed counter summary, or
    None when there is none or the kernels changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != kernel_source_digest():
        return None
    try:
        return float(vals[f"hbm_bytes_per_launch.{kernel}"])
    except (KeyError, ValueError):
        return None


def blas_threads() -> int:
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        n = [d["num_threads"] for d in info if d.get("user_api") == "blas"]
        if n:
            return int(n[0])
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine() or "unknown"


def cpu_baseline(w, n_sample: int):
    """The float64 oracle, as it stands, on the workload (all N tokens when
    n_sample >= N, else every (N // n_sample)-th token) with the full weight;
    tokens/s = tokens run / oracle time."""
    import numpy as np
    import torch
    from oracle import flce_oracle as orc
    N = w.N
    stride = max(1, N // n_sample)
    idx = torch.arange(0, N, stride)[:n_sample]
    h = w.h.reshape(-1, w.H)[idx].to(torch.float64).numpy()
    W = w.W.to(torch.float64).numpy()
    y = w.labels.reshape(-1)[idx].numpy()
    t0 = time.perf_counter()
    r = orc.flce_reference(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                           reduction=w.reduction)
    dt = time.perf_counter() - t0
    assert np.isfinite(r.loss64)
    what = (f"all {N} tokens" if len(idx) == N
            else f"{len(idx)} tokens (every {stride}th of the {N})")
    return {
        "value": len(idx) / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
        "sample": (f"{what} with the full W [{w.V},{w.H}]: one float64 forward+backward of "
                   f"the oracle (materialised logits per 1024 tokens) in {dt:.1f} s; "
                   "bf16->float64 widening not timed"),
        "host_cpu_count": os.cpu_count(), "blas_threads": blas_threads(),
        "cpu_model": cpu_model(),
        "seconds": dt,
    }


def time_steps(fn, steps: int, warmup: int):
    """(host-clock ms, event ms) per call of fn over `steps` timed calls, after
    `warmup` untimed ones, bracketed by device synchronisation."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def other_configs(steps: int, warmup: int, only=None):
    """The full step (flce_forward_backward, bf16) on the other full-size
    configurations: small, softcapped, and long, as one call and as its four
    micro-batches with the shared external token count and dW added up across
    them; each mode timed over at least `steps` calls and about a quarter
    second of them (a short step gets more). `only`: the names of the
    configurations to time (all three when None). Returns {name: figures}."""
    import torch
    import flce_inputs as fi
    import lm_head_linear_amd as m
    dev = torch.device("cuda:0")
    out = {}
    for k in (2, 4, 5):
        if only and fi.RECIPES[k]["name"] not in only:
            continue
        w = fi.make_workload(k)
        N, H, V = w.N, w.H, w.V
        h = w.h.reshape(N, H).to(dev)
        W = w.W.to(dev)
        y = w.labels.reshape(N).to(dev)
        dH, dW = torch.empty_like(h), torch.empty_like(W)
        loss = torch.empty((), dtype=torch.float32, device=dev)
        nt = torch.empty((), dtype=torch.int64, device=dev)
        kw = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
                  num_label_tokens=w.num_label_tokens, loss=loss, num_tokens=nt)
        # each mode with a workspace of its own, allocated for it alone, so
        # that the peak extra memory is that mode's
        def one_call(ws):
            m.flce_forward_backward(h, W, y, dH=dH, dW=dW, workspace=ws, **kw)

        def flops(lab, acc):
            n = lab.numel()
            return step_flops(n, int((lab != w.ignore_index).sum()), H, V,
                              m.flce_vocab_chunk(n, H, V, W.dtype),
                              m.flce_kept_chunks(n, H, V, W.dtype, acc))["step"]
        lab_all = w.labels.reshape(N)
        modes = {"one_call": (N, one_call, flops(lab_all, False))}
        if w.micro_batches > 1:
            nb = N // w.micro_batches

            def micro(ws):
                for i in range(w.micro_batches):
                    s = slice(i * nb, (i + 1) * nb)
                    m.flce_forward_backward(h[s], W, y[s], dH=dH[s], dW=dW, workspace=ws,
                                            accumulate_dW=i > 0,
                                            mb_scale=m.micro_batch_scale(0, 0, w.reduction), **kw)
            modes[f"{w.micro_batches}_micro_batches"] = (
                nb, micro, sum(flops(lab_all[i * nb:(i + 1) * nb], i > 0)
                               for i in range(w.micro_batches)))
        res = {"N": N, "H": H, "V": V, "softcap": w.softcap, "reduction": w.reduction,
               "num_label_tokens": w.num_label_tokens, "logits_f32_bytes_avoided": int(N * V * 4)}
        nhv = float(N) * H * V
        for name, (n_call, fn, xfl) in modes.items():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = torch.cuda.memory_allocated(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            ws = torch.empty(m.flce_workspace_size(n_call, H, V, W.dtype), dtype=torch.uint8,
                             device=dev)
            # at least `steps` timed calls, more for a short step: about a
            # quarter second of them, after a tenth as many warm-up calls
            for _ in range(warmup):
                fn(ws)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn(ws)
            torch.cuda.synchronize()
            est = max(time.perf_counter() - t0, 1e-5)
            n_steps = int(min(max(steps, 0.25 / est), 2000))
            ms, ev_ms = time_steps(lambda: fn(ws), n_steps, max(warmup, n_steps // 10))
            torch.cuda.synchronize()
            res[name] = {"ms_per_step": round(ms, 4), "event_ms_per_step": round(ev_ms, 4),
                         "steps": n_steps,
                         "tokens_per_s": round(N / ms * 1e3, 1),
                         "mfma_frac_8nhv": round(8.0 * nhv / (ms * 1e-3) / 1e12
                                                 / PEAK_BF16_TFLOPS, 4),
                         "mfma_frac_6nhv": round(6.0 * nhv / (ms * 1e-3) / 1e12
                                                 / PEAK_BF16_TFLOPS, 4),
                         "mfma_frac_executed": round(xfl / (ms * 1e-3) / 1e12
                                                     / PEAK_BF16_TFLOPS, 4),
                         "workspace_bytes": int(ws.numel()),
                         "extra_memory_bytes": int(torch.cuda.max_memory_allocated(dev) - base)}
            log(f"{w.name} {name}: {ms:.3f} ms/step, "
                f"{res[name]['extra_memory_bytes'] / 2**20:.0f} MiB extra")
            del ws
        out[w.name] = res
        del h, W, y, dH, dW
        torch.cuda.empty_cache()
    return out


def copy_calibration(size_mib: int, reps: int):
    """A plain device copy of known size, to scale the HBM byte counters."""
    import torch
    n = size_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {size_mib} MiB")


def other_modes(m, w, h, W, y, dH, dW, loss, nt, steps, timing, nhv):
    """The forward-only entry, float32 gradients and the no-recompute variant
    on the same inputs, each timed like the main step, after it (so they
    cannot disturb it)."""
    import torch
    N, H = h.shape
    V = W.shape[0]
    dev = h.device
    # The forward-only entry (loss and lse, no gradients) on the same inputs,
    # timed the same way, after the step timing so it cannot disturb it.
    fws = torch.empty(m.flce_forward_workspace_size(N, H, V, W.dtype), dtype=torch.uint8,
                      device=dev)

    def fwd():
        m.flce_forward(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                       reduction=w.reduction, workspace=fws, loss=loss, num_tokens=nt)

    for _ in range(2):
        fwd()
    torch.cuda.synchronize()
    tf0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    f_ms = (time.perf_counter() - tf0) * 1e3 / steps
    n_kept = int((w.labels != w.ignore_index).sum())
    forward_only = {"ms_per_call": round(f_ms, 4), "tokens_per_s": round(N / (f_ms * 1e-3), 1),
                    "tflops_executed": round(2.0 * n_kept * H * V / (f_ms * 1e-3) / 1e12, 1),
                    "workspace_bytes": int(fws.numel())}
    log(f"forward only: {f_ms:.3f} ms/call, {forward_only['tflops_executed']:.1f} TFLOP/s "
        f"over the {n_kept} kept tokens")

    # The same forward handing back the logits ([N, V], bf16 then float32):
    # the extra time is the logits' write.
    for name, dt in (("with_logits_bf16", torch.bfloat16), ("with_logits_f32", torch.float32)):
        lg = torch.empty(N, V, dtype=dt, device=dev)

        def fwd_logits():
            m.flce_forward_logits(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                                  reduction=w.reduction, workspace=fws, loss=loss,
                                  num_tokens=nt, logits=lg)

        for _ in range(2):
            fwd_logits()
        torch.cuda.synchronize()
        tl0 = time.perf_counter()
        for _ in range(steps):
            fwd_logits()
        torch.cuda.synchronize()
        l_ms = (time.perf_counter() - tl0) * 1e3 / steps
        nbytes = lg.numel() * lg.element_size()
        forward_only[name] = {"ms_per_call": round(l_ms, 4), "logits_bytes": int(nbytes),
                              "extra_ms": round(l_ms - f_ms, 4)}
        log(f"forward + {dt} logits: {l_ms:.3f} ms/call ({nbytes / 1e9:.2f} GB of logits, "
            f"+{l_ms - f_ms:.3f} ms)")
        del lg

    # Float32 gradients for the same bf16 inputs (G as a bf16 hi + lo pair,
    # twice the dW/dH work), timed the same way.
    gws = torch.empty(m.flce_workspace_size(N, H, V, W.dtype, torch.float32), dtype=torch.uint8,
                      device=dev)
    dH32 = torch.empty(N, H, dtype=torch.float32, device=dev)
    dW32 = torch.empty(V, H, dtype=torch.float32, device=dev)

    def step32():
        m.flce_forward_backward(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                                reduction=w.reduction, dH=dH32, dW=dW32, workspace=gws,
                                loss=loss, num_tokens=nt, grad_dtype=torch.float32)

    n32 = max(1, steps // 2)
    for _ in range(2):
        step32()
    torch.cuda.synchronize()
    tg0 = time.perf_counter()
    for _ in range(n32):
        step32()
    torch.cuda.synchronize()
    g_ms = (time.perf_counter() - tg0) * 1e3 / n32
    float32_grads = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(N / (g_ms * 1e-3), 1),
                     "steps": n32, "workspace_bytes": int(gws.numel())}
    log(f"float32 gradients: {g_ms:.3f} ms/step")
    del dH32, dW32, gws

    # The no-recompute variant on the same inputs (token chunks whose
    # probabilities are kept instead of recomputing the logits), timed the
    # same way, with its per-kernel split.
    nws = torch.empty(m.flce_workspace_size_nr(N, H, V, W.dtype), dtype=torch.uint8, device=dev)

    def step_nr():
        m.flce_forward_backward(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                                reduction=w.reduction, dH=dH, dW=dW, workspace=nws, loss=loss,
                                num_tokens=nt, recompute=False)

    for _ in range(2):
        step_nr()
    torch.cuda.synchronize()
    tn0 = time.perf_counter()
    for _ in range(steps):
        step_nr()
    torch.cuda.synchronize()
    n_ms = (time.perf_counter() - tn0) * 1e3 / steps
    nr_kernels = {}
    if timing:
        m.flce_profile_begin()
        for _ in range(3):
            step_nr()
        torch.cuda.synchronize()
        m.flce_profile_end()
        nr_kernels = {k: round(ms / 3, 4) for k, (ms, n) in m.flce_profile_query().items() if n}
    no_recompute = {"ms_per_step": round(n_ms, 4), "tokens_per_s": round(N / (n_ms * 1e-3), 1),
                    "tflops_executed": round(6.0 * n_kept * H * V / (n_ms * 1e-3) / 1e12, 1),
                    "token_chunk": m.flce_token_chunk_nr(N, H, V, W.dtype),
                    "workspace_bytes": int(nws.numel()), "kernels_ms_per_step": nr_kernels}
    log(f"no recompute: {n_ms:.3f} ms/step {nr_kernels}")
    del nws
    return forward_only, float32_grads, no_recompute


def step_flops(N: int, n_kept: int, H: int, V: int, vchunk: int, kept: int = 1,
               lse_out: bool = False) -> dict:
    """Matrix flops each GEMM kind executes per step of flce_forward_backward
    (bf16, bf16 gradients). The call gathers the non-ignored tokens first: an
    ignored token's loss is 0 and its logit gradient exactly zero, so the
    forward runs over the n_kept kept tokens (over all N when per-token lse is
    asked for) and the recompute, dW and dH over the kept ones. The forward
    keeps the probabilities of the first `kept` vocabulary chunks
    (flce_kept_chunks), so the recompute covers the other V - kept vchunk
    rows. dH_dW_gemm is a chunk's dH and dW in one grid; 'step' is the sum over
    the step."""
    fwd, bwd = 2.0 * (N if lse_out else n_kept) * H * V, 2.0 * n_kept * H * V
    rec = 2.0 * n_kept * H * max(V - kept * vchunk, 0)
    return {"lse_fwd_gemm": fwd, "grad_logits_gemm": rec, "dW_gemm": bwd, "dH_gemm": bwd,
            "dH_dW_gemm": 2.0 * bwd, "step": fwd + rec + 2.0 * bwd}


def kernel_pass(m, step, steps: int, flops: dict):
    """Per-kernel HIP-event timing over `steps` extra steps, run after the
    headline loop (events bracket every launch on the call's stream, so this
    pass is not the one `value` comes from). `flops`: executed matrix flops
    per step of each GEMM kind. Returns (kernels, roofline)."""
    import torch
    m.flce_profile_begin()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    m.flce_profile_end()
    kernels = {}
    for name, (ms, n) in m.flce_profile_query().items():
        if n == 0:
            continue
        e = {"ms_per_step": ms / steps, "launches_per_step": n / steps, "avg_launch_ms": ms / n}
        if name in GEMM_KINDS:
            e["tflops"] = flops[name] * steps / (ms * 1e-3) / 1e12
        kernels[name] = e
    dom = max(GEMM_KINDS, key=lambda k: kernels.get(k, {}).get("ms_per_step", 0.0))
    d = kernels[dom]
    flops_per_launch = flops[dom] / d["launches_per_step"]
    achieved = flops_per_launch / (d["avg_launch_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": read_traffic(dom), "kernel": dom,
                "flops_per_launch": flops_per_launch,
                "avg_launch_ms": round(d["avg_launch_ms"], 4),
                "timing": f"HIP events around each launch, {steps} steps after the timed loop"}
    for k, v in kernels.items():
        log(f"  {k:18s} {v['ms_per_step']:8.3f} ms/step  {v['launches_per_step']:.0f} launches"
            + (f"  {v['tflops']:7.1f} TFLOP/s" if "tflops" in v else ""))
    return kernels, roofline


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens the oracle baseline runs (0: all N)")
    ap.add_argument("--kernel-steps", type=int, default=-1,
                    help="steps of the separate per-kernel event pass (-1: --steps, 0: none)")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the main path (no other entry points and no other "
                         "configurations), e.g. for per-kernel counter runs")
    ap.add_argument("--no-configs", action="store_true",
                    help="leave out the small, softcapped and long configurations")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain copy of this size (counter calibration)")
    ap.add_argument("--configs", action="store_true",
                    help="only time the full step on the small, softcapped and long "
                         "configurations (one JSON line of its own)")
    ap.add_argument("--only", action="append", default=None, metavar="NAME",
                    choices=("small", "softcapped", "long_edge"),
                    help="with --configs: time this configuration (repeatable; default all)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 10)
        return

    import flce_inputs as fi
    import lm_head_linear_amd as m
    from lm_head_linear_amd import _lib
    _lib.load()
    if args.configs:
        print(json.dumps({"configs": other_configs(args.steps, args.warmup, args.only)}),
              flush=True)
        return

    dev = torch.device("cuda:0")
    t = time.perf_counter()
    w = fi.make_workload(3)
    N, H, V = w.N, w.H, w.V
    log(f"workload {w.name}: N={N} H={H} V={V} generated in {time.perf_counter() - t:.1f} s")
    h = w.h.reshape(N, H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(N).to(dev)
    dH = torch.empty_like(h)
    dW = torch.empty_like(W)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    nt = torch.empty((), dtype=torch.int64, device=dev)
    ws_bytes = m.flce_workspace_size(N, H, V, W.dtype)
    vchunk = m.flce_vocab_chunk(N, H, V, W.dtype)
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        m.flce_forward_backward(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                                reduction=w.reduction, dH=dH, dW=dW, workspace=ws, loss=loss,
                                num_tokens=nt)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); loss={loss.item():.6f} num_tokens={nt.item()}")

    # The headline loop: nothing but the steps (no per-launch events).
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_mem
    log(f"timed {args.steps} steps: {wall_ms:.3f} ms/step (host clock), {ev_ms:.3f} ms/step (events)")

    nhv = float(N) * H * V
    tflops_8 = 8 * nhv / (wall_ms * 1e-3) / 1e12
    tflops_6 = 6 * nhv / (wall_ms * 1e-3) / 1e12
    n_kept = int((w.labels != w.ignore_index).sum())
    kept_chunks = m.flce_kept_chunks(N, H, V, W.dtype)
    flops = step_flops(N, n_kept, H, V, vchunk, kept_chunks)
    x_step = flops["step"]
    tflops_x = x_step / (wall_ms * 1e-3) / 1e12
    kernels, roofline = {}, None
    ksteps = args.steps if args.kernel_steps < 0 else args.kernel_steps
    if ksteps > 0:
        kernels, roofline = kernel_pass(m, step, ksteps, flops)

    forward_only = float32_grads = no_recompute = None
    configs = None
    if not args.main_only:
        forward_only, float32_grads, no_recompute = other_modes(
            m, w, h, W, y, dH, dW, loss, nt, args.steps, ksteps > 0, nhv)
        if not args.no_configs:
            del h, W, y, dH, dW, ws
            torch.cuda.empty_cache()
            configs = other_configs(max(3, args.steps // 4), 2)

    cpu = None
    if not args.no_cpu_baseline:
        n_cpu = args.cpu_sample_tokens if args.cpu_sample_tokens > 0 else N
        log(f"cpu baseline: oracle on {n_cpu} of {N} tokens ...")
        cpu = cpu_baseline(w, n_cpu)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": round(N * args.steps / (t1 - t0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"large_vocab: h bf16 [2,4096,4096], W bf16 [131072,4096], "
                                "Zipf(1.1) labels, first quarter of each sequence ignored, "
                                "reduction=mean"),
                   "N": N, "H": H, "V": V, "vocab_chunk": vchunk,
                   "kept_chunks": kept_chunks},
        "mfma_frac_8nhv": round(tflops_8 / PEAK_BF16_TFLOPS, 4),
        "mfma_frac_6nhv": round(tflops_6 / PEAK_BF16_TFLOPS, 4),
        "tflops_8nhv": round(tflops_8, 1),
        "tokens_kept": n_kept,
        "executed_flops_per_step": x_step,
        "tflops_executed": round(tflops_x, 1),
        "mfma_frac_executed": round(tflops_x / PEAK_BF16_TFLOPS, 4),
        "event_ms_per_step": round(ev_ms, 4),
        "extra_memory_bytes": int(peak_extra),
        "workspace_bytes": int(ws_bytes),
        "roofline": roofline,
        "forward_only": forward_only,
        "float32_grads": float32_grads,
        "no_recompute": no_recompute,
        "configs": configs,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": ({k: (round(v, 3) if isinstance(v, float) else v)
                          for k, v in cpu.items() if k != "seconds"} if cpu else None),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
