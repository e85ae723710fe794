"""Throughput of batched speculative-sampling verification on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload selfdraft] [--gpus 1]

One step = one sv_verify call (sv_vat_labels for --workload vat, sv_vat_loss
for --workload vat_loss, sv_vat_loss_grad for --workload vat_loss_grad: the
gradient of the VAT loss with respect to the draft logits, kernel k_vat_grad,
after one sv_vat_loss call outside the timed region) over one
batch of synthetic logits already resident in HBM; the call is the whole path
(one launch of the task-grid kernel k_verify, or of k_vat_grad).  The default workload is the
quantized-self-drafter batch: B=128 sequences, k=5 draft positions,
V=151936, bf16 target and draft logits, T=1.  Prints ONE JSON line.

  value        verified draft positions per second = B*k*K / wall time of K
               steps (synchronised on both sides); VAT: labelled positions
  roofline     k_verify: algorithmic bytes per launch (every logit the path
               needs, read once: the k target and k draft rows of every
               sequence, and target row k of the sequences that kept all k
               drafts, the only ones that draw from it) / its mean duration, measured live with HIP
               events recorded on the launch stream around the K timed
               launches (per-launch events would add several microseconds
               of stream work between launches);
               `traffic` = HBM bytes per launch from committed rocprofv3
               FETCH_SIZE/WRITE_SIZE counters when they were taken on the
               current kernel source, else null
  cpu_baseline the fp64 oracle on a bounded sample of the same workload on
               the host (single thread)

Inputs rotate through enough copies that each timed sweep touches more than
twice the 256 MB last-level (MALL) cache, so the figures are HBM figures.
The default warm-up (200 calls, tens of milliseconds) lets the GPU reach its
steady clocks; with a few warm-up calls the first timed calls run slower.

    python bench.py --workload lmhead_selfdraft|lmhead_grpo [--steps K]

times greedy verification with the target's logits formed inside the call
from its hidden states and output layer (sv_verify_lm_head_greedy: the
GEMM with its argmax epilogue, then the per-sequence finisher), B(k+1)
hidden states of size D=4096 against a [151936][4096] bf16 output layer.
value = verified draft positions per second; roofline: the GEMM's
2 B(k+1) V D flops per launch / its mean duration (HIP events recorded
around every GEMM launch on the launch stream) against the bf16 dense MFMA
peak.  --workload lmhead_sample_selfdraft|lmhead_sample_grpo does the same
for sampling verification (sv_verify_lm_head, T > 0): the GEMM timed is the
statistics pass over the B(k+1) target and B k draft rows (which also stores
every row's fp32 logits); the step also holds the decisions and the draws.

    python bench.py --copy-probe [--steps K]

runs K plain device-to-device copies of 1 GiB (torch's copy kernel) and
nothing else: the known-size reference that scales rocprofv3's FETCH_SIZE and
WRITE_SIZE counters to bytes.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 * 2**20
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence
METRIC = "verified draft positions/sec + achieved HBM GB/s (V=151936 bf16, k=5..16)"


class HipEvents:
    """Raw hipEvent_t handles recorded on the launch stream (torch.cuda.Event
    would record on torch's current stream, which need not be it)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        # No system-scope fence at record time: the events only timestamp the
        # launch stream and should disturb it as little as possible.
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return ev.value

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_ms(self, a, b) -> float:
        self.hip.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("sv_kernels.hip", "sv_launch.h"):
        with open(os.path.join(ROOT, "speculative_decoding_verification_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, source_hash=None):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != (source_hash or kernel_source_hash()):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, seconds: float, loss: bool = False, grad: bool = False):
    """The oracle as it is (plain fp64 C, one thread) over whole sequences (VAT:
    blocks) of the same workload until `seconds` of CPU work have elapsed; the
    sample is drawn on the host by the same seeded generator.  With `grad`, the
    loss and then its gradient with respect to the draft logits."""
    import oracle
    import workloads

    n_sample = min(cfg.B, 32 if cfg.kind == "verify" else 4)
    wl = workloads.generate(cfg, 0, n_sample)
    done = 0
    t0 = time.perf_counter()
    step = 4 if cfg.kind == "verify" else 1
    while True:
        lo = done % n_sample
        hi = min(n_sample, lo + step)
        d = wl.draft[lo:hi] if wl.draft is not None else None
        if loss:
            r = oracle.vat_loss(wl.target[lo:hi], d, wl.tokens[lo:hi], wl.uniforms[lo:hi], wl.hard_tokens[lo:hi],
                                cfg.T, cfg.decay, 1.0)
            if grad:
                oracle.vat_loss_grad(wl.target[lo:hi], d, wl.hard_tokens[lo:hi], r.weights, cfg.T, 1.0)
        elif cfg.kind == "vat":
            oracle.vat_labels(wl.target[lo:hi], d, wl.tokens[lo:hi], wl.uniforms[lo:hi], cfg.T, cfg.decay)
        else:
            oracle.verify(wl.target[lo:hi], d, wl.tokens[lo:hi], wl.uniforms[lo:hi], cfg.T, onehot=cfg.onehot)
        done += hi - lo
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    what = "blocks" if cfg.kind == "vat" else "sequences"
    if loss:
        what = "blocks (labels, loss and its gradient)" if grad else "blocks (labels and loss)"
    return {"value": done * cfg.k / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": "%d whole %s (%d positions; cycling over the first %d) of the %s workload, fp64 C oracle, "
                      "1 thread, %.1f s" % (done, what, done * cfg.k, n_sample, cfg.name, dt),
            "host_cpu": platform.processor() or platform.machine(), "host_nproc": os.cpu_count()}


def lm_kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("sv_lmhead.hip", "sv_lmhead.h"):
        with open(os.path.join(ROOT, "speculative_decoding_verification_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def lm_cpu_baseline(cfg, wl, seconds: float):
    """The oracle as it is over whole sequences of the LM-head workload (fp64
    logits over the full vocabulary, one thread) until `seconds` elapsed."""
    import oracle

    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % cfg.B
        if cfg.T > 0:
            oracle.lm_head_verify(wl.target_hidden[b:b + 1], wl.target_weight, wl.draft_hidden[b:b + 1],
                                  wl.draft_weight, wl.tokens[b:b + 1], wl.uniforms[b:b + 1], cfg.T)
        else:
            oracle.lm_head_greedy(wl.hidden[b:b + 1], wl.weight, wl.tokens[b:b + 1])
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done * cfg.k / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": "%d whole sequences (%d positions, %d logits of dimension %d each) of the %s workload, fp64 C "
                      "oracle, 1 thread, %.1f s" % (done, done * cfg.k, done * (cfg.k + 1 + (cfg.k if cfg.T > 0 else 0))
                                                    * cfg.V, cfg.D, cfg.name, dt),
            "host_cpu": platform.processor() or platform.machine(), "host_nproc": os.cpu_count()}


def bench_lm_head(args) -> int:
    import torch

    import speculative_decoding_verification_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    cfg = workloads.LM_CONFIGS[args.workload]
    sample = cfg.T > 0
    print("bench: generating %s (B=%d k=%d V=%d D=%d T=%g)" % (cfg.name, cfg.B, cfg.k, cfg.V, cfg.D, cfg.T),
          file=sys.stderr, flush=True)
    if sample:
        wl = workloads.generate_lm_head_sample(cfg)
        th, tw, dh, dw, x, u = workloads.lm_head_sample_to_device(wl, dev)
        ver = sv.LmHeadSampler(th, tw, dh, dw, x, u, cfg.T)
        tensors = (th, tw, dh, dw, x, u)
    else:
        wl = workloads.generate_lm_head(cfg)
        h, w, x = workloads.lm_head_to_device(wl, dev)
        ver = sv.LmHeadVerifier(h, w, x)
        tensors = (h, w, x)
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    region = (ev.create(), ev.create())
    print("bench: %d warmup + %d timed steps" % (args.warmup, args.steps), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        ver(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(region[0], stream)
    for i in range(args.steps):
        ver.set_probe(pairs[i])
        ver(stream)
    ev.record(region[1], stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gemm_ms = sum(ev.elapsed_ms(a, b) for a, b in pairs) / args.steps
    step_device_ms = ev.elapsed_ms(*region) / args.steps
    ver.set_probe(None)
    for e in [e for p in pairs for e in p] + list(region):
        ev.destroy(e)
    acc = ver.accepted_len.float()
    # the GEMM the events bracket: target rows (and, sampling, draft rows)
    flops = cfg.flops() + (2 * cfg.B * cfg.k * cfg.V * cfg.D if sample else 0)
    tflops = flops / (gemm_ms * 1e-3) / 1e12
    ms_per_step = elapsed * 1e3 / args.steps
    res = {
        "metric": METRIC,
        "value": cfg.B * cfg.k * args.steps / elapsed,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": cfg.B, "draft_positions": cfg.k, "vocab": cfg.V,
                   "hidden": cfg.D, "temperature": cfg.T, "weights": "bf16", "accumulate": "f32",
                   "draft_output_layer": "shared with the target" if sample else None},
        "roofline": {"bound": "mfma", "kernel": "k_lmhead_gemm<stats>" if sample else "k_lmhead_gemm<argmax>",
                     "achieved": tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("k_lmhead_gemm", args.workload, lm_kernel_source_hash()),
                     "flops_per_launch": flops, "mean_launch_us": gemm_ms * 1e3,
                     "weight_bytes_per_launch": cfg.V * cfg.D * 2,
                     "hbm_floor_us": cfg.V * cfg.D * 2 / (HBM_PEAK_GBPS * 1e9) * 1e6},
        "device_ms_per_step": step_device_ms,
        "mean_accepted_len": acc.mean().item(),
        "full_acceptance": int((acc == cfg.k).sum().item()),
    }
    del ver, tensors
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (%.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        res["cpu_baseline"] = lm_cpu_baseline(cfg, wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def copy_probe(steps: int) -> int:
    import torch

    dev = torch.device("cuda:0")
    n = 2**30 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": steps + 1,
                      "us_per_copy": dt * 1e6, "gbps_read_plus_write": 2 * n * 4 / dt / 1e9}), flush=True)
    return 0


def _launchers(cfg, sets, sv, n, loss=False):
    """One prepared call per resident input copy (they rotate)."""
    out = []
    for i in range(n):
        if loss:
            t, d, x, u, h = sets[i % len(sets)]
            out.append(sv.VatLoss(t, d, x, u, h, cfg.T, cfg.decay, 1.0))
            continue
        t, d, x, u = sets[i % len(sets)]
        if cfg.kind == "vat":
            out.append(sv.VatLabeler(t, d, x, u, cfg.T, cfg.decay))
        else:
            out.append(sv.Verifier(t, d, x, u, cfg.T, onehot=cfg.onehot))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="selfdraft",
                    choices=["selfdraft", "ngram_tail", "grpo", "grpo_greedy", "vat", "vat_loss", "vat_loss_grad", "tiny",
                             "lmhead_selfdraft", "lmhead_grpo", "lmhead_sample_selfdraft", "lmhead_sample_grpo"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; --gpus %d is not supported (the path shards by sequence "
              "with no exchange, so N GPUs would each run this single-GPU step)" % args.gpus, file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no HIP device", file=sys.stderr)
        return 1
    if args.copy_probe:
        return copy_probe(args.steps)

    if args.workload.startswith("lmhead_"):
        return bench_lm_head(args)

    import speculative_decoding_verification_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    grad = args.workload == "vat_loss_grad"
    loss = args.workload in ("vat_loss", "vat_loss_grad")
    cfg = workloads.get_config("vat" if loss else args.workload)
    print("bench: generating %s (B=%d k=%d V=%d %s T=%g)" % (cfg.name, cfg.B, cfg.k, cfg.V, cfg.dtype, cfg.T),
          file=sys.stderr, flush=True)
    in_bytes = cfg.algorithmic_bytes()
    copies = max(1, math.ceil(2 * MALL_BYTES / in_bytes))
    if cfg.kind == "vat":
        # 33.6 GB: drawn on the device (same distributions, torch's generator)
        sets = [workloads.generate_on_device(cfg, dev)]
        if loss:
            sets[0] = sets[0] + (workloads.hard_tokens_on_device(cfg, sets[0][0], dev),)
        for _ in range(copies - 1):
            sets.append(tuple(a.clone() for a in sets[0]))
    else:
        wl = workloads.generate(cfg)
        sets = [workloads.to_device(wl, dev) for _ in range(copies)]
        del wl
    ev = HipEvents()
    n_launch = args.warmup + args.steps
    if grad:
        # the gradient pass consumes what sv_vat_loss wrote for the same logits
        t, d, x, u, h = sets[0]
        pre = sv.VatLoss(t, d, x, u, h, cfg.T, cfg.decay, 1.0, return_row_stats=True)()
        calls = [sv.VatLossGrad(t, d, h, pre.weights, pre.row_stats, cfg.T, 1.0)]
    else:
        calls = _launchers(cfg, sets, sv, len(sets), loss)
    stream = torch.cuda.current_stream(dev).cuda_stream
    region = (ev.create(), ev.create())

    print("bench: %d copies of %.1f MB, %d warmup + %d timed steps" % (copies, in_bytes / 1e6, args.warmup,
                                                                        args.steps), file=sys.stderr, flush=True)
    for i in range(args.warmup):
        calls[i % len(calls)](stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(region[0], stream)
    for i in range(args.warmup, n_launch):
        calls[i % len(calls)](stream)
    ev.record(region[1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    # The only work on the stream inside the region is the K launches of the
    # kernel, back to back: the region's device time over K is the kernel's
    # average launch duration (any gap between launches counts against it).
    k1_mean = ev.elapsed_ms(*region) / args.steps
    ms_per_step = elapsed * 1e3 / args.steps
    positions = cfg.positions() * args.steps
    value = positions / elapsed
    kernel = "k_vat_grad" if grad else "k_verify"
    last = calls[(n_launch - 1) % len(calls)]
    if grad:
        rows = cfg.B * cfg.k
        zero_rows = int((pre.weights == 0).sum().item())
        # every row's gradient is written (fp32); rows of weight 0 read no logits
        needed = rows * cfg.V * 4 + (rows - zero_rows) * cfg.V * 2 * cfg.elem_bytes
        extra = {"mean_block_loss": pre.block_loss.float().mean().item(), "zero_weight_rows": zero_rows}
        in_bytes = rows * cfg.V * (4 + 2 * cfg.elem_bytes)
    elif cfg.kind == "vat":
        fr = last.first_reject.float()
        extra = {"mean_first_reject": fr.mean().item(), "timeouts": int((fr == -2).sum().item())}
        if loss:
            extra["mean_block_loss"] = last.block_loss.float().mean().item()
        needed = in_bytes
    else:
        acc = last.accepted_len.float()
        full = int((acc == cfg.k).sum().item())
        extra = {"mean_accepted_len": acc.mean().item(), "timeouts": int((acc == -2).sum().item()),
                 "full_acceptance": full}
        # every input copy holds the same logits, so every call needs the
        # same rows: the decision rows of all sequences and the bonus row
        # (target position k) of those that kept all k drafts
        needed = in_bytes - (cfg.B - full) * cfg.V * cfg.elem_bytes
        # acceptance telemetry: the histogram of accepted lengths after a call
        hist = sv.accept_histogram(last.accepted_len, cfg.k)
        torch.cuda.synchronize()
        ev.record(region[0], stream)
        for _ in range(200):
            sv.accept_histogram(last.accepted_len, cfg.k, out=hist, stream=stream)
        ev.record(region[1], stream)
        torch.cuda.synchronize()
        ctl = sv.DraftLengthController()
        ctl.update(hist.cpu())
        extra["accept_histogram_us"] = ev.elapsed_ms(*region) / 200 * 1e3
        extra["block_efficiency"] = ctl.efficiency
    achieved = needed / (k1_mean * 1e-3) / 1e9
    for e in region:
        ev.destroy(e)
    del calls, sets

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": cfg.B, "draft_positions": cfg.k, "vocab": cfg.V,
                   "logits": cfg.dtype, "temperature": cfg.T, "draft": "one-hot" if cfg.onehot else "logits",
                   "input_copies_rotated": copies},
        "hbm_gbps_whole_step": needed / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(kernel, args.workload),
                     "algorithmic_bytes_per_launch": needed, "all_rows_bytes_per_launch": in_bytes,
                     "mean_launch_us": k1_mean * 1e3},
    }
    res.update(extra)
    if cfg.kind == "vat":
        res["config"]["decay"] = cfg.decay
    if loss:
        res["config"]["hard_weight"] = 1.0
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (%.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, loss, grad)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
