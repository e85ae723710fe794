"""Throughput of batched speculative-sampling verification on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload selfdraft] [--gpus 1]

One step = one sv_verify call over one batch of synthetic logits already
resident in HBM; the call is the whole path (one launch of the task-grid
kernel k_verify).  The default workload is the quantized-self-drafter batch:
B=128 sequences, k=5 draft positions, V=151936, bf16 target and draft
logits, T=1.  W untimed calls, then exactly K timed calls, synchronised on
both sides.  Prints ONE JSON line:

  value        verified draft positions per second = B*k*K / wall time of K
               steps
  dtype        the logits' storage type (the arithmetic is fp32: config)
  roofline     k_verify: algorithmic bytes per launch (every logit of the
               workload read once: k+1 target rows and, with draft logits,
               k draft rows per sequence) / its mean launch duration,
               measured live with HIP events recorded on the launch stream
               around the K timed launches (per-launch events would add
               stream work between launches); also the bytes this call
               needed (the bonus row only of sequences that kept all k) and
               that fraction; `traffic` = HBM bytes per launch from
               committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters when they
               were taken on the current kernel source, else null, and
               `traffic_gbps` = that over the mean launch
  sol          k_sol_read (sv_sol_read: a plain non-temporal read) over the
               needed bytes, buffers rotated the same way: its mean launch
               duration and sol/k_verify
  call_us      p10 / p50 / p90 of single calls' device time (each between
               its own events), 200 calls after the timed steps
  accept_rate, mean_accepted_len, full_acceptance, block_efficiency,
  accept_histogram
               acceptance of the last call (accept_rate = accepted drafts /
               tested drafts; the histogram counts accepted lengths 0..k,
               then invalid, timed out, other)
  parity_sample
               the fp64 oracle on the first 32 sequences next to the GPU's
               outputs for them, outside any timed region: positions whose
               acceptance test is within 1e-5 of its threshold, draws within
               1e-5 of an interval end (both may legitimately differ between
               fp32 and fp64; *_differ: those the GPU resolved otherwise)
               and sequences that differ anywhere else (expect 0)
  workloads    the same figures for the n-gram tail (B=8, k=16, one-hot
               drafts) and GRPO batches (B=320, k=7, T=0.6 and T=0), each
               after 200 warm-up calls over 500 timed calls
  cpu_baseline the fp64 oracle on a bounded sample of the same workload on
               the host: all the process's host threads, each taking whole
               sequences (reported), and one thread (nested)

Inputs rotate through enough copies that each timed sweep touches more than
twice the 256 MB last-level (MALL) cache, so the figures are HBM figures.
The side workloads run first and about 0.3 s of plain reads of the
headline's bytes (no kernel call) come right before its warm-up, so the GPU
is at its steady clocks before the headline's warm-up even when W is small.

    python bench.py --workload ngram_tail|grpo|grpo_greedy [--no-side]

makes that workload the headline.  --workload vat|vat_loss|vat_loss_grad
times sv_vat_labels, sv_vat_loss, or sv_vat_loss_grad (the gradient of the
VAT loss with respect to the draft logits, kernel k_vat_grad, after one
sv_vat_loss call outside the timed region) on N=2048 blocks of k=16 fp32
rows of V=128256; `sol` is then sv_sol_read over the logits, or, for the
gradient, sv_sol_read_write (both logit arrays read, the fp32 gradient
written) over the same buffers.

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

    python bench.py --blas-probe [--steps K]

times the library GEMM (torch.matmul, hipBLASLt) on the LM-head operands of
lmhead_selfdraft and lmhead_grpo, writing the bf16 logits instead of reducing
them: the reference for the LM-head GEMM's MFMA rate (one JSON line per
shape; a kernel trace names the kernel the library picks).
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

import numpy as np

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


def _oracle_call(cfg, wl, lo, hi, loss=False, grad=False):
    """The oracle on sequences (VAT: blocks) [lo, hi) of a host sample."""
    import oracle

    d = wl.draft[lo:hi] if wl.draft is not None else None
    if loss:
        r = oracle.vat_loss(wl.target[lo:hi], d, wl.tokens[lo:hi], wl.uniforms[lo:hi], wl.hard_tokens[lo:hi],
                            cfg.T, cfg.decay, 1.0)
        if grad:
            oracle.vat_loss_grad(wl.target[lo:hi], d, wl.hard_tokens[lo:hi], r.weights, cfg.T, 1.0)
        return r
    if cfg.kind == "vat":
        return oracle.vat_labels(wl.target[lo:hi], d, wl.tokens[lo:hi], wl.uniforms[lo:hi], cfg.T, cfg.decay)
    return oracle.verify(wl.target[lo:hi], d, wl.tokens[lo:hi], wl.uniforms[lo:hi], cfg.T, onehot=cfg.onehot)


HOST_THREADS_MAX = 16  # a GPU's share of its host's cores


def host_threads() -> int:
    """Host threads for the oracle: the process's CPU affinity (else the core
    count), bounded by OMP_NUM_THREADS when set and by one GPU's share."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, HOST_THREADS_MAX))


def cpu_baseline(cfg, seconds: float, loss: bool = False, grad: bool = False, threads: int = 1, wl=None):
    """The oracle as it is (plain fp64 C) over whole sequences (VAT: blocks) of
    the same workload until `seconds` of wall time have elapsed, on `threads`
    host threads that each take the next whole sequence (the C oracle runs
    without Python's lock held).  The sample is the workload's first
    sequences, drawn on the host by the same seeded generator.  With `grad`,
    the loss and then its gradient with respect to the draft logits."""
    import threading

    import workloads

    n_sample = min(cfg.B, 32 if cfg.kind == "verify" else 4)
    if wl is None:
        wl = workloads.generate(cfg, 0, n_sample)
    n_sample = min(n_sample, wl.n)
    lock = threading.Lock()
    state = {"next": 0, "done": 0}
    deadline = [0.0]

    def worker():
        while True:
            with lock:
                if time.perf_counter() >= deadline[0]:
                    return
                i = state["next"] % n_sample
                state["next"] += 1
            _oracle_call(cfg, wl, i, i + 1, loss, grad)
            with lock:
                state["done"] += 1

    t0 = time.perf_counter()
    deadline[0] = t0 + seconds
    if threads == 1:
        worker()
    else:
        pool = [threading.Thread(target=worker) for _ in range(threads)]
        for t in pool:
            t.start()
        for t in pool:
            t.join()
    dt = time.perf_counter() - t0
    done = state["done"]
    what = "blocks" if cfg.kind == "vat" else "sequences"
    if loss:
        what = "blocks (labels, loss and its gradient)" if grad else "blocks (labels and loss)"
    return {"value": done * cfg.k / dt, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole %s (%d positions; cycling over the first %d) of the %s workload, fp64 C oracle, "
                      "%s, %.1f s" % (done, what, done * cfg.k, n_sample, cfg.name,
                                     "1 thread" if threads == 1 else "%d threads over %s" % (threads, what.split()[0]),
                                     dt),
            "host_cpu": host_cpu_model(), "host_nproc": os.cpu_count()}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baselines(cfg, seconds: float, loss: bool = False, grad: bool = False):
    """All host threads (the reported figure) and one thread (nested)."""
    import workloads

    wl = workloads.generate(cfg, 0, min(cfg.B, 32 if cfg.kind == "verify" else 4))
    n = host_threads()
    res = cpu_baseline(cfg, seconds, loss, grad, threads=n, wl=wl)
    res["single_thread"] = cpu_baseline(cfg, seconds, loss, grad, threads=1, wl=wl)
    return res


def sample_parity(cfg, wl, acc_gpu, out_gpu, threads: int, band: float = 1e-5):
    """The oracle on the host sample's sequences next to the GPU's outputs for
    the same sequences (outside any timed region).  Counts, without
    asserting: positions whose acceptance test sits within `band` of the
    threshold (the fp32 and fp64 decisions may differ there; the sequence
    is compared only before it), draws whose u*Z lies within band*Z of an
    end of the chosen interval, and sequences that differ anywhere else
    (expected 0); of the first two, how many the GPU resolved differently
    from the oracle."""
    from concurrent.futures import ThreadPoolExecutor

    n = wl.n
    with ThreadPoolExecutor(max(1, min(threads, n))) as ex:
        res = list(ex.map(lambda b: _oracle_call(cfg, wl, b, b + 1), range(n)))
    greedy = cfg.T == 0
    amb_accept = amb_draw = mismatch = amb_accept_differ = amb_draw_differ = 0
    for b, r in enumerate(res):
        ro, rg = int(r.accepted_len[0]), int(acc_gpu[b])
        if ro < 0:
            mismatch += int(rg != ro)
            continue
        tested = range(min(ro + 1, cfg.k))
        amb = [i for i in tested if abs(r.accept_margin[0, i]) < band] if not greedy else []
        if amb:
            amb_accept += 1
            n_cmp = min(rg, ro)
            mismatch += int(rg < amb[0] or not np.array_equal(out_gpu[b, :n_cmp], r.out_tokens[0, :n_cmp]))
            amb_accept_differ += int(rg != ro or not np.array_equal(out_gpu[b], r.out_tokens[0]))
            continue
        if rg != ro or not np.array_equal(out_gpu[b, :ro], r.out_tokens[0, :ro]):
            mismatch += 1
            continue
        if not greedy and r.sample_margin[0] < band:
            amb_draw += 1
            amb_draw_differ += int(out_gpu[b, ro] != r.out_tokens[0, ro])
            continue
        mismatch += int(out_gpu[b, ro] != r.out_tokens[0, ro])
    return {"sequences": n, "ambiguous_accept": amb_accept, "ambiguous_accept_differ": amb_accept_differ,
            "ambiguous_draw": amb_draw, "ambiguous_draw_differ": amb_draw_differ, "mismatches": mismatch,
            "band": band}


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


SIDE_WORKLOADS = ("ngram_tail", "grpo", "grpo_greedy")
SIDE_WARMUP = 200
SIDE_STEPS = 500
PER_CALL_SAMPLES = 200
SETTLE_SECONDS = 0.3  # plain reads of the headline's size before its warm-up


class VerifyRun:
    """One verification workload resident on the device: the seeded inputs
    in enough copies that a sweep over them touches more than twice the MALL,
    one prepared sv_verify call per copy (they rotate), and the host copy of
    the first sequences for the oracle."""

    def __init__(self, name, dev, n_host=32):
        import speculative_decoding_verification_amd as sv
        import workloads

        self.cfg = cfg = workloads.get_config(name)
        print("bench: generating %s (B=%d k=%d V=%d %s T=%g)" % (cfg.name, cfg.B, cfg.k, cfg.V, cfg.dtype, cfg.T),
              file=sys.stderr, flush=True)
        wl = workloads.generate(cfg)
        self.spec_bytes = cfg.algorithmic_bytes()
        self.copies = max(1, math.ceil(2 * MALL_BYTES / self.spec_bytes))
        self.sets = [workloads.to_device(wl, dev) for _ in range(self.copies)]
        self.calls = _launchers(cfg, self.sets, sv, self.copies)
        n = min(cfg.B, n_host)
        self.host = workloads.Workload(cfg, 0, wl.target[:n].copy(),
                                       None if wl.draft is None else wl.draft[:n].copy(), wl.tokens[:n].copy(),
                                       wl.uniforms[:n].copy())
        del wl
        self.launched = 0

    def launch(self, stream):
        self.calls[self.launched % len(self.calls)](stream)
        self.launched += 1

    def last(self):
        return self.calls[(self.launched - 1) % len(self.calls)]

    def region_ms(self, ev, stream, warmup, steps):
        """Mean device time per call over `steps` back-to-back calls (one event
        pair around all of them, on the launch stream) and the wall time."""
        import torch

        for _ in range(warmup):
            self.launch(stream)
        torch.cuda.synchronize()
        a, b = ev.create(), ev.create()
        t0 = time.perf_counter()
        ev.record(a, stream)
        for _ in range(steps):
            self.launch(stream)
        ev.record(b, stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = ev.elapsed_ms(a, b) / steps
        ev.destroy(a)
        ev.destroy(b)
        return ms, wall

    def per_call_ms(self, ev, stream, n):
        """Device time of each of n calls, each bracketed by its own events
        (the events add a little stream work between calls)."""
        import torch

        pairs = [(ev.create(), ev.create()) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in pairs:
            ev.record(a, stream)
            self.launch(stream)
            ev.record(b, stream)
        torch.cuda.synchronize()
        out = np.array([ev.elapsed_ms(a, b) for a, b in pairs])
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        return out

    def outcome(self):
        import torch

        torch.cuda.synchronize()
        last = self.last()
        acc = last.accepted_len.cpu().numpy()
        out = last.out_tokens.cpu().numpy()
        return acc, out

    def needed_bytes(self, acc):
        """Every logit this call must read once: all decision rows, and the
        bonus row (target position k) only of sequences that kept all k."""
        cfg = self.cfg
        full = int((acc == cfg.k).sum())
        return self.spec_bytes - (cfg.B - full) * cfg.V * cfg.elem_bytes


def sol_read_ms(nbytes, dev, ev, stream, warmup=50, steps=200):
    """Mean duration of sv_sol_read over `nbytes` (rounded up to 16), the
    buffers rotated like the workload's inputs."""
    import torch

    import speculative_decoding_verification_amd as sv

    nbytes = (nbytes + 15) // 16 * 16
    copies = max(1, math.ceil(2 * MALL_BYTES / nbytes))
    bufs = [torch.full((nbytes // 4,), 0x3c003c00, dtype=torch.int32, device=dev) for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    sv.sol_read(bufs[0], sink, stream)  # checks the arguments once
    # then the bare C call, so that launches of a few microseconds are not
    # spaced out by the binding's checks
    lib = sv.load_library()
    calls = [(ctypes.c_void_p(t.data_ptr()), ctypes.c_size_t(nbytes), ctypes.c_void_p(sink.data_ptr()),
              ctypes.c_void_p(stream)) for t in bufs]
    f = lib.sv_sol_read
    for i in range(warmup):
        f(*calls[i % copies])
    torch.cuda.synchronize()
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    for i in range(steps):
        f(*calls[i % copies])
    ev.record(b, stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(a, b) / steps
    ev.destroy(a)
    ev.destroy(b)
    del bufs
    return ms


def acceptance_stats(acc, k):
    valid = acc[acc >= 0]
    tested = np.minimum(valid + 1, k).sum()
    return {"mean_accepted_len": float(valid.mean()) if valid.size else None,
            "accept_rate": float(valid.sum() / tested) if tested else None,
            "full_acceptance": int((acc == k).sum()), "invalid": int((acc == -1).sum()),
            "timeouts": int((acc == -2).sum())}


def workload_figures(run, ev, stream, dev, warmup, steps):
    """The side measurements of one workload (fixed warm-up and step count).
    The oracle comparison is left to the caller (`pending`: host sample and
    GPU outputs), so that no host work separates GPU measurements."""
    cfg = run.cfg
    ms, _ = run.region_ms(ev, stream, warmup, steps)
    calls = run.per_call_ms(ev, stream, PER_CALL_SAMPLES)
    acc, out = run.outcome()
    needed = run.needed_bytes(acc)
    sol = sol_read_ms(needed, dev, ev, stream)
    fig = {"B": cfg.B, "k": cfg.k, "V": cfg.V, "logits": cfg.dtype, "temperature": cfg.T,
           "draft": "one-hot" if cfg.onehot else ("none (greedy)" if cfg.T == 0 else "logits"),
           "warmup": warmup, "steps": steps, "mean_launch_us": ms * 1e3,
           "positions_per_s": cfg.positions() / (ms * 1e-3),
           "algorithmic_bytes": run.spec_bytes, "needed_bytes": needed,
           "frac": run.spec_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "frac_needed": needed / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "sol": {"kernel": "k_sol_read", "bytes": needed, "mean_launch_us": sol * 1e3, "frac": sol / ms},
           "call_us": {"p10": float(np.percentile(calls, 10) * 1e3), "p50": float(np.percentile(calls, 50) * 1e3),
                       "p90": float(np.percentile(calls, 90) * 1e3), "calls": len(calls)},
           "traffic": measured_traffic("k_verify", cfg.name)}
    fig.update(acceptance_stats(acc, cfg.k))
    fig["pending"] = (cfg, run.host, acc[:run.host.n], out[:run.host.n])
    return fig


def bench_verify(args) -> int:
    """Verification workloads (the default): the headline line for
    args.workload, with the side workloads measured in the same process."""
    import torch

    import speculative_decoding_verification_amd as sv

    dev = torch.device("cuda:0")
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    run = VerifyRun(args.workload, dev)  # prepared first: no host work right before its timing
    cfg = run.cfg
    side = {}
    if not args.no_side and args.workload not in ("tiny",):
        for name in SIDE_WORKLOADS:
            if name == args.workload:
                continue
            srun = VerifyRun(name, dev)
            print("bench: side workload %s: %d copies, %d warmup + %d steps" % (name, srun.copies, SIDE_WARMUP,
                                                                               SIDE_STEPS), file=sys.stderr,
                  flush=True)
            side[name] = workload_figures(srun, ev, stream, dev, SIDE_WARMUP, SIDE_STEPS)
            del srun
            torch.cuda.empty_cache()

    print("bench: %s: %d copies of %.1f MB, %d warmup + %d timed steps" % (cfg.name, run.copies, run.spec_bytes / 1e6,
                                                                        args.warmup, args.steps), file=sys.stderr,
          flush=True)
    # The device's clocks drop while the host prepares inputs; a short plain
    # read of the workload's size (no call of the kernel) brings them back
    # before the warm-up, so that a small W measures the same kernel.
    settle = int(min(5000, max(300, SETTLE_SECONDS / (run.spec_bytes / 6.5e12))))
    sol_read_ms(run.spec_bytes, dev, ev, stream, warmup=0, steps=settle)
    k1_mean, elapsed = run.region_ms(ev, stream, args.warmup, args.steps)
    ms_per_step = elapsed * 1e3 / args.steps
    value = cfg.positions() * args.steps / elapsed
    acc, out = run.outcome()
    needed = run.needed_bytes(acc)
    calls = run.per_call_ms(ev, stream, PER_CALL_SAMPLES)
    sol = sol_read_ms(needed, dev, ev, stream)
    achieved = run.spec_bytes / (k1_mean * 1e-3) / 1e9

    # acceptance telemetry: the histogram of accepted lengths after a call
    last = run.last()
    hist = sv.accept_histogram(last.accepted_len, cfg.k)
    torch.cuda.synchronize()
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    for _ in range(200):
        sv.accept_histogram(last.accepted_len, cfg.k, out=hist, stream=stream)
    ev.record(b, stream)
    torch.cuda.synchronize()
    hist_us = ev.elapsed_ms(a, b) / 200 * 1e3
    ev.destroy(a)
    ev.destroy(b)
    ctl = sv.DraftLengthController()
    ctl.update(hist.cpu())

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
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "draft_positions": cfg.k, "vocab": cfg.V,
                   "logits": cfg.dtype, "arithmetic": "f32", "temperature": cfg.T,
                   "draft": "one-hot" if cfg.onehot else ("none (greedy)" if cfg.T == 0 else "logits"),
                   "input_copies_rotated": run.copies},
        "hbm_gbps_whole_step": run.spec_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "k_verify", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("k_verify", cfg.name),
                     "algorithmic_bytes_per_launch": run.spec_bytes, "needed_bytes_per_launch": needed,
                     "frac_needed": needed / (k1_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "mean_launch_us": k1_mean * 1e3},
        "sol": {"kernel": "k_sol_read", "bytes": needed, "mean_launch_us": sol * 1e3, "frac": sol / k1_mean},
        "call_us": {"p10": float(np.percentile(calls, 10) * 1e3), "p50": float(np.percentile(calls, 50) * 1e3),
                    "p90": float(np.percentile(calls, 90) * 1e3), "calls": len(calls),
                    "how": "device time of single calls, each between its own HIP events, after the timed steps"},
        "accept_histogram_us": hist_us,
        "accept_histogram": hist.cpu().tolist(),
        "block_efficiency": ctl.efficiency,
    }
    tr = res["roofline"]["traffic"]
    res["roofline"]["traffic_gbps"] = tr / (k1_mean * 1e-3) / 1e9 if tr else None
    res.update(acceptance_stats(acc, cfg.k))
    res["parity_sample"] = sample_parity(cfg, run.host, acc[:run.host.n], out[:run.host.n], host_threads())
    del run
    torch.cuda.empty_cache()
    for fig in side.values():
        fig["parity_sample"] = sample_parity(*fig.pop("pending"), host_threads())
    if side:
        res["workloads"] = side
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (%.0f s, all host threads, then one)" % args.cpu_seconds, file=sys.stderr,
              flush=True)
        res["cpu_baseline"] = cpu_baselines(cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)
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


def blas_probe(steps: int) -> int:
    """torch.matmul (hipBLASLt) of the LM-head workloads' hidden states by
    their output layer's transpose, bf16 in and out, synthetic operands of
    the same shapes."""
    import torch

    import workloads

    dev = torch.device("cuda:0")
    for name in ("lmhead_selfdraft", "lmhead_grpo"):
        cfg = workloads.LM_CONFIGS[name]
        gen = torch.Generator(device=dev).manual_seed(cfg.seed)
        h = (torch.randn(cfg.rows, cfg.D, generator=gen, device=dev) * 0.05).to(torch.bfloat16)
        w = (torch.randn(cfg.V, cfg.D, generator=gen, device=dev) * 0.05).to(torch.bfloat16)
        wt = w.t()
        for _ in range(5):
            y = torch.matmul(h, wt)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            y = torch.matmul(h, wt)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        tflops = cfg.flops() / (ms * 1e-3) / 1e12
        print(json.dumps({"blas_probe": name, "rows": cfg.rows, "hidden": cfg.D, "vocab": cfg.V, "steps": steps,
                          "mean_us": ms * 1e3, "tflops": tflops, "frac_of_bf16_peak": tflops / MFMA_BF16_PEAK_TFLOPS,
                          "output": "bf16 logits written"}), flush=True)
        del h, w, wt, y
        torch.cuda.empty_cache()
    return 0


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
    ap.add_argument("--blas-probe", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="time only --workload (no ngram_tail / grpo / grpo_greedy side figures)")
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
    if args.blas_probe:
        return blas_probe(args.steps)

    if args.workload.startswith("lmhead_"):
        return bench_lm_head(args)
    if args.workload in ("selfdraft", "ngram_tail", "grpo", "grpo_greedy", "tiny"):
        return bench_verify(args)

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
    achieved = needed / (k1_mean * 1e-3) / 1e9
    # speed of light over the same buffers: the logits read once (labels,
    # loss), or both logit arrays read and one fp32 array written (gradient)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    t, d = sets[0][0], sets[0][1]
    sol_kernel = "k_sol_read_write" if grad else "k_sol_read"
    for rep in range(2):  # the first pass warms up
        torch.cuda.synchronize()
        ev.record(region[0], stream)
        for _ in range(5):
            if grad:
                sv.sol_read_write(t, d, calls[0].grad, stream)
            else:
                sv.sol_read(t, sink, stream)
                sv.sol_read(d, sink, stream)
        ev.record(region[1], stream)
        torch.cuda.synchronize()
    sol_ms = ev.elapsed_ms(*region) / 5
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
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "blocks": cfg.B, "draft_positions": cfg.k, "vocab": cfg.V,
                   "logits": cfg.dtype, "arithmetic": "f32", "temperature": cfg.T, "draft": "logits",
                   "input_copies_rotated": copies},
        "hbm_gbps_whole_step": needed / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(kernel, args.workload),
                     "algorithmic_bytes_per_launch": needed, "all_rows_bytes_per_launch": in_bytes,
                     "mean_launch_us": k1_mean * 1e3},
        "sol": {"kernel": sol_kernel, "bytes": in_bytes, "mean_launch_us": sol_ms * 1e3, "frac": sol_ms / k1_mean},
    }
    res.update(extra)
    if cfg.kind == "vat":
        res["config"]["decay"] = cfg.decay
    if loss:
        res["config"]["hard_weight"] = 1.0
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (%.0f s, all host threads, then one)" % args.cpu_seconds, file=sys.stderr,
              flush=True)
        res["cpu_baseline"] = cpu_baselines(cfg, args.cpu_seconds, loss, grad)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
