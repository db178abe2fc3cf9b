"""Benchmark: LCP forward + backward steps per second on one linear layer.

Workload: the LLaMA-7B down_proj-shaped layer, W 4096 x 11008 bf16, X 2048
tokens x 11008 bf16 with lognormal channel scales, block size 64, 5 Sinkhorn
iterations at tau = 1, 2:4 mask; seeded synthetic data (no model weights or
calibration text exist here).

One step = the whole hot path: per-layer setup (column norms, X transposed),
Sinkhorn, fused permute / importance / mask / un-permute, error GEMM and its
norm, backward GEMM, block adjoint and Sinkhorn adjoint, all in liblcp.so.
Inputs are resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--breakdown]

Warm-up runs at least W steps and at least --warmup-seconds (1 s) of steps
(`warmup_run` records both): on MI355X the clocks take longer than a few steps
to settle, and 5 warm-up steps leave the 20 timed ones about 7 % slower than
the steady state a training loop on one layer runs at.

Prints one JSON line. `value` is steps/s from the median step time (an event
at every step boundary of the K timed steps; `ms_per_step` is their mean).
`roofline` is computed from the average duration of the dominant kernel,
measured with HIP events recorded on the step's stream inside the timed
region, against the published peak and (`roofline.attainable`) against
hipBLASLt on the same GEMM shape in the same process. After the timed region
a per-kernel pass (`kernels`: µs, algorithmic bytes or flops, GB/s or
TFLOP/s, fractions of the published peak and of the measured copy / hipBLASLt
rates) and the attainable probes (`attainable`) run; `cpu_baseline` times the
float64 oracle on the host; `source` identifies the library sources.
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FWD_NAMES = ["sinkhorn_fwd", "permute_mask_unpermute", "error_gemm", "error_finalize"]
BWD_NAMES = ["dD_gemm", "block_adjoint", "sinkhorn_bwd"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up (whole steps) until at least this much time has passed as well as "
                         "--warmup steps: the GPU's clocks take longer than a few steps to settle")
    ap.add_argument("--config", type=int, default=None, help="layer config index (default: the bench layer)")
    ap.add_argument("--breakdown", action="store_true", help="also print the per-kernel times to stderr")
    ap.add_argument("--no-kernels", action="store_true",
                    help="skip the per-kernel pass and the attainable-peak probes after the timed region")
    ap.add_argument("--harden", action="store_true",
                    help="hardened forward + straight-through backward (another workload)")
    ap.add_argument("--cosine", action="store_true",
                    help="cosine objective of the layer outputs (another workload; the dense outputs are "
                         "part of the per-layer setup of every step)")
    ap.add_argument("--mask-ste", action="store_true",
                    help="straight-through gradient of the mask in the backward (another workload)")
    ap.add_argument("--deploy", action="store_true",
                    help="deploy path of a trained layer: channel gather + 2:4 sparse GEMM (another workload)")
    ap.add_argument("--adamw", action="store_true",
                    help="training step: the backward with the fused AdamW update of the logits")
    ap.add_argument("--saturate", action="store_true",
                    help="also time the Sinkhorn and the N:M mask at saturating sizes (to stderr)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured into a HIP graph (reported beside the eager value)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run 3 plain device copies of MIB MiB (HBM counter calibration)")
    return ap.parse_args()


# source files each timed kernel is built from (with the shared common.h):
# its HBM counters stay valid until one of them changes
KERNEL_SOURCES = {
    "layer_init": ["layer.hip"], "sinkhorn_fwd": ["sinkhorn.hip", "frag.h"],
    "sinkhorn_bwd": ["sinkhorn.hip"], "permute_mask_unpermute": ["permute.hip", "frag.h"],
    "error_gemm": ["gemm.hip"], "dD_gemm": ["gemm.hip"], "error_finalize": ["gemm.hip"],
    "dD_gemm_adjoint": ["gemm.hip", "frag.h"],
    "block_adjoint": ["adjoint.hip"], "harden": ["harden.hip", "frag.h"],
    "cosine_finalize": ["cosine.hip"], "cosine_grad": ["cosine.hip"],
    "sparse_gemm": ["deploy.hip"], "gather": ["deploy.hip"], "sparse_pack": ["deploy.hip"],
}


def _code_only(text):
    """Source text without comments and blank lines (a comment edit does not
    change the kernel the counters were taken on)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "learnable_channel_permutation_amd", "csrc")
    for f in ["common.h"] + sorted(KERNEL_SOURCES.get(kernel, [])):
        with open(os.path.join(csrc, f)) as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, shape):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel's current sources and on this layer shape
    ([cout, cin, T]); else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if k is None or kernel not in KERNEL_SOURCES or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    if list(k.get("shape", [])) != list(shape):
        return None
    return k.get("bytes_per_launch")


def fused_adjoint(spec, mask_ste=False):
    """Whether the step runs the block adjoint inside the dD GEMM (bf16 layers
    with B = 64 and the mask held constant); the library then records nothing
    between the block adjoint's timing events."""
    return spec.dtype == "bf16" and spec.B == 64 and not mask_ste and spec.backward


def kernel_work(spec, names):
    """Algorithmic work of one launch of each step kernel on this layer:
    ("bytes", n) for the HBM-bound kernels (every input read once, every
    output written once) or ("flops", n) for the two GEMMs. The dD GEMM with
    the fused block adjoint counts the GEMM's flops plus the adjoint's four
    products per block (W_b P_b, G_b P_b and the two sums over the rows,
    2 Cout B flops each per channel); its transposes are not counted."""
    cout, cin, T, B, L = spec.cout, spec.cin, spec.T, spec.B, spec.iters
    nb = cin // B
    es = 2 if spec.dtype == "bf16" else 4
    pitch = (T + 63) // 64 * 64
    KS, TT = B // 16, B // 32
    frag = TT * KS * 64 * 16                                      # bytes of one fragment set
    frags = nb * ((2 + (2 if B == 128 else 3)) * frag + frag) if spec.dtype == "bf16" else 0
    wk = {
        "layer_init": ("bytes", es * T * cin + (2 * cin * pitch if spec.dtype == "bf16" else 0) + 4 * cin),
        "sinkhorn_fwd": ("bytes", 8 * nb * B * B + 4 * nb * L * 2 * B + 4 * cin + frags),
        "permute_mask_unpermute": ("bytes", 2 * es * cout * cin + cout * cin // 8 + 4 * nb * B * B),
        "error_gemm": ("flops", 2.0 * cout * cin * T),
        "error_finalize": ("bytes", 4 * ((cout + 255) // 256) * ((pitch + 127) // 128)),
        "dD_gemm": ("flops", 2.0 * cout * cin * T),
        "dD_gemm_adjoint": ("flops", 2.0 * cout * cin * T + 8.0 * cout * cin * B),
        "block_adjoint": ("bytes", 2 * es * cout * cin + cout * cin // 8 + 4 * nb * B * B),
        "sinkhorn_bwd": ("bytes", 12 * nb * B * B + 4 * nb * L * 2 * B),
    }
    return {n: wk[n] for n in names if n in wk}


def attainable_peaks(torch, spec):
    """Measured-attainable denominators on this GPU, in this process: a plain
    device copy (torch's copy kernel, 1 GiB read + 1 GiB written) and
    hipBLASLt (torch.matmul) on the two GEMM shapes of the step with random
    bf16 operands. The step holds X both as [T, Cin] and as its transpose, so
    each product is timed with the right operand in either layout and the
    faster one is kept (hipBLASLt's speed depends on it). Each is the best of
    3 rounds of 10 timed calls. The same two, a weight-sized copy and the two
    hipBLASLt products, are also timed "cold": each call right after 1 GiB of
    other writes has flushed the caches, as the step's kernels mostly find
    their operands (median of 5 calls)."""
    dev = torch.device("cuda:0")
    out = {}
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def best(fn, reps=10, rounds=3):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(rounds):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b) / reps)
        return min(ms)

    ms = best(lambda: dst.copy_(src))
    out["copy_GB_per_s"] = round(2.0 * n * 4 / (ms * 1e-3) / 1e9, 1)

    def cold(fn, reps=5):
        ms = []
        for _ in range(reps + 1):
            dst.fill_(1.0)                                 # 1 GiB of other writes
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms[1:]))

    wn = spec.cout * spec.cin                              # a weight-sized bf16 copy
    wa = torch.ones(wn, dtype=torch.bfloat16, device=dev)
    wb = torch.empty_like(wa)
    ms = cold(lambda: wb.copy_(wa))
    out["copy_cold_weight_GB_per_s"] = round(2.0 * wn * 2 / (ms * 1e-3) / 1e9, 1)
    del src, wa, wb
    cout, cin, T = spec.cout, spec.cin, spec.T
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    R = torch.randn((cout, T), device=dev, generator=g).to(torch.bfloat16)
    X = torch.randn((T, cin), device=dev, generator=g).to(torch.bfloat16)
    D = torch.randn((cout, cin), device=dev, generator=g).to(torch.bfloat16)
    Xt = X.t().contiguous()
    flops = 2.0 * cout * cin * T
    # dD: G = R X with X as stored ([T, Cin]) or as the transposed copy's view;
    # error: R = D Xᵀ with X's view (K contiguous in both) or the copy itself.
    dd = {"nn": best(lambda: torch.matmul(R, X)), "nt": best(lambda: torch.matmul(R, Xt.t()))}
    er = {"nt": best(lambda: torch.matmul(D, X.t())), "nn": best(lambda: torch.matmul(D, Xt))}
    lay_dd, ms_dd = min(dd.items(), key=lambda kv: kv[1])
    lay_err, ms_err = min(er.items(), key=lambda kv: kv[1])
    out["hipblaslt_layouts"] = {"dD": lay_dd, "error": lay_err}
    out["hipblaslt_dD_TFLOP_per_s"] = round(flops / (ms_dd * 1e-3) / 1e12, 1)
    out["hipblaslt_error_TFLOP_per_s"] = round(flops / (ms_err * 1e-3) / 1e12, 1)
    out["hipblaslt_dD_us"] = round(ms_dd * 1e3, 1)
    out["hipblaslt_error_us"] = round(ms_err * 1e3, 1)
    mm = {"nn": lambda A, Bm, Bt: torch.matmul(A, Bm), "nt": lambda A, Bm, Bt: torch.matmul(A, Bt.t())}
    out["hipblaslt_dD_cold_us"] = round(cold(lambda: mm[lay_dd](R, X, Xt)) * 1e3, 1)
    out["hipblaslt_error_cold_us"] = round(cold(lambda: (torch.matmul(D, X.t()) if lay_err == "nt"
                                                         else torch.matmul(D, Xt))) * 1e3, 1)
    del R, X, D, Xt, dst
    torch.cuda.synchronize()
    return out


def source_identity():
    """sha256 (16 hex) of the library sources as built (code only), and the
    git commit when the tree is a checkout."""
    import subprocess
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "learnable_channel_permutation_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f)) as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    sha = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        if r.returncode == 0:
            sha = r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        sha = None
    return {"csrc_sha16": h.hexdigest()[:16], "git": sha}


class HipEvents:
    """hipEvent_t handles created and read through the HIP runtime (the library
    records them on the step's stream; torch's Event wrapper only accepts
    events it recorded itself)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.made = []

    def new(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.made.append(e)
        return e

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(out.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


class _Ev:
    """Adapter so make_timing() can take raw hipEvent_t handles."""

    def __init__(self, h):
        self.cuda_event = h.value


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        return os.cpu_count()


def cpu_baseline(spec, lay, hard=False, loss="frobenius", mask_ste=False):
    """The float64 oracle, untuned, for full forward + backward steps of the
    same layer on the host cores: the median step time of repeated steps,
    repeated until about 10 s of work (at least 3 steps, a single step for
    layers above 10^8 weights)."""
    import oracle
    big = spec.cout * spec.cin > 10 ** 8
    times = []
    while not times or (not big and (len(times) < 3 or sum(times) < 10.0) and len(times) < 200):
        t0 = time.perf_counter()
        fw = oracle.step_forward(lay.W, lay.X, lay.logits, spec.tau, spec.iters, spec.N, spec.M, hard=hard,
                                 loss=loss)
        if spec.backward:
            oracle.step_backward(fw, lay.X, lay.W, mask_ste=mask_ste)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": 1.0 / dt, "unit": "steps/s", "cores": int(_blas_threads()), "cpu_count": os.cpu_count(),
            "kind": "oracle",
            "sample": "median of %d full %s steps of the same %dx%d layer (T=%d), float64 NumPy, %.3f s each, %.1f s total"
                      % (len(times), "forward+backward" if spec.backward else "forward", spec.cout, spec.cin, spec.T,
                         dt, sum(times))}


def cpu_baseline_deploy(W, X, P, mask):
    """The float64 oracle's deployed-layer forward on the host cores: the
    median of repeated full forwards of the same layer (about 10 s of work,
    at least 3)."""
    import oracle
    times = []
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 200):
        t0 = time.perf_counter()
        oracle.deploy_forward(W, X, P, mask)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": 1.0 / dt, "unit": "forwards/s", "cores": int(_blas_threads()), "cpu_count": os.cpu_count(),
            "kind": "oracle",
            "sample": "median of %d full deployed-layer forwards (%dx%d weight, %d tokens), float64 NumPy, %.3f s each, %.1f s total"
                      % (len(times), W.shape[0], W.shape[1], X.shape[0], dt, sum(times))}


def run_deploy(args, torch, lcp, lcp_synth):
    """Deploy workload: Y = gather(X) Ws^T with the 2:4 packed weight, on the
    bench layer's shape (weight 4096 x 11008, 2048 tokens, B = 64)."""
    L = lcp._lib
    spec = lcp_synth.DOWN_PROJ_4096x11008
    cout, cin, T, B = spec.cout, spec.cin, spec.T, spec.B
    lay = lcp_synth.make_layer(spec)
    dev = torch.device("cuda:0")
    rng = np.random.Generator(np.random.PCG64(2024))
    nb = cin // B
    perm_np = np.stack([rng.permutation(B) for _ in range(nb)]).astype(np.int32)
    W = torch.from_numpy(lay.W).to(dev).to(torch.bfloat16)
    X = torch.from_numpy(lay.X).to(dev).to(torch.bfloat16)
    perm = torch.from_numpy(perm_np).to(dev)
    # a 2:4 mask in permuted positions from seeded random scores
    scores = torch.from_numpy(rng.random((cout, cin), dtype=np.float32)).to(dev)
    bits = torch.empty((cout, cin // 32), dtype=torch.int32, device=dev)
    L.lcp_nm_mask(scores, 2, 4, bits)
    vb, mb = L.lcp_sparse_pack_bytes(cout, cin)
    vals = torch.empty(vb, dtype=torch.uint8, device=dev)
    meta = torch.empty(mb, dtype=torch.uint8, device=dev)
    L.lcp_sparse_pack(W, B, perm, bits, vals, meta)
    Xp = torch.empty_like(X)
    Y = torch.empty((T, cout), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        L.lcp_deploy_forward(vals, meta, perm, B, X, cout, Xp, Y)
    torch.cuda.synchronize()
    K = args.steps
    he = HipEvents()
    ev = [(he.new(), he.new(), he.new()) for _ in range(K)]
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(K):
        he.record(ev[k][0], stream)
        L.lcp_gather_channels(X, B, perm, Xp)
        he.record(ev[k][1], stream)
        L.lcp_sparse_gemm(vals, meta, Xp, cout, Y)
        he.record(ev[k][2], stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_stop) / K
    g_ms = sum(he.ms(a, b) for a, b, _ in ev) / K
    s_ms = sum(he.ms(b, c) for _, b, c in ev) / K
    ms_median = float(np.median([he.ms(a, c) for a, _, c in ev]))
    he.close()
    # context on the same box: PyTorch's own gather and dense bf16 GEMM
    gidx = torch.from_numpy((np.arange(nb)[:, None] * B + perm_np).reshape(-1).astype(np.int64)).to(dev)
    Wd = W.contiguous()
    for _ in range(3):
        torch.index_select(X, 1, gidx)
        torch.matmul(X, Wd.t())
    torch.cuda.synchronize()
    reps = 20
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    for _ in range(reps):
        torch.index_select(X, 1, gidx)
    e1.record(stream)
    for _ in range(reps):
        torch.matmul(X, Wd.t())
    e2.record(stream)
    torch.cuda.synchronize()
    torch_gather_ms = e0.elapsed_time(e1) / reps
    torch_dense_ms = e1.elapsed_time(e2) / reps
    useful = 2.0 * T * cout * (cin // 2)          # nonzero multiply-adds of the 2:4 weight
    achieved = useful / (s_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        P = np.zeros((nb, B, B))
        for b in range(nb):
            P[b, perm_np[b], np.arange(B)] = 1.0
        import oracle
        mask = oracle.unpack_bits(bits.cpu().numpy().view(np.uint32), cin)
        cpu = cpu_baseline_deploy(lay.W, lay.X, P, mask)
    gather_bytes = 2.0 * 2 * T * cin
    out = {
        "metric": "LCP deployed-layer forwards/sec (%dx%d 2:4, %d tokens)" % (cout, cin, T),
        "value": round(1000.0 / ms, 2),
        "unit": "forwards/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded LLaMA-shaped layer, random block permutation and 2:4 mask)",
        "config": {"workload": "lcp_deploy_forward", "layer": spec.name, "cout": cout, "cin": cin, "T": T,
                   "B": B, "N": 2, "M": 4},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("sparse_gemm", [cout, cin, T]),
                     "kernel": "sparse_gemm", "kernel_ms": round(s_ms, 4),
                     "note": "flops = nonzero multiply-adds x 2, priced against the dense bf16 peak"},
        "gather": {"ms": round(g_ms, 4), "GB/s": round(gather_bytes / (g_ms * 1e-3) / 1e9, 1)},
        "context": {"torch_index_select_ms": round(torch_gather_ms, 4),
                    "torch_dense_matmul_ms": round(torch_dense_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def saturating_kernels(lcp, torch, he):
    """Sinkhorn forward over all B = 64 blocks of a LLaMA-7B-shaped model's
    projection layers (17,792 blocks) and lcp_nm_mask on 28672 x 8192 fp32
    scores, timed with HIP events; HBM bytes are the algorithmic ones (inputs
    read once, outputs written once)."""
    import numpy as np
    dev = torch.device("cuda:0")
    out = {}
    nb, B, L = 17792, 64, 5
    rng = np.random.Generator(np.random.PCG64(99))
    lg = torch.from_numpy((3.0 * np.eye(B, dtype=np.float32)[None] +
                           1e-3 * rng.standard_normal((1, B, B)).astype(np.float32)).repeat(nb, axis=0)).to(dev)
    P = torch.empty_like(lg)
    rows, cin = 28672, 8192
    scores = torch.rand((rows, cin), dtype=torch.float32, device=dev)
    bits = torch.empty((rows, cin // 32), dtype=torch.int32, device=dev)
    for _ in range(3):
        lcp.lcp_sinkhorn(lg, P, L, 1.0)
        lcp.lcp_nm_mask(scores, 2, 4, bits)
    torch.cuda.synchronize()
    reps = 10
    for name, fn, nbytes in (
            ("sinkhorn_fwd_17792x64x64", lambda: lcp.lcp_sinkhorn(lg, P, L, 1.0), 2 * nb * B * B * 4),
            ("nm_mask_28672x8192", lambda: lcp.lcp_nm_mask(scores, 2, 4, bits), rows * cin * 4 + rows * cin // 8)):
        evs = [(he.new(), he.new()) for _ in range(reps)]
        st = torch.cuda.current_stream()
        for a, b in evs:
            he.record(a, st)
            fn()
            he.record(b, st)
        torch.cuda.synchronize()
        ms = sum(he.ms(a, b) for a, b in evs) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 1), "GB_per_s": round(gbs, 1), "frac_of_8TBs": round(gbs / 8000.0, 3),
                     "bytes": nbytes}
    # the same traffic as a plain device copy (torch's copy kernel): the
    # Sinkhorn reads and writes nb B^2 floats, the mask reads the scores
    for name, nin, nout in (("sinkhorn_fwd_17792x64x64", nb * B * B, nb * B * B),
                            ("nm_mask_28672x8192", rows * cin, rows * cin // 32)):
        a = torch.ones(nin, dtype=torch.float32, device=dev)
        c = torch.empty(nout, dtype=torch.float32, device=dev)
        fn = (lambda: c.copy_(a)) if nin == nout else (lambda: torch.sum(a))
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / reps
        cgbs = (4 * nin + (4 * nout if nin == nout else 0)) / (cms * 1e-3) / 1e9
        out[name]["reference"] = {"kind": "device copy" if nin == nout else "torch.sum read", "us": round(cms * 1e3, 1),
                                  "GB_per_s": round(cgbs, 1)}
        out[name]["frac_of_reference"] = round(out[name]["GB_per_s"] / cgbs, 3)
        del a, c
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import lcp_synth
    import learnable_channel_permutation_amd as lcp

    if args.copy_probe > 0:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.deploy:
        run_deploy(args, torch, lcp, lcp_synth)
        return

    ci = lcp_synth.BENCH_CONFIG if args.config is None else args.config
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    W = torch.from_numpy(lay.W).to(dev).to(tdt)
    X = torch.from_numpy(lay.X).to(dev).to(tdt)
    logits = torch.from_numpy(lay.logits).to(dev)
    dlogits = torch.empty_like(logits)
    loss = "cosine" if args.cosine else "frobenius"
    sess = lcp.LayerSession(W, X, spec.B, spec.iters, spec.tau, spec.N, spec.M, harden=args.harden, loss=loss,
                            mask_ste=args.mask_ste)
    stream = torch.cuda.current_stream()

    m_state = torch.zeros_like(logits)
    v_state = torch.zeros_like(logits)
    acfg = lcp.make_adamw_cfg(5e-3)
    t_opt = [0]

    def step(tf=None, tb=None):
        sess.init()
        sess.forward(logits, timing=tf)
        if spec.backward and args.adamw:
            t_opt[0] += 1
            lcp.lcp_step_bwd_adamw(sess.layer, logits, sess.cfg, sess.ws, m_state, v_state, t_opt[0], acfg,
                                   timing=tb)
        elif spec.backward:
            sess.backward(logits, dlogits, timing=tb)

    # untimed warm-up: at least --warmup steps and at least --warmup-seconds
    # of stepping (synchronised every 8 steps so wall time follows the GPU)
    t_w0 = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w0 < args.warmup_seconds:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_info = {"steps": n_warm, "seconds": round(time.perf_counter() - t_w0, 3)}

    # timed region: whole steps, plus events around the two GEMMs on the same stream
    K = args.steps
    he = HipEvents()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    g_fwd = [(he.new(), he.new()) for _ in range(K)]
    g_bwd = [(he.new(), he.new()) for _ in range(K)]
    tfs = [lcp.make_timing([None, None, _Ev(a)], [None, None, _Ev(b)]) for a, b in g_fwd]
    tbs = [lcp.make_timing([_Ev(a)], [_Ev(b)]) for a, b in g_bwd]
    t_start, t_stop = ev(), ev()
    bounds = [ev() for _ in range(K + 1)]
    torch.cuda.synchronize()
    t_start.record(stream)
    bounds[0].record(stream)
    for k in range(K):
        step(tfs[k], tbs[k] if spec.backward else None)
        bounds[k + 1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_stop) / K
    ms_median = float(np.median([bounds[k].elapsed_time(bounds[k + 1]) for k in range(K)]))
    fwd_gemm_ms = sum(he.ms(a, b) for a, b in g_fwd) / K
    bwd_gemm_ms = sum(he.ms(a, b) for a, b in g_bwd) / K if spec.backward else 0.0

    fused = fused_adjoint(spec, args.mask_ste)
    dd_name = "dD_gemm_adjoint" if fused else "dD_gemm"
    flops_gemm = 2.0 * spec.cout * spec.cin * spec.T
    flops = {"error_gemm": flops_gemm, dd_name: kernel_work(spec, [dd_name])[dd_name][1]}
    dom_name, dom_ms = ("error_gemm", fwd_gemm_ms)
    if bwd_gemm_ms > fwd_gemm_ms:
        dom_name, dom_ms = (dd_name, bwd_gemm_ms)
    achieved = flops[dom_name] / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(dom_name, [spec.cout, spec.cin, spec.T])
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": dom_name,
            "kernel_ms": round(dom_ms, 4), "flops_per_launch": flops[dom_name],
            "other_gemm": {"kernel": dd_name if dom_name == "error_gemm" else "error_gemm",
                           "ms": round(bwd_gemm_ms if dom_name == "error_gemm" else fwd_gemm_ms, 4)}}

    kernels = None
    if not args.no_kernels:
        # per-kernel pass after the timed region: events around every kernel
        # of 20 further steps (kept out of the timed steps so that the extra
        # event records do not perturb them)
        fwd_names = FWD_NAMES[:3] + (["cosine_finalize"] if args.cosine else FWD_NAMES[3:]) \
            + (["harden"] if args.harden else [])
        bwd_names = [dd_name] + BWD_NAMES[1:] + (["cosine_grad"] if args.cosine else [])
        names = fwd_names + (bwd_names if spec.backward else [])
        reps = 20
        evs = {n: [(he.new(), he.new()) for _ in range(reps)] for n in names}
        init_ev = [(ev(), ev()) for _ in range(reps)]
        torch.cuda.synchronize()
        for r in range(reps):
            init_ev[r][0].record(stream)
            sess.init()
            init_ev[r][1].record(stream)
            tf = lcp.make_timing([_Ev(evs[n][r][0]) for n in fwd_names], [_Ev(evs[n][r][1]) for n in fwd_names])
            sess.forward(logits, timing=tf)
            if spec.backward:
                tb = lcp.make_timing([_Ev(evs[n][r][0]) for n in bwd_names],
                                     [_Ev(evs[n][r][1]) for n in bwd_names])
                sess.backward(logits, dlogits, timing=tb)
        torch.cuda.synchronize()
        per = {"layer_init": sum(a.elapsed_time(b) for a, b in init_ev) / reps}
        for n in names:
            if fused and n == "block_adjoint":
                continue                      # runs inside the dD GEMM
            per[n] = sum(he.ms(a, b) for a, b in evs[n]) / reps
        work = kernel_work(spec, list(per))
        kernels = {}
        for n, kms in per.items():
            e = {"us": round(kms * 1e3, 1)}
            if n in work:
                kind, amount = work[n]
                if kind == "bytes":
                    gbs = amount / (kms * 1e-3) / 1e9
                    e.update({"bytes": int(amount), "GB_per_s": round(gbs, 1),
                              "frac_hbm": round(gbs / PEAK_HBM_GBS, 3)})
                else:
                    tfs = amount / (kms * 1e-3) / 1e12
                    e.update({"flops": amount, "TFLOP_per_s": round(tfs, 1),
                              "frac_mfma": round(tfs / PEAK_BF16_TFLOPS, 3)})
            kernels[n] = e
        if args.breakdown:
            print("per-kernel ms (mean of %d):" % reps, file=sys.stderr)
            for n, kms in per.items():
                print("  %-24s %8.4f" % (n, kms), file=sys.stderr)
    graph = None
    if args.graph and not args.adamw:
        g = sess.capture_step(logits, dlogits, setup=True)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = ev(), ev()
        g0.record(stream)
        for _ in range(K):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / K
        graph = {"ms_per_step": round(gms, 4), "value": round(1000.0 / gms, 2), "unit": "steps/s"}
    if args.saturate:
        sat = saturating_kernels(lcp, torch, he)
        print("saturating sizes: " + json.dumps(sat), file=sys.stderr)
    he.close()

    attain = None
    if not args.no_kernels and spec.dtype == "bf16":
        attain = attainable_peaks(torch, spec)
        gemm_att = attain["hipblaslt_error_TFLOP_per_s"] if dom_name == "error_gemm" else attain["hipblaslt_dD_TFLOP_per_s"]
        gemm_achieved = flops_gemm / (dom_ms * 1e-3) / 1e12
        roof["attainable"] = {"peak": gemm_att, "unit": "TFLOP/s", "frac": round(gemm_achieved / gemm_att, 4),
                              "source": "hipBLASLt (torch.matmul) on the same GEMM shape, same process"
                                        + ("; GEMM flops only: hipBLASLt's time for the GEMM alone over this "
                                           "kernel's time for the GEMM and the block adjoint"
                                           if dom_name == "dD_gemm_adjoint" else "")}
        if kernels is not None:
            for n, e in kernels.items():
                if "GB_per_s" in e:
                    e["frac_copy"] = round(e["GB_per_s"] / attain["copy_GB_per_s"], 3)
                    e["frac_copy_cold"] = round(e["GB_per_s"] / attain["copy_cold_weight_GB_per_s"], 3)
                elif "TFLOP_per_s" in e:
                    if n == "error_gemm":
                        e["frac_hipblaslt"] = round(e["TFLOP_per_s"] / attain["hipblaslt_error_TFLOP_per_s"], 3)
                    elif n == "dD_gemm":
                        e["frac_hipblaslt"] = round(e["TFLOP_per_s"] / attain["hipblaslt_dD_TFLOP_per_s"], 3)
                    else:                       # fused: hipBLASLt's dD time over this kernel's
                        e["hipblaslt_dD_time_ratio"] = round(attain["hipblaslt_dD_us"] / e["us"], 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, lay, hard=args.harden, loss=loss, mask_ste=args.mask_ste)

    out = {
        "metric": "LCP %s steps/sec per layer (%dx%d, %d:%d)" % ("fwd+bwd" if spec.backward else "fwd",
                                                                 spec.cout, spec.cin, spec.N, spec.M),
        "value": round(1000.0 / ms_median, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "value_from": "median step time (event at every step boundary); ms_per_step is the mean over the K steps",
        "value_mean": round(1000.0 / ms, 2),
        "warmup_run": warm_info,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic (seeded LLaMA-shaped layer; no weights or calibration text available)",
        "config": {"workload": ("lcp_step_fwd_bwd" if spec.backward else "lcp_step_fwd")
                               + ("_hardened" if args.harden else "")
                               + ("_cosine" if args.cosine else "")
                               + ("_maskste" if (args.mask_ste and spec.backward) else "")
                               + ("_adamw" if (args.adamw and spec.backward) else ""),
                   "layer": spec.name, "cout": spec.cout, "cin": spec.cin,
                   "T": spec.T, "B": spec.B, "sinkhorn_iters": spec.iters, "tau": spec.tau,
                   "N": spec.N, "M": spec.M, "backward": spec.backward, "objective": loss,
                   "includes_layer_setup": True},
        "roofline": roof,
        "kernels": kernels,
        "attainable": attain,
        "cpu_baseline": cpu,
        "source": source_identity(),
    }
    if graph is not None:
        out["graph"] = graph
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
