"""Benchmark of the mHC hot path on one MI355X.

A step is one pass of the forward hot path over one batch: hc_pre (RMSNorm,
projection, gates, Sinkhorn, collapse) and hc_post (mix + expand), through the
C ABI, on the long-sequence workload B=1, S=4096 tokens, N=4 streams, D=5120,
bf16 storage of x / y / h / x_next and fp32 math: the configuration the
headline metric (pre+post tokens/s and HBM GB/s) is quoted on.  Inputs are
seeded synthetic tensors already resident in HBM; two input sets alternate
between steps so that no step finds its inputs in the 256 MB Infinity Cache
left warm by the step before.

Prints one JSON line.  `value` is tokens/s of the forward pair (wall clock
around exactly K steps, synchronised on both sides).  `roofline` is the
kernel that takes the most time in that step, timed with HIP events the
library records around each launch on its stream (a second pass over the same
K steps, so that the events do not enter the wall-clock figure).  The training
step of the same shape (forward plus both backward calls), the two fp32
configurations of the pages' measurement paragraph, the fused layer boundary,
the stabilised write-back, a graph-replayed step and the CPU oracle are
reported beside it.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
METRIC = "mHC pre+post tokens/s and HBM GB/s (% of peak) at S=4096,N=4,D=5120"

WORKLOADS = {
    # name: (T, N, D, io)
    "pro_s4096_bf16": (4096, 4, 5120, "bf16"),
    "pro_s1024_f32": (1024, 4, 5120, "f32"),
    "flash_s2048_f32": (2048, 4, 2560, "f32"),
}
WORKLOAD_TEXT = {
    "pro_s4096_bf16": "long-sequence forward: B=1, S=4096, N=4, D=5120, bf16 storage, fp32 math",
    "pro_s1024_f32": "Pro-width forward: B=1, S=1024, N=4, D=5120, fp32",
    "flash_s2048_f32": "Flash-width forward: B=1, S=2048, N=4, D=2560, fp32",
}


def algo_bytes(T, N, D, io):
    """Algorithmic HBM bytes per call: every tensor read or written once, the
    fp32 coefficients counted, φ (and dφ) counted once per call."""
    e = 2 if io == "bf16" else 4
    K, C = N * D, N * N + 2 * N
    coef = (N + N * N) * 4  # H_post + H_res (or their gradients), fp32
    phi = K * C * 4 + C * 4
    return {
        "mhc_pre": T * (K * e + D * e + C * 4) + phi,
        "mhc_post": T * (K * e + D * e + coef + K * e),
        "mhc_post_bwd": T * (3 * K * e + 2 * D * e + 2 * coef),
        "mhc_pre_bwd": T * (D * e + 3 * K * e + coef) + 2 * phi,
        # the backward pair of the training step: hc_post's backward without
        # dx, then the hc_pre backward forming dx = H_resᵀ·dx_next + its own
        # part (dx_next read where mhc_pre_bwd reads dx, and H_res)
        "mhc_post_bwd_nodx": T * (2 * K * e + 2 * D * e + 2 * coef),
        "mhc_pre_bwd_mix": T * (D * e + 3 * K * e + coef + N * N * 4) + 2 * phi,
        # hc_post(l) + hc_pre(l+1) with x_next not read back: x, y, H_post/H_res
        # in; x_next, h, H out
        "mhc_post_pre": T * (K * e + D * e + coef + K * e + D * e + C * 4) + phi,
        # stabilised write-back: as mhc_post / mhc_post_bwd plus the norm
        # weights read (and their gradients written) once per call
        "mhc_post_stable_sw": T * (K * e + D * e + coef + K * e) + D * 4,
        "mhc_post_stable_both": T * (K * e + D * e + coef + K * e) + (D + K) * 4,
        "mhc_post_stable_bwd_sw": T * (3 * K * e + 2 * D * e + 2 * coef) + 2 * D * 4,
        "mhc_post_stable_bwd_both": T * (3 * K * e + 2 * D * e + 2 * coef) + 2 * (D + K) * 4,
    }


def kernel_bytes(name, T, N, D, io):
    """Algorithmic bytes of one launch of a kernel, by its short name (see
    short_name): the method's tensors it must read or write once, φ counted
    once; workspace intermediates (partial sums, coefficient records, the
    packed φ copy a later kernel reads) are not counted.  None for kernels
    without such a figure."""
    e = 2 if io == "bf16" else 4
    K, C = N * D, N * N + 2 * N
    phi = K * C * 4
    coef = (N + N * N) * 4
    if name.startswith(("phi_pack_tile_kernel", "phi_pack_kernel")):  # fp32 φ in, its packed copy out
        return 2 * phi
    if name.startswith(("hc_pre_tile_kernel", "hc_pre_mfma_kernel", "hc_pre_generic")):
        return T * (K * e + D * e + C * 4) + phi + C * 4  # x in; h, H_pre/H_post/H_res out; φ, bias in
    if name.startswith("hc_post_generic"):  # x, y, H_post, H_res in; x_next out
        return T * (2 * K * e + D * e + coef)
    if name.startswith("hc_post_bwd_generic"):  # dx_next, x, y, H in; dy, dH (and dx) out
        return T * ((3 if "true" in name else 2) * K * e + 2 * D * e + 2 * coef)
    if name.startswith("res_mix_t_kernel"):  # dx_next, H_res in; dx out
        return T * (2 * K * e + N * N * 4)
    if name.startswith("bwd_proj"):  # x and dh in, φ
        return T * (K * e + D * e) + phi
    if name.startswith("bwd_coef"):  # dH_post and dH_res in (the rest is workspace)
        return T * coef + C * 4
    if name.startswith("bwd_dx"):  # x, dh in; dx out; dx (accumulated) or dx_next and H_res in; φ
        return T * (3 * K * e + D * e + (N * N * 4 if "true" in name else 0)) + phi
    if name.startswith("dphi_bias_sum"):  # dφ and dbias out
        return phi + C * 4
    return None


def short_name(name):
    """Kernel name as the library reports it, without the launch's
    parentheses and namespaces."""
    n = name.strip().strip("()")
    head, sep, tail = n.partition("<")
    return head.split("::")[-1] + sep + tail


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "residual_stream_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, src_hash, workload):
    """HBM traffic per launch of a kernel from the committed rocprofv3 counter
    runs, if they were taken on the current kernel sources and on this
    workload; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("workload") != workload or doc.get("source_hash") != src_hash:
        return None
    ent = doc.get("kernels", {}).get(kernel)
    return ent.get("bytes_per_launch") if ent else None


def cpu_baseline(T, N, D, io, seed, budget_s=10.0):
    """The fp64 oracle (as it stands) on the host: the forward pair over the
    whole batch, repeated until about `budget_s` seconds of work (at least one
    pass, at most 16); matmuls on every core BLAS uses."""
    from threadpoolctl import threadpool_info

    from oracle import mhc_oracle as O
    from residual_stream_amd.inputs import make_inputs

    inp = make_inputs(T, N, D, io=io, seed=seed)
    runs, t0 = 0, time.perf_counter()
    while True:
        pre = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
        O.hc_post(inp.x, inp.y, pre["H_post"], pre["H_res"])
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or runs >= 16:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": runs * T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"forward pair (hc_pre + hc_post) of the whole {T}-token batch (N={N}, D={D}, "
                      f"{io} inputs upcast to fp64), {runs} passes in {dt:.1f} s; matmuls on {threads} "
                      f"BLAS threads, the rest single-threaded; {len(os.sched_getaffinity(0))} host "
                      f"cores available"}


def cpu_train_step(T, N, D, io, seed):
    """One fp64 oracle pass of the training step (forward and backward)."""
    from oracle import mhc_oracle as O
    from residual_stream_amd.inputs import make_inputs

    inp = make_inputs(T, N, D, io=io, seed=seed, grads=True)
    t0 = time.perf_counter()
    pre = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    O.hc_post(inp.x, inp.y, pre["H_post"], pre["H_res"])
    dx, dy, dHp, dHr = O.hc_post_bwd(inp.dx_next, inp.x, inp.y, pre["H_post"], pre["H_res"])
    O.hc_pre_bwd(inp.dh, inp.x, inp.phi, inp.bias, dHp, dHr, inp.alphas, inp.eps, inp.iters)
    dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s", "kind": "oracle",
            "sample": f"one forward + backward pass of the {T}-token batch in {dt:.1f} s"}


class Workload:
    """Two seeded input sets of one workload, resident on the GPU, with every
    output preallocated, and the C-ABI calls of a step on them."""

    def __init__(self, name, seed, dev):
        import torch

        from residual_stream_amd import mhc
        from residual_stream_amd.inputs import make_inputs, make_norm_weights

        self.mhc, self.torch = mhc, torch
        self.name = name
        T, N, D, io = WORKLOADS[name]
        self.T, self.N, self.D, self.io = T, N, D, io
        K, C = N * D, N * N + 2 * N
        tdt = torch.bfloat16 if io == "bf16" else torch.float32
        self.mio = mhc.MHC_BF16 if io == "bf16" else mhc.MHC_F32
        self.kw = dict(iters=20, eps=1e-6, alphas=(0.01, 0.01, 0.01))
        f32 = dict(dtype=torch.float32, device=dev)
        self.sets = []
        for s in range(2):
            inp = make_inputs(T, N, D, io=io, seed=seed + s, grads=True)

            def t(a, dt=None):
                x = torch.from_numpy(a)
                return (x.to(dt) if dt is not None else x).to(dev)

            st = {"x": t(inp.x, tdt), "y": t(inp.y, tdt), "phi": t(inp.phi), "bias": t(inp.bias),
                  "dh": t(inp.dh, tdt), "dxn": t(inp.dx_next, tdt)}
            st["h"] = torch.empty((T, D), dtype=tdt, device=dev)
            st["Hp"] = torch.empty((T, N), **f32)
            st["Hq"] = torch.empty((T, N), **f32)
            st["Hr"] = torch.empty((T, N, N), **f32)
            st["xn"] = torch.empty((T, N, D), dtype=tdt, device=dev)
            st["pp"] = (torch.empty((T, N, D), dtype=tdt, device=dev), torch.empty((T, D), dtype=tdt, device=dev),
                        torch.empty((T, N), **f32), torch.empty((T, N), **f32), torch.empty((T, N, N), **f32))
            st["dx"] = torch.empty((T, N, D), dtype=tdt, device=dev)
            st["dy"] = torch.empty((T, D), dtype=tdt, device=dev)
            st["dHp"] = torch.empty((T, N), **f32)
            st["dHr"] = torch.empty((T, N, N), **f32)
            st["dphi"] = torch.empty((K, C), **f32)
            st["dbias"] = torch.empty((C,), **f32)
            st["dalpha"] = torch.empty((4,), **f32)
            wy, wx = make_norm_weights(N, D, seed=seed + 10 + s)
            st["wy"], st["wx"] = t(wy), t(wx)
            st["dwy"] = torch.empty((D,), **f32)
            st["dwx"] = torch.empty((K,), **f32)
            self.sets.append(st)
            del inp
        ws_pre = mhc.workspace_bytes("pre", T, N, D, self.mio)
        ws_bwd = mhc.workspace_bytes("pre_bwd", T, N, D, self.mio)
        self.ws_pre = torch.empty(max(ws_pre, 256), dtype=torch.uint8, device=dev)
        self.ws_bwd = torch.empty(max(ws_bwd, 256), dtype=torch.uint8, device=dev)
        self.stab_ok = N * ((D + 5119) // 5120) <= 4
        self.ws_stab = {}
        if self.stab_ok:
            for pn in (False, True):
                n = mhc.workspace_bytes("post_stable_bwd", T, N, D, self.mio, y_weight=True, out_weight=pn)
                self.ws_stab[pn] = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        self.fuses = mhc.mix_fuses(N, D, self.mio)

    # -- the calls ---------------------------------------------------------
    def pre(self, st):
        self.mhc.mhc_pre(st["x"], st["phi"], st["bias"], out=(st["h"], st["Hp"], st["Hq"], st["Hr"]),
                         workspace=self.ws_pre, **self.kw)

    def post(self, st):
        self.mhc.mhc_post(st["x"], st["y"], st["Hq"], st["Hr"], out=st["xn"])

    def post_pre(self, st):
        self.mhc.mhc_post_pre(st["x"], st["y"], st["Hq"], st["Hr"], st["phi"], st["bias"], out=st["pp"],
                              workspace=self.ws_pre, **self.kw)

    def post_bwd(self, st, with_dx):
        self.mhc.mhc_post_bwd(st["dxn"], st["x"], st["y"], st["Hq"], st["Hr"],
                              out=(st["dx"] if with_dx else None, st["dy"], st["dHp"], st["dHr"]))

    def pre_bwd_mix(self, st):
        self.mhc.mhc_pre_bwd_mix(st["dh"], st["x"], st["phi"], st["bias"], st["dHp"], st["dHr"], st["dxn"],
                                 st["Hr"], out=(st["dx"], st["dphi"], st["dbias"], st["dalpha"]),
                                 workspace=self.ws_bwd, **self.kw)

    def pre_bwd(self, st):
        self.mhc.mhc_pre_bwd(st["dh"], st["x"], st["phi"], st["bias"], st["dHp"], st["dHr"], st["dx"],
                             out=(st["dphi"], st["dbias"], st["dalpha"]), workspace=self.ws_bwd, **self.kw)

    def stable(self, st, pn):
        self.mhc.mhc_post_stable(st["x"], st["y"], st["Hq"], st["Hr"], y_weight=st["wy"],
                                 out_weight=st["wx"] if pn else None, eps=1e-6, out=st["xn"])

    def stable_bwd(self, st, pn):
        self.mhc.mhc_post_stable_bwd(st["dxn"], st["x"], st["y"], st["Hq"], st["Hr"], y_weight=st["wy"],
                                     out_weight=st["wx"] if pn else None, eps=1e-6,
                                     out=(st["dx"], st["dy"], st["dHp"], st["dHr"], st["dwy"],
                                          st["dwx"] if pn else None), workspace=self.ws_stab[pn])

    def forward_calls(self):
        return [("mhc_pre", self.pre), ("mhc_post", self.post)]

    def train_calls(self):
        # the backward pair: hc_post's backward without dx and the hc_pre
        # backward forming it, where the library fuses that mix into its dx
        # pass; else the two-call backward (the faster one there)
        if self.fuses:
            bwd = [("mhc_post_bwd_nodx", lambda st: self.post_bwd(st, False)), ("mhc_pre_bwd_mix", self.pre_bwd_mix)]
        else:
            bwd = [("mhc_post_bwd", lambda st: self.post_bwd(st, True)), ("mhc_pre_bwd", self.pre_bwd)]
        return self.forward_calls() + bwd

    # -- timing ------------------------------------------------------------
    def wall(self, calls, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            for _, f in calls:
                f(self.sets[i % 2])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            for _, f in calls:
                f(self.sets[i % 2])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def kernel_times(self, calls, steps):
        """Per-kernel durations (µs, averaged over the steps) from HIP events
        the library records around each launch on the stream it runs on."""
        torch = self.torch
        probe = self.mhc.KernelTrace(64)
        with probe:
            for _, f in calls:
                f(self.sets[0])
        torch.cuda.synchronize()
        per_step = len(probe.durations_us())
        tr = self.mhc.KernelTrace(per_step * steps)
        with tr:
            for i in range(steps):
                for _, f in calls:
                    f(self.sets[i % 2])
        torch.cuda.synchronize()
        rec = tr.durations_us()
        out = {}
        for k, (name, us) in enumerate(rec):
            key = f"{k % per_step}:{short_name(name)}"
            out.setdefault(key, []).append(us)
        return {k: {"avg_us": sum(v) / len(v), "min_us": min(v), "max_us": max(v), "launches": len(v)}
                for k, v in out.items()}

    def call_times(self, calls, which, steps):
        """HIP-event time of the calls named in `which` (one event pair around
        them), the rest of the step run on the other input set in between."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            st = self.sets[i % 2]
            evs[i][0].record(self.stream)
            for name, f in calls:
                if name in which:
                    f(st)
            evs[i][1].record(self.stream)
            for name, f in calls:
                if name not in which:
                    f(self.sets[(i + 1) % 2])
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return {"avg_us": sum(ts) / len(ts), "median_us": ts[len(ts) // 2],
                "p10_us": ts[int(0.1 * (len(ts) - 1))], "p90_us": ts[int(round(0.9 * (len(ts) - 1)))]}

    def extra_call_time(self, f, steps, calls):
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record(self.stream)
            f(self.sets[i % 2])
            evs[i][1].record(self.stream)
            for _, g in calls:
                g(self.sets[(i + 1) % 2])
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return sum(ts) / len(ts)


def roofline_of(kernels, T, N, D, io, workload, src_hash):
    """The kernel with the largest average duration and its HBM figures."""
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    name = dom.split(":", 1)[1]
    ab = kernel_bytes(name, T, N, D, io)
    avg = kernels[dom]["avg_us"]
    achieved = ab / (avg * 1e-6) / 1e9 if ab else None
    return {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS if achieved else None,
            "traffic": load_traffic(name, src_hash, workload), "algo_bytes_per_launch": ab, "avg_us": avg,
            "timing": "HIP events the library records around each launch on its stream, averaged over the "
                      "traced pass of the K steps"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="pro_s4096_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the timed step, its roofline and the CPU baseline")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the fp32 configurations (so that counter runs see one workload's launches)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of one x-sized bf16 tensor (5 times), "
                         "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the mHC hot path is token-local and this "
              "build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from residual_stream_amd import mhc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, N, D, io = WORKLOADS[args.workload]
    if args.calibrate_copy:
        n = T * N * D
        a = torch.ones(n, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 2 * n, "calibrate_copy_bytes_written": 2 * n,
                          "launches": 5}))
        return
    mhc.load()
    src_hash = kernel_source_hash()
    say = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)  # noqa: E731

    W = Workload(args.workload, args.seed, dev)
    ab = algo_bytes(T, N, D, io)
    fwd = W.forward_calls()
    say(f"workload {args.workload}: T={T} N={N} D={D} io={io}; warmup {args.warmup}, {args.steps} steps")

    # ---- timed region: exactly K forward steps ----
    ms_step = W.wall(fwd, args.steps, args.warmup)
    say(f"forward step {ms_step:.4f} ms")
    fwd_bytes = ab["mhc_pre"] + ab["mhc_post"]
    kernels = W.kernel_times(fwd, args.steps)
    roof = roofline_of(kernels, T, N, D, io, args.workload, src_hash)

    out = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": io,
        "data": "synthetic (seeded Gaussian x, y; phi ~ N(0, 1/(N*D)); bias ~ N(0, 0.1))",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": T, "N": N, "D": D, "io": io,
                   "sinkhorn_iters": 20, "alpha": 0.01, "step": "mhc_pre + mhc_post"},
        "step_algo_bytes": fwd_bytes,
        "step_gbps": fwd_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": fwd_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernels": {k: dict(v, algo_bytes=kernel_bytes(k.split(":", 1)[1], T, N, D, io)) for k, v in kernels.items()},
        "roofline": roof,
        "kernel_source_hash": src_hash,
    }

    if not args.no_extras:
        # forward calls one at a time, and the pair, with HIP events
        per_call = {}
        for name, _ in fwd:
            r = W.call_times(fwd, {name}, args.steps)
            r.update(algo_bytes=ab[name], gbps=ab[name] / (r["avg_us"] * 1e-6) / 1e9)
            per_call[name] = r
        pair = W.call_times(fwd, {"mhc_pre", "mhc_post"}, args.steps)
        pair.update(algo_bytes=fwd_bytes, gbps=fwd_bytes / (pair["avg_us"] * 1e-6) / 1e9,
                    frac_of_peak=fwd_bytes / (pair["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS)
        # an on-box device copy moving the pair's bytes (half read, half written)
        n_cp = fwd_bytes // 4
        cp_src = torch.ones(n_cp, dtype=torch.bfloat16, device=dev)
        cp_dst = torch.empty_like(cp_src)
        cp_us = W.extra_call_time(lambda st: cp_dst.copy_(cp_src), args.steps, fwd)
        del cp_src, cp_dst
        pair["copy_gbps"] = 4 * n_cp / (cp_us * 1e-6) / 1e9
        pair["frac_of_copy"] = pair["gbps"] / pair["copy_gbps"]
        out["forward"] = {"pair_events": pair, "per_call": per_call}

        # the forward step on each input set, both captured in one HIP graph
        # (so a replay's launch is shared by two steps)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s_idx in range(2):
                for _, f in fwd:
                    f(W.sets[s_idx])
        for i in range((args.warmup + 1) // 2):
            g.replay()
        torch.cuda.synchronize()
        replays = max(1, (args.steps + 1) // 2)
        t0 = time.perf_counter()
        for i in range(replays):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / (2 * replays)
        del g
        out["graph_step"] = {"ms_per_step": graph_ms, "tokens_per_s": T / (graph_ms * 1e-3),
                             "note": "the forward step replayed from a HIP graph holding one step per input set"}

        # the training step of the same shape (configuration: forward plus backward)
        train = W.train_calls()
        tr_ms = W.wall(train, args.steps, 2)
        tr_kernels = W.kernel_times(train, args.steps)
        tr_bytes = sum(ab[n] for n, _ in train)
        tr_calls = {}
        for name, _ in train[2:]:
            r = W.call_times(train, {name}, args.steps)
            r.update(algo_bytes=ab[name], gbps=ab[name] / (r["avg_us"] * 1e-6) / 1e9)
            tr_calls[name] = r
        out["train_step"] = {
            "step": " + ".join(n for n, _ in train), "ms_per_step": tr_ms, "tokens_per_s": T / (tr_ms * 1e-3),
            "algo_bytes": tr_bytes, "gbps": tr_bytes / (tr_ms * 1e-3) / 1e9,
            "kernels": {k: dict(v, algo_bytes=kernel_bytes(k.split(":", 1)[1], T, N, D, io))
                        for k, v in tr_kernels.items()},
            "roofline": roofline_of(tr_kernels, T, N, D, io, args.workload, src_hash),
            "backward_calls": tr_calls}

        # hc_post of a layer with hc_pre of the next (one call per boundary)
        pp_us = W.extra_call_time(W.post_pre, args.steps, fwd)
        out["post_pre"] = {"call": "mhc_post_pre (hc_post of a layer + hc_pre of the next)", "avg_us": pp_us,
                           "algo_bytes": ab["mhc_post_pre"], "gbps": ab["mhc_post_pre"] / (pp_us * 1e-6) / 1e9}

        # openPangu's stabilised write-back: sandwich norm (every layer), block
        # post-norm as well (every fifth)
        if W.stab_ok:
            stabilised = {}
            for name, f in (("mhc_post_stable_sw", lambda st: W.stable(st, False)),
                            ("mhc_post_stable_both", lambda st: W.stable(st, True)),
                            ("mhc_post_stable_bwd_sw", lambda st: W.stable_bwd(st, False)),
                            ("mhc_post_stable_bwd_both", lambda st: W.stable_bwd(st, True))):
                us = W.extra_call_time(f, args.steps, fwd)
                gbps = ab[name] / (us * 1e-6) / 1e9
                stabilised[name] = {"avg_us": us, "algo_bytes": ab[name], "gbps": gbps,
                                    "frac_of_peak": gbps / HBM_PEAK_GBPS}
            out["stabilised_write_back"] = stabilised

        # the fp32 configurations of the pages' measurement paragraph
        others = {}
        for wname in ("pro_s1024_f32", "flash_s2048_f32"):
            if wname == args.workload or args.no_other_workloads:
                continue
            del W
            torch.cuda.empty_cache()
            W = Workload(wname, args.seed, dev)
            Tw, Nw, Dw, iow = WORKLOADS[wname]
            abw = algo_bytes(Tw, Nw, Dw, iow)
            fw = W.forward_calls()
            f_ms = W.wall(fw, args.steps, args.warmup)
            f_kernels = W.kernel_times(fw, args.steps)
            f_bytes = abw["mhc_pre"] + abw["mhc_post"]
            tw = W.train_calls()
            t_ms = W.wall(tw, args.steps, 2)
            t_kernels = W.kernel_times(tw, args.steps)
            others[wname] = {
                "workload": WORKLOAD_TEXT[wname],
                "forward": {"ms_per_step": f_ms, "tokens_per_s": Tw / (f_ms * 1e-3), "algo_bytes": f_bytes,
                            "gbps": f_bytes / (f_ms * 1e-3) / 1e9,
                            "frac_of_peak": f_bytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                            "kernels": f_kernels, "roofline": roofline_of(f_kernels, Tw, Nw, Dw, iow, wname, src_hash)},
                "train_step": {"step": " + ".join(n for n, _ in tw), "ms_per_step": t_ms,
                               "tokens_per_s": Tw / (t_ms * 1e-3), "kernels": t_kernels}}
        out["other_workloads"] = others

    if not args.no_cpu_baseline:
        say("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(T, N, D, io, args.seed)
        if not args.no_extras:
            out["train_step"]["cpu_baseline"] = cpu_train_step(T, N, D, io, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
