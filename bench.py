"""Benchmark: causal HyperAttention forward on one MI355X.

One step is one full hyperattn_forward (hash, V-norm weights, sortLSH sorts,
samples, bucket/sample attention on every recursion level, exact base case
with the merge) over one batch of synthetic inputs already resident in HBM.
Default workload: batch 1, 32 heads, n = 131072, d = 128, bf16, b = m = 256,
r = 8, recursion base 4096 (RoPE on Q and K).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (timed
live with the library's hipEvents on the launch stream, in a second pass of
the same steps after the timed region), the library's own
exact causal attention at the same shape, and the CPU oracle timed on a
bounded sample (one head of the same workload).
"""

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal HyperAttention fwd tokens/s at n=131k,d=128,32 heads; % MFMA peak"


def metric_for(w):
    """The headline metric for the headline workload; the same wording with
    the workload's own shape for the others."""
    from approximate_softmax_attention_amd import workloads as wl
    if w.name == wl.HEADLINE:
        return METRIC
    kind = "causal" if w.causal else "non-causal"
    return f"{kind} HyperAttention fwd tokens/s at n={w.n},d={w.d},{w.heads} heads"


def data_for(w):
    parts = ["seeded iid N(0,1)"]
    if w.planted:
        parts.append(f"{w.planted} planted keys per query")
    if w.rope:
        parts.append("RoPE on Q,K")
    return "synthetic (" + ", ".join(parts) + ")"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()
PEAK_BF16 = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12         # bytes/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_pass(torch, api, fn, steps):
    """Per-kernel durations over `steps` more calls of fn, after the timed
    region: the library's kernel timer records two HIP events on the launch
    stream around every launch, which add a few microseconds each, so the
    step time is measured without it and the kernels are timed in this
    identical pass. Returns (the timer, ms per step of this pass)."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with api.KernelTimer() as kt:
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
    return kt, e0.elapsed_time(e1) / steps


def kernel_source_hash(backward=False):
    """sha256 over the sources of the forward pass's kernels (file names and
    code), or with backward=True over every kernel source. Comments and blank
    lines are left out, so that editing a comment keeps a profile valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    src = os.path.join(ROOT, "approximate_softmax_attention_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".h", ".cpp")) and (backward or name != "backward.hip"):
            h.update(name.encode())
            with open(os.path.join(src, name)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            code = [re.sub(r"//.*", "", line).rstrip() for line in text.splitlines()]
            h.update("\n".join(line for line in code if line.strip()).encode())
    return h.hexdigest()


def profiled_traffic(workload, kernel, backward=False):
    """HBM bytes per launch of `kernel` (read + written, scaled by the plain
    copy calibration) from the committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    name = "backward_hbm_traffic" if backward else "hbm_traffic"
    path = os.path.join(ROOT, "profiles", f"hyperattn_{workload}_{name}.md")
    if not os.path.exists(path):
        return None
    sha, val = None, None
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`")
            if line.startswith("source-sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith(f"bytes-per-launch {kernel}:"):
                val = int(line.split(":", 1)[1])
    if sha is None or sha != kernel_source_hash(backward):
        return None
    return val


def profiled_mfma(workload, kernel, backward=False):
    """(MFMA-busy fraction, clock in GHz) of `kernel` from the committed
    rocprofv3 MFMA counter summary (the forward pass's, or with backward=True
    the forward + backward call's), or None when there is none or the kernel
    sources changed since it was taken."""
    name = "backward_mfma_counters" if backward else "mfma_counters"
    path = os.path.join(ROOT, "profiles", f"hyperattn_{workload}_{name}.md")
    if not os.path.exists(path):
        return None
    sha, busy, clock = None, None, None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("source-sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith(f"mfma-busy {kernel}:"):
                busy = float(line.split(":", 1)[1])
            elif line.startswith(f"clock-ghz {kernel}:"):
                clock = float(line.split(":", 1)[1])
    if sha is None or sha != kernel_source_hash(backward) or busy is None:
        return None
    return busy, clock


def algorithmic_flops(w):
    """MFMA flops the method must do, per kernel (per launch)."""
    H, n, d, b, m = w.heads, w.n, w.d, w.b, w.m
    out = {}
    if w.causal:
        L, size = 0, n
        while size > w.recursion_base:
            size //= 2
            L += 1
        rows = 0
        per_row = 0.0
        for lv in range(L):
            h = n >> (lv + 1)
            be = min(b, h)
            mm = min(m, h)
            per_row += (n // 2) * (4 * be * d + 2 * mm * d + 4 * mm * d)
        out["bucket_attention"] = H * per_row
        B = size
        out["exact_base_merge"] = H * (n // B) * 4.0 * d * B * (B + 1) / 2
    else:
        be, mm = min(b, n), min(m, n)
        out["bucket_attention"] = H * n * (4 * be * d + 2 * mm * d + 4 * mm * d)
    return out


def hbm_bytes(w):
    """Algorithmic HBM bytes per launch of the bandwidth-bound forward
    kernels: the hash reads Q and K and writes one code byte per row; the
    V-norm pass reads V and writes the fp64 squared norms; the sort scatter
    reads a code byte and writes a 4-byte perm and a 4-byte rank entry per
    element of every level's segments (n per head per level)."""
    H, n, d = w.heads, w.n, w.d
    es = 2 if w.dtype == "bf16" else 4
    levels = 0
    if w.causal:
        size = n
        while size > w.recursion_base:
            size //= 2
            levels += 1
    else:
        levels = 1
    return {"hash": 2 * H * n * d * es + 2 * H * n,
            "vnorm_rows": H * n * d * es + H * n * 8,
            "sort_scatter": levels * H * n * 9}


def levels_of(w):
    """Sub-problem sizes of the causal recursion (non-causal: [n])."""
    if not w.causal:
        return [w.n]
    out, size = [], w.n
    while size > w.recursion_base:
        size //= 2
        out.append(size)
    return out


def attention_bytes(w):
    """Algorithmic HBM bytes per launch of the attention kernels: the bucket
    kernel reads each query, key and value row of every level's sub-problems
    once (gathered in bucket order) and writes each query row's partial
    output and lse once; the base case reads Q, K and V once, reads every
    level's partials once and writes O and lse."""
    H, n, d = w.heads, w.n, w.d
    es = 2 if w.dtype == "bf16" else 4
    row, out_row = d * es, d * es + 4
    lv = levels_of(w)
    rows = n // 2 if w.causal else n
    out = {"bucket_attention": H * len(lv) * rows * (3 * row + out_row)}
    if w.causal:
        out["exact_base_merge"] = H * (3 * n * row + len(lv) * rows * out_row + n * out_row)
    return out


def exact_flops(w):
    H, n, d = w.heads, w.n, w.d
    return H * 4.0 * d * (n * (n + 1) / 2 if w.causal else n * n)


def make_device_inputs(w, torch, pairs=None):
    """Q, K, V on the device; the planted pairs of each head go to `pairs`
    (a list) when given."""
    from approximate_softmax_attention_amd import workloads as wl
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Q = torch.empty((w.heads, w.n, w.d), dtype=dt, device="cuda")
    K, V = torch.empty_like(Q), torch.empty_like(Q)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))

    def one(h):
        q, k, v, pr = wl.make_head(w, h)
        return h, q, k, v, pr

    with cf.ThreadPoolExecutor(workers) as ex:
        for h, q, k, v, pr in ex.map(one, range(w.heads)):
            Q[h].copy_(torch.from_numpy(q).to(dt))
            K[h].copy_(torch.from_numpy(k).to(dt))
            V[h].copy_(torch.from_numpy(v).to(dt))
            if pairs is not None:
                pairs.append(pr)
    torch.cuda.synchronize()
    return Q, K, V


def planted_recall(w, api, Q, K, V, pairs):
    """Fraction of planted (query, key) pairs whose query and key land in the
    same sortLSH bucket, from the library's own sorted orders."""
    import numpy as np
    art = api.debug_artifacts(Q, K, V, causal=w.causal, b=w.b, m=w.m, r=w.r,
                              recursion_base=w.recursion_base, seed=w.method_seed)
    perm_q = art["PERM_Q"].reshape(w.heads, w.n)
    perm_k = art["PERM_K"].reshape(w.heads, w.n)
    be = min(w.b, w.n)
    hits = tot = 0
    for h in range(w.heads):
        bq = np.empty(w.n, dtype=np.int64)
        bq[perm_q[h]] = np.arange(w.n) // be
        bk = np.empty(w.n, dtype=np.int64)
        bk[perm_k[h]] = np.arange(w.n) // be
        p = pairs[h]
        hits += int((bq[p[:, 0]] == bk[p[:, 1]]).sum())
        tot += len(p)
    return {"recall": hits / tot, "pairs": tot,
            "meaning": "planted pairs whose query and key share a sortLSH bucket"}


def cpu_baseline(w):
    """The oracle as it stands, on one head of the workload, scaled to all heads."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from approximate_softmax_attention_amd import workloads as wl
    from oracle import hyperattention as oha
    q, k, v, _ = wl.make_head(w, 0)
    t0 = time.perf_counter()
    oha.hyperattention(q[None], k[None], v[None], causal=w.causal, b=w.b, m=w.m, r=w.r,
                       recursion_base=w.recursion_base, seed=w.method_seed)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    per_forward = dt * w.heads
    return {"value": w.n / per_forward, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"1 of {w.heads} heads of the same workload (full n={w.n} "
                      f"forward, fp64 numpy), {dt:.1f} s, scaled x{w.heads}",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "exact_oracle": cpu_baseline_exact(w)}


def cpu_baseline_exact(w):
    """The oracle's exact attention as it stands: the whole workload when its
    score matrices are small (heads * n^2 <= 2^31), else 4096 position-
    stratified query rows of head 0 scaled by the number of (query, key)
    pairs of the whole forward ("extrapolated"; about 25 s at n = 131072)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from approximate_softmax_attention_amd import workloads as wl
    from oracle import exact as oexact
    pairs_total = w.heads * (w.n * (w.n + 1) / 2 if w.causal else float(w.n) * w.n)
    if w.heads * w.n * w.n <= (1 << 31):
        Q, K, V, _ = wl.make_inputs(w)
        t0 = time.perf_counter()
        for h in range(w.heads):
            oexact.exact_attention(Q[h], K[h], V[h], causal=w.causal)
        dt = time.perf_counter() - t0
        full, sample = dt, f"the whole workload ({w.heads} heads), {dt:.1f} s"
    else:
        q, k, v, _ = wl.make_head(w, 0)
        nrows = 4096
        edges = np.linspace(0, w.n, nrows + 1).astype(np.int64)
        rs = np.random.default_rng(0)
        rows = np.array([rs.integers(lo, hi) for lo, hi in zip(edges[:-1], edges[1:])])
        t0 = time.perf_counter()
        oexact.exact_attention_rows(q, k, v, rows, causal=w.causal)
        dt = time.perf_counter() - t0
        pairs = float((rows + 1).sum()) if w.causal else float(len(rows)) * w.n
        full = dt * pairs_total / pairs
        sample = (f"{nrows} position-stratified rows of head 0, {dt:.1f} s, extrapolated "
                  f"by (query, key) pairs to all {w.heads} heads")
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": w.n / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "extrapolated": w.heads * w.n * w.n > (1 << 31)}


def sweep(args, torch, api):
    """HA page, "Single self-attention layer": one layer's forward time and
    forward + backward time against n, causal and non-causal, with exact
    attention beside it. Inputs are seeded iid N(0, 1) bf16 tensors of the
    page's shape (d = 64, 12 heads); dO likewise."""
    H, d = args.sweep_heads, args.sweep_d
    g = torch.Generator(device="cuda")
    g.manual_seed(20231009)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for causal in (False, True):
        n = 4096
        while n <= 131072:
            q, k, v = (torch.randn(H, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
                       for _ in range(3))
            kw = dict(causal=causal, b=256, m=256, r=8, recursion_base=4096, seed=7)
            ws = api.alloc_workspace(api.workspace_bytes(n, d, H, **{x: kw[x] for x in (
                "causal", "b", "m", "r", "recursion_base")}), "cuda")
            o = torch.empty_like(q)
            oe = torch.empty_like(q)
            reps = max(2, min(20, (1 << 22) // n))
            t_h = timed(lambda: api.forward(q, k, v, workspace=ws, out=o, **kw), reps)
            t_e = timed(lambda: api.exact(q, k, v, causal=causal, out=oe), max(2, reps // 4))
            rec = {"sweep": "single layer", "heads": H, "head_dim": d,
                   "seq_len": n, "causal": causal, "dtype": "bf16",
                   "hyperattention_ms": t_h, "exact_ms": t_e, "speedup": t_e / t_h}
            if not args.no_backward:
                do = torch.randn(q.shape, device="cuda", dtype=torch.bfloat16, generator=g)
                lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
                le = torch.empty_like(lse)
                wsb = api.alloc_workspace(api.backward_workspace_bytes(n, d, H, **{
                    x: kw[x] for x in ("causal", "b", "m", "r", "recursion_base")}), "cuda")

                def h_fb():
                    api.forward(q, k, v, workspace=ws, out=o, lse_out=lse, return_lse=True, **kw)
                    api.backward(q, k, v, o, lse, do, workspace=wsb, **kw)

                def e_fb():
                    api.exact(q, k, v, causal=causal, out=oe, lse_out=le, return_lse=True)
                    api.exact_backward(q, k, v, oe, le, do, causal=causal)

                rec["hyperattention_fwd_bwd_ms"] = timed(h_fb, max(2, reps // 2))
                rec["exact_fwd_bwd_ms"] = timed(e_fb, max(2, reps // 8))
                rec["fwd_bwd_speedup"] = rec["exact_fwd_bwd_ms"] / rec["hyperattention_fwd_bwd_ms"]
                del do, lse, le, wsb
            print(json.dumps(rec), flush=True)
            del q, k, v, ws, o, oe
            torch.cuda.empty_cache()
            n *= 2


def rope_mode(args, torch, api, wl):
    """The headline workload with its rotary embedding applied by the library
    (hyperattn_forward_rope on the rows before RoPE): one JSON line with the
    forward time and the per-kernel breakdown, the fused rotate-and-hash pass
    included."""
    w = wl.scaled(wl.WORKLOADS[args.workload or wl.HEADLINE], rope=False)
    log(f"workload {w.name} before RoPE: generating inputs")
    Q, K, V = make_device_inputs(w, torch)
    nb = api.workspace_bytes(w.n, w.d, w.heads, causal=w.causal, b=w.b, m=w.m, r=w.r,
                             recursion_base=w.recursion_base,
                             dtype=api.HA_BF16 if w.dtype == "bf16" else api.HA_F32)
    ws = api.alloc_workspace(nb, "cuda")
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              seed=w.method_seed, workspace=ws)
    for _ in range(args.warmup):
        api.forward_rope(Q, K, V, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        api.forward_rope(Q, K, V, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kt, ms_inst = kernel_pass(torch, api, lambda: api.forward_rope(Q, K, V, **kw), args.steps)
    kernels = {k: {"launches": n, "avg_ms": t / n} for k, (n, t) in kt.stats.items()}
    rh = kernels.get("rope_hash", {}).get("avg_ms")
    # rope_hash reads Q and K, writes them rotated, reads the cos/sin table once
    moved = 2 * 2 * w.heads * w.n * w.d * (2 if w.dtype == "bf16" else 4) + w.n * w.d * 8
    print(json.dumps({"mode": "forward_rope", "workload": w.name + " (RoPE on the device)",
                      "steps": args.steps, "ms_per_step": ms, "tokens_per_s": w.n / (ms / 1e3),
                      "ms_per_step_kernel_pass": ms_inst,
                      "rope_hash_gbs": moved / (rh / 1e3) / 1e9 if rh else None,
                      "rope_hash_hbm_frac": moved / (rh / 1e3) / PEAK_HBM if rh else None,
                      "kernels": kernels}), flush=True)


def backward_flops(w):
    """MFMA flops the backward pass must do (the products the gradient
    formulas need, counted once), per kernel group: per query row of a level,
    the bucket's keys need S, dP, dQ, dK, dV (5 products of 2bd), the uniform
    sample S, dQ, dK (3 of 2md) and the V-norm sample all five; the base case
    needs the five products over its causal half."""
    H, n, d, b, m = w.heads, w.n, w.d, w.b, w.m
    out = {}
    if w.causal:
        L, size = 0, n
        while size > w.recursion_base:
            size //= 2
            L += 1
        lv_flops = 0.0
        for lv in range(L):
            h = n >> (lv + 1)
            be, mm = min(b, h), min(m, h)
            lv_flops += (n // 2) * 2 * d * (5 * be + 8 * mm)
        out["levels"] = H * lv_flops
        out["base"] = H * (n // size) * 5 * 2.0 * d * size * (size + 1) / 2
    else:
        be, mm = min(b, n), min(m, n)
        out["levels"] = H * n * 2 * d * (5 * be + 8 * mm)
    return out


def copy_calibration(torch):
    """A plain 1 GiB copy (reads 1 GiB, writes 1 GiB) for scaling HBM byte
    counters against known traffic."""
    log("plain copy of 1 GiB (reads 1 GiB, writes 1 GiB)")
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1, out=dst)
    torch.cuda.synchronize()
    del src, dst


def backward_kernel_flops(w):
    """MFMA flops each backward kernel needs (per launch), counting the
    products that kernel's own results require: the key-major kernels need
    S, dP, dV and dK, the query-major ones S, dP and dQ (so S and dP count in
    both); uniform sample slots need no dP, dV (query-major: no dP)."""
    H, n, d, b, m = w.heads, w.n, w.d, w.b, w.m
    out = {"bwd_bucket_q": 0.0, "bwd_bucket_kv": 0.0, "bwd_sample_kv": 0.0}
    size = n
    levels = []
    if w.causal:
        while size > w.recursion_base:
            size //= 2
            levels.append(size)
    else:
        levels = [n]
    for h in levels:
        be, mm = min(b, h), min(m, h)
        rows = n // 2 if w.causal else n
        out["bwd_bucket_q"] += H * rows * 2 * d * (3 * be + 2 * mm + 3 * mm)
        out["bwd_bucket_kv"] += H * rows * 2 * d * 4 * be
        out["bwd_sample_kv"] += H * rows * 2 * d * (2 * mm + 4 * mm)
    if w.causal:
        pairs = H * (n // size) * size * (size + 1) / 2
        out["bwd_base_q"] = 3 * 2.0 * d * pairs
        out["bwd_base_kv"] = 4 * 2.0 * d * pairs
    return out


def backward_mode(args, torch, api, wl):
    """The headline workload's forward and backward pass (the HA page times
    forward + backward in its single-layer experiment), with exact attention's
    forward + backward beside it; one JSON line with the per-kernel
    breakdown."""
    w = wl.WORKLOADS[args.workload or wl.HEADLINE]
    log(f"workload {w.name}: generating inputs")
    Q, K, V = make_device_inputs(w, torch)
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    dO = torch.randn(Q.shape, device="cuda", dtype=Q.dtype, generator=g)
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              seed=w.method_seed)
    wsf = api.alloc_workspace(api.workspace_bytes(w.n, w.d, w.heads, causal=w.causal, b=w.b,
                                                  m=w.m, r=w.r,
                                                  recursion_base=w.recursion_base), "cuda")
    wsb = api.alloc_workspace(api.backward_workspace_bytes(w.n, w.d, w.heads, causal=w.causal,
                                                           b=w.b, m=w.m, r=w.r,
                                                           recursion_base=w.recursion_base),
                              "cuda")
    O = torch.empty_like(Q)
    lse = torch.empty((w.heads, w.n), dtype=torch.float32, device="cuda")

    def step():
        api.forward(Q, K, V, workspace=wsf, out=O, lse_out=lse, return_lse=True, **kw)
        return api.backward(Q, K, V, O, lse, dO, workspace=wsb, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kt, ms_inst = kernel_pass(torch, api, step, args.steps)
    kernels = {k: {"launches": n, "avg_ms": t / n} for k, (n, t) in kt.stats.items()}
    fl = backward_flops(w)
    groups = {"levels": ("bwd_sample_kv", "bwd_bucket_q", "bwd_bucket_kv"),
              "base": ("bwd_base_q", "bwd_base_kv")}
    mfma = {}
    for grp, names in groups.items():
        t = sum(kernels.get(k, {}).get("avg_ms", 0.0) for k in names)
        if grp in fl and t > 0:
            mfma[grp] = {"tflops": fl[grp] / (t / 1e3) / 1e12,
                         "frac": fl[grp] / (t / 1e3) / PEAK_BF16}
    bwd_ms = sum(v["avg_ms"] for k, v in kernels.items() if k.startswith("bwd_")) + sum(
        kernels.get(k, {}).get("avg_ms", 0.0) for k in ("hash", "vnorm_rows", "vnorm_weights",
                                                          "vnorm_prefix", "sort_hist",
                                                          "sort_scatter", "samples")) / 2
    kfl = backward_kernel_flops(w)
    dom = max((k for k in kfl if k in kernels), key=lambda k: kernels[k]["avg_ms"])
    achieved = kfl[dom] / (kernels[dom]["avg_ms"] / 1e3)
    traffic = profiled_traffic(w.name, dom, backward=True)
    for k in kfl:
        if k in kernels:
            kernels[k]["tflops"] = kfl[k] / (kernels[k]["avg_ms"] / 1e3) / 1e12
    rec = {"mode": "forward_backward",
           "metric": "causal HyperAttention fwd+bwd tokens/s at the same workload",
           "value": w.n / (ms / 1e3), "unit": "tokens/s", "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic", "workload": w.name, "steps": args.steps,
           "ms_per_step": ms, "tokens_per_s": w.n / (ms / 1e3), "kernels": kernels,
           "backward_ms_approx": bwd_ms, "backward_mfma": mfma,
           "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16 / 1e12,
                        "unit": "TFLOP/s", "frac": achieved / PEAK_BF16, "traffic": traffic,
                        "kernel": dom, "flops_per_launch": kfl[dom]}}
    counters = profiled_mfma(w.name, dom, backward=True)
    if counters is not None:
        rec["roofline"]["mfma_busy"], rec["roofline"]["clock_ghz"] = counters
    if not args.no_exact:
        Oe = torch.empty_like(Q)
        le = torch.empty_like(lse)

        def exact_step():
            api.exact(Q, K, V, causal=w.causal, out=Oe, lse_out=le, return_lse=True)
            return api.exact_backward(Q, K, V, Oe, le, dO, causal=w.causal)

        exact_step()
        torch.cuda.synchronize()
        e0.record(stream)
        exact_step()
        e1.record(stream)
        torch.cuda.synchronize()
        rec["exact_ms_per_step"] = e0.elapsed_time(e1)
        rec["speedup_vs_exact"] = rec["exact_ms_per_step"] / ms
    if args.copy_calibration:
        copy_calibration(torch)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle's forward + backward on one head")
        rec["cpu_baseline"] = cpu_baseline_backward(w)
    print(json.dumps(rec), flush=True)


def cpu_baseline_backward(w):
    """The oracle's forward + backward (oracle.backward recomputes the
    forward) on one head of the workload, scaled to all heads."""
    from threadpoolctl import threadpool_info

    from approximate_softmax_attention_amd import workloads as wl
    from oracle import backward as obw
    q, k, v, _ = wl.make_head(w, 0)
    do = wl.make_grad(w, heads=[0])[0]
    t0 = time.perf_counter()
    obw.hyperattention_backward(q[None], k[None], v[None], do[None], causal=w.causal, b=w.b,
                                m=w.m, r=w.r, recursion_base=w.recursion_base,
                                seed=w.method_seed)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": w.n / (dt * w.heads), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"1 of {w.heads} heads of the same workload (full n={w.n} forward + "
                      f"backward, fp64 numpy), {dt:.1f} s, scaled x{w.heads}",
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="the single-layer sweep of the HA page's experiment: forward time "
                         "of HyperAttention and of exact attention for n = 4096 .. 131072, "
                         "causal and not; one JSON line per point")
    ap.add_argument("--rope", action="store_true",
                    help="time the headline workload with RoPE applied by the library "
                         "(hyperattn_forward_rope on the rows before RoPE); one JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward on the headline workload (and exact "
                         "attention's forward + backward); one JSON line")
    ap.add_argument("--no-backward", action="store_true",
                    help="with --sweep: forward times only")
    ap.add_argument("--sweep-heads", type=int, default=12)
    ap.add_argument("--sweep-d", type=int, default=64)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (torch elementwise kernel) "
                         "so that HBM byte counters can be scaled against known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "HyperAttention shards by head with no communication, so the "
              "whole-job rate at N GPUs is not measured here.", file=sys.stderr)
        sys.exit(2)

    import torch

    from approximate_softmax_attention_amd import api, workloads as wl
    from approximate_softmax_attention_amd._lib import HA_BF16, HA_F32

    if args.sweep:
        sweep(args, torch, api)
        return
    if args.rope:
        rope_mode(args, torch, api, wl)
        return
    if args.backward:
        backward_mode(args, torch, api, wl)
        return

    w = wl.WORKLOADS[args.workload or wl.HEADLINE]
    log(f"workload {w.name}: generating inputs")
    pairs = [] if w.planted and not w.causal else None
    Q, K, V = make_device_inputs(w, torch, pairs)
    dtc = HA_BF16 if w.dtype == "bf16" else HA_F32
    nb = api.workspace_bytes(w.n, w.d, w.heads, causal=w.causal, b=w.b, m=w.m, r=w.r,
                             recursion_base=w.recursion_base, dtype=dtc)
    ws = api.alloc_workspace(nb, "cuda")
    O = torch.empty_like(Q)
    lse = torch.empty((w.heads, w.n), dtype=torch.float32, device="cuda")
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              seed=w.method_seed, workspace=ws, out=O, lse_out=lse)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        api.forward(Q, K, V, **kw)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    e0.record(stream)
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        api.forward(Q, K, V, **kw)
        marks[i + 1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    tokens_per_s = w.n / (ms / 1e3)
    log(f"{ms:.3f} ms/step, {tokens_per_s:.4g} tokens/s (wall {wall / args.steps * 1e3:.3f} ms)")
    log(f"per-kernel pass: {args.steps} more steps under the library's kernel timer")
    kt, ms_inst = kernel_pass(torch, api, lambda: api.forward(Q, K, V, **kw), args.steps)

    flops = algorithmic_flops(w)
    kernels = {}
    for name, (launches, total) in kt.stats.items():
        kernels[name] = {"launches": launches, "avg_ms": total / launches}
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    peak = PEAK_BF16 if w.dtype == "bf16" else PEAK_FP32_MFMA
    for name, f in flops.items():
        if name in kernels:
            kernels[name]["tflops"] = f / (kernels[name]["avg_ms"] / 1e3) / 1e12
            kernels[name]["mfma_frac"] = f / (kernels[name]["avg_ms"] / 1e3) / peak
    for name, nbytes in hbm_bytes(w).items():
        if name in kernels:
            t = kernels[name]["avg_ms"] / 1e3
            kernels[name]["gbs"] = nbytes / t / 1e9
            kernels[name]["hbm_frac"] = nbytes / t / PEAK_HBM
            counted = profiled_traffic(w.name, name)
            if counted is not None:
                kernels[name]["counter_gbs"] = counted / t / 1e9
    abytes = attention_bytes(w)
    for name, nbytes in abytes.items():
        if name in kernels:
            kernels[name]["bytes"] = nbytes
            kernels[name]["alg_gbs"] = nbytes / (kernels[name]["avg_ms"] / 1e3) / 1e9
    if dom in flops:
        t = kernels[dom]["avg_ms"] / 1e3
        # the bound is whichever floor is longer at the published peaks
        mfma_floor, hbm_floor = flops[dom] / peak, abytes.get(dom, 0) / PEAK_HBM
        if mfma_floor >= hbm_floor:
            roofline = {"bound": "mfma", "achieved": flops[dom] / t / 1e12, "peak": peak / 1e12,
                        "unit": "TFLOP/s", "frac": flops[dom] / t / peak}
        else:
            roofline = {"bound": "hbm", "achieved": abytes[dom] / t / 1e9,
                        "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": abytes[dom] / t / PEAK_HBM}
        roofline.update({"traffic": profiled_traffic(w.name, dom), "kernel": dom,
                         "flops_per_launch": flops[dom], "bytes_per_launch": abytes.get(dom),
                         "mfma_floor_ms": mfma_floor * 1e3, "hbm_floor_ms": hbm_floor * 1e3})
        counters = profiled_mfma(w.name, dom)
        if counters is not None:
            roofline["mfma_busy"], roofline["clock_ghz"] = counters
    else:
        roofline = {"bound": "hbm", "achieved": None, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                    "frac": None, "traffic": None, "kernel": dom}
    total_flops = sum(flops.values())

    # whole forward: the longer of its MFMA floor and its HBM floor (all
    # kernels' algorithmic bytes) against the measured step
    fwd_bytes = sum(hbm_bytes(w).values()) + sum(abytes.values())
    floors = {"mfma": sum(flops.values()) / peak * 1e3, "hbm": fwd_bytes / PEAK_HBM * 1e3}
    fbound = max(floors, key=floors.get)
    whole = {"bound": fbound, "floor_ms": floors[fbound], "frac": floors[fbound] / ms,
             "mfma_floor_ms": floors["mfma"], "hbm_floor_ms": floors["hbm"],
             "alg_bytes": fwd_bytes}
    result = {
        "metric": metric_for(w), "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": per_step[len(per_step) // 2], "ms_per_step_min": per_step[0],
        "ms_per_step_kernel_pass": ms_inst,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": data_for(w),
        "config": {"workload": w.name, "batch": 1, "heads": w.heads, "seq_len": w.n,
                   "head_dim": w.d, "causal": w.causal, "b": w.b, "m": w.m, "r": w.r,
                   "recursion_base": w.recursion_base, "parallelism": "single-gpu"},
        "mfma_frac_whole_forward": total_flops / (ms / 1e3) / peak,
        "whole_forward": whole,
        "roofline": roofline,
        "kernels": kernels,
    }

    if not args.no_exact:
        log("timing the library's exact attention at the same shape")
        Oe = torch.empty_like(Q)
        api.exact(Q, K, V, causal=w.causal, out=Oe)
        torch.cuda.synchronize()
        reps = 2
        e0.record(stream)
        for _ in range(reps):
            api.exact(Q, K, V, causal=w.causal, out=Oe)
        e1.record(stream)
        torch.cuda.synchronize()
        ems = e0.elapsed_time(e1) / reps
        diff = (O.float() - Oe.float()).pow(2).sum().sqrt() / Oe.float().pow(2).sum().sqrt()
        result["exact_baseline"] = {
            "ms": ems, "tokens_per_s": w.n / (ems / 1e3),
            "tflops": exact_flops(w) / (ems / 1e3) / 1e12,
            "mfma_frac": exact_flops(w) / (ems / 1e3) / peak,
            "speedup_of_hyperattention": ems / ms,
            "rel_frobenius_err_vs_exact": float(diff)}
        if not w.causal and not w.planted:
            # iid N(0, 1) inputs: the sampled part's noise against the exact
            # output predicts a relative error of about sqrt(n_k / m)
            result["exact_baseline"]["predicted_rel_err"] = (w.n / min(w.m, w.n)) ** 0.5
        del Oe

    if pairs is not None:
        log("planted recall from the library's sorted orders")
        result["planted"] = planted_recall(w, api, Q, K, V, pairs)

    if args.copy_calibration:
        copy_calibration(torch)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one head")
        result["cpu_baseline"] = cpu_baseline(w)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
