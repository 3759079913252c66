"""Benchmark: one layer decode step of low-rank KV-cache attention on one MI355X.

A step is one pass of the whole hot path for one layer and one new token per sequence:
lowrank_decode_step, i.e. the append (project the new K/V rows with the caller's pseudo-inverse,
store them in the cache format, advance the lengths) and the decode (fold, split-token latent
decode, combine + up-projection, the exact window if any), in three launches: append + fold, the
latent kernel, the combine. Inputs are seeded synthetic data already resident in HBM.

Prints ONE JSON line on stdout (progress goes to stderr).
Default workload: batch 16, 32768 cached tokens per sequence, rank 256 for K and V, bf16 latents
(the long-context point of the TraceKV latency setting: batch 16, 4K-32K context). --config 4
times the whole 28-layer step instead (per-layer ranks, ragged lengths, exact recent window).
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_TBS = 8.0   # MI355X HBM3E peak, TB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime the process already uses (torch's)."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime first)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(ctypes.c_void_p(e))

    def record(self, e: int, stream: int) -> None:
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rc = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")


def latent_bytes_per_token(latent: str, rank: int) -> int:
    if latent == "bf16":
        return 2 * rank
    if latent == "f32":
        return 4 * rank
    g = (rank + 31) // 32
    return (rank + 1) // 2 + 4 * g          # packed nibbles + fp16 scale and zero per group


def step_bytes(cfg, rk, rv, lat_len, win_len, n_new):
    """Algorithmic HBM bytes of one layer step (append + decode), see the benchmark notes."""
    D, Hq, d, B = cfg.kv_width, cfg.n_q_heads, cfg.head_dim, cfg.batch
    base_e = 4 if cfg.latent == "f32" else 2
    lat = int(np.sum(lat_len)) * (latent_bytes_per_token(cfg.latent, rk) + latent_bytes_per_token(cfg.latent, rv))
    win = int(np.sum(win_len)) * 2 * D * 2
    bases = (rk + rv) * D * base_e
    q_out = B * Hq * d * (base_e + 4)
    append = (B * n_new * 2 * D * 2 + (rk + rv) * D * base_e
              + B * n_new * (latent_bytes_per_token(cfg.latent, rk) + latent_bytes_per_token(cfg.latent, rv)))
    return dict(latents=lat, window=win, bases=bases, q_out=q_out, append=append,
                total=lat + win + bases + q_out + append)


def cpu_baseline(cfg, li, budget_s: float = 8.0, reps: int = 3, d1_budget_s: float = 4.0):
    """Times the fp64 oracle on the host cores, in the same run as the GPU measurement:
    D2 (latent domain, the algorithmic counterpart of the kernels) over whole sequences of the same
    workload, as many as fit a third of `budget_s` (at least one), then that sample repeated until
    `budget_s` of CPU time is spent (at least `reps` runs; median); and D1 (reconstruct K = Zk Bk,
    V = Zv Bv, then plain attention) over one whole sequence, repeated the same way within
    `d1_budget_s`. About 10-15 s of host work in all."""
    from threadpoolctl import threadpool_info
    from oracle import attention as OA
    from oracle import quant as OQ

    def oracle_latents(which, b):
        z = li.zk if which == "k" else li.zv
        r = li.rank_k if which == "k" else li.rank_v
        rows = z[b, :int(li.lat_len[b]), :r].float().numpy()
        if cfg.latent == "i4g32":
            rows = OQ.dequant_rows(*OQ.quantize_rows(rows), r)
        return rows.astype(np.float64)

    class One:
        def __init__(self, rows):
            self.rows = rows

        def __getitem__(self, i):
            return self.rows

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    q = li.q.float().numpy()
    bk = li.bk.float().numpy()
    bv = li.bv.float().numpy()
    win = {}
    if cfg.window:
        win = dict(kwin=li.kwin.float().numpy(), vwin=li.vwin.float().numpy(), win_len=li.win_len,
                   window=cfg.window)

    def seq_bytes(b):
        n = int(li.lat_len[b]) * (latent_bytes_per_token(cfg.latent, li.rank_k)
                                  + latent_bytes_per_token(cfg.latent, li.rank_v))
        return n + (int(li.win_len[b]) * 2 * cfg.kv_width * 2 if cfg.window else 0)

    lat = {}   # each sequence's oracle latents, built once (untimed) and kept for the repeats

    def run(fn, b):
        if b not in lat:
            lat[b] = (oracle_latents("k", b), oracle_latents("v", b))
        zk, zv = lat[b]
        t0 = time.perf_counter()
        fn(q, One(zk), One(zv), bk, bv, li.lat_len, li.rank_k, li.rank_v, cfg.n_kv_heads, cfg.sm_scale,
           batches=[b], **win)
        return time.perf_counter() - t0

    def repeated(once, first, budget):
        times = [first]
        while len(times) < reps or (sum(times) < budget and len(times) < 100):
            times.append(once())
        return float(np.median(times)), len(times)

    # D2: as many whole sequences as fit a third of the budget, then that sample repeated
    done, t_first = 0, 0.0
    while done < cfg.batch and (done == 0 or t_first < budget_s / reps):
        t_first += run(OA.decode_latent, done)
        done += 1
    t2, n2 = repeated(lambda: sum(run(OA.decode_latent, b) for b in range(done)), t_first, budget_s)
    nbytes = sum(seq_bytes(b) for b in range(done))
    t1, n1 = repeated(lambda: run(OA.decode_reconstruct, 0), run(OA.decode_reconstruct, 0), d1_budget_s)
    lens = "x".join(str(int(x)) for x in li.lat_len[:done]) if cfg.len_range else str(int(li.lat_len[0]))
    return dict(value=nbytes / t2 / 1e12, unit="TB/s", cores=int(threads), kind="oracle",
                sample=f"D2 (latent-domain fp64 oracle): {done} of {cfg.batch} sequences x {lens} tokens"
                       f"{' (+ window)' if cfg.window else ''} of layer {li.layer}, median of {n2} runs "
                       f"{t2:.3f} s; latent bytes per second in the benchmark's units",
                us_per_layer_step=t2 / done * cfg.batch * 1e6,
                d1={"value": seq_bytes(0) / t1 / 1e12, "unit": "TB/s", "sample": f"D1 (reconstruct K, V then "
                    f"attend, fp64): sequence 0 ({int(li.lat_len[0])} tokens), median of {n1} runs {t1:.3f} s",
                    "us_per_layer_step": t1 * cfg.batch * 1e6})


def oracle_time(fn, budget_s: float = 4.0, reps: int = 3):
    """Median wall time (s) of fn() on the host over at least `reps` runs, repeated until `budget_s`
    is spent (at most 50 runs), and the number of runs: the oracle beside an operation's GPU line."""
    times = []
    while len(times) < reps or (sum(times) < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def host_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def copy_ceiling(torch, dev, nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of `nbytes` (read once, written once), timed with events in the same run:
    the practical ceiling of a 1:1 read/write stream on this GPU (median of `reps`)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = float(np.median(ts))
    del src, dst
    return {"GB/s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1), "bytes_moved": 2 * nbytes,
            "kind": "device-to-device copy (read + write), median of %d" % reps}


KERNEL_SOURCES = {
    "lr_decode": ("decode.hip", "fold.h", "device_common.h", "internal.h", "abi.cpp"),
    "lr_rebase_bf16": ("rebase.hip", "device_common.h"),
}


def kernel_source_hash(kernel: str = "lr_decode") -> str:
    """sha256 over a kernel's sources: counter figures are valid only for this code."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_kv_cache_lowrank_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str = "lr_decode"):
    """HBM bytes per launch of a kernel from its committed counter summary (FETCH_SIZE and
    WRITE_SIZE runs, scaled by a copy kernel of known size), or None when there is none for
    this workload or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get("workloads", {}).get(workload)
    if entry is None or rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return int(entry["hbm_bytes_per_launch"])


def copy_probe(torch, dev):
    """One elementwise kernel that reads 256 MiB and writes 256 MiB (the counter calibration)."""
    src = torch.zeros(64 * 2**20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: {src.numel() * 4} bytes read, {dst.numel() * 4} bytes written")


def capture_graph(torch, fn):
    """One HIP graph holding the launches fn makes on the current stream (captured on a side
    stream: nothing runs during capture; every replay runs all of them again)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def decode28_bench(args):
    """The full 28-layer decode step of the global-rank-allocation workload: batch 16, total
    lengths per sequence drawn from U{2048..8192} with the last 128 tokens kept exact in the
    window ring, per-layer ranks rK, rV drawn independently from {128, 136, ..., 512}, bf16
    latents. A step = for each of the 28 layers, lowrank_decode_step (one new token per sequence
    enters the window, the oldest window token is projected and stored as a latent row, and the
    layer's attention runs). The lengths start W + 2K tokens short, so the last step of the
    event pass attends over exactly the drawn lengths. With --graph the timed pass replays one
    HIP graph of the 28 layers' launches. The caches of all layers (~5 GB) far exceed the 256 MB
    Infinity Cache, so every step streams from HBM."""
    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth
    from synth.device import device_layer

    dev = "cuda"
    cfg = synth.CONFIGS[4]
    K, W = args.steps, args.warmup
    NL = cfg.n_layers
    n_new = 1
    ranks = [synth.layer_ranks(cfg, l) for l in range(NL)]
    model = lr.Model(NL, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, [r[0] for r in ranks],
                     [r[1] for r in ranks], cfg.sm_scale, cfg.window, cfg.latent)
    ll, wl = synth.split_lengths(cfg)
    total = W + 2 * K
    start_len = (ll - total * n_new).astype(np.int32)
    assert np.all(start_len >= 0)
    max_len = int(ll.max())
    caches, qs, li0 = [], [], None
    t0 = time.time()
    for l in range(NL):
        li = synth.make_layer(cfg, l, t_cap=max_len)
        _, cache = device_layer(li, dev, with_proj=True)
        cache.tensors["lat_len"].copy_(torch.from_numpy(start_len).to(dev))
        caches.append(cache)
        qs.append(li.q.to(dev))
        if l == 0:
            li0 = li
        log(f"layer {l}: ranks {li.rank_k}/{li.rank_v} staged ({time.time() - t0:.1f} s)")
    gen = np.random.default_rng(12345)
    k_new = torch.from_numpy(gen.standard_normal((cfg.batch, n_new, cfg.kv_width), dtype=np.float32)).to(
        torch.bfloat16).to(dev)
    v_new = torch.from_numpy(gen.standard_normal((cfg.batch, n_new, cfg.kv_width), dtype=np.float32)).to(
        torch.bfloat16).to(dev)
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
    ws_bytes = max(lr.lowrank_attn_decode_workspace_size(model, l, cfg.batch, max_len, args.nsplit)
                   for l in range(NL))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def full_step(events=None):
        for l in range(NL):
            lr.lowrank_decode_step(model, l, caches[l], k_new, v_new, qs[l], out, max_len, ws, nsplit=args.nsplit,
                                   events=events[l] if events is not None else None)

    # W warm-up steps, pass A (timed, no per-dispatch events), pass B (events on every layer's latent
    # kernel dispatch and around every step); one step = the 28 layers' lowrank_decode_step calls
    for i in range(W):
        full_step()
        if i % 5 == 0:
            log(f"warm-up step {i} enqueued")
    torch.cuda.synchronize()
    graph = capture_graph(torch, full_step) if args.graph else None
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()                 # no collector pause while the host enqueues the timed steps
    start.record()
    for i in range(K):
        if graph is not None:
            graph.replay()
        else:
            full_step()
    stop.record()
    torch.cuda.synchronize()
    gc.enable()
    ms_per_step = start.elapsed_time(stop) / K
    evs = [[(ev.create(), ev.create()) for _ in range(NL)] for _ in range(K)]
    sev = [(ev.create(), ev.create()) for _ in range(K)]
    for k in range(K):
        ev.record(sev[k][0], stream)
        full_step(evs[k])
        ev.record(sev[k][1], stream)
    torch.cuda.synchronize()
    kern_ms = np.array([[ev.elapsed_ms(a, b) for a, b in row] for row in evs])   # [K, NL]
    span_ms = [ev.elapsed_ms(a, b) for a, b in sev]
    for row in evs:
        for a, b in row:
            ev.destroy(a)
            ev.destroy(b)
    for a, b in sev:
        ev.destroy(a)
        ev.destroy(b)
    assert torch.isfinite(out).all(), "non-finite output"
    for l in range(NL):
        got = caches[l].tensors["lat_len"].cpu().numpy()
        assert np.array_equal(got, ll), "lengths did not advance to the drawn lengths"

    ceiling = copy_ceiling(torch, dev)
    # bytes of each step: lat_len after that step's append = start + (i + 1)
    def step_total_at(i):
        L = start_len + (i + 1) * n_new
        return sum(step_bytes(cfg, ranks[l][0], ranks[l][1], L, wl, n_new)["total"] for l in range(NL))

    step_total = float(np.mean([step_total_at(W + k) for k in range(K)]))
    kern_bytes = np.zeros((K, NL))
    for k in range(K):
        L = start_len + (W + K + k + 1) * n_new
        for l in range(NL):
            kern_bytes[k, l] = step_bytes(cfg, ranks[l][0], ranks[l][1], L, wl, n_new)["latents"]
    value = step_total / (ms_per_step * 1e-3) / 1e12
    kern_avg_ms = float(kern_ms.mean())
    bytes_per_launch = float(kern_bytes.mean())
    achieved = bytes_per_launch / (kern_avg_ms * 1e-3) / 1e9
    per_layer_us = (kern_ms.mean(axis=0) * 1e3).round(2).tolist()
    log(f"ms/step {ms_per_step:.4f} ({NL} layers)  decode kernel avg {kern_avg_ms * 1e3:.2f} us  "
        f"step span (events) {np.median(span_ms):.4f} ms  step {value:.3f} TB/s  kernel {achieved / 1e3:.3f} TB/s")

    rec = {
        "metric": "µs per layer decode step & achieved HBM TB/s (B=16, T=4K–32K)",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_layer_step": round(ms_per_step * 1e3 / NL, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.latent,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "layers": NL,
                   "total_len_range": list(cfg.len_range), "window": cfg.window,
                   "rank_range": [int(min(cfg.rank_choices)), int(max(cfg.rank_choices))],
                   "latent": cfg.latent, "q_heads": cfg.n_q_heads, "kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "new_tokens_per_step": n_new,
                   "step": "28 x lowrank_decode_step (append + fold + window, latent kernel, combine)"
                           + ("; timed pass replayed from one HIP graph" if args.graph else ""),
                   "parallelism": "single GPU"},
        "step_bytes": int(step_total),
        "step_span_ms_events": round(float(np.median(span_ms)), 5),
        "decode_kernel_us_per_layer": per_layer_us,
        "roofline": {"bound": "hbm", "kernel": "lr_decode", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_TBS * 1000, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM_TBS * 1000), 4), "traffic": None,
                     "kernel_us": round(kern_avg_ms * 1e3, 2), "bytes_per_launch": int(bytes_per_launch)},
        "copy_ceiling": ceiling,
    }
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        li0.lat_len = ll
        rec["cpu_baseline"] = cpu_baseline(cfg, li0)
    print(json.dumps(rec), flush=True)


def rebase_bench(args):
    """Historical-coordinate sync of a whole layer cache (every stored K and V row re-expressed
    in an updated basis), timed per call. One call = one launch of lr_rebase_bf16 over K and V.
    Algorithmic bytes: each row's old coordinates read once and new coordinates written once."""
    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth

    dev = "cuda"
    cfg = synth.CONFIGS[args.config]
    if cfg.n_layers != 1 or cfg.latent != "bf16":
        raise SystemExit("--op rebase times single-layer bf16 configurations (1 or 2)")
    K, W = args.steps, args.warmup
    B, T = cfg.batch, cfg.seq_len
    rk, rv = synth.layer_ranks(cfg, 0)
    rk2 = args.rank_new or rk
    rv2 = args.rank_new or rv
    log(f"generating inputs for {cfg.name} ...")
    li = synth.make_layer(cfg, t_cap=T, lat_len=np.full(B, T, np.int32))
    bk, bv = li.bk.double().numpy(), li.bv.double().numpy()
    wk64 = synth.sync_projection(bk, synth.gen_basis_update(cfg, "k", 0, bk, rk2))
    wv64 = synth.sync_projection(bv, synth.gen_basis_update(cfg, "v", 0, bv, rv2))
    wk = synth.w_storage(wk64, "bf16").to(dev)
    wv = synth.w_storage(wv64, "bf16").to(dev)
    model = lr.Model(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, [rk], [rv], cfg.sm_scale, 0, "bf16")
    lat = torch.full((B,), T, dtype=torch.int32, device=dev)
    ldk2, ldv2 = synth.latent_ld(rk2), synth.latent_ld(rv2)
    bytes_call = B * T * 2 * (rk + rk2 + rv + rv2)
    # src and dst pairs rotated so that the pairs together exceed 2 x the 256 MB Infinity Cache
    n_pairs = max(1, min(4, -(-(2 * 256 * 2**20) // bytes_call)))
    pairs = []
    for _ in range(n_pairs):
        src = lr.Cache(li.zk.to(dev), li.zv.to(dev), None, None, lat, T, li.ld_k, li.ld_v)
        dk = torch.empty(B, T, ldk2, dtype=torch.bfloat16, device=dev)
        dv = torch.empty(B, T, ldv2, dtype=torch.bfloat16, device=dev)
        pairs.append((src, lr.Cache(dk, dv, None, None, None, T, ldk2, ldv2)))
    log(f"{n_pairs} src/dst pair(s) of {bytes_call / 1e6:.1f} MB moved per call")
    ev = HipEvents()
    evs = [(ev.create(), ev.create()) for _ in range(K)]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    for i in range(W + K):
        if i == W:
            torch.cuda.synchronize()
            start.record()
        src, dst = pairs[i % n_pairs]
        if i >= W:
            ev.record(evs[i - W][0], stream)
        lr.lowrank_kv_rebase(model, 0, src, dst, T, rk2, rv2, wk, wv, stream=stream)
        if i >= W:
            ev.record(evs[i - W][1], stream)
    stop.record()
    torch.cuda.synchronize()
    ms_per_call = start.elapsed_time(stop) / K
    kern_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in evs]))
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    assert torch.isfinite(pairs[0][1].zk[:, :, :rk2].float()).all(), "non-finite output"
    if args.copy_probe:
        copy_probe(torch, dev)
    value = bytes_call / (ms_per_call * 1e-3) / 1e9
    achieved = bytes_call / (kern_ms * 1e-3) / 1e9
    workload = f"rebase {cfg.name} r{rk}->r{rk2}"
    log(f"ms/call {ms_per_call:.4f}  kernel {kern_ms * 1e3:.2f} us  {value:.1f} GB/s  kernel {achieved:.1f} GB/s")
    rec = {
        "metric": "historical-coordinate sync of one layer cache: algorithmic HBM GB/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_call, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "batch": B, "seq_len": T,
                   "rank_k": rk, "rank_v": rv, "rank_k_new": rk2, "rank_v_new": rv2,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "lr_rebase_bf16", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_TBS * 1000, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM_TBS * 1000), 4),
                     "traffic": measured_traffic(workload, "lr_rebase_bf16"),
                     "kernel_us": round(kern_ms * 1e3, 2), "bytes_per_launch": int(bytes_call),
                     "mfma_tflops": round(2.0 * B * T * (rk * rk2 + rv * rv2) / (kern_ms * 1e-3) / 1e12, 1)},
    }
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        from oracle import rebase as ORB
        zk0 = li.zk[0, :T, :rk].float().numpy()
        zv0 = li.zv[0, :T, :rv].float().numpy()
        w_k = synth.w_storage(wk64, "bf16")[:, :rk].float().numpy()
        w_v = synth.w_storage(wv64, "bf16")[:, :rv].float().numpy()
        t, n = oracle_time(lambda: (ORB.store(ORB.rebase_rows(zk0, w_k), "bf16"),
                                    ORB.store(ORB.rebase_rows(zv0, w_v), "bf16")))
        sample_bytes = T * 2 * (rk + rk2 + rv + rv2)
        rec["cpu_baseline"] = {
            "value": round(sample_bytes / t / 1e9, 3), "unit": "GB/s", "cores": host_threads(), "kind": "oracle",
            "sample": f"rebase_rows + store (fp64 oracle) of sequence 0's K and V rows ({T} each), "
                      f"median of {n} runs {t:.4f} s; algorithmic bytes per second as the GPU line"}
    print(json.dumps(rec), flush=True)


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def prefill_bench(args):
    """Chunked prefill attention of one layer: every sequence's chunk of --chunk new tokens
    attends over its latent history and, causally, over itself. One call = fold, the latent
    kernel (timed with HIP events attached to its dispatch), the exact-keys workgroups and the
    combine. Algorithmic FLOPs of the latent kernel: 2 * Hq * (rank_k + rank_v) per (query
    token, latent token)."""
    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth
    from synth.device import device_layer

    dev = "cuda"
    cfg = synth.CONFIGS[args.config]
    if cfg.n_layers != 1:
        raise SystemExit("--op prefill times single-layer configurations (0-3)")
    K, W = args.steps, args.warmup
    B, T, C = cfg.batch, cfg.seq_len, args.chunk
    log(f"generating inputs for {cfg.name} ...")
    li = synth.make_layer(cfg, t_cap=T, lat_len=np.full(B, T, np.int32))
    model, cache = device_layer(li, dev)
    q, k, v = synth.gen_chunk(cfg, 0, C)
    qdt = torch.float32 if cfg.latent == "f32" else torch.bfloat16
    q = torch.from_numpy(q).to(qdt).to(dev)
    k = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    out = torch.empty(B, C, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
    ws = lr.prefill_workspace(model, 0, B, C, T, args.nsplit)
    ev = HipEvents()
    evs = [(ev.create(), ev.create()) for _ in range(K)]
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    for i in range(W + K):
        if i == W:
            torch.cuda.synchronize()
            start.record()
        lr.lowrank_attn_prefill(model, 0, cache, q, k, v, out, T, ws, nsplit=args.nsplit,
                                events=evs[i - W] if i >= W else None)
    stop.record()
    torch.cuda.synchronize()
    ms_per_call = start.elapsed_time(stop) / K
    kern_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in evs]))
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    assert torch.isfinite(out).all(), "non-finite output"
    flops = 2.0 * B * C * T * cfg.n_q_heads * (li.rank_k + li.rank_v)
    tflops = flops / (kern_ms * 1e-3) / 1e12
    value = B * C / (ms_per_call * 1e-3)
    log(f"ms/call {ms_per_call:.4f}  latent kernel {kern_ms * 1e3:.2f} us  {tflops:.1f} TFLOP/s  "
        f"{value:.0f} query tokens/s")
    rec = {
        "metric": "chunked prefill attention over the latent cache: query tokens per second",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_call, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.latent,
        "data": "synthetic",
        "config": {"workload": f"prefill {cfg.name} chunk{C}", "batch": B, "seq_len": T, "chunk": C,
                   "rank_k": li.rank_k, "rank_v": li.rank_v, "latent": cfg.latent, "q_heads": cfg.n_q_heads,
                   "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "lr_prefill_latent" if cfg.latent == "bf16" else "lr_decode (prefill query sequences)", "achieved": round(tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel_us": round(kern_ms * 1e3, 2), "flops_per_launch": flops},
    }
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        from oracle import prefill as OP
        from oracle import quant as OQ

        def rows(z, r):
            x = z[0, :T, :r].float().numpy()
            return OQ.dequant_rows(*OQ.quantize_rows(x), r) if cfg.latent == "i4g32" else x.astype(np.float64)

        class One:
            def __init__(self, x):
                self.x = x

            def __getitem__(self, b):
                return self.x

        zk0, zv0 = One(rows(li.zk, li.rank_k)), One(rows(li.zv, li.rank_v))
        qn, kn, vn = q.float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy()
        bkn, bvn = li.bk.float().numpy(), li.bv.float().numpy()
        t, n = oracle_time(lambda: OP.prefill_latent(qn, zk0, zv0, bkn, bvn, li.lat_len, li.rank_k, li.rank_v,
                                                     cfg.n_kv_heads, cfg.sm_scale, kn, vn, batches=[0]))
        rec["cpu_baseline"] = {
            "value": round(C / t, 1), "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
            "sample": f"prefill_latent (P2, fp64 oracle): sequence 0, {C} query tokens over {T} latent rows, "
                      f"median of {n} runs {t:.3f} s"}
    print(json.dumps(rec), flush=True)


def _timed_calls(fn, K, W):
    """Mean ms per call of fn over K calls after W warm-up calls (torch events, same stream)."""
    import torch
    for _ in range(W):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / K


def sensvd_bench(args):
    """Sensitivity-weighted SVD of one KV matrix's calibration rows (256 samples x 512 tokens =
    131072 rows of dim 512, rank 358), or with --matrices M of M matrices in one batched call: the
    weighted Gram on the matrix cores, then block Jacobi.
    The roofline line is the Gram's algorithmic FLOPs (N * D * (D + 1), the symmetric half plus
    the diagonal) over the whole call: the Jacobi rounds are launch-latency bound."""
    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth

    dev = "cuda"
    M, dim, rank = args.matrices, 512, 358
    if M == 1:
        n = args.samples
        x, w = synth.gen_kv_samples(synth.CONFIGS[4], n, dim)
        xd = torch.from_numpy(x).to(torch.bfloat16).to(dev)
        wd = torch.from_numpy(w).to(dev)
        basis = torch.empty(rank, dim, dtype=torch.bfloat16, device=dev)
        sigma = torch.empty(dim, dtype=torch.float32, device=dev)
        ws = torch.empty(lr.lowrank_sens_svd_workspace_size(n, dim), dtype=torch.uint8, device=dev)
        call = lambda: lr.lowrank_sens_svd(xd, wd, rank, basis, sigma, ws)   # noqa: E731
        n_rows = n
        metric = "sensitivity-weighted SVD basis of one KV matrix: ms per call"
        workload = f"sensvd N{n} D{dim} r{rank}"
    else:
        # a model's K and V matrices in one batched call; each matrix its own spectrum decay
        n = args.samples if args.samples != 131072 else 16384
        log(f"generating {M} x {n} samples ...")
        xs = np.empty((M, n, dim), np.float32)
        wv = np.empty((M, n), np.float32)
        for m in range(M):
            xs[m], wv[m] = synth.gen_kv_samples(synth.CONFIGS[4], n, dim, 0.6 + 0.01 * m)
        xd = torch.from_numpy(xs).to(torch.bfloat16).to(dev)
        wd = torch.from_numpy(wv).to(dev)
        xs0, ws0, n_rows = xs[0].copy(), wv[0].copy(), n
        del xs
        basis = torch.empty(M, rank, dim, dtype=torch.bfloat16, device=dev)
        sigma = torch.empty(M, dim, dtype=torch.float32, device=dev)
        ws = torch.empty(lr.lowrank_sens_svd_batched_workspace_size(M, n, dim), dtype=torch.uint8, device=dev)
        call = lambda: lr.lowrank_sens_svd_batched(xd, wd, rank, basis, sigma, ws)   # noqa: E731
        metric = f"sensitivity-weighted SVD bases of {M} KV matrices in one batched call: ms per call"
        workload = f"sensvd {M}x N{n} D{dim} r{rank}"
    ms = _timed_calls(call, args.steps, args.warmup)
    assert torch.isfinite(sigma).all()
    flops = float(M) * n * dim * (dim + 1)
    rec = {"metric": metric, "value": round(ms, 4),
           "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": workload, "matrices": M, "samples": n, "dim": dim, "rank": rank,
                      "sweeps": 10, "parallelism": "single GPU"},
           "roofline": {"bound": "mfma", "kernel": "lr_svd_gram + block Jacobi (whole call)",
                        "achieved": round(flops / (ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
                        "traffic": None, "flops_per_launch": flops}}
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        from oracle import sensvd as OS
        xs, wsm = (x, w) if M == 1 else (xs0, ws0)
        ns = min(xs.shape[0], 16384)
        t, n = oracle_time(lambda: OS.basis(xs[:ns], wsm[:ns], rank))
        n_all = M * n_rows
        rec["cpu_baseline"] = {
            "value": round(t * 1e3 * n_all / ns, 1), "unit": "ms", "cores": host_threads(), "kind": "oracle",
            "sample": f"basis (fp64 oracle: weighted rows, thin SVD) of the first {ns} rows of matrix 0, median "
                      f"of {n} runs {t:.3f} s, scaled by rows to the call's {n_all} rows"}
    print(json.dumps(rec), flush=True)


def basisupd_bench(args):
    """Block-incremental basis update of one KV matrix: a rank-256 history (D = 512) takes the 128
    tokens of one window's worth of evictions and keeps rank 256 (bf16 basis): staging, the Gram of
    the 384 stacked rows on the matrix cores, block Jacobi, and the sync weights W = B' B^T. Once
    per block of evictions, not per token; the Jacobi rounds are launch-latency bound."""
    import torch
    import rank_kv_cache_lowrank_amd as lr

    dev = "cuda"
    r, n, dim = 256, 128, 512
    rng = np.random.default_rng(21)
    q, rr = np.linalg.qr(rng.standard_normal((dim, r)))
    B = (q * np.sign(np.diag(rr))[None, :]).T
    sigma = np.sqrt(4096.0 / np.arange(1, r + 1))
    Y = rng.standard_normal((n, dim)) / np.sqrt(dim) * sigma[0]
    bd = torch.from_numpy(B.astype(np.float32)).to(torch.bfloat16).to(dev)
    sd = torch.from_numpy(sigma.astype(np.float32)).to(dev)
    yd = torch.from_numpy(Y.astype(np.float32)).to(torch.bfloat16).to(dev)
    bn = torch.empty(r, dim, dtype=torch.bfloat16, device=dev)
    sn = torch.empty(r, dtype=torch.float32, device=dev)
    w = torch.empty(r, (r + 7) // 8 * 8, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lr.lowrank_basis_update_workspace_size(r, n, dim), dtype=torch.uint8, device=dev)
    ms = _timed_calls(lambda: lr.lowrank_basis_update(bd, sd, yd, r, bn, sn, w, ws), args.steps, args.warmup)
    assert torch.isfinite(sn).all()
    flops = float(r + n) * dim * (dim + 1)
    rec = {"metric": "block-incremental basis update of one KV matrix: ms per call", "value": round(ms, 4),
           "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"basis update r{r} + {n} rows D{dim} -> r{r}", "rank": r, "rows": n,
                      "dim": dim, "rank_new": r, "sweeps": 10, "parallelism": "single GPU"},
           "roofline": {"bound": "latency", "kernel": "whole call (stage, Gram, block Jacobi, finish)",
                        "achieved": round(flops / (ms * 1e-3) / 1e12, 4), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 7),
                        "traffic": None, "flops_per_launch": flops}}
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        from oracle import basis_update as OB
        b64 = bd.float().cpu().numpy().astype(np.float64)
        s64 = sd.cpu().numpy().astype(np.float64)
        y64 = yd.float().cpu().numpy().astype(np.float64)

        def upd():
            b2, _ = OB.incremental_update(s64, b64, y64, r)
            return OB.sync_weights(b64, b2)

        t, n = oracle_time(upd)
        rec["cpu_baseline"] = {
            "value": round(t * 1e3, 3), "unit": "ms", "cores": host_threads(), "kind": "oracle",
            "sample": f"incremental_update + sync_weights (fp64 oracle), the whole call, median of {n} runs"}
    print(json.dumps(rec), flush=True)


def append_bench(args):
    """Storing a chunk of new tokens per sequence (lowrank_kv_append with n_new = --chunk), as after
    a prefill chunk: the projection and storage of every new (or evicted) row, the window ring
    and the lengths. --config 1 (B=16, r=358 bf16, no window, 2000 stored rows) or 4 (the
    28-layer workload's layer 0 shape with W = 128, full windows: every new token evicts one).
    Algorithmic bytes per call: the new dense rows read (2 D bf16 each) and the latent rows
    written."""
    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth
    from synth.device import device_layer

    dev = "cuda"
    C = args.chunk
    K, W = args.steps, args.warmup
    cfg = synth.CONFIGS[args.config]
    calls = K + W
    if cfg.window:
        cfg = cfg.replace(rank_choices=None, rank_k=358, rank_v=358)
        lat = np.full(cfg.batch, 3000, np.int32)
        li = synth.make_layer(cfg, 0, lat_len=lat, win_len=np.full(cfg.batch, cfg.window, np.int32),
                              t_cap=3000 + C * calls)
    elif cfg.n_layers == 1:
        li = synth.make_layer(cfg, t_cap=2000 + C * calls, lat_len=np.full(cfg.batch, 2000, np.int32))
    else:
        raise SystemExit("--op append takes --config 1 or 4")
    model, cache = device_layer(li, dev, with_proj=True)
    B, D = cfg.batch, cfg.kv_width
    gen = np.random.default_rng(5)
    k = torch.from_numpy(gen.standard_normal((B, C, D), dtype=np.float32)).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(gen.standard_normal((B, C, D), dtype=np.float32)).to(torch.bfloat16).to(dev)
    ms = _timed_calls(lambda: lr.lowrank_kv_append(model, 0, cache, k, v), K, W)
    got = cache.tensors["lat_len"].cpu().numpy()
    assert np.all(got == li.lat_len + C * calls), "lengths did not advance by the chunk"
    row_bytes = latent_bytes_per_token(cfg.latent, li.rank_k) + latent_bytes_per_token(cfg.latent, li.rank_v)
    nbytes = B * C * (2 * D * 2 + row_bytes)
    rec = {"metric": "storing a chunk of new tokens per sequence: us per call", "value": round(ms * 1e3, 2),
           "unit": "us", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 5),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": cfg.latent,
           "data": "synthetic",
           "config": {"workload": f"{cfg.name} append chunk {C}", "batch": B, "new_tokens_per_sequence": C,
                      "rank_k": li.rank_k, "rank_v": li.rank_v, "window": cfg.window,
                      "parallelism": "single GPU"},
           "tokens_per_s": round(B * C / (ms * 1e-3), 1),
           "roofline": {"bound": "latency", "kernel": "lr_append_rows + lr_append_finish (n_new > 1), lr_append (1)",
                        "achieved": round(nbytes / (ms * 1e-3) / 1e9, 2), "peak": PEAK_HBM_TBS * 1000,
                        "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / (PEAK_HBM_TBS * 1000), 5),
                        "traffic": None, "bytes_per_launch": nbytes}}
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        from oracle import append as OA
        # the stored down-projections are rank-major [r][D]; the oracle takes P [D, r]
        pk = cache.tensors["pk"].float().cpu().numpy().astype(np.float64).T
        pv = cache.tensors["pv"].float().cpu().numpy().astype(np.float64).T
        kn, vn = k[0].float().cpu().numpy(), v[0].float().cpu().numpy()

        def one_seq():
            st = OA.SeqState(cfg.window, D)
            if cfg.window:
                st.win_len = cfg.window
            for c in range(C):
                OA.append_token(st, kn[c], vn[c], pk, pv, pos_base=int(li.lat_len[0]))
            if st.lat_len:
                OA.store_rows(np.asarray(st.lat_z_k), cfg.latent)
                OA.store_rows(np.asarray(st.lat_z_v), cfg.latent)

        t, n = oracle_time(one_seq, budget_s=2.0)
        rec["cpu_baseline"] = {
            "value": round(t * B * 1e6, 2), "unit": "us", "cores": host_threads(), "kind": "oracle",
            "sample": f"append_token x {C} + store_rows (fp64 oracle) for sequence 0, median of {n} runs "
                      f"{t * 1e6:.1f} us, times the {B} sequences of the call"}
    print(json.dumps(rec), flush=True)


def rankalloc_bench(args):
    """Global rank allocation for the 28-layer model (56 spectra of 512, ranks 128..512 by 8,
    budget 70% of full rank): three short launches (gains, split ordered counts, selection)."""
    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth

    dev = "cuda"
    s = torch.from_numpy(synth.gen_spectra(synth.CONFIGS[4], 56, 512)).to(dev)
    ranks = torch.empty(56, dtype=torch.int32, device=dev)
    ws = torch.empty(lr.lowrank_rank_allocate_workspace_size(56, 128, 512, 8), dtype=torch.uint8, device=dev)
    budget = int(0.7 * 56 * 512)
    ms = _timed_calls(lambda: lr.lowrank_rank_allocate(s, budget, 128, 512, 8, ranks, ws), args.steps,
                      args.warmup)
    n_gran = 56 * (512 - 128) // 8
    rec = {"metric": "global rank allocation of a 28-layer model: us per call", "value": round(ms * 1e3, 2),
           "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f64 gains",
           "data": "synthetic",
           "config": {"workload": "rankalloc 56x512 r128..512/8 budget0.7", "matrices": 56, "granules": n_gran,
                      "parallelism": "single GPU"},
           "roofline": {"bound": "alu", "kernel": "whole call (lr_rank_gains, lr_rank_count, lr_rank_select)", "achieved": round(n_gran ** 2 / (ms * 1e-3) / 1e12, 6),
                        "peak": 78.6, "unit": "T compares/s", "frac": round(n_gran ** 2 / (ms * 1e-3) / 1e12 / 78.6, 8),
                        "traffic": None}}
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        from oracle import rankalloc as ORA
        sn = s.cpu().numpy()
        t, n = oracle_time(lambda: ORA.allocate(sn, budget, 128, 512, 8), budget_s=2.0, reps=1)
        rec["cpu_baseline"] = {
            "value": round(t * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
            "sample": f"allocate (the literal greedy oracle, pure Python), the whole call, median of {n} runs"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--nsplit", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copies", type=int, default=0,
                    help="cache copies rotated over the steps (0: enough that the copies exceed 2 x 256 MB)")
    ap.add_argument("--graph", action="store_true",
                    help="decode: time the steps as replays of HIP graphs captured from them")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 256 MiB device copy (the counter calibration reference)")
    ap.add_argument("--op", choices=("decode", "rebase", "prefill", "sensvd", "rankalloc", "basisupdate", "append"),
                    default="decode",
                    help="decode: the decode step (default); rebase: the historical-coordinate sync; "
                         "prefill: chunked prefill attention; sensvd: sensitivity-weighted SVD basis; "
                         "rankalloc: global rank allocation; basisupdate: block-incremental basis update; "
                         "append: storing a chunk of new tokens")
    ap.add_argument("--samples", type=int, default=131072,
                    help="--op sensvd: calibration rows per matrix (batched default: 16384)")
    ap.add_argument("--matrices", type=int, default=1, help="--op sensvd: matrices per (batched) call")
    ap.add_argument("--chunk", type=int, default=32, help="--op prefill / append: new tokens per sequence")
    ap.add_argument("--rank-new", type=int, default=0, help="--op rebase: new rank (0: unchanged)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (single-GPU build)")
        sys.exit(2)

    import torch
    import rank_kv_cache_lowrank_amd as lr
    import synth

    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.op == "rebase":
        rebase_bench(args)
        return
    if args.op == "prefill":
        prefill_bench(args)
        return
    if args.op == "sensvd":
        sensvd_bench(args)
        return
    if args.op == "rankalloc":
        rankalloc_bench(args)
        return
    if args.op == "basisupdate":
        basisupd_bench(args)
        return
    if args.op == "append":
        append_bench(args)
        return
    dev = "cuda"
    cfg = synth.CONFIGS[args.config]
    if cfg.n_layers == 28 and cfg.window:
        decode28_bench(args)
        return
    if cfg.n_layers != 1 or cfg.window:
        raise SystemExit("bench.py times the single-layer configurations 0-3 and the 28-layer step (4)")
    K, W = args.steps, args.warmup
    T = cfg.seq_len
    n_new = 1
    log(f"generating inputs for {cfg.name} ...")
    t0 = time.time()
    li = synth.make_layer(cfg, t_cap=T, lat_len=np.full(cfg.batch, T, np.int32))
    log(f"inputs ready in {time.time() - t0:.1f} s")
    from synth.device import device_layer
    # The MI355X Infinity Cache holds 256 MB: workloads smaller than that rotate over copies of
    # the cache so that every step streams its latents from HBM.
    lat_bytes = step_bytes(cfg, li.rank_k, li.rank_v, li.lat_len, np.zeros_like(li.lat_len), 0)["latents"]
    n_copies = args.copies if args.copies > 0 else max(1, min(8, -(-(2 * 256 * 2**20) // lat_bytes)))
    caches = []
    for _ in range(n_copies):
        model, cache = device_layer(li, dev, with_proj=True)
        caches.append(cache)
    log(f"{n_copies} cache cop{'y' if n_copies == 1 else 'ies'} of {lat_bytes / 1e6:.1f} MB")
    q = li.q.to(dev)
    gen = np.random.default_rng(12345)
    k_new = torch.from_numpy(gen.standard_normal((cfg.batch, n_new, cfg.kv_width), dtype=np.float32)).to(
        torch.bfloat16).to(dev)
    v_new = torch.from_numpy(gen.standard_normal((cfg.batch, n_new, cfg.kv_width), dtype=np.float32)).to(
        torch.bfloat16).to(dev)
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
    ws = lr.workspace(model, 0, cfg.batch, T, args.nsplit)
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    # Two passes of K steps after W warm-up steps: pass A is the timed region (no per-dispatch
    # events: they lengthen the gaps around the dispatch they are attached to); pass B repeats the
    # steps with HIP events attached to the latent kernel's dispatch (its duration) and recorded
    # around each step call (the step's span). Every copy takes the same number of steps; the
    # lengths start short so that the last step of pass B attends over exactly T tokens.
    total = W + 2 * K
    steps_per_copy = -(-total // n_copies)
    L0 = T - steps_per_copy * n_new
    for cache in caches:
        cache.tensors["lat_len"].copy_(torch.from_numpy(np.full(cfg.batch, L0, np.int32)).to(dev))

    def launch(c, events=None):
        lr.lowrank_decode_step(model, 0, caches[c], k_new, v_new, q, out, T, ws, nsplit=args.nsplit, events=events)

    def step(i, events=None):
        launch(i % n_copies, events)
        return np.full(cfg.batch, L0 + (i // n_copies + 1) * n_new, np.int32)   # lengths the step attends

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graphs = [capture_graph(torch, lambda c=c: launch(c)) for c in range(n_copies)] if args.graph else None
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    lens_a = []
    gc.collect()
    gc.disable()                 # no collector pause while the host enqueues the timed steps
    start.record()
    for i in range(W, W + K):
        if graphs is not None:
            graphs[i % n_copies].replay()
            lens_a.append(np.full(cfg.batch, L0 + (i // n_copies + 1) * n_new, np.int32))
        else:
            lens_a.append(step(i))
    stop.record()
    torch.cuda.synchronize()
    gc.enable()
    ms_per_step = start.elapsed_time(stop) / K
    # pass B
    kev = [(ev.create(), ev.create()) for _ in range(K)]
    sev = [(ev.create(), ev.create()) for _ in range(K)]
    lens_b = []
    for k in range(K):
        i = W + K + k
        ev.record(sev[k][0], stream)
        lens_b.append(step(i, events=kev[k]))
        ev.record(sev[k][1], stream)
    torch.cuda.synchronize()
    kern_ms = [ev.elapsed_ms(a, b) for a, b in kev]
    span_ms = [ev.elapsed_ms(a, b) for a, b in sev]
    for a, b in kev + sev:
        ev.destroy(a)
        ev.destroy(b)
    assert torch.isfinite(out).all(), "non-finite output"
    got = caches[(W + 2 * K - 1) % n_copies].tensors["lat_len"].cpu().numpy()
    assert np.all(got <= T), "lengths past the cache capacity"

    ceiling = copy_ceiling(torch, dev)
    if args.copy_probe:
        copy_probe(torch, dev)

    by = [step_bytes(cfg, li.rank_k, li.rank_v, L, np.zeros_like(L), n_new) for L in lens_a]
    step_total = float(np.mean([x["total"] for x in by]))
    by_b = [step_bytes(cfg, li.rank_k, li.rank_v, L, np.zeros_like(L), n_new) for L in lens_b]
    lat_avg = float(np.mean([x["latents"] + x["window"] for x in by_b]))
    kern_avg_ms = float(np.mean(kern_ms))
    value = step_total / (ms_per_step * 1e-3) / 1e12
    achieved = lat_avg / (kern_avg_ms * 1e-3) / 1e9
    log(f"ms/step {ms_per_step:.4f}  decode kernel {kern_avg_ms * 1e3:.2f} us  step span (events) "
        f"{np.median(span_ms) * 1e3:.2f} us  step {value:.3f} TB/s  kernel {achieved / 1e3:.3f} TB/s  "
        f"copy ceiling {ceiling['GB/s'] / 1e3:.2f} TB/s")

    rec = {
        "metric": "µs per layer decode step & achieved HBM TB/s (B=16, T=4K–32K)",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_layer_step": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.latent,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": T, "rank_k": li.rank_k,
                   "rank_v": li.rank_v, "latent": cfg.latent, "q_heads": cfg.n_q_heads,
                   "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "new_tokens_per_step": n_new,
                   "step": "lowrank_decode_step (append + fold, latent kernel, combine)"
                           + ("; timed pass replayed from HIP graphs" if args.graph else ""),
                   "parallelism": "single GPU"},
        "step_bytes": int(step_total),
        "step_span_us_events": round(float(np.median(span_ms)) * 1e3, 2),
        "roofline": {"bound": "hbm", "kernel": "lr_decode", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_TBS * 1000, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM_TBS * 1000), 4),
                     "traffic": measured_traffic(cfg.name),
                     "kernel_us": round(kern_avg_ms * 1e3, 2), "bytes_per_launch": int(lat_avg)},
        "copy_ceiling": ceiling,
        "cache_copies": n_copies,
    }
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, li)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
