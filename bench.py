#!/usr/bin/env python3
"""Benchmark of the rotary-embedding apply on one MI355X.

A step is one rope_apply call of the fp16 prefill workload (X (4, 2048, 4096)
in 32 heads of 128, int64 position ids gathering an (8192, 64) fp16 table,
split-half pairing): read the ids, gather one cos/sin row per token, rotate
every pair of every head in fp32 with one rounding, write Y. Inputs are
seeded synthetic tensors resident in HBM before the timed region; launches
rotate over independent (X, Y, ids) sets totalling >= 1 GiB so that the 256 MB
last-level cache cannot hold them and the rate measured is HBM's.

Workloads under 64 MiB per step (decode steps, a tensor-parallel share) are
bound by the host's per-call cost when launched one by one; for them the
rates come from the same launches captured in one HIP graph and replayed (the
eager time is reported too).

Timing: the K launches run in batches (10 by default) with a pair of HIP
events on the launch stream around each batch; ms_per_step is the median of
the batches' per-launch times, and the line also gives the batches' minimum,
maximum and the mean over all K launches.

Prints ONE JSON line on stdout. Also reported (in "also"): the M-RoPE
prefill in both section layouts, the fp32 partial interleaved case, the fp16
decode Q+K step (table and on the fly), the prefill and M-RoPE stored in
bfloat16, the packed [Q|K|V] decode step, the decode step with the
key/value cache append, QK-norm + RoPE (prefill with a table, decode on the
fly), the QK-norm decode step with the cache append, an M-RoPE decode step,
one GPU's share of the fp16 prefill and of the decode Q+K step under 8-way
tensor parallelism (4 of the 32 query heads, 1 of the 8 key heads), and its
share of the fp16 prefill under 8-way sequence parallelism (256 of the 2048
tokens of each sequence), a prompt of 4 x 2048 tokens written to the
key/value caches, and prefills of other model shapes: 64 heads of 64, 64
heads of 96 with 24 dimensions rotated (GPT-NeoX-20B), QK-norm with heads of
256.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "RoPE apply achieved HBM GB/s and % of MI355X peak (fp16 prefill, M-RoPE)"
PEAK_GBS = 8000.0            # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30       # >= 4x the 256 MB last-level cache
HEADLINE = "c2_rope_f16_prefill"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c2_rope_f16_prefill.json")
BATCHES = 10                 # event-timed batches per measurement (median reported)
CPU_THREADS_MAX = 16         # host cores one GPU's share of the machine offers


# kernel variant prefix (as the *_check functions report it) -> kernel function
KERNEL_FUNCTIONS = {"vec16": "rope_vec_kernel", "row16": "rope_row_kernel", "scalar": "rope_scalar_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha():
    """SHA-256 of every source the library is built from (the hash its build
    records beside it)."""
    from rotary_position_embedding_amd import build
    return build.source_hash()


# ---------------------------------------------------------------------------
# workload set-up: inputs generated on the host from the seeded generators,
# tables built on the GPU by the library itself

def to_device(a, dev):
    """numpy -> device tensor (uint16 arrays are bfloat16 bit patterns)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def setup(w, onthefly=False):
    import torch
    import rotary_position_embedding_amd as rpe
    dev = torch.device("cuda:0")
    dt = {np.dtype(np.float16): torch.float16, np.dtype(np.float32): torch.float32,
          np.dtype(np.uint16): torch.bfloat16}[np.dtype(w.dtype)]
    x0 = to_device(w.make_x(), dev)
    if w.op in ("kv_append", "kv_append_norm"):
        return setup_kv_append(w, x0, dt, dev)
    ids_h = w.make_ids()
    ids0 = None if ids_h is None else torch.from_numpy(ids_h).to(dev)
    k0 = to_device(w.make_k(), dev) if w.op in ("rope_qk", "qk_norm") else None
    wts = [to_device(a, dev) for a in w.make_norm_weights()] if w.op == "qk_norm" else None
    inv = rpe.rope_inv_freq(w.rotary_dim, w.cache_base, device=dev)
    if w.op == "rope" and not w.has_ids:
        cos, sin = rpe.rope_cos_sin_cache(inv, w.seq, dt, w.scaling)
        cos = cos.unsqueeze(0).expand(w.batch, -1, -1).contiguous()
        sin = sin.unsqueeze(0).expand(w.batch, -1, -1).contiguous()
    else:
        cos, sin = rpe.rope_cos_sin_cache(inv, w.cache_rows, dt, w.scaling)
    set_bytes = 2 * x0.numel() * x0.element_size()
    if k0 is not None:
        set_bytes += 2 * k0.numel() * k0.element_size()
    nsets = max(2, -(-ROTATE_BYTES // set_bytes))
    launchers = []
    for _ in range(nsets):
        x = x0.clone()
        ids = None if ids0 is None else ids0.clone()
        if w.op == "rope":
            y = torch.empty_like(x)
            launchers.append(rpe.rope_apply_launcher(
                x, cos, sin, ids, y, interleaved=w.interleaved,
                num_heads=w.num_heads if w.rank == 3 else 0,
                rotary_embedding_dim=w.rotary_embedding_dim))
        elif w.op == "qk_norm":
            k = k0.clone()
            yq, yk = torch.empty_like(x), torch.empty_like(k)
            tabs = dict(inv_freq=inv, attention_scaling=w.scaling) if onthefly else {}
            launchers.append(rpe.rope_apply_qk_norm_launcher(
                x, k, wts[0], wts[1], None if onthefly else cos, None if onthefly else sin, ids, yq, yk,
                epsilon=1e-6, num_heads=w.num_heads, kv_num_heads=w.kv_num_heads, **tabs))
        elif w.op == "qkv_packed":
            y = torch.empty_like(x)
            launchers.append(rpe.rope_apply_qkv_packed_launcher(
                x, cos, sin, ids, y, num_heads=w.num_heads, kv_num_heads=w.kv_num_heads))
        elif w.op == "mrope":
            y = torch.empty_like(x)
            launchers.append(rpe.mrope_apply_launcher(
                x, ids, cos, sin, y, mrope_section=w.mrope_section, mrope_layout=w.mrope_layout,
                interleaved=w.interleaved, num_heads=w.num_heads,
                rotary_embedding_dim=w.rotary_embedding_dim, scale=w.scale))
        else:
            k = k0.clone()
            yq, yk = torch.empty_like(x), torch.empty_like(k)
            if onthefly:
                launchers.append(rpe.rope_apply_qk_launcher(
                    x, k, None, None, ids, yq, yk, num_heads=w.num_heads,
                    kv_num_heads=w.kv_num_heads, inv_freq=inv, attention_scaling=w.scaling))
            else:
                launchers.append(rpe.rope_apply_qk_launcher(
                    x, k, cos, sin, ids, yq, yk, num_heads=w.num_heads,
                    kv_num_heads=w.kv_num_heads))
    torch.cuda.synchronize()
    return launchers, nsets * set_bytes


def setup_kv_append(w, q0, dt, dev):
    """Decode with cache append: sets of (Q, K, V, q_out, lengths) rotate;
    the two caches are shared, and each set's lengths are the base lengths
    shifted by a set-dependent offset (mod the cache length) so that the
    rows written differ from set to set. A prompt (every sequence starts at
    0, rows 0..S-1 written): each set has caches of its own."""
    import torch
    import rotary_position_embedding_amd as rpe
    smax = w.extra["cache_seq"]
    B, Hk, D = w.batch, w.kv_num_heads, w.head_size
    k0 = to_device(w.make_k(), dev)
    v0 = to_device(w.make_v(), dev)
    lens0 = w.make_lengths()
    inv = rpe.rope_inv_freq(w.rotary_dim, w.cache_base, device=dev)
    cos, sin = rpe.rope_cos_sin_cache(inv, w.cache_rows, dt, w.scaling)
    prompt = bool(w.extra.get("prompt"))
    pk = torch.zeros(B, Hk, smax, D, dtype=dt, device=dev)
    pv = torch.zeros_like(pk)
    set_bytes = 2 * (q0.numel() + 2 * k0.numel()) * q0.element_size()
    nsets = max(2, -(-ROTATE_BYTES // set_bytes))
    launchers = []
    wts = [to_device(a, dev) for a in w.make_norm_weights()] if w.op == "kv_append_norm" else None
    for i in range(nsets):
        if prompt:
            lens_h = lens0.copy()
            pk, pv = torch.zeros_like(pk), torch.zeros_like(pv)
        else:
            lens_h = ((lens0.astype(np.int64) - 1 + 997 * i) % smax + 1).astype(np.int32)
        q, k, v = q0.clone(), k0.clone(), v0.clone()
        lens = torch.from_numpy(lens_h).to(dev)
        if wts is None:
            launchers.append(rpe.rope_kv_append_launcher(
                q, k, v, pk, pv, lens, int(lens_h.max()), cos, sin, torch.empty_like(q),
                num_heads=w.num_heads, kv_num_heads=Hk))
        else:
            launchers.append(rpe.rope_kv_append_qk_norm_launcher(
                q, k, v, pk, pv, lens, int(lens_h.max()), cos, sin, torch.empty_like(q), wts[0], wts[1],
                epsilon=1e-6, num_heads=w.num_heads, kv_num_heads=Hk))
    torch.cuda.synchronize()
    return launchers, nsets * set_bytes


def _batches(steps):
    """Split K launches into at most BATCHES nearly equal batches."""
    nb = max(1, min(BATCHES, steps))
    return [steps // nb + (1 if i < steps % nb else 0) for i in range(nb)]


def _summary(per_launch, counts):
    """ms per launch: the median over batches, their spread and the mean over
    all launches."""
    total = sum(ms * n for ms, n in zip(per_launch, counts))
    return {"median": float(np.median(per_launch)), "min": float(min(per_launch)),
            "max": float(max(per_launch)), "mean": total / sum(counts), "batches": len(counts)}


def time_steps(launchers, steps, warmup):
    """K back-to-back launches in batches, a pair of HIP events around each
    batch on the launch stream (the current stream, which the launchers were
    bound to), synchronised on both sides of the K launches. Each step is
    one kernel, so a batch's time over its launch count is the kernel's
    average launch duration in that batch."""
    import torch
    n = len(launchers)
    for i in range(warmup):
        launchers[i % n]()
    torch.cuda.synchronize()
    counts = _batches(steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in counts]
    k = 0
    for (e0, e1), c in zip(evs, counts):
        e0.record()
        for _ in range(c):
            launchers[k % n]()
            k += 1
        e1.record()
    torch.cuda.synchronize()
    return _summary([e0.elapsed_time(e1) / c for (e0, e1), c in zip(evs, counts)], counts)


def time_steps_graph(launchers, steps, warmup):
    """The K launches captured in one HIP graph (rotating over the input
    sets as the eager launches do) and the graph replayed once per batch,
    each replay between a pair of events: what the GPU takes per step once
    the host's per-call cost is out of the way (decode steps are that
    small). The launchers were bound to the capture stream when they were
    made."""
    import torch
    n = len(launchers)
    for i in range(warmup):
        launchers[i % n]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
        for i in range(steps):
            launchers[i % n]()
    g.replay()                       # the first replay uploads the graph
    torch.cuda.synchronize()
    nb = max(5, min(BATCHES, 10))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nb)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    return _summary([e0.elapsed_time(e1) / steps for e0, e1 in evs], [steps] * nb)


def copy_reference(nbytes, steps, warmup):
    """A plain device copy (torch copy_) of `nbytes` read and the same written,
    N(0,1) fp16 data, rotating over >= 1 GiB like the kernels: the rate a pure
    stream of this size reaches on this GPU, for context (GB/s, ms)."""
    import torch
    n = nbytes // 2
    nsets = max(2, -(-ROTATE_BYTES // (2 * nbytes)))
    pairs = []
    for _ in range(nsets):
        a = torch.empty(n, dtype=torch.float16, device="cuda:0").normal_()
        pairs.append((a, torch.empty_like(a)))
    launchers = [lambda a=a, b=b: b.copy_(a) for a, b in pairs]
    ms = time_steps(launchers, steps, warmup)["median"]
    del pairs, launchers
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9, ms


# hand-written plain copies (libstream_copy.so): pattern, workgroups of the
# persistent patterns, description
STREAM_COPY_PATTERNS = [(1, 0, "one 1 KiB run per wave"), (2, 0, "one 16 KiB run per wave"),
                        (3, 1024, "persistent, 4 KiB chunks, 1024 workgroups"),
                        (4, 1024, "persistent, 8 KiB chunks, 1024 workgroups")]


def stream_copy_ceiling(nbytes, steps, warmup):
    """The best of the hand-written plain copies of `nbytes` read and the same
    written (no rotation), timed like the steps (same >= 1 GiB rotation over
    independent buffers, event-timed batches, median): the rate this GPU
    reaches for a pure stream of this size in this run."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "rotary_position_embedding_amd", "libstream_copy.so"))
    fn = lib.stream_copy
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    nsets = max(2, -(-ROTATE_BYTES // (2 * nbytes)))
    side = torch.cuda.Stream()
    out = []
    with torch.cuda.stream(side):
        pairs = []
        for _ in range(nsets):
            a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda:0").normal_()
            pairs.append((a, torch.empty_like(a)))
        st = side.cuda_stream
        for pattern, blocks, what in STREAM_COPY_PATTERNS:
            def make(a, b, pattern=pattern, blocks=blocks):
                args = (a.data_ptr(), b.data_ptr(), nbytes, pattern, blocks, st)

                def launch():
                    rc = fn(*args)
                    if rc != 0:
                        raise RuntimeError("stream_copy failed: %d" % rc)
                return launch
            t = time_steps([make(a, b) for a, b in pairs], steps, warmup)
            out.append({"pattern": what, "us": round(t["median"] * 1e3, 3),
                        "gbs": round(2 * nbytes / (t["median"] * 1e-3) / 1e9, 1)})
    torch.cuda.synchronize()
    del pairs
    torch.cuda.empty_cache()
    best = min(out, key=lambda r: r["us"])
    return {"bytes_read": nbytes, "bytes_written": nbytes, "patterns": out, "best_us": best["us"],
            "best_gbs": best["gbs"], "best_frac_of_peak": round(best["gbs"] / PEAK_GBS, 4)}


# Launches moving less than this are timed in a HIP graph replay: eager, the
# host's per-call cost (several µs) would set their rate.
GRAPH_BELOW_BYTES = 64 << 20


def small(w):
    return w.algorithmic_bytes() < GRAPH_BELOW_BYTES


def measure(w, steps, warmup, onthefly=False, graph=False):
    """Eager timing; with graph=True also the HIP-graph replay timing, which
    then gives the rates (the launch-bound decode steps)."""
    import torch
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):    # launchers bind the stream they are made on
        launchers, rot = setup(w, onthefly)
        eager = time_steps(launchers, steps, warmup)
        in_graph = time_steps_graph(launchers, steps, warmup) if graph else None
    torch.cuda.synchronize()
    nbytes = w.algorithmic_bytes(onthefly)
    t = in_graph if graph else eager
    ms_rate = t["median"]
    gbs = nbytes / (ms_rate * 1e-3) / 1e9
    r = {
        "workload": w.name + ("_onthefly" if onthefly else ""),
        "bytes_per_step": nbytes,
        "ms_per_step": ms_rate,
        "ms_per_step_min": t["min"],
        "ms_per_step_max": t["max"],
        "ms_per_step_mean": t["mean"],
        "batches": t["batches"],
        "gbs": gbs,
        "frac_of_peak": gbs / PEAK_GBS,
        "tokens_heads_per_s": w.tokens_heads() / (ms_rate * 1e-3),
        "rotation_sets_bytes": rot,
        "kernel_variant": launchers[0].variant,
    }
    if graph:
        r["ms_per_step_eager"] = eager["median"]
        r["rates_from"] = "hip_graph"
    return r


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores of this machine

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, min_reps=5, single_s=8.0, pool_s=2.0):
    """The oracle as it stands on the whole workload input: single-threaded,
    and on all the host cores this GPU's share allows (up to 16) by running
    the unmodified oracle on token slices in a thread pool (its C calls
    release the interpreter lock; every slice is an independent
    RotaryEmbedding call, so the result is the same, which is checked).
    Median of at least `min_reps` runs each, repeated until the leg has run
    `single_s` / `pool_s` seconds (a bounded sample of about 10 s)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    x = w.make_x()
    ids = w.make_ids()
    cos, sin = oracle.table_for(w)
    nh = w.num_heads if w.rank == 3 else 0
    kw = dict(interleaved=w.interleaved, num_heads=nh, rotary_embedding_dim=w.rotary_embedding_dim)

    def whole():
        return oracle.rope_apply(x, cos, sin, ids, **kw)

    # token slices: rank 3 (B, S, H*D) with ids (B, S) -> x[b, s0:s1], ids[b, s0:s1]
    if w.rank != 3 or ids is None:
        raise ValueError("the CPU baseline slices rank-3 inputs with position ids")
    B, S = ids.shape
    step = 128
    slices = [(b, s0, min(S, s0 + step)) for b in range(B) for s0 in range(0, S, step)]

    def one(sl):
        b, s0, s1 = sl
        return oracle.rope_apply(x[b:b + 1, s0:s1], cos, sin, ids[b:b + 1, s0:s1], **kw)

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(CPU_THREADS_MAX, avail))
    nbytes = w.algorithmic_bytes()
    t_single = []
    ref = None
    while len(t_single) < min_reps or sum(t_single) < single_s:
        t0 = time.perf_counter()
        ref = whole()
        t_single.append(time.perf_counter() - t0)
    t_par = []
    with ThreadPoolExecutor(max_workers=threads) as pool:
        while len(t_par) < min_reps or sum(t_par) < pool_s:
            t0 = time.perf_counter()
            parts = list(pool.map(one, slices))
            t_par.append(time.perf_counter() - t0)
    got = np.concatenate([np.concatenate([p for sl, p in zip(slices, parts) if sl[0] == b], axis=1)
                          for b in range(B)], axis=0)
    if not np.array_equal(got.view(np.uint8), ref.view(np.uint8)):
        raise AssertionError("oracle on token slices differs from the whole-input oracle")
    single = nbytes / float(np.median(t_single)) / 1e9
    par = nbytes / float(np.median(t_par)) / 1e9
    return {"value": round(par, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the whole %s input (%d tokens x %d heads, %d algorithmic bytes); scalar C oracle in "
                      "binary64 on %d token slices of %d in a pool of %d threads, median of %d runs (%.1f s)"
                      % (w.name, w.tokens, w.heads, nbytes, len(slices), step, threads, len(t_par), sum(t_par)),
            "single_thread": {"value": round(single, 4), "unit": "GB/s", "cores": 1,
                              "median_s": round(float(np.median(t_single)), 3),
                              "runs": len(t_single), "total_s": round(sum(t_single), 1)},
            "all_cores_median_s": round(float(np.median(t_par)), 3),
            "host": {"nproc": os.cpu_count(), "affinity_cpus": avail, "cpu_model": cpu_model()}}


def traffic_for_headline():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel source as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_sha():
        return None
    return t.get("traffic_bytes_per_launch")


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE,
                    help="workload to time alone (for profiler runs); implies --no-extra")
    ap.add_argument("--onthefly", action="store_true", help="with the decode Q+K workload")
    ap.add_argument("--dtype", choices=["bf16", "f32", "f16"], default=None,
                    help="time the workload stored in this type instead of its own")
    ap.add_argument("--interleaved", type=int, choices=[0, 1], default=None,
                    help="time the workload with this pairing instead of its own")
    ap.add_argument("--mrope-layout", type=int, choices=[0, 1], default=None,
                    help="time an M-RoPE workload with this mrope_layout instead of its own")
    ap.add_argument("--rotary-dim", type=int, default=None,
                    help="time the workload with this rotary_embedding_dim instead of its own")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-policy", type=int, default=0, choices=[0, 1, 2, 3],
                    help="rope_set_kernel_policy: 0 automatic, 1 scalar, 2 vector kernel only, "
                         "3 row kernel wherever its shape rules allow (kernel comparisons)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time plain 128 MiB device copies instead (counter calibration)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time only the hand-written plain copies of the prefill workloads' X/Y sizes")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU (the rotary apply has no cross-GPU step); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    # the library must be the build of the sources in this tree
    from rotary_position_embedding_amd import build as product_build
    product_build.ensure_current()

    import torch
    import rope_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.kernel_policy:
        import rotary_position_embedding_amd as rpe
        rpe.set_kernel_policy(args.kernel_policy)

    if args.copy_calibration:
        n = 64 << 20
        a = torch.ones(n, dtype=torch.float16, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(args.warmup):
            b.copy_(a)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        log("copy %d bytes x %d: %.1f GB/s" % (2 * n, args.steps, 2 * 2 * n * args.steps / el / 1e9))
        print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "steps": args.steps}))
        return

    if args.copy_ceiling:
        res = []
        for name in (HEADLINE, "c4_mrope_f16_prefill", "c3_rope_f32_partial_interleaved"):
            cw = rope_inputs.get(name)
            nx = int(np.prod(cw.x_shape)) * np.dtype(cw.dtype).itemsize
            log("plain copies of %s's X bytes (%d read, %d written)" % (name, nx, nx))
            c = stream_copy_ceiling(nx, args.steps, args.warmup)
            for r in c["patterns"]:
                log("  %-45s %8.2f us  %7.1f GB/s" % (r["pattern"], r["us"], r["gbs"]))
            res.append(dict(c, workload=name))
        print(json.dumps({"copy_ceiling": res}), flush=True)
        return

    only = args.workload != HEADLINE or args.no_extra
    w = rope_inputs.get(args.workload)
    if args.dtype:
        dt = {"bf16": rope_inputs.BFLOAT16, "f32": np.float32, "f16": np.float16}[args.dtype]
        w = rope_inputs.with_dtype(w, dt, args.dtype)
    if args.mrope_layout is not None:
        w = rope_inputs.with_layout(w, args.mrope_layout)
    if args.interleaved is not None or args.rotary_dim is not None:
        from dataclasses import replace
        w = replace(w, interleaved=w.interleaved if args.interleaved is None else args.interleaved,
                    rotary_embedding_dim=w.rotary_embedding_dim if args.rotary_dim is None else args.rotary_dim,
                    name="%s_il%s_r%s" % (w.name, args.interleaved, args.rotary_dim))
    log("timing %s: %d warmup + %d steps" % (w.name, args.warmup, args.steps))
    head = measure(w, args.steps, args.warmup, args.onthefly, graph=small(w))
    log("  %.2f us/step (median of %d batches; %.2f-%.2f), %.1f GB/s (%.1f%% of %g)" % (
        head["ms_per_step"] * 1e3, head["batches"], head["ms_per_step_min"] * 1e3,
        head["ms_per_step_max"] * 1e3, head["gbs"], 100 * head["frac_of_peak"], PEAK_GBS))

    also = []
    if not only:
        extra = [(rope_inputs.with_layout(rope_inputs.get("c4_mrope_f16_prefill"), 0), False),
                 (rope_inputs.with_layout(rope_inputs.get("c4_mrope_f16_prefill"), 1), False),
                 (rope_inputs.get("c3_rope_f32_partial_interleaved"), False),
                 (rope_inputs.get("c5_rope_qk_f16_decode"), False),
                 (rope_inputs.get("c5_rope_qk_f16_decode"), True),
                 (rope_inputs.with_dtype(rope_inputs.get(HEADLINE), rope_inputs.BFLOAT16, "bf16"), False),
                 (rope_inputs.with_dtype(rope_inputs.with_layout(rope_inputs.get("c4_mrope_f16_prefill"), 0),
                                         rope_inputs.BFLOAT16, "bf16"), False),
                 (rope_inputs.get("qkv_packed_f16_decode"), False),
                 (rope_inputs.get("kv_append_f16_decode"), False),
                 (rope_inputs.get("qk_norm_f16_prefill"), False),
                 (rope_inputs.get("qk_norm_f16_decode"), True),
                 (rope_inputs.get("qk_norm_kv_append_f16_decode"), False),
                 (rope_inputs.get("mrope_f16_decode"), False),
                 (rope_inputs.get("c2_rope_f16_prefill_tp8"), False),
                 (rope_inputs.get("c5_rope_qk_f16_decode_tp8"), False),
                 (rope_inputs.get("c2_rope_f16_prefill_sp8"), False),
                 (rope_inputs.get("kv_append_f16_prompt"), False),
                 (rope_inputs.get("rope_f16_prefill_heads64"), False),
                 (rope_inputs.get("rope_f16_prefill_neox_partial"), False),
                 (rope_inputs.get("qk_norm_f16_prefill_heads256"), False)]
        for ew, otf in extra:
            log("timing %s%s" % (ew.name, " on the fly" if otf else ""))
            decode = small(ew)
            r = measure(ew, min(args.steps, 100), min(args.warmup, 10), otf, graph=decode)
            if decode:
                log("  %.2f us/step in a HIP graph (%.2f eager): %.1f GB/s (%.1f%% of peak)" % (
                    r["ms_per_step"] * 1e3, r["ms_per_step_eager"] * 1e3, r["gbs"], 100 * r["frac_of_peak"]))
            else:
                log("  %.2f us/step, %.1f GB/s (%.1f%% of peak)" % (
                    r["ms_per_step"] * 1e3, r["gbs"], 100 * r["frac_of_peak"]))
            also.append({k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()})

    cpu = None
    if not args.no_cpu_baseline and w.op == "rope" and w.rank == 3 and w.has_ids:
        log("cpu baseline (oracle) on %s" % w.name)
        cpu = cpu_baseline(w)
        log("  %.3f GB/s on %d threads, %.3f GB/s single-threaded" % (
            cpu["value"], cpu["cores"], cpu["single_thread"]["value"]))

    traffic = traffic_for_headline() if w.name == HEADLINE else None
    copy_ref = None
    ceiling = None
    if not only and w.op == "rope":
        # the activation bytes of the step (X read, Y written) as a plain copy
        nx = int(np.prod(w.x_shape)) * np.dtype(w.dtype).itemsize
        log("timing a plain device copy of the same %d bytes (read and written)" % nx)
        cgbs, cms = copy_reference(nx, args.steps, args.warmup)
        log("  %.2f us/copy, %.1f GB/s" % (cms * 1e3, cgbs))
        copy_ref = {"what": "torch copy_ of the step's X bytes into Y (N(0,1) fp16 data, same >= 1 GiB rotation)",
                    "bytes_per_copy": 2 * nx, "us": round(cms * 1e3, 3), "gbs": round(cgbs, 1),
                    "frac_of_peak": round(cgbs / PEAK_GBS, 4),
                    "step_rate_over_copy_rate": round(head["gbs"] / cgbs, 4)}
        log("timing hand-written plain copies of the same %d bytes (read and written)" % nx)
        ceiling = stream_copy_ceiling(nx, args.steps, args.warmup)
        for r in ceiling["patterns"]:
            log("  %-45s %8.2f us  %7.1f GB/s" % (r["pattern"], r["us"], r["gbs"]))
        # the step moves X, Y and the coefficient rows and ids; the copy X and Y only
        ceiling["step_us_over_best_copy_us"] = round(head["ms_per_step"] * 1e3 / ceiling["best_us"], 4)
    result = {
        "metric": METRIC,
        "value": round(head["gbs"], 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: binary32 for 16-bit storage, binary64 products
        # and sums for float32 storage
        "dtype": "f64" if np.dtype(w.dtype) == np.float32 else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "storage_dtype": "bfloat16" if np.dtype(w.dtype) == np.uint16 else np.dtype(w.dtype).name,
            "x_shape": list(w.x_shape),
            "bytes_per_step": head["bytes_per_step"],
            "tokens_heads_per_s": round(head["tokens_heads_per_s"], 1),
            "rotation_sets_bytes": head["rotation_sets_bytes"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["gbs"], 3),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["gbs"] / PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "%s, variant %s" % (KERNEL_FUNCTIONS.get(head["kernel_variant"].split("/")[0], "?"),
                                          head["kernel_variant"]),
            "algorithmic_bytes_per_launch": head["bytes_per_step"],
            # HIP events on the launch stream: the median over batches of the
            # batch time per launch (one kernel per launch), and the spread
            "event_us_per_launch": round(head["ms_per_step"] * 1e3, 3),
            "event_us_batches": {"min": round(head["ms_per_step_min"] * 1e3, 3),
                                 "max": round(head["ms_per_step_max"] * 1e3, 3),
                                 "mean_all_launches": round(head["ms_per_step_mean"] * 1e3, 3),
                                 "batches": head["batches"]},
            "frac_range": [round(head["bytes_per_step"] / (head["ms_per_step_max"] * 1e-3) / 1e9 / PEAK_GBS, 4),
                           round(head["bytes_per_step"] / (head["ms_per_step_min"] * 1e-3) / 1e9 / PEAK_GBS, 4)],
        },
        "cpu_baseline": cpu,
        "source_sha256": kernel_source_sha(),
        "copy_reference": copy_ref,
        "copy_ceiling": ceiling,
        "also": also,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
