"""Decode throughput and HBM bandwidth of pool-indexed recurrent-state decode.

One step = one library call (gather, per-token prologue, decay, read-outs,
rank-1 update, outputs, optional per-token cache, writeback) over one batch
of synthetic input resident in HBM. Prints one JSON line.

Timing: untimed calls for 0.3 s of wall time (the GPU reaches its steady
clocks after the idle setup), W untimed warm-up calls, then K timed calls
bracketed by torch.cuda.synchronize(). Two HIP events on the stream the kernels are
launched on bracket the K back-to-back launches; their elapsed time / K is
the kernel's average launch duration used for the roofline. The calls
rotate over R independent copies of the pool and inputs, R x bytes-per-call
>= 4 GiB (16 times the 256 MB Infinity Cache; at most 512 copies, a limit only
the launch-bound small workload reaches), so that no call finds its tiles in
the cache: on MI355X a 1 GiB rotation still let cached loads reuse lines
across calls (GDN B=128 with cached loads: 77 % of peak at 1 GiB, 63 % at
3 GiB).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode tokens/sec and achieved HBM GB/s (% of peak), K=V=128 fp32 "
          "state")
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
ROTATE_BYTES = 4 << 30  # bytes the rotated copies span (16 x the MALL)
ROTATE_MAX = 512
SETTLE_SECONDS = 0.3  # untimed calls before the warm-up (steady clocks)
DEFAULT_WORKLOAD = "kda_b256_t8"
KERNEL_SRC = os.path.join(ROOT, "linear_attention_recurrent_slot_amd", "csrc",
                          "la_decode.hip")
PROFILES = os.path.join(ROOT, "profiles")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=0,
                    help="pool copies to rotate over (0: enough for 4 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline (0: skip)")
    ap.add_argument("--no-copy-probe", action="store_true")
    ap.add_argument("--head-shards", type=int, default=1,
                    help="measure one GPU's share when this many GPUs split "
                         "the value heads (1: the whole workload)")
    return ap.parse_args()


def source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = os.path.join(PROFILES, "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                key, val = ln.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_copies(wl, R, dev):
    """R independent device copies of the workload's tensors. Copy 0 is the
    seeded workload; the others redraw the pool and activations on the
    device with their own seeds (same shapes, distributions, indices)."""
    import torch
    copies = []
    for i in range(R):
        d = wl.to(dev)
        if i > 0:
            gen = torch.Generator(device=dev).manual_seed(1000 + i)
            std = float(wl.backing.float().std())
            d.backing.normal_(0.0, std, generator=gen)
            for name in ("q", "k", "v"):
                t = getattr(d, name)
                t.copy_(torch.randn(t.shape, generator=gen, device=dev))
        # (B, T), or the packed token count of a variable-length batch
        lead = tuple(wl.q.shape[:-2])
        inter = None
        if wl.inter:
            inter = torch.empty(lead + (wl.HV, wl.V, wl.K),
                                dtype=wl.backing.dtype, device=dev)
        out = torch.empty(lead + (wl.HV, wl.V), dtype=wl.out_dtype,
                          device=dev)
        if wl.replay_tokens is not None:
            d.records = torch.empty((wl.B, wl.T, wl.HV, wl.record_floats),
                                    dtype=torch.float32, device=dev)
            d.nowrite = torch.full((wl.B,), -1, dtype=torch.int32,
                                   device=dev)
        copies.append((d, inter, out))
    return copies


def make_call(wl, d, inter, out, stream):
    """A zero-argument callable launching one decode: the C argument struct
    is built (and shape-checked) once, so the timed loop costs one ctypes
    call per launch."""
    import ctypes
    from linear_attention_recurrent_slot_amd import _binding as bnd
    flags = 0
    if wl.variant != "lightning":
        flags = ((bnd.LA_F_L2NORM_QK if wl.l2norm else 0)
                 | (bnd.LA_F_BETA_LOGIT if wl.beta_logit else 0))
    vl = dict(cu_seqlens=d.cu_seqlens, max_tokens=wl.T)
    if d.token_slots is not None:
        args = bnd.build_args(wl.variant, d.q, d.k, d.v, d.g, d.beta,
                              d.pool(), None, None, out, inter, flags,
                              d.token_slots, d.num_accepted, **vl)
    elif d.replay_tokens is not None:
        # verify: no writeback, one update record per token
        args = bnd.build_args(wl.variant, d.q, d.k, d.v, d.g, d.beta,
                              d.pool(), d.read_idx, d.nowrite, out, inter,
                              flags, factors=d.records)
        rargs = bnd.build_replay_args(d.records, d.pool(), d.read_idx,
                                      d.write_idx, d.replay_tokens)
    else:
        args = bnd.build_args(wl.variant, d.q, d.k, d.v, d.g, d.beta,
                              d.pool(), d.read_idx, d.write_idx, out, inter,
                              flags, **vl)
    entry = getattr(bnd.lib(), {"lightning": "la_decode",
                                "gdn": "gdn_decode_mtp",
                                "kda": "kda_decode_mtp"}[wl.variant])
    ref = ctypes.byref(args)
    handle = ctypes.c_void_p(stream.cuda_stream)
    keep = (args, d, inter, out)

    if d.replay_tokens is not None:
        rref = ctypes.byref(rargs)
        replay = bnd.lib().la_replay
        keep = keep + (rargs,)

        def step():
            st = entry(ref, handle)
            if st != 0:
                raise bnd.LaDecodeError(st, "decode call")
            st = replay(rref, handle)
            if st != 0:
                raise bnd.LaDecodeError(st, "replay call")
            return keep
        step.args = args
        return step

    def call():
        st = entry(ref, handle)
        if st != 0:
            raise bnd.LaDecodeError(st, "decode call")
        return keep
    call.args = args  # the decode call's argument struct
    return call


def copy_probe(dev, stream):
    """Device-to-device copy of 1 GiB: achievable-bandwidth context, and the
    known-size kernel that calibrates the rocprofv3 byte counters."""
    import torch
    n = 1 << 28  # floats
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(
            enable_timing=True)
        s.record(stream)
        reps = 10
        for _ in range(reps):
            dst.copy_(src)
        e.record(stream)
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def _host():
    """CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu": model, "available_cores": len(os.sched_getaffinity(0))}


def _oracle_inputs(wl, lo, hi):
    """Arguments of one fp64 oracle call on requests [lo, hi) of the
    workload, as fp64 / int32 numpy arrays, with a sub-pool of exactly the
    slots those requests read or write (indices remapped; the work per
    request is unchanged)."""
    import numpy as np
    import oracle
    import torch
    variant = {"lightning": oracle.LIGHTNING, "gdn": oracle.GDN,
               "kda": oracle.KDA}[wl.variant]
    flags = ((oracle.L2NORM_QK if wl.l2norm else 0)
             | (oracle.BETA_LOGIT if wl.beta_logit else 0))

    def f64(t):
        return None if t is None else t.double().numpy().copy()

    def i32(t):
        return None if t is None else t.numpy().astype(np.int32)
    sel = slice(lo, hi)
    kw = dict(flags=flags, inter=wl.inter)
    tsel = sel  # per-token rows of the requests
    if wl.cu_seqlens is not None:
        cu = wl.cu_seqlens.tolist()
        tsel = slice(cu[lo], cu[hi])
        kw.update(cu_seqlens=i32(wl.cu_seqlens[lo:hi + 1]) - cu[lo],
                  max_tokens=wl.T)
    if wl.token_slots is not None:
        used = [i32(wl.token_slots[sel]).ravel()]
    else:
        used = [i32(wl.read_idx[sel])]
        if wl.write_idx is not None:
            used.append(i32(wl.write_idx[sel]))
    slots = np.unique(np.concatenate(used))
    slots = slots[slots >= 0]
    remap = np.full(wl.pool_size, -1, dtype=np.int32)
    remap[slots] = np.arange(len(slots), dtype=np.int32)

    def local(idx):
        return np.where(idx >= 0, remap[np.maximum(idx, 0)], idx).astype(
            np.int32)
    pool = wl.pool()[torch.from_numpy(slots.astype(np.int64))].double() \
        .numpy()
    ridx = widx = None
    if wl.token_slots is not None:
        kw.update(token_slots=local(i32(wl.token_slots[sel])),
                  num_accepted=i32(wl.num_accepted[sel]))
    else:
        ridx = local(i32(wl.read_idx[sel]))
        if wl.write_idx is not None:
            widx = local(i32(wl.write_idx[sel]))
    g = f64(wl.g) if wl.variant == "lightning" else f64(wl.g[tsel])
    beta = None if wl.beta is None else f64(wl.beta[tsel])
    args = (variant, f64(wl.q[tsel]), f64(wl.k[tsel]), f64(wl.v[tsel]), g,
            beta, pool, ridx, widx)
    return args, kw


def _time_oracle(inputs):
    import oracle
    args, kw = inputs
    t0 = time.perf_counter()
    oracle.decode(*args, **kw)
    return time.perf_counter() - t0


def cpu_baseline(wl, seconds):
    """The fp64 oracle as it stands, timed on the host on inputs already
    converted to fp64: single-threaded, and with one thread per available
    core (at most 16, the host share of one GPU) running it on disjoint
    request ranges at once (the oracle's C loop runs without the Python
    lock), about `seconds` each. A call covers the whole workload, or a
    leading part of its requests when one call would exceed the budget. The
    faster mode is the reported value; both are listed."""
    from concurrent.futures import ThreadPoolExecutor
    import torch
    counts = wl.counts()
    host = _host()
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        nb = wl.B
        inp = _oracle_inputs(wl, 0, nb)
        first = _time_oracle(inp)
        if first > seconds / 4:
            nb = max(1, int(wl.B * seconds / first / 8))
            inp = _oracle_inputs(wl, 0, nb)
        calls, tokens, spent = 0, 0, 0.0
        while spent < seconds / 2:
            spent += _time_oracle(inp)
            calls += 1
            tokens += sum(counts[:nb])
        st = {"value": tokens / spent, "cores": 1,
              "sample": "%d calls on %d of %d requests (%d tokens), %.1f s"
                        % (calls, nb, wl.B, sum(counts[:nb]), spent)}

        threads = max(1, min(16, host["available_cores"], wl.B))
        nbp = min(wl.B, max(threads, nb * threads))
        bounds = [nbp * i // threads for i in range(threads + 1)]
        ranges = [(bounds[i], bounds[i + 1]) for i in range(threads)
                  if bounds[i + 1] > bounds[i]]
        inps = [_oracle_inputs(wl, lo, hi) for lo, hi in ranges]
        calls, tokens, wall = 0, 0, 0.0
        with ThreadPoolExecutor(len(ranges)) as ex:
            while wall < seconds / 2:
                t0 = time.perf_counter()
                list(ex.map(_time_oracle, inps))
                wall += time.perf_counter() - t0
                calls += 1
                tokens += sum(counts[:nbp])
    finally:
        torch.set_num_threads(torch_threads)
    mt = {"value": tokens / wall, "cores": len(ranges),
          "sample": "%d parallel calls on %d of %d requests (%d tokens) in "
                    "%d threads, each on its request range and the pool "
                    "slots it touches, %.1f s"
                    % (calls, nbp, wl.B, sum(counts[:nbp]), len(ranges),
                       wall)}
    best = mt if mt["value"] >= st["value"] else st
    return {"value": best["value"], "unit": "tokens/s",
            "cores": best["cores"], "kind": "oracle", "host": host,
            "sample": "fp64 oracle on %s, inputs converted to fp64 "
                      "beforehand; %s" % (wl.name, best["sample"]),
            "threads": mt, "single_thread": st}


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(the decode shards by request or by value head with no "
              "exchange between GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_recurrent_slot_amd as lad
    import workloads

    lad.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wl = workloads.named(args.workload)
    if args.head_shards > 1:
        wl = workloads.head_shard(wl, args.head_shards)
    per_call = wl.state_bytes() + wl.io_bytes()
    pool_bytes = wl.backing.numel() * wl.backing.element_size()
    R = args.rotate or min(ROTATE_MAX, max(2, math.ceil(ROTATE_BYTES / per_call)))
    print("[bench] workload %s: B=%d T=%d H=%d HV=%d K=%d V=%d pool=%d, "
          "%.1f MB per call, rotating %d copies (%.2f GB of pools)"
          % (wl.name, wl.B, wl.T, wl.H, wl.HV, wl.K, wl.V, wl.pool_size,
             per_call / 1e6, R, R * pool_bytes / 1e9), file=sys.stderr,
          flush=True)
    copies = make_copies(wl, R, dev)
    calls = [make_call(wl, d, inter, out, stream) for d, inter, out in copies]
    for c in copies:
        if wl.token_slots is not None:
            bad = lad.check_token_slots(c[0].token_slots, c[0].num_accepted,
                                        wl.pool_size, wl.T)
        else:
            bad = lad.check_indices(c[0].read_idx, c[0].write_idx,
                                    wl.pool_size)
        if int(bad.item()) != 0:
            raise RuntimeError("workload index set violates the preconditions")

    # Bring the GPU to its steady clocks before the W warm-up calls: the
    # setup above leaves it idle, and a short timed run (K = 20) would
    # otherwise see the first calls at a lower clock. Untimed calls for
    # SETTLE_SECONDS of wall time.
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < SETTLE_SECONDS:
        calls[i % R]()
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()

    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        calls[i % R]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the timed region holds only the K back-to-back launches on `stream`
    avg_launch_ms = ev0.elapsed_time(ev1) / K
    ms_per_step = wall * 1e3 / K

    copy_gbps = None if args.no_copy_probe else copy_probe(dev, stream)

    tokens = wl.tokens  # B T, or the packed tokens of a varlen batch
    achieved = per_call / (avg_launch_ms * 1e-3) / 1e9
    state_gbps = wl.state_bytes() / (avg_launch_ms * 1e-3) / 1e9
    traffic = read_traffic(wl.name)
    from linear_attention_recurrent_slot_amd import _binding as bnd
    kinfo = bnd.kernel_info_of(wl.variant, calls[0].args)
    rec = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "variant": wl.variant, "B": wl.B,
                   "T": wl.T, "H": wl.H, "HV": wl.HV, "K": wl.K, "V": wl.V,
                   "pool_size": wl.pool_size, "qkv_dtype":
                   str(wl.q.dtype).replace("torch.", ""),
                   "state_dtype": str(wl.backing.dtype).replace("torch.", ""),
                   "stride_mult": wl.stride_mult,
                   "inter_cache": wl.inter,
                   "paged_slots": wl.token_slots is not None,
                   "spec_records_replay": wl.replay_tokens is not None,
                   "varlen_tokens": (wl.tokens if wl.cu_seqlens is not None
                                     else None),
                   "rotation": R, "head_shards": args.head_shards},
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic},
        "kernel_avg_us": avg_launch_ms * 1e3,
        "state_GBps": state_gbps,
        "state_frac_of_peak": state_gbps / PEAK_HBM_GBPS,
        "bytes_per_call": per_call,
        "state_bytes_per_call": wl.state_bytes(),
        "device_copy_GBps": copy_gbps,
        "kernel": kinfo,  # the decode call's kernel (the replay's is not listed)
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
