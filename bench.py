"""Decode throughput and HBM bandwidth of pool-indexed recurrent-state decode.

One step = one library call (gather, per-token prologue, decay, read-outs,
rank-1 update, outputs, optional per-token cache, writeback) over one batch
of synthetic input resident in HBM. Prints one JSON line.

Timing: W untimed warm-up calls, then K timed calls bracketed by
torch.cuda.synchronize(). Two HIP events on the stream the kernels are
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
DEFAULT_WORKLOAD = "lightning_b33_h64"
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


def cpu_baseline(wl, seconds):
    """The fp64 oracle as it stands, single-threaded on the host, repeated
    over the full workload (or a leading slice of its requests when one call
    would exceed the budget) for about `seconds`."""
    import oracle
    import torch
    variant = {"lightning": oracle.LIGHTNING, "gdn": oracle.GDN,
               "kda": oracle.KDA}[wl.variant]
    flags = ((oracle.L2NORM_QK if wl.l2norm else 0)
             | (oracle.BETA_LOGIT if wl.beta_logit else 0))

    counts = wl.counts()

    def run(nb):
        sel = slice(0, nb)
        extra = {}
        tsel = sel  # per-token rows of the first nb requests
        if wl.cu_seqlens is not None:
            tsel = slice(0, sum(counts[:nb]))
            extra = dict(cu_seqlens=wl.cu_seqlens[: nb + 1], max_tokens=wl.T)
        g = wl.g if wl.variant == "lightning" else wl.g[tsel]
        beta = None if wl.beta is None else wl.beta[tsel]
        widx = None if wl.write_idx is None else wl.write_idx[sel]
        t0 = time.perf_counter()
        if wl.token_slots is not None:
            extra.update(token_slots=wl.token_slots[sel],
                         num_accepted=wl.num_accepted[sel])
        oracle.decode(variant, wl.q[tsel], wl.k[tsel], wl.v[tsel], g, beta,
                      wl.pool(), wl.read_idx[sel], widx, flags=flags,
                      inter=wl.inter, **extra)
        return time.perf_counter() - t0

    nb = wl.B
    first = run(nb)
    if first > seconds:
        nb = max(1, int(wl.B * seconds / first / 2))
    calls, tokens, spent = 0, 0, 0.0
    while spent < seconds:
        spent += run(nb)
        calls += 1
        tokens += sum(counts[:nb])
    return {"value": tokens / spent, "unit": "tokens/s", "cores": 1,
            "kind": "oracle", "host": _host(),
            "sample": "%d calls of the fp64 oracle on %d of %d requests "
                      "(%d tokens) of %s (pool conversion included), %.1f s"
                      % (calls, nb, wl.B, sum(counts[:nb]), wl.name, spent)}


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the decode shards by request or head with no exchange; see "
              "the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_recurrent_slot_amd as lad
    import workloads

    lad.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wl = workloads.named(args.workload)
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
                   "rotation": R},
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
