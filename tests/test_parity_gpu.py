"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Element by element on the same seeded inputs (workloads.py), for every
variant, dtype and tile shape, index patterns from the pages' tests, strided
pools, packed views, token splitting, padding and skipped writes, plus
bytewise checks that every slot the call must not write is untouched.

Tolerances (max over a tensor of |gpu - oracle|):
  fp32 q/k/v: relative to max |oracle|, <= 1e-4 for outputs and states;
  bf16 q/k/v with the fp32 state: absolute <= 2e-3 (outputs), <= 1e-3
  (states and cached intermediates).
  bf16 state pool: stored states within one bf16 step of the oracle rounded
  to bf16, on top of the tolerance above (the kernel computes in fp32 and
  rounds to nearest even only when it stores).
"""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
VARIANT_CODE = {W.LIGHTNING: oracle.LIGHTNING, W.GDN: oracle.GDN,
                W.KDA: oracle.KDA}


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu-test] %s" % request.node.nodeid, flush=True)
    yield


def _lad():
    import linear_attention_recurrent_slot_amd as lad
    lad.lib()  # raises if the HIP library is missing
    return lad


# ------------------------------------------------------------------ runners


def gpu_run(wl, *, q=None, k=None, v=None, backing=None, stream=None,
            inter_fill=float("nan")):
    """Run the workload on the GPU. Returns CPU copies of out, backing and
    inter (inter pre-filled with NaN so untouched rows stay NaN)."""
    lad = _lad()
    d = wl.to(DEV)
    if backing is None:
        backing = d.backing
    pool = backing[:: wl.stride_mult]
    q = d.q if q is None else q
    k = d.k if k is None else k
    v = d.v if v is None else v
    # every index set must satisfy the device preconditions before a launch
    bad = lad.check_indices(d.read_idx, d.write_idx, wl.pool_size)
    assert int(bad.item()) == 0, "invalid index set in a test case"
    inter = None
    if wl.inter:
        inter = torch.full((wl.B, wl.T, wl.HV, wl.V, wl.K), inter_fill,
                           dtype=wl.backing.dtype, device=DEV)
    if wl.variant == W.LIGHTNING:
        out, _ = lad.la_decode(q, k, v, pool, d.read_idx, d.write_idx,
                               lam=d.g, inter=inter, out_dtype=wl.out_dtype,
                               stream=stream)
    else:
        fn = lad.gdn_decode_mtp if wl.variant == W.GDN else lad.kda_decode_mtp
        out, _ = fn(q, k, v, d.g, d.beta, pool, d.read_idx, d.write_idx,
                    inter=inter, l2norm_qk=wl.l2norm,
                    beta_logit=wl.beta_logit, out_dtype=wl.out_dtype,
                    stream=stream)
    torch.cuda.synchronize()
    return {"out": out.cpu(), "backing": backing.cpu(),
            "inter": None if inter is None else inter.cpu()}


def _flags(wl):
    return ((oracle.L2NORM_QK if wl.l2norm else 0)
            | (oracle.BETA_LOGIT if wl.beta_logit else 0))


def _oracle_chunk(wl, reqs):
    """Oracle on the requests `reqs`, on a mini pool made of their read
    slots (reads at 0..n-1, writes at n..2n-1). Returns their outputs, cache
    rows and written states (None where nothing is written), in order."""
    n = len(reqs)
    pool = wl.pool()
    ridx = wl.read_idx.tolist()
    widx = wl.write_idx.tolist() if wl.write_idx is not None else ridx
    mini = torch.zeros((2 * n,) + tuple(pool.shape[1:]), dtype=torch.float64)
    mr, mw = [], []
    for i, b in enumerate(reqs):
        if ridx[b] >= 0:
            mini[i] = pool[ridx[b]].double()
            mr.append(i)
            mw.append(n + i if widx[b] >= 0 else -1)
        else:
            mr.append(-1)
            mw.append(-1)
    sel = torch.tensor(reqs)
    g = wl.g
    if wl.variant != W.LIGHTNING:
        g = g[sel]
    beta = None if wl.beta is None else wl.beta[sel]
    res = oracle.decode(VARIANT_CODE[wl.variant], wl.q[sel], wl.k[sel],
                        wl.v[sel], g, beta, mini, mr, mw, flags=_flags(wl),
                        inter=wl.inter)
    return {"out": res["out"], "inter": res["inter"],
            "state": [None if w < 0 else res["pool"][w] for w in mw]}


ORACLE_CHUNK = 8  # requests per oracle call
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_run(wl):
    """The oracle on every request of `wl`: chunks of ORACLE_CHUNK requests,
    each on its own mini pool (bounded host memory), run on threads (the
    oracle's C loop runs without the Python lock). Returns the outputs
    [B,T,HV,V], the cache [B,T,HV,V,K] (or None) and, per request, the state
    it writes (or None)."""
    reqs = list(range(wl.B))
    chunks = [reqs[i:i + ORACLE_CHUNK]
              for i in range(0, len(reqs), ORACLE_CHUNK)]
    with ThreadPoolExecutor(min(ORACLE_THREADS, max(1, len(chunks)))) as ex:
        parts = list(ex.map(lambda c: _oracle_chunk(wl, c), chunks))
    if not parts:
        return {"out": np.zeros((0,)), "inter": None, "state": []}
    return {"out": np.concatenate([p["out"] for p in parts]),
            "inter": (np.concatenate([p["inter"] for p in parts])
                      if wl.inter else None),
            "state": [s for p in parts for s in p["state"]]}


def _tol(wl):
    if wl.q.dtype == torch.float32:
        return ("rel", 1e-4, 1e-4)
    return ("abs", 2e-3, 1e-3)


def _err(kind, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite GPU values"
    e = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if kind == "rel":
        e /= max(float(np.max(np.abs(ref))), 1e-30)
    return e


def _state_err(wl, kind, tol_state, got, ref):
    """Error of a stored state; for a bf16 pool, the excess over one bf16
    step of the oracle rounded to nearest even (0 when within it)."""
    if wl.backing.dtype != torch.bfloat16:
        return _err(kind, got, ref)
    g = torch.as_tensor(np.asarray(got, dtype=np.float64))
    rb = torch.as_tensor(np.asarray(ref, dtype=np.float64)).to(
        torch.bfloat16).double()
    assert torch.isfinite(g).all(), "non-finite GPU values"
    floor = tol_state if kind == "abs" else tol_state * float(rb.abs().max())
    excess = (g - rb).abs() - rb.abs() * 2.0 ** -7 - floor
    return max(float(excess.max()), 0.0)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def check_parity(wl, got, before_backing):
    """Compare every request with the oracle; check every untouched byte of
    the backing buffer over the whole pool."""
    ref = oracle_run(wl)
    kind, tol_out, tol_state = _tol(wl)
    ridx = wl.read_idx.tolist()
    widx = wl.write_idx.tolist() if wl.write_idx is not None else ridx
    m = wl.stride_mult
    errs = {"out": 0.0, "state": 0.0, "inter": 0.0}
    out = got["out"].float().numpy()
    # the fp32 tolerance of a bf16 output in absolute terms: relative
    # tolerances are taken against the largest output of the call
    out_floor = tol_out if kind == "abs" else \
        tol_out * float(np.max(np.abs(ref["out"]))) if ref["out"].size else 0
    for b in range(wl.B):
        if wl.out_dtype == torch.bfloat16:
            # the kernel rounds its fp32 result to nearest even: allow one
            # bf16 step on top of the fp32 tolerance (near zero the fp32
            # tolerance is the larger one)
            ref_b = torch.tensor(ref["out"][b]).to(torch.bfloat16).float()
            step = torch.abs(ref_b) * 2.0 ** -7 + 1e-30
            diff = torch.abs(torch.tensor(out[b]) - ref_b)
            assert bool((diff <= step + out_floor).all()), \
                "bf16 output off by more than one step"
        else:
            errs["out"] = max(errs["out"], _err(kind, out[b], ref["out"][b]))
        if ridx[b] < 0:
            assert not np.any(out[b]), "padded request must output zeros"
            if wl.inter:
                assert torch.isnan(got["inter"][b].float()).all(), \
                    "padded request must not touch the cache"
            continue
        if wl.inter:
            errs["inter"] = max(errs["inter"], _state_err(
                wl, kind, tol_state, got["inter"][b].float().numpy(),
                ref["inter"][b]))
        if widx[b] >= 0:
            errs["state"] = max(errs["state"], _state_err(
                wl, kind, tol_state, got["backing"][m * widx[b]].float().numpy(),
                ref["state"][b]))
    bf = wl.backing.dtype == torch.bfloat16
    assert errs["out"] <= tol_out, errs
    assert errs["state"] <= (0.0 if bf else tol_state), errs
    assert errs["inter"] <= (0.0 if bf else tol_state), errs
    # bytewise: only the backing slots of non-negative write slots of active
    # requests may change
    written = {m * w for r, w in zip(ridx, widx) if r >= 0 and w >= 0}
    a = _bits(got["backing"])
    b0 = _bits(before_backing)
    keep = torch.ones(a.shape[0], dtype=torch.bool)
    if written:
        keep[torch.tensor(sorted(written))] = False
    assert torch.equal(a[keep], b0[keep]), "a slot that must not change did"
    return errs


def run_and_check(wl):
    before = wl.backing.clone()
    got = gpu_run(wl)
    errs = check_parity(wl, got, before)
    print("  %s errors %s" % (wl.name, {k: "%.2e" % v for k, v in errs.items()}),
          flush=True)
    return got


# ------------------------------------------------------- named workloads

@pytest.mark.parametrize("name", [n for n in W.NAMED
                                  if "paged" not in n and "varlen" not in n])
def test_named_workload_parity(name):
    """Every request of the named workload against the oracle, at its full
    size and in the launch configuration the benchmark times."""
    run_and_check(W.named(name))


def test_named_paged_workload_parity():
    wl = W.named("gdn_paged_b64_t4")
    got = gpu_run_paged(wl, wl.token_slots, wl.num_accepted)
    check_paged(wl, wl.token_slots, wl.num_accepted, got)


def test_small_workload_host_normalised_inputs():
    """q and k normalised before the call (flag off) give the same result
    as raw inputs normalised in the kernel."""
    wl = W.gdn_small_k64()
    qn = wl.q / wl.q.norm(dim=-1, keepdim=True)
    kn = wl.k / wl.k.norm(dim=-1, keepdim=True)
    wl2 = W.gdn_small_k64()
    wl2.q, wl2.k, wl2.l2norm = qn, kn, False
    run_and_check(wl2)


# ------------------------------------------------- shapes, dtypes, tokens


SHAPES = [(64, 64), (128, 128), (64, 128), (128, 64)]


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 3, 9])
def test_shapes_dtypes_tokens(variant, K, V, dtype, T):
    seed = (1000 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant)
            + 10 * SHAPES.index((K, V)) + T
            + (500 if dtype == torch.bfloat16 else 0))
    wl = W.make("shape", variant, B=3, T=T, H=2, HV=4, K=K, V=V,
                pool_size=7, seed=seed, act_dtype=dtype, pool_std=0.1,
                l2norm=variant != W.LIGHTNING, separate_write=True,
                write_skip=0.34, inter=True)
    run_and_check(wl)


def test_long_multi_token_run_crosses_chunks():
    """T = 17: three prologue chunks of up to 8 tokens."""
    wl = W.make("long", W.KDA, B=5, T=17, H=1, HV=2, K=128, V=128,
                pool_size=9, seed=21, inter=True)
    run_and_check(wl)


# ------------------------------------------- index patterns of the pages


def _gdn_pool_case(B, pool_size, read_idx, T=1, seed=30, **kw):
    return W.make("pool", W.GDN, B=B, T=T, H=2, HV=4, K=128, V=128,
                  pool_size=pool_size, seed=seed, read_idx=read_idx,
                  act_dtype=torch.float32, **kw)


@pytest.mark.parametrize("B,pool_size,read_idx", [
    (4, 4, [0, 1, 2, 3]),           # identity offsets
    (4, 6, [2, 0, 5, 1]),           # non-identity, pool larger than batch
    (4, 4, [3, 2, 1, 0]),           # reversed, pool = batch
    (33, 40, None),                 # big batch in a pool of 40
], ids=["identity", "non_identity", "reversed", "b33_pool40"])
def test_page_index_patterns(B, pool_size, read_idx):
    wl = _gdn_pool_case(B, pool_size, read_idx)
    run_and_check(wl)


@pytest.mark.parametrize("B,pool_size,read_idx", [
    (4, 6, [2, 0, 5, 1]), (4, 4, [3, 2, 1, 0]), (33, 40, None)])
def test_index_equivariance_bit_identical(B, pool_size, read_idx):
    """Batched results equal one-request calls on the same slots, bit for
    bit: the arithmetic does not depend on B or the slot."""
    wl = _gdn_pool_case(B, pool_size, read_idx, T=2)
    whole = gpu_run(wl)
    for b in range(B):
        one = W.make("one", W.GDN, B=1, T=2, H=2, HV=4, K=128, V=128,
                     pool_size=pool_size, seed=0, act_dtype=torch.float32,
                     read_idx=[int(wl.read_idx[b])])
        one.q, one.k, one.v = wl.q[b:b + 1], wl.k[b:b + 1], wl.v[b:b + 1]
        one.g, one.beta = wl.g[b:b + 1], wl.beta[b:b + 1]
        one.backing = wl.backing.clone()
        got = gpu_run(one)
        assert torch.equal(got["out"][0], whole["out"][b])
        r = int(wl.read_idx[b])
        assert torch.equal(got["backing"][r], whole["backing"][r])


@pytest.mark.parametrize("B", [1, 4, 16])
@pytest.mark.parametrize("T", [2, 4])
@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("cache", [False, True])
def test_mtp_fp32_state_pool(B, T, separate, cache):
    """The FlashInfer fp32 MTP pool matrix: batch x seq_len x separate
    output indices x intermediate caching."""
    wl = W.make("mtp", W.GDN, B=B, T=T, H=16, HV=32, K=128, V=128,
                pool_size=2 * B + 3, seed=100 + B * 10 + T, act_dtype=torch.float32,
                separate_write=separate, write_skip=0.25 if separate else 0.0,
                inter=cache)
    run_and_check(wl)


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("T", [2, 4])
@pytest.mark.parametrize("mult", [2, 3])
def test_mtp_fp32_state_pool_non_contiguous(B, T, mult):
    """Strided pools cut from an oversized buffer are updated in place and
    the gap slots stay untouched."""
    wl = W.make("strided", W.GDN, B=B, T=T, H=16, HV=32, K=128, V=128,
                pool_size=2 * B + 2, seed=200 + B * 10 + T + mult,
                act_dtype=torch.float32, stride_mult=mult,
                separate_write=True, inter=True)
    run_and_check(wl)


@pytest.mark.parametrize("mult", [2, 3])
def test_strided_pool_bit_identical_to_contiguous(mult):
    wl = W.make("s", W.KDA, B=4, T=3, H=2, HV=4, K=128, V=128, pool_size=9,
                seed=40 + mult, stride_mult=mult, separate_write=True)
    got_s = gpu_run(wl)
    wl_c = W.make("c", W.KDA, B=4, T=3, H=2, HV=4, K=128, V=128, pool_size=9,
                  seed=40 + mult, stride_mult=mult, separate_write=True)
    wl_c.backing = wl.pool().contiguous()
    wl_c.stride_mult = 1
    got_c = gpu_run(wl_c)
    assert torch.equal(got_s["out"], got_c["out"])
    assert torch.equal(got_s["backing"][::mult], got_c["backing"])


# ------------------------------------------------------ packed q/k/v views


@pytest.mark.parametrize("variant", [W.GDN, W.KDA, W.LIGHTNING])
def test_packed_qkv_views_bit_identical(variant):
    """q/k/v as head-dim slices of one fused [B, T, 2HK + HV V] buffer give
    exactly the contiguous result."""
    wl = W.make("pk", variant, B=5, T=2, H=2, HV=4, K=128, V=64, pool_size=8,
                seed=50, l2norm=variant != W.LIGHTNING)
    B, T, H, HV, K, V = wl.B, wl.T, wl.H, wl.HV, wl.K, wl.V
    fused = torch.cat([wl.q.reshape(B, T, H * K), wl.k.reshape(B, T, H * K),
                       wl.v.reshape(B, T, HV * V)], dim=-1).to(DEV)
    qv = fused[..., : H * K].unflatten(-1, (H, K))
    kv = fused[..., H * K: 2 * H * K].unflatten(-1, (H, K))
    vv = fused[..., 2 * H * K:].unflatten(-1, (HV, V))
    assert not qv.is_contiguous()
    packed = gpu_run(wl, q=qv, k=kv, v=vv)
    plain = gpu_run(W.make("pk", variant, B=5, T=2, H=2, HV=4, K=128, V=64,
                           pool_size=8, seed=50,
                           l2norm=variant != W.LIGHTNING))
    assert torch.equal(packed["out"], plain["out"])
    assert torch.equal(packed["backing"], plain["backing"])


def _scrambled_like(x, inner, rng):
    """A view with x's shape whose outer dimensions (all but the last
    `inner`) are laid out in a random order with padding, inside a
    NaN-filled buffer on the device; the inner dimension keeps unit
    stride. Holds x's values."""
    outer = x.dim() - inner
    order = list(range(outer))
    rng.shuffle(order)
    pads = [rng.randint(0, 2) for _ in range(outer)]
    shape = [x.shape[d] + pads[d] for d in order] + list(x.shape[outer:])
    buf = torch.full(shape, float("nan"), dtype=x.dtype, device=DEV)
    view = buf[tuple(slice(0, x.shape[d]) for d in order)]
    back = [order.index(d) for d in range(outer)] + list(
        range(outer, x.dim()))
    view = view.permute(back)
    view.copy_(x.to(DEV))
    return view


LAYOUT_CASES = {
    # name: (variant, B, T, H, HV, K, V, act, out, state, kernel)
    "general_gdn_t3": (W.GDN, 5, 3, 2, 4, 128, 64, torch.bfloat16,
                       torch.float32, torch.float32, "decode_kernel"),
    "general_kda_t5": (W.KDA, 4, 5, 2, 2, 64, 128, torch.float32,
                       torch.bfloat16, torch.float32, "decode_kernel"),
    "general_lightning_t2": (W.LIGHTNING, 6, 2, 3, 3, 64, 64, torch.bfloat16,
                             torch.bfloat16, torch.bfloat16, "decode_kernel"),
    "general_kda_bf16_state_t9": (W.KDA, 3, 9, 1, 2, 128, 128, torch.bfloat16,
                                  torch.float32, torch.bfloat16,
                                  "decode_kernel"),
    "general_32_rows_gdn_t3": (W.GDN, 40, 3, 8, 16, 128, 128, torch.bfloat16,
                               torch.float32, torch.float32, "decode_kernel"),
    "general_32_rows_kda_t8": (W.KDA, 24, 8, 24, 24, 128, 128,
                               torch.bfloat16, torch.float32, torch.float32,
                               "decode_kernel"),
    "one_token_gdn": (W.GDN, 40, 1, 16, 32, 128, 128, torch.bfloat16,
                      torch.float32, torch.float32, "decode1_kernel"),
    "one_token_kda": (W.KDA, 48, 1, 24, 24, 128, 128, torch.float32,
                      torch.bfloat16, torch.float32, "decode1_kernel"),
    "packed_gdn_bf16_state": (W.GDN, 16, 1, 8, 16, 128, 128, torch.bfloat16,
                              torch.float32, torch.bfloat16,
                              "decode_packed_kernel"),
}


@pytest.mark.parametrize("name", sorted(LAYOUT_CASES))
def test_scrambled_activation_layouts_bit_identical(name):
    """q, k, v, g, beta and out as views whose outer dimensions lie in
    memory in a random order with padding (any non-negative strides, the
    innermost dimension unit-stride) give exactly the bits of the same call
    on contiguous tensors, in every kernel; the padding of the output
    buffer stays NaN."""
    import random
    (variant, B, T, H, HV, K, V, act, outd, state,
     kernel) = LAYOUT_CASES[name]
    seed = 5600 + sorted(LAYOUT_CASES).index(name)
    rng = random.Random(seed)

    def make():
        return W.make("layout", variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
                      pool_size=2 * B + 1, seed=seed, act_dtype=act,
                      out_dtype=outd, state_dtype=state, separate_write=True,
                      write_skip=0.2, l2norm=variant != W.LIGHTNING)
    wl = make()
    assert _kernel_name(wl) == kernel
    lad = _lad()
    results = []
    for scrambled in (False, True):
        d = make().to(DEV)
        pool = d.backing[:: wl.stride_mult]
        q, k, v, g, beta = d.q, d.k, d.v, d.g, d.beta
        out = torch.full((B, T, HV, V), float("nan"), dtype=outd, device=DEV)
        if scrambled:
            q = _scrambled_like(q, 1, rng)
            k = _scrambled_like(k, 1, rng)
            v = _scrambled_like(v, 1, rng)
            out = _scrambled_like(out, 1, rng)
            if variant != W.LIGHTNING:
                g = _scrambled_like(g, 1 if variant == W.KDA else 0, rng)
                beta = _scrambled_like(beta, 0, rng)
            assert not q.is_contiguous() or not out.is_contiguous()
        if variant == W.LIGHTNING:
            lad.la_decode(q, k, v, pool, d.read_idx, d.write_idx, lam=g,
                          out=out, out_dtype=outd)
        else:
            fn = lad.gdn_decode_mtp if variant == W.GDN else \
                lad.kda_decode_mtp
            fn(q, k, v, g, beta, pool, d.read_idx, d.write_idx,
               l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit, out=out,
               out_dtype=outd)
        torch.cuda.synchronize()
        if scrambled:
            base = out._base
            assert int(torch.isnan(base.float()).sum()) == \
                base.numel() - out.numel(), "a write outside the output view"
        results.append((out.contiguous().cpu(), d.backing.cpu()))
    assert not torch.isnan(results[0][0].float()).any()
    assert torch.equal(_bits(results[1][0]), _bits(results[0][0]))
    assert torch.equal(_bits(results[1][1]), _bits(results[0][1]))


PACKED_QKV_KERNELS = {
    # name: (variant, B, T, H, HV, state dtype, kernel)
    "one_token_gdn": (W.GDN, 64, 1, 16, 32, torch.float32, "decode1_kernel"),
    "one_token_lightning": (W.LIGHTNING, 33, 1, 64, 64, torch.float32,
                            "decode1_kernel"),
    "packed_bf16_kda": (W.KDA, 8, 1, 8, 8, torch.bfloat16,
                        "decode_packed_kernel"),
    "one_token_kda": (W.KDA, 96, 1, 24, 24, torch.float32, "decode1_kernel"),
    "general_32_rows_gdn": (W.GDN, 40, 2, 16, 32, torch.float32,
                            "decode_kernel"),
}


@pytest.mark.parametrize("name", sorted(PACKED_QKV_KERNELS))
def test_packed_qkv_views_every_kernel(name):
    """Fused q/k/v views give the contiguous bits in each kernel, with
    their own strides read per request, token and head."""
    variant, B, T, H, HV, state, kernel = PACKED_QKV_KERNELS[name]
    K = V = 128

    def make():
        return W.make("pkk", variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
                      pool_size=2 * B, seed=5100 + B + T, state_dtype=state,
                      separate_write=True, l2norm=variant != W.LIGHTNING)
    wl = make()
    assert _kernel_name(wl) == kernel
    fused = torch.cat([wl.q.reshape(B, T, H * K), wl.k.reshape(B, T, H * K),
                       wl.v.reshape(B, T, HV * V)], dim=-1).to(DEV)
    qv = fused[..., : H * K].unflatten(-1, (H, K))
    kv = fused[..., H * K: 2 * H * K].unflatten(-1, (H, K))
    vv = fused[..., 2 * H * K:].unflatten(-1, (HV, V))
    packed = gpu_run(wl, q=qv, k=kv, v=vv)
    plain = gpu_run(make())
    assert torch.equal(_bits(packed["out"]), _bits(plain["out"]))
    assert torch.equal(_bits(packed["backing"]), _bits(plain["backing"]))


# --------------------------------------------------------- token splitting


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
def test_token_split_bit_identical(variant):
    """T single-token calls chained through the pool = one T-token call,
    bit for bit (outputs and final state)."""
    T = 5
    wl = W.make("split", variant, B=3, T=T, H=2, HV=4, K=128, V=128,
                pool_size=5, seed=60, l2norm=variant != W.LIGHTNING)
    whole = gpu_run(wl)
    backing = wl.backing.clone().to(DEV)
    for t in range(T):
        step = W.make("split", variant, B=3, T=T, H=2, HV=4, K=128, V=128,
                      pool_size=5, seed=60, l2norm=variant != W.LIGHTNING)
        step.T = 1
        step.q, step.k, step.v = (x[:, t:t + 1] for x in (wl.q, wl.k, wl.v))
        if variant != W.LIGHTNING:
            step.g = wl.g[:, t:t + 1]
            step.beta = wl.beta[:, t:t + 1]
        got = gpu_run(step, backing=backing)
        assert torch.equal(got["out"][:, 0], whole["out"][:, t])
    assert torch.equal(backing.cpu(), whole["backing"])


# ------------------------------------------------- padding and degenerate


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
def test_padding_and_skipped_writes(variant):
    wl = W.make("pad", variant, B=6, T=2, H=2, HV=2, K=64, V=128, pool_size=9,
                seed=70, read_idx=[3, -1, 0, 8, -1, 5],
                write_idx=[1, 2, -1, 7, 4, -1], inter=True)
    got = run_and_check(wl)
    assert not got["out"][1].any() and not got["out"][4].any()


def test_zero_beta_zero_gate_leaves_state():
    wl = W.make("z", W.GDN, B=3, T=2, H=1, HV=2, K=128, V=128, pool_size=4,
                seed=80, act_dtype=torch.float32, beta_logit=False)
    wl.g = torch.zeros_like(wl.g)
    wl.beta = torch.zeros_like(wl.beta)
    before = wl.backing.clone()
    got = gpu_run(wl)
    assert torch.equal(got["backing"], before)
    check_parity(wl, got, before)


def test_zero_query_and_key_stay_finite():
    wl = W.make("zq", W.KDA, B=2, T=2, H=1, HV=2, K=128, V=128, pool_size=3,
                seed=81)
    wl.q = torch.zeros_like(wl.q)
    wl.k = torch.zeros_like(wl.k)
    got = run_and_check(wl)
    assert not got["out"].any()


def test_unit_key_beta_one_writes_value():
    """beta = 1, |k| = 1 (l2norm on): the new state maps k to v."""
    wl = W.make("uk", W.GDN, B=2, T=1, H=1, HV=2, K=128, V=128, pool_size=2,
                seed=82, act_dtype=torch.float32, beta_logit=False,
                inter=True)
    wl.beta = torch.ones_like(wl.beta)
    got = gpu_run(wl)
    kn = wl.k / torch.sqrt((wl.k.double() ** 2).sum(-1, keepdim=True) + 1e-6)
    for b in range(2):
        for hv in range(2):
            S = got["inter"][b, 0, hv].double()
            err = (S @ kn[b, 0, 0].double() - wl.v[b, 0, hv].double()).abs().max()
            assert float(err) < 1e-4


def test_empty_batch_noop():
    lad = _lad()
    wl = W.make("e", W.GDN, B=1, T=1, H=1, HV=1, K=64, V=64, pool_size=2,
                seed=83)
    d = wl.to(DEV)
    out, _ = lad.gdn_decode_mtp(d.q[:0], d.k[:0], d.v[:0], d.g[:0],
                                d.beta[:0], d.pool(), d.read_idx[:0])
    torch.cuda.synchronize()
    assert out.shape[0] == 0
    assert torch.equal(d.backing.cpu(), wl.backing)


def test_bf16_output():
    wl = W.make("bo", W.GDN, B=4, T=2, H=2, HV=4, K=128, V=128, pool_size=6,
                seed=84, out_dtype=torch.bfloat16)
    run_and_check(wl)


def test_int64_pool_addressing():
    """A slot beyond 2^31 elements from the pool base (8.6 GB buffer)."""
    K = V = 128
    tile = V * K
    slot_stride = 2 ** 31 + tile
    n = slot_stride + tile
    buf = torch.empty(n, dtype=torch.float32, device=DEV)
    gen = torch.Generator().manual_seed(90)
    tiles = torch.randn((2, 1, V, K), generator=gen) * 0.05
    pool = torch.as_strided(buf, (2, 1, V, K), (slot_stride, tile, K, 1))
    pool.copy_(tiles.to(DEV))
    wl = W.make("big", W.GDN, B=2, T=2, H=1, HV=1, K=K, V=V, pool_size=2,
                seed=91, read_idx=[1, 0])
    wl.backing = tiles
    lad = _lad()
    d = wl.to(DEV)
    out, _ = lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx,
                                d.write_idx, l2norm_qk=True, beta_logit=True)
    torch.cuda.synchronize()
    ref = oracle_run(wl)
    kind, tol_out, tol_state = _tol(wl)
    assert _err(kind, out.cpu().numpy(), ref["out"]) <= tol_out
    after = pool.cpu()
    # request 0 read and wrote slot 1, request 1 slot 0
    assert _err(kind, after[1].numpy(), ref["state"][0]) <= tol_state
    assert _err(kind, after[0].numpy(), ref["state"][1]) <= tol_state
    del buf, pool


# ------------------------------------------------------- index validator


@pytest.mark.parametrize("ridx,widx,expect", [
    ([0, 1, 2], None, 0),
    ([0, 1, 2], [3, 4, -1], 0),
    ([0, -1, 2], [3, 0, 5], 0),     # a padded request writes nothing
    ([0, 1, 9], None, 3),           # the default write slot is out of range too
    ([0, 1, 9], [2, 3, 4], 1),
    ([0, 1, 2], [3, 9, 4], 2),
    ([0, 1, 2], [3, 3, 4], 4),
    ([0, 1, 2], [1, 4, 5], 8),
    ([0, 0, 2], None, 12),          # two requests write back one slot
    ([0, 0, 2], [3, 4, 5], 0),      # shared read slot, distinct writes
])
def test_check_indices(ridx, widx, expect):
    lad = _lad()
    r = torch.tensor(ridx, dtype=torch.int32, device=DEV)
    w = None if widx is None else torch.tensor(widx, dtype=torch.int32,
                                               device=DEV)
    res = lad.check_indices(r, w, pool_size=6)
    assert int(res.item()) == expect


def test_check_indices_empty_and_large():
    lad = _lad()
    r = torch.empty(0, dtype=torch.int32, device=DEV)
    assert int(lad.check_indices(r, None, pool_size=4).item()) == 0
    perm = torch.randperm(4096, generator=torch.Generator().manual_seed(3))
    r = perm[:2000].to(torch.int32).to(DEV)
    w = perm[2000:4000].to(torch.int32).to(DEV)
    assert int(lad.check_indices(r, w, pool_size=4096).item()) == 0
    w2 = w.clone()
    w2[1999] = w2[0]
    assert int(lad.check_indices(r, w2, pool_size=4096).item()) == 4


def _indices_rule(ridx, widx, P):
    """The bits la_check_indices documents, restated over host lists: a
    padded request (negative read slot) reads and writes nothing."""
    w = list(ridx) if widx is None else list(widx)
    f = 0
    for i, r in enumerate(ridx):
        if r >= P:
            f |= 1
        if r < 0:
            continue
        if w[i] >= P:
            f |= 2
        if w[i] < 0:
            continue
        for j, rj in enumerate(ridx):
            if j != i and rj >= 0:
                f |= 4 if w[j] == w[i] else 0
                f |= 8 if rj == w[i] else 0
    return f


def _token_slots_rule(tab, acc, T, P):
    """The bits la_check_token_slots documents: a request with an accepted
    count outside [1, T] or a negative seed is padding and writes nothing;
    an active request writes the entries of its row (negatives skip)."""
    def seed(i):
        return tab[i][acc[i] - 1] if 1 <= acc[i] <= T else -1
    f = 0
    for i in range(len(acc)):
        if not 1 <= acc[i] <= T:
            f |= 16
            continue
        if seed(i) >= P:
            f |= 1
        if seed(i) < 0:
            continue
        if any(s >= P for s in tab[i][:T]):
            f |= 2
        for j in range(len(acc)):
            if j == i or seed(j) < 0:
                continue
            for s in tab[i][:T]:
                if s >= 0:
                    f |= 8 if s == seed(j) else 0
                    f |= 4 if s in tab[j][:T] else 0
    return f


def _cu_seqlens_rule(cu, T, total):
    """The bits la_check_cu_seqlens documents."""
    f = 0
    for c0, c1 in zip(cu[:-1], cu[1:]):
        if not (0 <= c0 <= total and 0 <= c1 <= total):
            f |= 1
        if c1 < c0 or c1 - c0 > T:
            f |= 2
    return f


def test_validators_follow_their_rules_on_random_inputs():
    """200 random inputs per validator (valid sets, and sets with negative,
    repeated and out-of-range entries): each validator's bits equal its
    documented rules evaluated on the host."""
    import random
    lad = _lad()
    rng = random.Random(4242)

    def slot(P):
        u = rng.random()
        return -1 if u < 0.1 else (P + rng.randrange(3) if u < 0.15
                                   else rng.randrange(P))
    seen = {"indices": set(), "slots": set(), "cu": set()}
    for _ in range(200):
        B = rng.randint(1, 24)
        P = rng.randint(1, 2 * B + 4)
        if rng.random() < 0.3 and P >= 2 * B:
            perm = rng.sample(range(P), 2 * B)
            ridx, widx = perm[:B], perm[B:]
        else:
            ridx = [slot(P) for _ in range(B)]
            widx = [slot(P) for _ in range(B)]
        if rng.random() < 0.3:
            widx = None
        r = torch.tensor(ridx, dtype=torch.int32, device=DEV)
        w = None if widx is None else torch.tensor(widx, dtype=torch.int32,
                                                   device=DEV)
        got = int(lad.check_indices(r, w, pool_size=P).item())
        assert got == _indices_rule(ridx, widx, P), (ridx, widx, P)
        seen["indices"].add(got)

        T = rng.randint(1, 5)
        P = rng.randint(1, 2 * B * T + 2)
        tab = [[slot(P) for _ in range(T)] for _ in range(B)]
        if rng.random() < 0.3 and P >= B * T:
            flat = rng.sample(range(P), B * T)
            tab = [flat[b * T:(b + 1) * T] for b in range(B)]
        acc = [rng.choice([0, T + 1]) if rng.random() < 0.1
               else rng.randint(1, T) for _ in range(B)]
        t = torch.tensor(tab, dtype=torch.int32, device=DEV)
        a = torch.tensor(acc, dtype=torch.int32, device=DEV)
        got = int(lad.check_token_slots(t, a, P, T).item())
        assert got == _token_slots_rule(tab, acc, T, P), (tab, acc, T, P)
        seen["slots"].add(got)

        lengths = [rng.randint(0, T) for _ in range(B)]
        cu = [0]
        for n in lengths:
            cu.append(cu[-1] + n)
        total = cu[-1]
        if rng.random() < 0.4:
            i = rng.randrange(B + 1)
            cu[i] += rng.choice([-2, -1, 1, T + 1])
        if rng.random() < 0.2:
            total = max(0, total - 1)
        c = torch.tensor(cu, dtype=torch.int32, device=DEV)
        got = int(lad.check_cu_seqlens(c, T, total).item())
        assert got == _cu_seqlens_rule(cu, T, total), (cu, T, total)
        seen["cu"].add(got)
    # the draws reach the valid case and several failure bits of each
    assert 0 in seen["indices"] and len(seen["indices"]) >= 6, seen
    assert 0 in seen["slots"] and len(seen["slots"]) >= 6, seen
    assert seen["cu"] >= {0, 1, 2, 3}, seen


def test_workload_index_sets_are_valid():
    lad = _lad()
    for name in W.NAMED:
        wl = W.named(name)
        if wl.token_slots is not None:
            res = lad.check_token_slots(wl.token_slots.to(DEV),
                                        wl.num_accepted.to(DEV),
                                        wl.pool_size, wl.T)
            assert int(res.item()) == 0, name
            continue
        r = wl.read_idx.to(DEV)
        w = None if wl.write_idx is None else wl.write_idx.to(DEV)
        assert int(lad.check_indices(r, w, wl.pool_size).item()) == 0, name


def test_side_stream():
    """Calls honour the caller's stream."""
    wl = W.make("st", W.GDN, B=3, T=2, H=1, HV=2, K=128, V=128, pool_size=4,
                seed=95)
    s = torch.cuda.Stream()
    before = wl.backing.clone()
    with torch.cuda.stream(s):
        got = gpu_run(wl, stream=s)
    check_parity(wl, got, before)


@pytest.mark.parametrize("variant,T", [(W.GDN, 1), (W.KDA, 2)],
                         ids=["gdn_t1", "kda_t2"])
def test_concurrent_streams_on_disjoint_slots(variant, T):
    """Two calls on two streams, issued back to back with no synchronisation
    between them, on disjoint halves of one batch (disjoint read and write
    slots of one pool): the pool and outputs equal those of the single call
    over the whole batch, bit for bit."""
    lad = _lad()
    B, HV = 64, 32 if variant == W.GDN else 24
    H = HV // 2 if variant == W.GDN else HV
    wl = W.make("streams", variant, B=B, T=T, H=H, HV=HV, K=128, V=128,
                pool_size=3 * B, seed=9300 + T, separate_write=True)
    d = wl.to(DEV)
    fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp

    def call(pool, sl):
        return fn(d.q[sl], d.k[sl], d.v[sl], d.g[sl], d.beta[sl], pool,
                  d.read_idx[sl], d.write_idx[sl], l2norm_qk=wl.l2norm,
                  beta_logit=wl.beta_logit)[0]
    whole_pool = d.backing.clone()
    whole = call(whole_pool, slice(0, B))
    torch.cuda.synchronize()
    pool = d.backing.clone()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for s, sl in zip(streams, (slice(0, B // 2), slice(B // 2, B))):
        with torch.cuda.stream(s):
            outs.append(call(pool, sl))
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch.cat(outs).cpu()), _bits(whole.cpu()))
    assert torch.equal(_bits(pool.cpu()), _bits(whole_pool.cpu()))


def test_host_threads_share_the_library():
    """The library keeps no state between calls: four host threads, each
    with its own stream, pool and inputs, call it at the same time and get
    the results of the same calls made one after another."""
    import threading
    lad = _lad()
    wls = [W.make("thr%d" % i, W.GDN, B=16, T=2, H=8, HV=16, K=128, V=128,
                  pool_size=32, seed=9400 + i, separate_write=True)
           for i in range(4)]
    devs = [wl.to(DEV) for wl in wls]

    def call(d, wl, pool):
        return lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, pool,
                                  d.read_idx, d.write_idx,
                                  l2norm_qk=wl.l2norm,
                                  beta_logit=wl.beta_logit)[0]
    serial = []
    for d, wl in zip(devs, wls):
        pool = d.backing.clone()
        serial.append((call(d, wl, pool), pool))
    torch.cuda.synchronize()
    pools = [d.backing.clone() for d in devs]
    torch.cuda.synchronize()
    results = [None] * 4
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                results[i] = call(devs[i], wls[i], pools[i])
            s.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(_bits(results[i].cpu()), _bits(serial[i][0].cpu()))
        assert torch.equal(_bits(pools[i].cpu()), _bits(serial[i][1].cpu()))


# ------------------------------------------------ paged per-token state slots


def _paged_case(variant, seed, B=4, T=3, HV=4, K=128, V=128, inter=False,
                state_dtype=torch.float32):
    """A workload plus a [B, T+2] slot table (wider than T: the row stride is
    explicit), accepted counts in [1, T], disjoint rows, some -1 entries."""
    pool_size = B * T + 5
    wl = W.make("paged", variant, B=B, T=T, H=2, HV=HV, K=K, V=V,
                pool_size=pool_size, seed=seed, inter=inter,
                state_dtype=state_dtype)
    gen = torch.Generator().manual_seed(seed + 1)
    perm = torch.randperm(pool_size, generator=gen).to(torch.int32)
    table = torch.full((B, T + 2), 99, dtype=torch.int32)  # padding columns
    table[:, :T] = perm[: B * T].view(B, T)
    accepted = torch.randint(1, T + 1, (B,), generator=gen, dtype=torch.int32)
    # a skipped snapshot on a token that is not any request's seed
    for b in range(B):
        t = (int(accepted[b]) % T)
        if t != int(accepted[b]) - 1:
            table[b, t] = -1
            break
    return wl, table, accepted


def gpu_run_paged(wl, table, accepted, inter_fill=float("nan")):
    lad = _lad()
    d = wl.to(DEV)
    tab, acc = table.to(DEV), accepted.to(DEV)
    bad = lad.check_token_slots(tab, acc, wl.pool_size, wl.T)
    assert int(bad.item()) in (0, 16), "invalid slot table in a test case"
    pool = d.backing[:: wl.stride_mult]
    inter = None
    if wl.inter:
        inter = torch.full((wl.B, wl.T, wl.HV, wl.V, wl.K), inter_fill,
                           dtype=wl.backing.dtype, device=DEV)
    kw = dict(inter=inter, out_dtype=wl.out_dtype, token_slots=tab,
              num_accepted=acc)
    if wl.variant == W.LIGHTNING:
        out, _ = lad.la_decode(d.q, d.k, d.v, pool, lam=d.g, **kw)
    else:
        fn = lad.gdn_decode_mtp if wl.variant == W.GDN else lad.kda_decode_mtp
        out, _ = fn(d.q, d.k, d.v, d.g, d.beta, pool, l2norm_qk=wl.l2norm,
                    beta_logit=wl.beta_logit, **kw)
    torch.cuda.synchronize()
    return {"out": out.cpu(), "backing": d.backing.cpu(),
            "inter": None if inter is None else inter.cpu()}


def check_paged(wl, table, accepted, got):
    ref = oracle.decode(VARIANT_CODE[wl.variant], wl.q, wl.k, wl.v, wl.g,
                        wl.beta, wl.pool(), [0] * wl.B, flags=_flags(wl),
                        inter=wl.inter, token_slots=table[:, : wl.T],
                        num_accepted=accepted)
    kind, tol_out, tol_state = _tol(wl)
    bf = wl.backing.dtype == torch.bfloat16
    assert _err(kind, got["out"].numpy(), ref["out"]) <= tol_out
    written = set()
    for b in range(wl.B):
        na = int(accepted[b])
        if not 1 <= na <= wl.T or int(table[b, na - 1]) < 0:
            assert not got["out"][b].any()
            if wl.inter:
                assert torch.isnan(got["inter"][b].float()).all()
            continue
        for t in range(wl.T):
            s = int(table[b, t])
            if s >= 0:
                written.add(s)
        if wl.inter:
            e = _state_err(wl, kind, tol_state, got["inter"][b].float().numpy(),
                           ref["inter"][b])
            assert e <= (0.0 if bf else tol_state)
    for s in sorted(written):
        e = _state_err(wl, kind, tol_state, got["backing"][s].float().numpy(),
                       ref["pool"][s])
        assert e <= (0.0 if bf else tol_state)
    keep = torch.ones(wl.backing.shape[0], dtype=torch.bool)
    if written:
        keep[torch.tensor(sorted(written))] = False
    assert torch.equal(_bits(got["backing"])[keep], _bits(wl.backing)[keep])


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("T", [1, 3, 9])
def test_paged_slots_parity(variant, T):
    wl, table, accepted = _paged_case(variant, 300 + T, T=T, inter=True)
    got = gpu_run_paged(wl, table, accepted)
    check_paged(wl, table, accepted, got)


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
def test_paged_slots_equal_scattered_cache_bitwise(variant):
    """Paged mode = classic mode reading the seed slot with the cache on,
    cache rows scattered to the table's slots, bit for bit."""
    wl, table, accepted = _paged_case(variant, 310, B=5, T=4)
    got = gpu_run_paged(wl, table, accepted)
    seeds = [int(table[b, int(accepted[b]) - 1]) for b in range(wl.B)]
    dense = W.make("paged", variant, B=5, T=4, H=2, HV=4, K=128, V=128,
                   pool_size=wl.pool_size, seed=310, inter=True,
                   read_idx=seeds, write_idx=[-1] * wl.B)
    dgot = gpu_run(dense)
    assert torch.equal(got["out"], dgot["out"])
    want = wl.backing.clone()
    for b in range(wl.B):
        for t in range(wl.T):
            s = int(table[b, t])
            if s >= 0:
                want[s] = dgot["inter"][b, t]
    assert torch.equal(got["backing"], want)


def test_paged_slots_out_of_range_accepted_is_padding():
    wl, table, accepted = _paged_case(W.KDA, 320, B=4, T=3, inter=True)
    accepted[1] = 0
    accepted[3] = 4
    got = gpu_run_paged(wl, table, accepted)
    check_paged(wl, table, accepted, got)
    lad = _lad()
    res = lad.check_token_slots(table.to(DEV), accepted.to(DEV),
                                wl.pool_size, wl.T)
    assert int(res.item()) == 16


def test_paged_slots_flat_table_rejected():
    """A flat table cannot be read as [B, T]: the explicit stride must cover
    T (the aiter reviewer's corruption case is refused, not guessed)."""
    lad = _lad()
    wl, table, accepted = _paged_case(W.GDN, 330, B=2, T=2)
    d = wl.to(DEV)
    flat = table[:, :2].reshape(-1).to(DEV)
    narrow = flat.as_strided((2, 2), (1, 1))  # rows overlapping: stride 1
    with pytest.raises(lad.LaDecodeError):
        lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, d.pool(),
                           token_slots=narrow, num_accepted=accepted.to(DEV))
    with pytest.raises(lad.LaDecodeError):
        lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, d.pool(), d.read_idx,
                           token_slots=table.to(DEV),
                           num_accepted=accepted.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(d.backing.cpu(), wl.backing)


@pytest.mark.parametrize("tab,acc,expect", [
    ([[0, 1], [2, 3]], [1, 2], 0),
    ([[0, 9], [2, 3]], [1, 2], 2),
    ([[9, 1], [2, 3]], [1, 2], 3),
    ([[0, 1], [1, 3]], [2, 2], 12),   # slot 1: both write it, it seeds 0
    ([[0, 1], [2, 1]], [1, 1], 4),
    ([[0, 1], [2, 3]], [0, 2], 16),
    ([[0, -1], [2, 3]], [1, 1], 0),
])
def test_check_token_slots(tab, acc, expect):
    lad = _lad()
    t = torch.tensor(tab, dtype=torch.int32, device=DEV)
    a = torch.tensor(acc, dtype=torch.int32, device=DEV)
    assert int(lad.check_token_slots(t, a, 6, 2).item()) == expect


# --------------------------------------------------------- bf16 state pool


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 3, 9])
def test_bf16_state_pool(variant, K, V, dtype, T):
    seed = (2000 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant)
            + 10 * SHAPES.index((K, V)) + T
            + (500 if dtype == torch.bfloat16 else 0))
    wl = W.make("bf16state", variant, B=3, T=T, H=2, HV=4, K=K, V=V,
                pool_size=7, seed=seed, act_dtype=dtype, pool_std=0.1,
                separate_write=True, write_skip=0.34, inter=True,
                state_dtype=torch.bfloat16)
    run_and_check(wl)


@pytest.mark.parametrize("mult", [1, 3])
def test_bf16_state_pool_strided_and_padded(mult):
    wl = W.make("bf16pad", W.GDN, B=6, T=2, H=2, HV=2, K=128, V=128,
                pool_size=9, seed=2900 + mult, stride_mult=mult,
                read_idx=[3, -1, 0, 8, -1, 5], write_idx=[1, 2, -1, 7, 4, -1],
                inter=True, state_dtype=torch.bfloat16)
    got = run_and_check(wl)
    assert not got["out"][1].any() and not got["out"][4].any()


def test_bf16_state_pool_paged():
    wl, table, accepted = _paged_case(W.KDA, 2950, T=4, inter=True,
                                      state_dtype=torch.bfloat16)
    got = gpu_run_paged(wl, table, accepted)
    check_paged(wl, table, accepted, got)


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
def test_bf16_state_one_token_packed(variant, K, V, dtype):
    """One token on a bf16 pool with no per-token cache: the kernel that
    keeps the tile packed in registers."""
    seed = (3100 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant)
            + 10 * SHAPES.index((K, V))
            + (5 if dtype == torch.bfloat16 else 0))
    wl = W.make("bf16t1", variant, B=5, T=1, H=2, HV=4, K=K, V=V,
                pool_size=11, seed=seed, act_dtype=dtype, pool_std=0.1,
                separate_write=True, write_skip=0.34,
                state_dtype=torch.bfloat16)
    run_and_check(wl)


@pytest.mark.parametrize("mult", [1, 3])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16],
                         ids=["out_f32", "out_bf16"])
def test_bf16_state_one_token_packed_strided_and_padded(mult, out_dtype):
    wl = W.make("bf16t1pad", W.KDA, B=6, T=1, H=2, HV=2, K=128, V=128,
                pool_size=9, seed=3050 + mult, stride_mult=mult,
                read_idx=[3, -1, 0, 8, -1, 5], write_idx=[1, 2, -1, 7, 4, -1],
                state_dtype=torch.bfloat16, out_dtype=out_dtype)
    got = run_and_check(wl)
    assert not got["out"][1].any() and not got["out"][4].any()


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 128)])
def test_bf16_state_packed_kernel_bit_identical_to_general(variant, K, V):
    """The packed one-token kernel and the general kernel (which runs when a
    per-token cache is asked for) do the same fp32 operations in the same
    order, so outputs and stored states agree bit for bit."""
    wl = W.make("bf16same", variant, B=7, T=1, H=2, HV=4, K=K, V=V,
                pool_size=16, seed=3200 + [W.LIGHTNING, W.GDN,
                                           W.KDA].index(variant),
                separate_write=True, write_skip=0.3,
                state_dtype=torch.bfloat16)
    packed = gpu_run(wl)
    general = gpu_run(dataclasses.replace(wl, inter=True))
    assert torch.equal(_bits(packed["out"]), _bits(general["out"]))
    assert torch.equal(_bits(packed["backing"]), _bits(general["backing"]))


def test_bf16_state_roundtrip_is_exact_when_unchanged():
    """beta = 0 and g = 0 leave the state unchanged: widening bf16 to fp32
    and rounding back must reproduce the stored bits exactly."""
    wl = W.make("bf16id", W.GDN, B=3, T=2, H=1, HV=2, K=128, V=128,
                pool_size=4, seed=2960, act_dtype=torch.float32,
                beta_logit=False, state_dtype=torch.bfloat16)
    wl.g = torch.zeros_like(wl.g)
    wl.beta = torch.zeros_like(wl.beta)
    before = wl.backing.clone()
    got = gpu_run(wl)
    assert torch.equal(_bits(got["backing"]), _bits(before))


# ------------------------------------------- update records and la_replay


def _records_case(variant, seed, K=128, V=128, T=4, dtype=torch.bfloat16,
                  state_dtype=torch.float32, B=4):
    return W.make("rec", variant, B=B, T=T, H=2, HV=4, K=K, V=V,
                  pool_size=2 * B + 3, seed=seed, act_dtype=dtype,
                  pool_std=0.1, separate_write=True, inter=True,
                  state_dtype=state_dtype)


def _decode_with_records(wl):
    """Decode without writeback, with the per-token cache and the records."""
    lad = _lad()
    d = wl.to(DEV)
    pool = d.pool()
    inter = torch.full((wl.B, wl.T, wl.HV, wl.V, wl.K), float("nan"),
                       dtype=wl.backing.dtype, device=DEV)
    fac = torch.full((wl.B, wl.T, wl.HV, 2 * wl.K + wl.V), float("nan"),
                     dtype=torch.float32, device=DEV)
    nowrite = torch.full((wl.B,), -1, dtype=torch.int32, device=DEV)
    if wl.variant == W.LIGHTNING:
        out, _ = lad.la_decode(d.q, d.k, d.v, pool, d.read_idx, nowrite,
                               lam=d.g, inter=inter, factors=fac)
    else:
        fn = lad.gdn_decode_mtp if wl.variant == W.GDN else lad.kda_decode_mtp
        out, _ = fn(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx, nowrite,
                    inter=inter, factors=fac, l2norm_qk=wl.l2norm,
                    beta_logit=wl.beta_logit)
    torch.cuda.synchronize()
    return d, out, inter, fac


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
def test_update_records_match_oracle(variant, K, V, dtype):
    seed = (3000 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant)
            + 10 * [(128, 128), (64, 128), (128, 64)].index((K, V))
            + (5 if dtype == torch.bfloat16 else 0))
    wl = _records_case(variant, seed, K=K, V=V, dtype=dtype)
    d, out, inter, fac = _decode_with_records(wl)
    ref = oracle.decode(VARIANT_CODE[wl.variant], wl.q, wl.k, wl.v, wl.g,
                        wl.beta, wl.pool(), wl.read_idx, [-1] * wl.B,
                        flags=_flags(wl), inter=True, factors=True)
    kind, tol_out, tol_state = _tol(wl)
    got = fac.cpu().numpy()
    a, kk, err = (got[..., :K], got[..., K:2 * K], got[..., 2 * K:])
    ra, rk, re_ = (ref["factors"][..., :K], ref["factors"][..., K:2 * K],
                   ref["factors"][..., 2 * K:])
    assert _err("rel", a, ra) <= 1e-5
    assert _err("rel", kk, rk) <= (1e-5 if dtype == torch.float32 else 1e-3)
    assert _err(kind, err, re_) <= tol_out
    assert _err(kind, out.cpu().numpy(), ref["out"]) <= tol_out
    # no writeback: the pool is untouched
    assert torch.equal(_bits(d.backing.cpu()), _bits(wl.backing))


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16],
                         ids=["f32state", "bf16state"])
@pytest.mark.parametrize("T", [1, 4, 11])
def test_replay_equals_per_token_cache_bitwise(variant, state_dtype, T):
    """Replaying n records from the seed reproduces the decode's state after
    token n-1 bit for bit (same fp32 operations on the same values)."""
    seed = 3500 + 10 * [W.LIGHTNING, W.GDN, W.KDA].index(variant) + T + (
        1000 if state_dtype == torch.bfloat16 else 0)
    wl = _records_case(variant, seed, T=T, state_dtype=state_dtype)
    lad = _lad()
    d, out, inter, fac = _decode_with_records(wl)
    pool = d.pool()
    assert torch.isfinite(fac).all()
    for n in sorted({0, 1, T // 2, T}):
        ntok = torch.full((wl.B,), n, dtype=torch.int32, device=DEV)
        lad.replay(fac, pool, d.read_idx, d.write_idx, ntok)
        torch.cuda.synchronize()
        for b in range(wl.B):
            w = int(wl.write_idx[b])
            if w < 0:
                continue
            want = (pool[int(wl.read_idx[b])] if n == 0
                    else inter[b, n - 1])
            assert torch.equal(_bits(pool[w]), _bits(want)), (b, n)
    # the read slots and every slot nobody writes keep their bytes
    written = {int(x) for x in wl.write_idx.tolist() if x >= 0}
    keep = torch.ones(wl.pool_size, dtype=torch.bool)
    keep[torch.tensor(sorted(written))] = False
    assert torch.equal(_bits(pool.cpu())[keep], _bits(wl.pool())[keep])


def test_replay_skips_out_of_range_counts_and_padding():
    wl = _records_case(W.KDA, 3900, T=3)
    lad = _lad()
    d, out, inter, fac = _decode_with_records(wl)
    pool = d.pool()
    before = pool.cpu().clone()
    ridx = d.read_idx.clone()
    ridx[0] = -1
    ntok = torch.tensor([2, -1, 4, 3], dtype=torch.int32, device=DEV)
    lad.replay(fac, pool, ridx, d.write_idx, ntok)
    torch.cuda.synchronize()
    after = pool.cpu()
    for b in range(3):  # padded read, negative count, count > T
        w = int(wl.write_idx[b])
        if w >= 0:
            assert torch.equal(_bits(after[w]), _bits(before[w]))
    w3 = int(wl.write_idx[3])
    if w3 >= 0:
        assert torch.equal(_bits(after[w3]), _bits(inter[3, 2].cpu()))


def test_named_spec_step_parity():
    """The speculative step the benchmark times: verify with records (no
    state write), then replay the accepted tokens into the write slots;
    compared with the oracle's records and replay."""
    lad = _lad()
    wl = W.named("kda_spec_b64_t4")
    d = wl.to(DEV)
    pool = d.pool()
    rec = torch.full((wl.B, wl.T, wl.HV, wl.record_floats), float("nan"),
                     dtype=torch.float32, device=DEV)
    nowrite = torch.full((wl.B,), -1, dtype=torch.int32, device=DEV)
    out, _ = lad.kda_decode_mtp(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx,
                                nowrite, factors=rec, l2norm_qk=True,
                                beta_logit=True)
    lad.replay(rec, pool, d.read_idx, d.write_idx, d.replay_tokens)
    torch.cuda.synchronize()
    ref = oracle.decode(oracle.KDA, wl.q, wl.k, wl.v, wl.g, wl.beta,
                        wl.pool(), wl.read_idx, [-1] * wl.B, flags=_flags(wl),
                        factors=True)
    refpool = oracle.replay(ref["factors"], wl.pool(), wl.read_idx,
                            wl.write_idx, wl.replay_tokens)
    kind, tol_out, tol_state = _tol(wl)
    assert _err(kind, out.cpu().numpy(), ref["out"]) <= tol_out
    got = pool.cpu()
    written = [int(w) for w in wl.write_idx.tolist() if w >= 0]
    for w in written:
        assert _err(kind, got[w].numpy(), refpool[w]) <= tol_state
    keep = torch.ones(wl.pool_size, dtype=torch.bool)
    keep[torch.tensor(written)] = False
    assert torch.equal(_bits(got)[keep], _bits(wl.pool())[keep])


# ----------------------------------------------------- variable-length batches


def gpu_run_varlen(wl, factors=False):
    """Run a token-packed workload (wl.cu_seqlens set). Outputs, cache and
    records are pre-filled with NaN."""
    lad = _lad()
    d = wl.to(DEV)
    pool = d.backing[:: wl.stride_mult]
    total = wl.q.shape[0]
    assert int(lad.check_cu_seqlens(d.cu_seqlens, wl.T, total).item()) == 0
    paged = wl.token_slots is not None
    if not paged:
        assert int(lad.check_indices(d.read_idx, d.write_idx,
                                     wl.pool_size).item()) == 0
    out = torch.full((total, wl.HV, wl.V), float("nan"), dtype=wl.out_dtype,
                     device=DEV)
    inter = (torch.full((total, wl.HV, wl.V, wl.K), float("nan"),
                        dtype=wl.backing.dtype, device=DEV)
             if wl.inter else None)
    fac = (torch.full((total, wl.HV, 2 * wl.K + wl.V), float("nan"),
                      dtype=torch.float32, device=DEV) if factors else None)
    kw = dict(out=out, inter=inter, factors=fac, cu_seqlens=d.cu_seqlens,
              max_tokens=wl.T, token_slots=d.token_slots,
              num_accepted=d.num_accepted, out_dtype=wl.out_dtype)
    ridx = None if paged else d.read_idx
    widx = None if paged else d.write_idx
    if wl.variant == W.LIGHTNING:
        lad.la_decode(d.q, d.k, d.v, pool, ridx, widx, lam=d.g, **kw)
    else:
        fn = lad.gdn_decode_mtp if wl.variant == W.GDN else lad.kda_decode_mtp
        fn(d.q, d.k, d.v, d.g, d.beta, pool, ridx, widx,
           l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit, **kw)
    torch.cuda.synchronize()
    return {"out": out.cpu(), "backing": d.backing.cpu(),
            "inter": None if inter is None else inter.cpu(),
            "factors": None if fac is None else fac.cpu()}


def oracle_run_varlen(wl, factors=False):
    """The oracle on every request of a token-packed workload, over the
    whole pool."""
    reqs = list(range(wl.B))
    cu = wl.cu_seqlens.tolist()
    rows = [r for b in reqs for r in range(cu[b], cu[b + 1])]
    counts = [cu[b + 1] - cu[b] for b in reqs]
    cu_sub = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sel = torch.tensor(rows, dtype=torch.long)
    bsel = torch.tensor(reqs, dtype=torch.long)
    g = wl.g if wl.variant == W.LIGHTNING else wl.g[sel]
    beta = None if wl.beta is None else wl.beta[sel]
    kw = {}
    if wl.token_slots is not None:
        kw = dict(token_slots=wl.token_slots[bsel],
                  num_accepted=wl.num_accepted[bsel])
        ridx, widx = None, None
    else:
        ridx = wl.read_idx[bsel]
        widx = None if wl.write_idx is None else wl.write_idx[bsel]
    res = oracle.decode(VARIANT_CODE[wl.variant], wl.q[sel], wl.k[sel],
                        wl.v[sel], g, beta, wl.pool(), ridx, widx,
                        flags=_flags(wl), inter=wl.inter, factors=factors,
                        cu_seqlens=cu_sub, max_tokens=wl.T, **kw)
    res["reqs"], res["cu_sub"] = reqs, cu_sub
    return res


def _varlen_active(wl, b):
    """Whether request b of a varlen workload runs (is not padding)."""
    n = wl.counts()[b]
    if wl.token_slots is not None:
        na = int(wl.num_accepted[b])
        return 1 <= na <= n and int(wl.token_slots[b, na - 1]) >= 0
    return int(wl.read_idx[b]) >= 0


def check_varlen(wl, got, before):
    ref = oracle_run_varlen(wl)
    kind, tol_out, tol_state = _tol(wl)
    cu = wl.cu_seqlens.tolist()
    m = wl.stride_mult
    errs = {"out": 0.0, "state": 0.0, "inter": 0.0}
    assert not torch.isnan(got["out"].float()).any()
    for i, b in enumerate(ref["reqs"]):
        g0, g1 = cu[b], cu[b + 1]
        r0, r1 = ref["cu_sub"][i], ref["cu_sub"][i + 1]
        if g1 == g0:
            continue  # no tokens: only its state write is checked (below)
        errs["out"] = max(errs["out"], _err(kind, got["out"][g0:g1].float(),
                                            ref["out"][r0:r1]))
        if not _varlen_active(wl, b):
            assert not got["out"][g0:g1].float().any(), "padding outputs 0"
            if wl.inter:
                assert torch.isnan(got["inter"][g0:g1].float()).all(), \
                    "padded request must not touch the cache"
            continue
        if wl.inter:
            errs["inter"] = max(errs["inter"], _state_err(
                wl, kind, tol_state, got["inter"][g0:g1].float().numpy(),
                ref["inter"][r0:r1]))
    # every slot of the pool: the oracle ran on the whole pool
    errs["state"] = _state_err(wl, kind, tol_state,
                               got["backing"][::m].float().numpy(),
                               ref["pool"])
    bf = wl.backing.dtype == torch.bfloat16
    assert errs["out"] <= tol_out, errs
    assert errs["state"] <= (0.0 if bf else tol_state), errs
    assert errs["inter"] <= (0.0 if bf else tol_state), errs
    # bytewise: only the slots active requests write may change (a request
    # with no tokens still writes its state unchanged); the gaps between
    # logical slots never
    counts = wl.counts()
    written = set()
    for b in range(wl.B):
        if not _varlen_active(wl, b):
            continue
        if wl.token_slots is not None:
            written.update(m * s for s in wl.token_slots[b, :counts[b]].tolist()
                           if s >= 0)
        else:
            w = int((wl.write_idx if wl.write_idx is not None
                     else wl.read_idx)[b])
            if w >= 0:
                written.add(m * w)
    keep = torch.ones(got["backing"].shape[0], dtype=torch.bool)
    if written:
        keep[torch.tensor(sorted(written))] = False
    assert torch.equal(_bits(got["backing"][keep]), _bits(before[keep])), \
        "a slot that must not change did"
    print("  %s errors %s" % (wl.name, {k: "%.2e" % v
                                        for k, v in errs.items()}),
          flush=True)
    return ref


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
def test_varlen_parity(variant, K, V, dtype):
    """Variable-length batch with a zero-token request, a padded request,
    separate write slots (some skipped), strided pool and token cache."""
    seed = (4000 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant)
            + 10 * [(128, 128), (64, 128), (128, 64)].index((K, V))
            + (5 if dtype == torch.bfloat16 else 0))
    wl = W.make("varlen", variant, B=7, T=5, H=2, HV=4, K=K, V=V,
                pool_size=20, seed=seed, act_dtype=dtype, pool_std=0.1,
                stride_mult=2, separate_write=True, write_skip=0.3,
                inter=True, varlen_min=0)
    ridx = wl.read_idx.clone()
    ridx[3] = -1  # padded
    wl.read_idx = ridx
    before = wl.backing.clone()
    got = gpu_run_varlen(wl)
    check_varlen(wl, got, before)


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
def test_varlen_zero_and_full_length_requests(variant):
    """Explicit lengths 0, T, 1: a zero-token request copies its read state
    to its write slot; outputs of the others match the oracle."""
    wl = W.make("varlen0", variant, B=3, T=4, H=1, HV=2, K=128, V=128,
                pool_size=8, seed=4300 + len(variant), separate_write=True,
                inter=True)
    lengths = [0, 4, 1]
    cu = torch.tensor([0, 0, 4, 5], dtype=torch.int32)

    def pack(x):
        return torch.cat([x[b, :n] for b, n in enumerate(lengths)], 0)
    wl.q, wl.k, wl.v = pack(wl.q), pack(wl.k), pack(wl.v)
    if variant != W.LIGHTNING:
        wl.g, wl.beta = pack(wl.g), pack(wl.beta)
    wl.cu_seqlens = cu
    before = wl.backing.clone()
    got = gpu_run_varlen(wl)
    check_varlen(wl, got, before)
    r0, w0 = int(wl.read_idx[0]), int(wl.write_idx[0])
    assert torch.equal(_bits(got["backing"][w0]), _bits(before[r0]))


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16],
                         ids=["f32_state", "bf16_state"])
def test_varlen_batch_without_tokens(variant, state):
    """Every request has zero tokens (offsets all 0): the token-packed
    inputs, outputs and cache are empty tensors, whose NULL addresses the
    library accepts because nothing indexes them. Each active request copies
    its read state to its write slot bit for bit; the padded request and the
    skipped write touch nothing."""
    wl = W.make("varlen_empty", variant, B=4, T=3, H=1, HV=2, K=128, V=64,
                pool_size=12, seed=4350 + len(variant), separate_write=True,
                inter=True, state_dtype=state)
    wl.write_idx[2] = -1
    wl.read_idx[1] = -1
    empty = slice(0, 0)
    wl.q, wl.k, wl.v = wl.q[0, empty], wl.k[0, empty], wl.v[0, empty]
    if variant != W.LIGHTNING:
        wl.g, wl.beta = wl.g[0, empty], wl.beta[0, empty]
    wl.cu_seqlens = torch.zeros(wl.B + 1, dtype=torch.int32)
    assert wl.q.shape[0] == 0
    before = wl.backing.clone()
    got = gpu_run_varlen(wl)
    check_varlen(wl, got, before)
    for b in (0, 3):
        r, w = int(wl.read_idx[b]), int(wl.write_idx[b])
        assert torch.equal(_bits(got["backing"][w]), _bits(before[r]))


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
def test_varlen_equal_lengths_bit_identical_to_dense(variant):
    """Offsets 0, T, 2T, ... over token-packed inputs give the dense call's
    bits (same kernels, same arithmetic)."""
    wl = W.make("vdense", variant, B=5, T=3, H=2, HV=4, K=128, V=128,
                pool_size=12, seed=4400 + len(variant), separate_write=True,
                inter=True)
    dense = gpu_run(wl)
    B, T = wl.B, wl.T
    vl = dataclasses.replace(
        wl, q=wl.q.reshape((B * T,) + wl.q.shape[2:]),
        k=wl.k.reshape((B * T,) + wl.k.shape[2:]),
        v=wl.v.reshape((B * T,) + wl.v.shape[2:]),
        g=wl.g if variant == W.LIGHTNING else wl.g.reshape(
            (B * T,) + wl.g.shape[2:]),
        beta=None if wl.beta is None else wl.beta.reshape(B * T, wl.HV),
        cu_seqlens=torch.arange(0, B * T + 1, T, dtype=torch.int32))
    got = gpu_run_varlen(vl)
    assert torch.equal(_bits(got["out"].reshape(dense["out"].shape)),
                       _bits(dense["out"]))
    assert torch.equal(_bits(got["backing"]), _bits(dense["backing"]))
    assert torch.equal(_bits(got["inter"].reshape(dense["inter"].shape)),
                       _bits(dense["inter"]))


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
def test_varlen_paged_slots(variant):
    """Paged per-token slots over a variable-length batch: the accepted
    count is checked against each request's own token count."""
    wl = W.make("vpaged", variant, B=4, T=3, H=2, HV=2, K=128, V=128,
                pool_size=16, seed=4500 + len(variant), paged=True,
                inter=True, varlen_min=1)
    counts = wl.counts()
    acc = wl.num_accepted.clone()
    for b, n in enumerate(counts):
        acc[b] = min(int(acc[b]), n)
    acc[1] = counts[1] + 1  # beyond its own tokens: padding
    wl.num_accepted = acc
    before = wl.backing.clone()
    got = gpu_run_varlen(wl)
    check_varlen(wl, got, before)
    cu = wl.cu_seqlens.tolist()
    assert not got["out"][cu[1]:cu[2]].any()


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
def test_varlen_records_replay_equal_cache_bitwise(variant):
    """Records written by a varlen decode, replayed for n_b <= T_b tokens,
    rebuild the token cache's state bit for bit (fp32 pool)."""
    lad = _lad()
    wl = W.make("vrec", variant, B=6, T=4, H=2, HV=2, K=128, V=128,
                pool_size=14, seed=4600 + len(variant), separate_write=True,
                inter=True, varlen_min=0)
    got = gpu_run_varlen(wl, factors=True)
    counts = wl.counts()
    ntok = torch.tensor([min(c, 2) for c in counts], dtype=torch.int32)
    d = wl.to(DEV)  # a fresh copy of the pool as it was before the decode
    pool = d.backing[:: wl.stride_mult]
    lad.replay(got["factors"].to(DEV), pool, d.read_idx, d.write_idx,
               ntok.to(DEV), cu_seqlens=d.cu_seqlens, max_tokens=wl.T)
    torch.cuda.synchronize()
    after = d.backing.cpu()
    cu = wl.cu_seqlens.tolist()
    for b, n in enumerate(ntok.tolist()):
        w = int(wl.write_idx[b])
        if w < 0:
            continue
        want = (wl.backing[int(wl.read_idx[b])] if n == 0
                else got["inter"][cu[b] + n - 1])
        assert torch.equal(_bits(after[w]), _bits(want)), b
    ref = oracle_run_varlen(wl, factors=True)
    fac = got["factors"].double().numpy()
    assert np.isfinite(fac).all()
    # the records against the oracle's, part by part, at the tolerances of
    # the dense records test
    kind, tol_out, _ = _tol(wl)
    K = wl.K
    rf = ref["factors"]
    assert _err("rel", fac[..., :K], rf[..., :K]) <= 1e-5
    assert _err("rel", fac[..., K:2 * K], rf[..., K:2 * K]) <= (
        1e-5 if wl.q.dtype == torch.float32 else 1e-3)
    assert _err(kind, fac[..., 2 * K:], rf[..., 2 * K:]) <= tol_out


@pytest.mark.parametrize("cu,T,total,expect", [
    ([0, 2, 3, 6], 3, 6, 0),
    ([0, 2, 3, 7], 4, 6, 1),
    ([0, 4, 5, 6], 3, 6, 2),
    ([0, 3, 2, 6], 3, 6, 2),
    ([-1, 2, 3, 6], 3, 6, 1),
    ([0, 0, 0, 0], 1, 0, 0),
])
def test_check_cu_seqlens(cu, T, total, expect):
    lad = _lad()
    t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    assert int(lad.check_cu_seqlens(t, T, total).item()) == expect


def test_varlen_bad_offsets_skip_the_request():
    """A request whose offsets break the precondition is skipped entirely:
    its pool slots stay untouched and the other requests are unaffected."""
    lad = _lad()
    wl = W.make("vbad", W.GDN, B=3, T=2, H=1, HV=2, K=128, V=128,
                pool_size=8, seed=4700, separate_write=True, varlen_min=2)
    # request 2 claims tokens 4..6 of a 5-token buffer: past the end
    wl.q, wl.k, wl.v = wl.q[:5], wl.k[:5], wl.v[:5]
    wl.g, wl.beta = wl.g[:5], wl.beta[:5]
    cu_bad = torch.tensor([0, 2, 4, 6], dtype=torch.int32)
    d = wl.to(DEV)
    assert int(lad.check_cu_seqlens(cu_bad.to(DEV), 2, 5).item()) == 1
    pool = d.backing[:: wl.stride_mult]
    out = torch.full((5, wl.HV, wl.V), float("nan"), device=DEV)
    lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx,
                       d.write_idx, out=out, cu_seqlens=cu_bad.to(DEV),
                       max_tokens=2, l2norm_qk=True, beta_logit=True)
    torch.cuda.synchronize()
    after = d.backing.cpu()
    w2 = int(wl.write_idx[2])
    assert torch.equal(after[w2], wl.backing[w2])
    assert torch.isnan(out[4].cpu()).all()  # the skipped request's row
    good = dataclasses.replace(wl, B=2, read_idx=wl.read_idx[:2],
                               write_idx=wl.write_idx[:2], q=wl.q[:4],
                               k=wl.k[:4], v=wl.v[:4], g=wl.g[:4],
                               beta=wl.beta[:4],
                               cu_seqlens=torch.tensor([0, 2, 4],
                                                       dtype=torch.int32))
    ref = oracle_run_varlen(good)
    _, tol_out, _ = _tol(wl)
    assert _err("abs", out[:4].cpu().float(), ref["out"]) <= tol_out


def test_named_varlen_workload_parity():
    wl = W.named("gdn_varlen_b64_t4")
    before = wl.backing.clone()
    got = gpu_run_varlen(wl)
    check_varlen(wl, got, before)


# ------------------------------------------------ in-kernel gate chain


def _gate_inputs(variant, HV, K, seed):
    gen = torch.Generator().manual_seed(seed)
    a_log = torch.log(1 + 15 * torch.rand(HV, generator=gen))  # A in [1, 16]
    dt = torch.randn((HV,) if variant == W.GDN else (HV, K), generator=gen)
    return a_log.float(), dt.float()


def _gate_run(wl, a_log, dt, lower_bound):
    """GPU and oracle runs of a gated workload (wl.g holds raw gates)."""
    lad = _lad()
    d = wl.to(DEV)
    pool = d.backing[:: wl.stride_mult]
    fn = lad.gdn_decode_mtp if wl.variant == W.GDN else lad.kda_decode_mtp
    fac = torch.full((wl.B, wl.T, wl.HV, 2 * wl.K + wl.V), float("nan"),
                     device=DEV)
    out, inter = fn(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx,
                    d.write_idx, inter=wl.inter, l2norm_qk=wl.l2norm,
                    beta_logit=wl.beta_logit, factors=fac,
                    A_log=a_log.to(DEV), dt_bias=dt.to(DEV),
                    lower_bound=lower_bound)
    torch.cuda.synchronize()
    ref = oracle.decode(VARIANT_CODE[wl.variant], wl.q, wl.k, wl.v, wl.g,
                        wl.beta, wl.pool(), wl.read_idx, wl.write_idx,
                        flags=_flags(wl), inter=wl.inter, factors=True,
                        A_log=a_log, dt_bias=dt, lower_bound=lower_bound)
    return {"out": out.cpu(), "backing": d.backing.cpu(),
            "inter": None if inter is None else inter.cpu(),
            "factors": fac.cpu()}, ref


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
@pytest.mark.parametrize("lower_bound", [None, -5.0], ids=["softplus", "lb"])
@pytest.mark.parametrize("T,state", [(3, torch.float32), (1, torch.float32),
                                     (1, torch.bfloat16)],
                         ids=["t3", "t1", "t1_bf16_state"])
def test_gate_chain_parity(variant, lower_bound, T, state):
    """The in-kernel gate chain (this library's reading of the pages' A_log
    / dt_bias / lower_bound inputs) against the oracle's, with the raw gate
    ~ N(0, 2^2), A in [1, 16], dt_bias ~ N(0, 1); one bf16-state case runs
    the packed one-token kernel."""
    seed = 5000 + 10 * [W.GDN, W.KDA].index(variant) + T + (
        5 if lower_bound is None else 0) + (100 if state != torch.float32
                                           else 0)
    wl = W.make("gate", variant, B=5, T=T, H=2, HV=4, K=128, V=128,
                pool_size=12, seed=seed, separate_write=True,
                write_skip=0.2, inter=state == torch.float32,
                state_dtype=state)
    wl.g = 2 * torch.randn(wl.g.shape, generator=torch.Generator()
                           .manual_seed(seed + 1))
    a_log, dt = _gate_inputs(variant, wl.HV, wl.K, seed + 2)
    got, ref = _gate_run(wl, a_log, dt, lower_bound)
    kind, tol_out, tol_state = _tol(wl)
    assert _err(kind, got["out"].float(), ref["out"]) <= tol_out
    m = wl.stride_mult
    widx = wl.write_idx.tolist()
    for b, w in enumerate(widx):
        if w >= 0:
            err = _state_err(wl, kind, tol_state,
                             got["backing"][m * w].float().numpy(),
                             ref["pool"][w])
            assert err <= (0.0 if state != torch.float32 else tol_state), b
    if wl.inter:
        assert _err(kind, got["inter"].float(), ref["inter"]) <= tol_state
    # the decays themselves (record field a): fp32 exp/log vs fp64. A few
    # ulp of error in the log-decay g' become |g'| times that, relative, in
    # exp(g'); decays below fp32 range (exp(-128) at A = 16) flush to 0,
    # hence the floor
    a_gpu = got["factors"][..., :wl.K].double().numpy()
    a_ref = ref["factors"][..., :wl.K]
    bound = 1e-6 * (1 + np.abs(np.log(a_ref))) * a_ref + 1e-12
    assert np.all(np.abs(a_gpu - a_ref) <= bound)


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
@pytest.mark.parametrize("lower_bound", [None, -5.0], ids=["softplus", "lb"])
def test_gate_chain_general_kernel_32_rows(variant, lower_bound):
    """The gate chain in the general kernel at 32 rows per wave (a grid of
    1280 tiles, T = 2, no update records) against the oracle."""
    lad = _lad()
    seed = 5200 + 10 * [W.GDN, W.KDA].index(variant) + (
        5 if lower_bound is None else 0)
    HV = 32
    wl = W.make("gate32", variant, B=40, T=2, H=16 if variant == W.GDN
                else HV, HV=HV, K=128, V=128, pool_size=96, seed=seed,
                separate_write=True, write_skip=0.1)
    wl.g = 2 * torch.randn(wl.g.shape, generator=torch.Generator()
                           .manual_seed(seed + 1))
    a_log, dt = _gate_inputs(variant, HV, wl.K, seed + 2)
    d = wl.to(DEV)
    fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp
    kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit,
              A_log=a_log.to(DEV), dt_bias=dt.to(DEV),
              lower_bound=lower_bound)
    info = lad.kernel_info(variant, d.q, d.k, d.v, d.g, d.beta, d.pool(),
                           d.read_idx, d.write_idx, **kw)
    assert info["kernel"] == "decode_kernel" and info["block_threads"] == 256
    out, _ = fn(d.q, d.k, d.v, d.g, d.beta, d.pool(), d.read_idx,
                d.write_idx, **kw)
    torch.cuda.synchronize()
    ref = oracle.decode(VARIANT_CODE[variant], wl.q, wl.k, wl.v, wl.g,
                        wl.beta, wl.pool(), wl.read_idx, wl.write_idx,
                        flags=_flags(wl), A_log=a_log, dt_bias=dt,
                        lower_bound=lower_bound)
    kind, tol_out, tol_state = _tol(wl)
    assert _err(kind, out.cpu().float(), ref["out"]) <= tol_out
    backing = d.backing.cpu()
    for b, w in enumerate(wl.write_idx.tolist()):
        if w >= 0:
            assert _err(kind, backing[w].float(), ref["pool"][w]) <= \
                tol_state, b


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
def test_gate_chain_closed_form_on_gpu(variant):
    """x + dt_bias = 0 with A_log = 0: every decay is 1/2 (softplus(0) =
    ln 2); in the bounded form exp(lb / 2) for any A_log."""
    wl = W.make("gatecf", variant, B=3, T=2, H=1, HV=2, K=128, V=128,
                pool_size=6, seed=5100 + len(variant))
    a_log, dt = _gate_inputs(variant, wl.HV, wl.K, 5101)
    raw = -dt.expand(wl.g.shape) if variant == W.KDA else \
        -dt.view(1, 1, -1).expand(wl.g.shape)
    wl.g = raw.contiguous()
    got, _ = _gate_run(wl, torch.zeros_like(a_log), dt, None)
    np.testing.assert_allclose(got["factors"][..., :wl.K].numpy(), 0.5,
                               rtol=2e-6)
    got, _ = _gate_run(wl, a_log, dt, -3.0)
    np.testing.assert_allclose(got["factors"][..., :wl.K].numpy(),
                               np.exp(-1.5), rtol=2e-6)


# --------------------------------------------- untouched-slot sentinels


def _fill_sentinels(wl):
    """Overwrite every backing slot that no active request reads or writes
    (stride gaps included) with NaN bit patterns carrying payloads, so that
    any stray read-modify-write (which would canonicalise or recompute them)
    changes bits."""
    m = wl.stride_mult
    ridx = wl.read_idx.tolist()
    widx = (wl.write_idx if wl.write_idx is not None else wl.read_idx).tolist()
    used = {m * r for r in ridx if r >= 0}
    used |= {m * w for r, w in zip(ridx, widx) if r >= 0 and w >= 0}
    bits = _bits(wl.backing)  # int32 or int16 view, shares storage
    if wl.backing.dtype == torch.float32:
        pats = torch.tensor([0x7FA5A5A5, -0x003F4111, 0x7F800001,
                             -0x00000001], dtype=torch.int32)
    else:
        pats = torch.tensor([0x7FA5, -0x007F, 0x7F81, -0x0001],
                            dtype=torch.int16)
    flat_n = bits[0].numel()
    pattern = pats.repeat(flat_n // 4 + 1)[:flat_n].view(bits.shape[1:])
    filled = []
    for s in range(bits.shape[0]):
        if s not in used:
            bits[s] = pattern
            filled.append(s)
    return filled


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16],
                         ids=["f32state", "bf16state"])
@pytest.mark.parametrize("T", [1, 3])
def test_untouched_slots_keep_nan_payload_sentinels(variant, state, T):
    wl = W.make("sentinel", variant, B=5, T=T, H=2, HV=2, K=128, V=128,
                pool_size=14, seed=5200 + 10 * T + len(variant)
                + (7 if state == torch.bfloat16 else 0), stride_mult=2,
                read_idx=[3, -1, 9, 0, 12], write_idx=[5, 7, -1, 0, 1],
                inter=True, state_dtype=state)
    filled = _fill_sentinels(wl)
    assert len(filled) > wl.pool_size  # gaps and unused logical slots
    snapshot = _bits(wl.backing).clone()
    got = run_and_check(wl)  # parity, plus the bytewise check of every slot
    after = _bits(got["backing"])
    for s in filled:
        assert torch.equal(after[s], snapshot[s]), s


# ------------------------------------------------------- HIP graph capture


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
def test_hip_graph_capture_replays_match_eager(variant):
    """A decode captured in a HIP graph and replayed four times (with eager
    work and synchronisation between replays) reproduces the eager call bit
    for bit: the call launches one kernel and allocates, clears and
    synchronises nothing. Read and write slots are disjoint, so every replay
    starts from the same states."""
    lad = _lad()
    wl = W.make("graph", variant, B=4, T=3, H=2, HV=4, K=128, V=128,
                pool_size=12, seed=5300 + len(variant), separate_write=True,
                inter=True)
    d = wl.to(DEV)
    pool = d.backing[:: wl.stride_mult]
    fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp
    kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)
    out = torch.empty((wl.B, wl.T, wl.HV, wl.V), device=DEV)
    inter = torch.empty((wl.B, wl.T, wl.HV, wl.V, wl.K), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream
        fn(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx, d.write_idx,
           out=out, inter=inter, **kw)
    torch.cuda.synchronize()
    eager = (out.clone(), inter.clone(), d.backing.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx, d.write_idx,
           out=out, inter=inter, **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        inter.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(eager[0])), rep
        assert torch.equal(_bits(inter), _bits(eager[1])), rep
        assert torch.equal(_bits(d.backing), _bits(eager[2])), rep


# ------- one-token kernel (fp32 pools beyond 1024 tiles, bf16 beyond one packed round)


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("dtype,out", [(torch.float32, torch.float32),
                                       (torch.bfloat16, torch.float32),
                                       (torch.bfloat16, torch.bfloat16)],
                         ids=["f32", "bf16", "bf16_out_bf16"])
def test_one_token_kernel_parity(variant, K, V, dtype, out):
    """T = 1, fp32 pool, B * HV = 2048 tiles at K = V = 128 and 4096 at the
    other shapes: the contiguous-row one-token kernel (4 workgroups per
    tile). Padded requests, separate and skipped writes on a strided pool;
    every request against the oracle, every untouched byte checked."""
    seed = (6000 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant)
            + 10 * SHAPES.index((K, V)) + (5 if dtype != torch.float32 else 0)
            + (2 if out != torch.float32 else 0))
    B, HV = (64 if (K, V) == (128, 128) else 128), 32
    ridx = list(range(0, 2 * B, 2))
    widx = [s + 1 for s in ridx]
    for b in (3, 17, 40):
        ridx[b] = -1  # padded
    for b in (5, 22, 63):
        widx[b] = -1  # skipped write
    wl = W.make("one", variant, B=B, T=1, H=16, HV=HV, K=K, V=V,
                pool_size=2 * B, seed=seed, act_dtype=dtype, pool_std=0.1,
                stride_mult=2 if K == V else 1, read_idx=ridx,
                write_idx=widx, out_dtype=out)
    assert _kernel_name(wl) == "decode1_kernel"
    run_and_check(wl)


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
def test_one_token_kernel_gate_chain(variant):
    """The gate chain (both forms) in the one-token kernel (a call without
    update records, which would take the general kernel)."""
    lad = _lad()
    seed = 6300 + 10 * [W.GDN, W.KDA].index(variant)
    wl = W.make("onegate", variant, B=64, T=1, H=16, HV=32, K=128, V=128,
                pool_size=128, seed=seed, separate_write=True)
    wl.g = 2 * torch.randn(wl.g.shape, generator=torch.Generator()
                           .manual_seed(seed + 1))
    a_log, dt = _gate_inputs(variant, wl.HV, wl.K, seed + 2)
    fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp
    for lb in (None, -5.0):
        d = wl.to(DEV)
        kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit,
                  A_log=a_log.to(DEV), dt_bias=dt.to(DEV), lower_bound=lb)
        info = lad.kernel_info(variant, d.q, d.k, d.v, d.g, d.beta,
                               d.pool(), d.read_idx, d.write_idx, **kw)
        assert info["kernel"] == "decode1_kernel"
        out, _ = fn(d.q, d.k, d.v, d.g, d.beta, d.pool(), d.read_idx,
                    d.write_idx, **kw)
        torch.cuda.synchronize()
        ref = oracle.decode(VARIANT_CODE[variant], wl.q, wl.k, wl.v, wl.g,
                            wl.beta, wl.pool(), wl.read_idx, wl.write_idx,
                            flags=_flags(wl), A_log=a_log, dt_bias=dt,
                            lower_bound=lb)
        kind, tol_out, tol_state = _tol(wl)
        assert _err(kind, out.cpu().float(), ref["out"]) <= tol_out
        got = d.backing.cpu()
        for b, w in enumerate(wl.write_idx.tolist()):
            if w >= 0:
                assert _err(kind, got[w].float(), ref["pool"][w]) <= \
                    tol_state, b


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
def test_one_token_kernel_token_split_bit_identical(variant, dtype):
    """T single-token calls of 2048 tiles (one-token kernel) chained through
    the pool = one T-token call (decode_kernel), bit for bit: the two
    kernels perform the same operations in the same order."""
    lad = _lad()
    T = 3
    wl = W.make("onesplit", variant, B=64, T=T, H=16, HV=32, K=128, V=128,
                pool_size=64, seed=6400 + len(variant) + T * (dtype ==
                                                              torch.bfloat16),
                act_dtype=dtype)
    step = dataclasses.replace(wl, T=1, q=wl.q[:, :1], k=wl.k[:, :1],
                               v=wl.v[:, :1],
                               g=wl.g if variant == W.LIGHTNING
                               else wl.g[:, :1],
                               beta=None if wl.beta is None else wl.beta[:, :1])
    assert _kernel_name(step) == "decode1_kernel"
    whole = gpu_run(wl)
    d = wl.to(DEV)
    pool = d.backing
    outs = []
    for t in range(T):
        sl = slice(t, t + 1)
        if variant == W.LIGHTNING:
            o, _ = lad.la_decode(d.q[:, sl], d.k[:, sl], d.v[:, sl], pool,
                                 d.read_idx, lam=d.g)
        else:
            fn = (lad.gdn_decode_mtp if variant == W.GDN
                  else lad.kda_decode_mtp)
            o, _ = fn(d.q[:, sl], d.k[:, sl], d.v[:, sl], d.g[:, sl],
                      d.beta[:, sl], pool, d.read_idx, l2norm_qk=wl.l2norm,
                      beta_logit=wl.beta_logit)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch.cat(outs, 1).cpu()), _bits(whole["out"]))
    assert torch.equal(_bits(pool.cpu()), _bits(whole["backing"]))


def _kernel_name(wl):
    """The kernel la_decode_kernel_info names for wl's call."""
    lad = _lad()
    d = wl.to(DEV)
    kw = {}
    if wl.variant != W.LIGHTNING:
        kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)
    return lad.kernel_info(wl.variant, d.q, d.k, d.v, d.g, d.beta, d.pool(),
                           d.read_idx, d.write_idx, **kw)["kernel"]


def _one_token_batch_invariance(wl, sub=8, **kw):
    """Outputs and pool of one call over wl's whole batch, and of the same
    requests in calls of `sub` requests on a second copy of the pool."""
    lad = _lad()
    d = wl.to(DEV)
    pools = [d.backing.clone(), d.backing.clone()]
    results = []
    for pool, step in zip(pools, (wl.B, sub)):
        outs = []
        for s in range(0, wl.B, step):
            sl = slice(s, s + step)
            if wl.variant == W.LIGHTNING:
                o, _ = lad.la_decode(d.q[sl], d.k[sl], d.v[sl], pool,
                                     d.read_idx[sl], d.write_idx[sl],
                                     lam=d.g)
            else:
                fn = (lad.gdn_decode_mtp if wl.variant == W.GDN
                      else lad.kda_decode_mtp)
                o, _ = fn(
                    d.q[sl], d.k[sl], d.v[sl], d.g[sl], d.beta[sl], pool,
                    d.read_idx[sl], d.write_idx[sl], l2norm_qk=wl.l2norm,
                    beta_logit=wl.beta_logit, **kw)
            outs.append(o)
        torch.cuda.synchronize()
        results.append((torch.cat(outs).cpu(), pool.cpu()))
    return results


@pytest.mark.parametrize("variant,raw", [(W.LIGHTNING, False), (W.GDN, False),
                                         (W.GDN, True), (W.KDA, False)],
                         ids=["lightning", "gdn", "gdn_raw", "kda"])
@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16],
                         ids=["f32_state", "bf16_state"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
def test_one_token_kernel_batch_invariant(variant, raw, K, V, state, dtype):
    """The same requests in one call of 2304 tiles (one-token kernel; 4352
    for an fp32 pool at the shapes other than K = V = 128) and in calls of
    8 requests (256 tiles: decode_kernel, or the packed kernel on a bf16
    pool) give the same bits, outputs and stored states; `raw` passes q, k
    without l2norm and beta without the sigmoid."""
    B, HV = 72, 32
    if state == torch.float32 and (K, V) != (128, 128):
        B = 136
    seed = (6700 + 10 * SHAPES.index((K, V)) + (1 if raw else 0)
            + (2 if state != torch.float32 else 0)
            + (4 if dtype != torch.float32 else 0)
            + (100 if variant == W.GDN else 0)
            + (200 if variant == W.KDA else 0))
    wl = W.make("inv", variant, B=B, T=1, H=16, HV=HV, K=K, V=V,
                pool_size=2 * B, seed=seed, act_dtype=dtype, pool_std=0.1,
                separate_write=True, state_dtype=state,
                l2norm=not raw, beta_logit=not raw)
    if raw:  # small raw keys keep the delta rule contractive
        wl.q = (wl.q.float() / K ** 0.5).to(dtype)
        wl.k = (wl.k.float() / K ** 0.5).to(dtype)
        wl.beta = torch.rand(wl.beta.shape, generator=torch.Generator()
                             .manual_seed(seed))
    assert _kernel_name(wl) == "decode1_kernel"
    (wo, wp), (so, sp) = _one_token_batch_invariance(wl)
    assert torch.isfinite(wo).all()
    assert torch.equal(_bits(wo), _bits(so))
    assert torch.equal(_bits(wp), _bits(sp))


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
@pytest.mark.parametrize("lower_bound", [None, -5.0], ids=["softplus", "lb"])
def test_one_token_kernel_batch_invariant_gate_chain(variant, lower_bound):
    """Batch invariance across the one-token kernel's grid threshold with
    the in-kernel gate chain."""
    seed = 6900 + 10 * [W.GDN, W.KDA].index(variant)
    wl = W.make("invgate", variant, B=72, T=1, H=16, HV=32, K=128, V=128,
                pool_size=144, seed=seed, separate_write=True)
    wl.g = 2 * torch.randn(wl.g.shape, generator=torch.Generator()
                           .manual_seed(seed + 1))
    a_log, dt = _gate_inputs(variant, wl.HV, wl.K, seed + 2)
    (wo, wp), (so, sp) = _one_token_batch_invariance(
        wl, A_log=a_log.to(DEV), dt_bias=dt.to(DEV), lower_bound=lower_bound)
    assert torch.equal(_bits(wo), _bits(so))
    assert torch.equal(_bits(wp), _bits(sp))


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("K,V", SHAPES)
def test_one_token_kernel_bf16_state(variant, K, V):
    """The one-token kernel on a bf16 pool (2304 tiles; at 2048 and below a
    bf16 pool takes the packed kernel): states widened to fp32, rounded once
    to nearest even on store; padded and skipped-write requests; sampled
    against the oracle, every untouched byte checked."""
    seed = 6500 + 100 * [W.LIGHTNING, W.GDN, W.KDA].index(variant) + \
        10 * SHAPES.index((K, V))
    B = 72
    ridx = list(range(0, 2 * B, 2))
    widx = [s + 1 for s in ridx]
    ridx[9] = -1
    widx[30] = -1
    wl = W.make("onebf", variant, B=B, T=1, H=16, HV=32, K=K, V=V,
                pool_size=2 * B, seed=seed, pool_std=0.1, read_idx=ridx,
                write_idx=widx, state_dtype=torch.bfloat16)
    assert _kernel_name(wl) == "decode1_kernel"
    run_and_check(wl)


@pytest.mark.parametrize("variant,B,T,H,HV,K,kernel", [
    # one range per XCD, 3 pairs past them
    (W.GDN, 67, 1, 5, 25, 64, "decode_kernel"),
    # 32-pair blocks, 48 pairs past them (816 tiles: below the one-token
    # kernel's threshold)
    (W.LIGHTNING, 17, 1, 48, 48, 128, "decode_kernel"),
    # 2079 pairs in the one-token kernel: 8316 workgroups (4 per tile),
    # blocks of 4 whole tiles (16 workgroups) dealt to the XCDs in turn, 124
    # workgroups past the last whole round of blocks
    (W.GDN, 63, 1, 11, 33, 128, "decode1_kernel"),
    # dense KDA with more than four tokens: the plain order (1080 pairs)
    (W.KDA, 45, 8, 24, 24, 128, "decode_kernel"),
], ids=["ranges_gdn", "blocks_lightning", "ranges_one_token", "plain_kda_t8"])
def test_xcd_block_order_covers_every_pair(variant, B, T, H, HV, K, kernel):
    """Workgroups take their pairs in XCD blocks (general kernel: whole
    ranges below 48 value heads, 32-pair blocks from 48, the plain order for
    dense KDA calls of more than four tokens without per-token writes; split
    one-token kernel: blocks of four whole tiles) with the workgroups past
    the last whole round in plain order: every request's outputs and stored
    state match the oracle, and nothing else in the pool changes."""
    wl = W.make("xcd", variant, B=B, T=T, H=H, HV=HV, K=K, V=K,
                pool_size=2 * B + 1, seed=9900 + B, separate_write=True,
                act_dtype=torch.float32, l2norm=variant != W.LIGHTNING)
    assert _kernel_name(wl) == kernel
    run_and_check(wl)


# ------------------------------------------------ small-grid instance


@pytest.mark.parametrize("variant", [W.LIGHTNING, W.GDN, W.KDA])
@pytest.mark.parametrize("T,state", [(1, torch.float32), (4, torch.float32),
                                     (4, torch.bfloat16)],
                         ids=["t1_f32_state", "t4_f32_state", "t4_bf16_state"])
def test_small_grid_instance_bit_identical(variant, T, state):
    """Grids of at most 512 tiles (V = 128) run the general kernel at 16
    rows per wave, larger ones at 32. The same requests give the same bits
    in a call of 1280 tiles and in calls of 512 tiles; padded and
    skipped-write requests included. (One bf16 token runs the packed kernel
    at these sizes.)"""
    lad = _lad()
    B, HV = 40, 32
    H = HV // 2 if variant == W.GDN else HV
    seed = 8100 + 10 * T + [W.LIGHTNING, W.GDN, W.KDA].index(variant) + \
        (5 if state != torch.float32 else 0)
    ridx = torch.randperm(2 * B, generator=torch.Generator()
                          .manual_seed(seed))[:B].tolist()
    ridx[7] = -1
    wl = W.make("small", variant, B=B, T=T, H=H, HV=HV, K=128, V=128,
                pool_size=3 * B, seed=seed, separate_write=True,
                write_skip=0.1, read_idx=ridx, state_dtype=state,
                l2norm=variant != W.LIGHTNING)
    d = wl.to(DEV)
    kw = {}
    if variant != W.LIGHTNING:
        kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)

    def call(pool, sl):
        if variant == W.LIGHTNING:
            return lad.la_decode(d.q[sl], d.k[sl], d.v[sl], pool,
                                 d.read_idx[sl], d.write_idx[sl], lam=d.g)[0]
        fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp
        return fn(d.q[sl], d.k[sl], d.v[sl], d.g[sl], d.beta[sl], pool,
                  d.read_idx[sl], d.write_idx[sl], **kw)[0]

    def threads(sl):
        g = d.g if variant == W.LIGHTNING else d.g[sl]
        beta = None if d.beta is None else d.beta[sl]
        return lad.kernel_info(variant, d.q[sl], d.k[sl], d.v[sl], g, beta,
                               d.pool(), d.read_idx[sl], d.write_idx[sl],
                               **kw)["block_threads"]
    assert threads(slice(0, B)) == 256 and threads(slice(0, 16)) == 512
    whole_pool = d.backing.clone()
    whole = call(whole_pool, slice(0, B))
    part_pool = d.backing.clone()
    parts = torch.cat([call(part_pool, slice(s, min(s + 16, B)))
                       for s in range(0, B, 16)])
    torch.cuda.synchronize()
    assert torch.isfinite(whole.float()).all()
    assert torch.equal(_bits(whole.cpu()), _bits(parts.cpu()))
    assert torch.equal(_bits(whole_pool.cpu()), _bits(part_pool.cpu()))
    run_and_check(wl)


# ------------------------------------------------------------ kernel query


@pytest.mark.parametrize("case", [
    # (variant, B, T, HV, state dtype, expected kernel, threads, cache,
    #  tokens per LDS round)
    # one token: the one-token kernel (4 workgroups of 64 threads per tile
    # row group: 256 threads) on fp32 pools at K = V = 128 beyond 1024
    # tiles, or from 1024 tiles with 48 or more value heads; on bf16 pools
    # beyond 2048 tiles, 1536 for KDA (the packed kernel up to there)
    ("gdn", 64, 1, 32, torch.float32, "decode1_kernel", 256, False, 0),
    ("lightning", 33, 1, 64, torch.float32, "decode1_kernel", 256, False, 0),
    ("kda", 96, 1, 24, torch.float32, "decode1_kernel", 256, False, 0),
    ("gdn", 128, 1, 16, torch.float32, "decode1_kernel", 256, False, 0),
    ("lightning", 96, 1, 24, torch.float32, "decode1_kernel", 256, False, 0),
    ("gdn", 136, 1, 32, torch.float32, "decode1_kernel", 256, False, 0),
    ("gdn", 96, 1, 48, torch.float32, "decode1_kernel", 256, False, 0),
    ("lightning", 16, 1, 64, torch.float32, "decode1_kernel", 256, False, 0),
    ("lightning", 15, 1, 64, torch.float32, "decode_kernel", 256, False, 8),
    ("gdn", 32, 1, 32, torch.float32, "decode_kernel", 256, False, 8),
    ("gdn", 33, 1, 32, torch.float32, "decode1_kernel", 256, False, 0),
    ("kda", 43, 1, 24, torch.float32, "decode1_kernel", 256, False, 0),
    ("kda", 42, 1, 24, torch.float32, "decode_kernel", 256, False, 8),
    ("gdn", 8, 1, 32, torch.float32, "decode_kernel", 512, False, 8),
    ("kda", 21, 1, 24, torch.float32, "decode_kernel", 512, False, 8),
    ("kda", 22, 1, 24, torch.float32, "decode_kernel", 256, False, 8),
    ("gdn", 64, 1, 32, torch.bfloat16, "decode_packed_kernel", 128, False, 1),
    ("kda", 8, 1, 24, torch.bfloat16, "decode_packed_kernel", 128, False, 1),
    ("kda", 64, 1, 24, torch.bfloat16, "decode_packed_kernel", 128, False, 1),
    ("kda", 65, 1, 24, torch.bfloat16, "decode1_kernel", 256, False, 0),
    ("gdn", 72, 1, 32, torch.bfloat16, "decode1_kernel", 256, False, 0),
    ("kda", 128, 1, 24, torch.bfloat16, "decode1_kernel", 256, False, 0),
    ("gdn", 136, 1, 16, torch.bfloat16, "decode1_kernel", 256, False, 0),
    # several tokens: the general kernel
    ("gdn", 16, 4, 32, torch.float32, "decode_kernel", 512, False, 8),
    ("gdn", 17, 4, 32, torch.float32, "decode_kernel", 256, False, 8),
    # tokens per LDS round: four for KDA beyond four tokens on 32-row grids
    # (a partial last round at T = 5..7), two on 32-row grids that cache
    # every token, eight on small grids and otherwise
    ("kda", 96, 8, 24, torch.float32, "decode_kernel", 256, False, 4),
    ("kda", 96, 6, 24, torch.float32, "decode_kernel", 256, False, 4),
    ("kda", 96, 4, 24, torch.float32, "decode_kernel", 256, False, 8),
    ("kda", 16, 8, 24, torch.float32, "decode_kernel", 512, False, 8),
    ("gdn", 32, 4, 32, torch.float32, "decode_kernel", 256, True, 2),
    ("gdn", 16, 4, 32, torch.float32, "decode_kernel", 512, True, 8),
    ("kda", 64, 4, 24, torch.float32, "decode_kernel", 256, True, 2),
], ids=lambda c: "%s_b%d_t%d_hv%d_%s%s" % (c[0], c[1], c[2], c[3],
                                          str(c[4])[6:],
                                          "_cache" if c[7] else ""))
def test_kernel_info_reports_the_dispatch(case):
    """la_decode_kernel_info names the kernel the call runs, with a launch
    shape that matches the dispatch rule and a plausible register budget;
    the call itself then runs and matches the oracle."""
    variant, B, T, HV, state, kernel, threads, cache, ch = case
    lad = _lad()
    wl = W.make("info", variant, B=B, T=T, H=HV // 2 if variant == "gdn"
                else HV, HV=HV, K=128, V=128, pool_size=2 * B, seed=7100 + B,
                separate_write=True, state_dtype=state, inter=cache,
                l2norm=variant != W.LIGHTNING)
    d = wl.to(DEV)
    kw = {}
    if variant != W.LIGHTNING:
        kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)
    inter = (torch.empty((B, T, HV, 128, 128), dtype=state, device=DEV)
             if cache else None)
    info = lad.kernel_info(variant, d.q, d.k, d.v, d.g, d.beta, d.pool(),
                           d.read_idx, d.write_idx, inter=inter, **kw)
    assert info["kernel"] == kernel
    # the one-token kernel runs each tile as 4 workgroups of 4 waves
    assert info["grid_blocks"] == B * HV * (4 if kernel == "decode1_kernel"
                                            else 1)
    assert info["block_threads"] == threads
    assert info["scratch_bytes"] == 0
    assert 0 < info["vgprs"] <= 512
    assert info["blocks_per_cu"] >= 1
    assert info["waves_per_simd"] == info["blocks_per_cu"] * threads // 64 // 4
    assert info["tokens_per_round"] == ch
    per_token = (3 if variant == "kda" else 2) * 128 + 128 + 4
    # 32-row instances without per-token writes on an fp32 pool also stage
    # their final write-back: 8 rows of 132 floats per wave
    stage = (threads // 64) * 8 * 132 if (
        kernel == "decode_kernel" and threads == 256 and ch != 2
        and state == torch.float32) else 0
    assert info["lds_bytes"] == (min(T, ch) * per_token + stage) * 4
    if kernel == "decode1_kernel":
        assert info["lds_bytes"] == 0 and info["waves_per_simd"] == 8
    if kernel == "decode_kernel":
        assert info["waves_per_simd"] >= 3
    run_and_check(wl)


@pytest.mark.parametrize("T", [5, 6, 7])
def test_kda_partial_last_round(T):
    """KDA beyond four tokens on a 32-row grid stages four tokens per LDS
    round, so T = 5..7 ends on a partial round: every request against the
    oracle, with a padded request and skipped writes."""
    B, HV = 48, 24
    ridx = torch.randperm(3 * B, generator=torch.Generator()
                          .manual_seed(7400 + T))[:B].tolist()
    ridx[5] = -1
    wl = W.make("kda_partial", W.KDA, B=B, T=T, H=HV, HV=HV, K=128, V=128,
                pool_size=3 * B, seed=7400 + T, read_idx=ridx,
                separate_write=True, write_skip=0.2)
    d = wl.to(DEV)
    info = _lad().kernel_info("kda", d.q, d.k, d.v, d.g, d.beta, d.pool(),
                              d.read_idx, d.write_idx, l2norm_qk=True,
                              beta_logit=True)
    assert info["block_threads"] == 256 and info["tokens_per_round"] == 4
    run_and_check(wl)


def test_varlen_kda_32_row_grid():
    """A variable-length KDA batch of 960 tiles (32 rows per wave, four
    tokens per LDS round): requests of 0..8 tokens end on every partial
    round; every request and slot against the oracle."""
    wl = W.make("vkda", W.KDA, B=40, T=8, H=24, HV=24, K=128, V=128,
                pool_size=96, seed=7450, separate_write=True,
                write_skip=0.2, varlen_min=0)
    d = wl.to(DEV)
    total = wl.q.shape[0]
    info = _lad().kernel_info("kda", d.q, d.k, d.v, d.g, d.beta, d.pool(),
                              d.read_idx, d.write_idx, l2norm_qk=True,
                              beta_logit=True, cu_seqlens=d.cu_seqlens,
                              max_tokens=wl.T)
    assert info["block_threads"] == 256 and info["tokens_per_round"] == 4
    assert total > 0
    before = wl.backing.clone()
    got = gpu_run_varlen(wl)
    check_varlen(wl, got, before)


def test_kernel_info_empty_batch():
    lad = _lad()
    wl = W.make("info0", W.GDN, B=2, T=1, H=2, HV=4, K=128, V=128,
                pool_size=4, seed=7199)
    d = wl.to(DEV)
    info = lad.kernel_info("gdn", d.q[:0], d.k[:0], d.v[:0], d.g[:0],
                           d.beta[:0], d.pool(), d.read_idx[:0])
    assert info["kernel"] == "none" and info["grid_blocks"] == 0


# ------------------------------------- pools with padded rows and heads

# NaN payloads that no kernel result equals
_SENTINEL = {torch.float32: 0x7FC0DEAD, torch.bfloat16: 0x7F81}


def _padded_pool(wl, row_pad, head_pad):
    """A device buffer [P, HV + head_pad, V, K + row_pad] filled with a
    NaN-payload sentinel whose [:, :HV, :, :K] view holds the workload's
    pool: row and head strides larger than the tile, gaps in between."""
    P, HV, V, K = wl.backing.shape
    big = torch.empty((P, HV + head_pad, V, K + row_pad),
                      dtype=wl.backing.dtype, device=DEV)
    _bits(big).fill_(_SENTINEL[wl.backing.dtype])
    big[:, :HV, :, :K] = wl.backing.to(DEV)
    return big, big[:, :HV, :, :K]


def _check_padding(wl, big, row_pad, head_pad):
    HV, K = wl.HV, wl.K
    s = _SENTINEL[wl.backing.dtype]
    b = _bits(big.cpu())
    if row_pad:
        assert bool((b[:, :HV, :, K:] == s).all()), "row padding changed"
    if head_pad:
        assert bool((b[:, HV:] == s).all()), "head padding changed"


PADDED_CASES = {
    # general kernel, three tokens with the per-token cache
    "general_gdn_t3": dict(variant=W.GDN, B=5, T=3, H=2, HV=4, K=128, V=128,
                           pool_size=12, inter=True, pads=(4, 1)),
    "general_kda_t1_v64": dict(variant=W.KDA, B=8, T=1, H=4, HV=4, K=128,
                               V=64, pool_size=16, pads=(4, 1)),
    # 32-row instances whose final write-back goes through LDS: rows of the
    # padded pool are K + pad floats apart
    "general_staged_gdn_t2": dict(variant=W.GDN, B=40, T=2, H=8, HV=16,
                                  K=128, V=128, pool_size=88, pads=(4, 1)),
    "general_staged_kda_t6": dict(variant=W.KDA, B=24, T=6, H=24, HV=24,
                                  K=128, V=128, pool_size=52, pads=(8, 1)),
    # one-token kernel (fp32: beyond 1024 tiles at K = V = 128, the split
    # form; from 4096 tiles at the other shapes, one workgroup per tile)
    "one_token_gdn": dict(variant=W.GDN, B=64, T=1, H=16, HV=32, K=128,
                          V=128, pool_size=128, pads=(4, 1)),
    "one_token_lightning_k64": dict(variant=W.LIGHTNING, B=128, T=1, H=32,
                                    HV=32, K=64, V=128, pool_size=256,
                                    pads=(8, 0)),
    # bf16 pools: packed kernel, one-token kernel, general kernel
    "packed_bf16_lightning": dict(variant=W.LIGHTNING, B=8, T=1, H=4, HV=4,
                                  K=128, V=128, pool_size=16, pads=(8, 1),
                                  state_dtype=torch.bfloat16),
    "one_token_bf16_gdn": dict(variant=W.GDN, B=72, T=1, H=16, HV=32, K=128,
                               V=128, pool_size=144, pads=(8, 1),
                               state_dtype=torch.bfloat16),
    "general_bf16_kda_t2": dict(variant=W.KDA, B=6, T=2, H=2, HV=2, K=128,
                                V=128, pool_size=12, pads=(16, 1),
                                state_dtype=torch.bfloat16),
}


@pytest.mark.parametrize("name", sorted(PADDED_CASES))
def test_padded_rows_and_heads(name):
    """Pools whose rows and heads are padded (row stride K + pad, head
    stride with a gap): every kernel path agrees with the oracle, writes
    only the write slots' tiles, and leaves every padding element's bits
    as they were."""
    case = dict(PADDED_CASES[name])
    row_pad, head_pad = case.pop("pads")
    variant = case.pop("variant")
    seed = 7300 + sorted(PADDED_CASES).index(name)
    wl = W.make("padded_" + name, variant, seed=seed, separate_write=True,
                write_skip=0.2, l2norm=variant != W.LIGHTNING, **case)
    # the case's name says which kernel it is for
    assert _kernel_name(wl) == ("decode1_kernel" if name.startswith("one_")
                                else "decode_packed_kernel"
                                if name.startswith("packed_")
                                else "decode_kernel"), name
    lad = _lad()
    d = wl.to(DEV)
    if "_staged_" in name:  # 32 rows per wave and the write-back's LDS area
        kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)
        info = lad.kernel_info(variant, d.q, d.k, d.v, d.g, d.beta, d.pool(),
                               d.read_idx, d.write_idx, **kw)
        assert info["block_threads"] == 256, info
        assert info["lds_bytes"] >= 4 * 8 * 132 * 4, info
    big, pool = _padded_pool(wl, row_pad, head_pad)
    assert pool.stride(2) == wl.K + row_pad
    inter = None
    if wl.inter:
        inter = torch.full((wl.B, wl.T, wl.HV, wl.V, wl.K), float("nan"),
                           dtype=wl.backing.dtype, device=DEV)
    if variant == W.LIGHTNING:
        out, _ = lad.la_decode(d.q, d.k, d.v, pool, d.read_idx, d.write_idx,
                               lam=d.g, inter=inter)
    else:
        fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp
        out, _ = fn(d.q, d.k, d.v, d.g, d.beta, pool, d.read_idx,
                    d.write_idx, inter=inter, l2norm_qk=wl.l2norm,
                    beta_logit=wl.beta_logit)
    torch.cuda.synchronize()
    got = {"out": out.cpu(), "backing": pool.contiguous().cpu(),
           "inter": None if inter is None else inter.cpu()}
    errs = check_parity(wl, got, wl.backing)
    print("  %s errors %s" % (name, errs), flush=True)
    _check_padding(wl, big, row_pad, head_pad)


@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16],
                         ids=["f32", "bf16"])
def test_replay_into_padded_pool(state):
    """Replay into a pool with padded rows and heads gives the same bits as
    replay into a contiguous pool, and leaves the padding untouched."""
    lad = _lad()
    wl = W.make("padrep", W.KDA, B=6, T=3, H=2, HV=4, K=128, V=128,
                pool_size=12, seed=7400, separate_write=True,
                state_dtype=state)
    d = wl.to(DEV)
    fac = torch.full((wl.B, wl.T, wl.HV, 2 * wl.K + wl.V), float("nan"),
                     device=DEV)
    lad.kda_decode_mtp(d.q, d.k, d.v, d.g, d.beta, d.backing.clone(),
                       d.read_idx, None, factors=fac, l2norm_qk=True,
                       beta_logit=True)
    ntok = torch.tensor([3, 0, 1, 2, 3, 2], dtype=torch.int32, device=DEV)
    plain = d.backing.clone()
    lad.replay(fac, plain, d.read_idx, d.write_idx, ntok)
    pad = 16 if state == torch.bfloat16 else 4
    big, pool = _padded_pool(wl, pad, 1)
    lad.replay(fac, pool, d.read_idx, d.write_idx, ntok)
    torch.cuda.synchronize()
    assert torch.equal(_bits(pool.contiguous()), _bits(plain))
    _check_padding(wl, big, pad, 1)


# ------------------------------------------------- extreme decays and gates


SUBNORMAL_CASES = {
    # name: (variant, B, T, H, HV, state dtype, kernel)
    "general_gdn": (W.GDN, 4, 2, 8, 8, torch.float32, "decode_kernel"),
    "general_kda_t3": (W.KDA, 4, 3, 8, 8, torch.float32, "decode_kernel"),
    "one_token_gdn": (W.GDN, 40, 1, 16, 32, torch.float32, "decode1_kernel"),
    "packed_bf16_gdn": (W.GDN, 16, 1, 8, 16, torch.bfloat16,
                        "decode_packed_kernel"),
}


@pytest.mark.parametrize("name", sorted(SUBNORMAL_CASES))
def test_subnormal_states_are_not_flushed(name):
    """A pool of subnormal states through calls whose decay is exactly 1
    (g = 0) and whose update is exactly 0 (beta logit -1e30, so beta = 0):
    S * 1 + 0 * k returns every nonzero element bit for bit, subnormals
    included, in each kernel; zeros stay zero (IEEE addition may turn -0
    into +0, as the fp64 oracle's would)."""
    variant, B, T, H, HV, state, kernel = SUBNORMAL_CASES[name]
    wl = W.make("subnormal", variant, B=B, T=T, H=H, HV=HV, K=128, V=128,
                pool_size=2 * B, seed=12, state_dtype=state,
                separate_write=True, l2norm=True)
    gen = torch.Generator().manual_seed(5)
    if state == torch.float32:
        # every element subnormal: random 23-bit mantissa, random sign
        mant = torch.randint(1, 1 << 23, wl.backing.shape, generator=gen,
                             dtype=torch.int32)
        sign = torch.randint(0, 2, wl.backing.shape, generator=gen,
                             dtype=torch.int32) << 31
        wl.backing = (mant | sign).view(torch.float32)
    else:
        wl.backing = (wl.backing.float() * 1e-38).to(state)
    wl.g = torch.zeros_like(wl.g)
    wl.beta = torch.full_like(wl.beta, -1e30)
    assert _kernel_name(wl) == kernel
    before = wl.backing.clone()
    got = gpu_run(wl)
    checked = 0
    for b in range(B):
        r, w = int(wl.read_idx[b]), int(wl.write_idx[b])
        if w < 0:
            continue
        x, y = before[r], got["backing"][w]
        nz = x.float() != 0
        assert int(nz.sum()) > 0
        assert torch.equal(_bits(x)[nz], _bits(y)[nz]), "a state changed"
        assert bool((y.float()[~nz] == 0).all()), "a zero changed"
        checked += 1
    assert checked > 0


@pytest.mark.parametrize("name", sorted(SUBNORMAL_CASES))
def test_nonfinite_values_stay_in_their_request(name):
    """NaN and Inf planted in one request's read tile and in another
    request's query reach only those requests: every other request's
    outputs and written state equal those of a clean call bit for bit."""
    variant, B, T, H, HV, state, kernel = SUBNORMAL_CASES[name]

    def make():
        return W.make("nonfinite", variant, B=B, T=T, H=H, HV=HV, K=128,
                      V=128, pool_size=2 * B, seed=13, state_dtype=state,
                      separate_write=True, l2norm=True)
    clean = make()
    assert _kernel_name(clean) == kernel
    ref = gpu_run(clean)
    bad = make()
    r1 = int(bad.read_idx[1])
    bad.backing[r1, 0, 3, 5] = float("nan")
    bad.backing[r1, HV - 1, 100, 7] = float("inf")
    bad.q[2, T - 1, 0, 9] = float("nan")
    got = gpu_run(bad)
    for b in range(B):
        w = int(bad.write_idx[b])
        if b in (1, 2):
            assert not torch.isfinite(got["out"][b].float()).all()
            continue
        assert torch.equal(_bits(got["out"][b]), _bits(ref["out"][b])), b
        if w >= 0:
            assert torch.equal(_bits(got["backing"][w]),
                               _bits(ref["backing"][w])), b


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
@pytest.mark.parametrize("T,B,HV", [(3, 5, 4), (1, 64, 32)],
                         ids=["t3_general", "t1_large"])
def test_extreme_log_decays(variant, T, B, HV):
    """Log-decays of -60 (the state all but erased: exp(-60) ~ 9e-27), -20
    and 0 mixed per head and token (per channel for KDA); the T = 1 GDN case
    runs the one-token kernel."""
    wl = W.make("xdecay", variant, B=B, T=T, H=HV // 2, HV=HV, K=128,
                V=128, pool_size=2 * B, seed=7500 + T, separate_write=True,
                act_dtype=torch.float32)
    gen = torch.Generator().manual_seed(7501 + T)
    choice = torch.tensor([-60.0, -20.0, 0.0])
    wl.g = choice[torch.randint(0, 3, wl.g.shape, generator=gen)]
    run_and_check(wl)


@pytest.mark.parametrize("variant", [W.GDN, W.KDA])
@pytest.mark.parametrize("lower_bound", [None, -5.0], ids=["softplus", "lb"])
def test_gate_chain_extreme_arguments(variant, lower_bound):
    """The gate chain far into its tails: x + dt_bias in {-40, -5, 0, 5, 40}
    (softplus then ~exp(-40), or exactly its argument above 20; the bounded
    form's sigmoid saturating at both ends)."""
    wl = W.make("xgate", variant, B=5, T=3, H=2, HV=4, K=128, V=128,
                pool_size=12, seed=7600, separate_write=True,
                act_dtype=torch.float32)
    a_log, dt = _gate_inputs(variant, wl.HV, wl.K, 7601)
    gen = torch.Generator().manual_seed(7602)
    z = torch.tensor([-40.0, -5.0, 0.0, 5.0, 40.0])
    zz = z[torch.randint(0, 5, wl.g.shape, generator=gen)]
    dt_b = dt.view((1, 1) + tuple(dt.shape))
    wl.g = (zz - dt_b).float()  # raw gate x = z - dt_bias
    got, ref = _gate_run(wl, a_log, dt, lower_bound)
    kind, tol_out, tol_state = _tol(wl)
    assert _err(kind, got["out"].float(), ref["out"]) <= tol_out
    for b, w in enumerate(wl.write_idx.tolist()):
        if w >= 0:
            assert _err(kind, got["backing"][w].float(),
                        ref["pool"][w]) <= tol_state, b


# ------------------------------- slots beyond 2^31 elements, every kernel


def _far_pool(wl):
    """The workload's pool as a strided view whose slot stride puts its last
    slots beyond 2^31 elements from the base (a 4-9 GB buffer)."""
    P, HV, V, K = wl.backing.shape
    es = wl.backing.element_size()
    epc = 16 // es  # slot starts stay 16-byte aligned
    tile = HV * V * K
    stride = max(tile, -(-(2 ** 31) // (P - 1)))
    stride = -(-stride // epc) * epc
    buf = torch.empty((P - 1) * stride + tile, dtype=wl.backing.dtype,
                      device=DEV)
    pool = torch.as_strided(buf, (P, HV, V, K), (stride, V * K, K, 1))
    pool.copy_(wl.backing.to(DEV))
    assert (P - 1) * stride >= 2 ** 31
    return buf, pool


FAR_CASES = {
    "one_token_f32": dict(variant=W.GDN, B=64, H=16, HV=32, pool_size=64),
    "one_token_bf16": dict(variant=W.GDN, B=72, H=16, HV=32, pool_size=72,
                           state_dtype=torch.bfloat16),
    "packed_bf16": dict(variant=W.LIGHTNING, B=8, H=4, HV=4, pool_size=8,
                        state_dtype=torch.bfloat16),
}


@pytest.mark.parametrize("name", sorted(FAR_CASES))
def test_far_slots_bit_identical_to_contiguous(name):
    """One-token calls (the one-token and the packed kernel) whose read and
    write slots lie beyond 2^31 elements from the pool base give the same
    bits as the same call on a contiguous pool."""
    case = dict(FAR_CASES[name])
    variant = case.pop("variant")
    wl = W.make("far_" + name, variant, T=1, K=128, V=128,
                seed=7700 + sorted(FAR_CASES).index(name),
                l2norm=variant != W.LIGHTNING, **case)
    assert _kernel_name(wl) == ("decode1_kernel" if name.startswith("one_")
                                else "decode_packed_kernel"), name
    lad = _lad()
    d = wl.to(DEV)
    buf, far = _far_pool(wl)
    near = d.backing.clone()
    outs = []
    for pool in (near, far):
        if variant == W.LIGHTNING:
            o, _ = lad.la_decode(d.q, d.k, d.v, pool, d.read_idx, lam=d.g)
        else:
            o, _ = lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, pool,
                                      d.read_idx, l2norm_qk=wl.l2norm,
                                      beta_logit=wl.beta_logit)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(_bits(outs[0]), _bits(outs[1]))
    assert torch.equal(_bits(near), _bits(far.contiguous()))
    assert not torch.equal(_bits(near), _bits(d.backing))  # states moved
    del buf, far


def test_replay_far_slots_bit_identical_to_contiguous():
    """Replay with seed and write slots beyond 2^31 elements."""
    lad = _lad()
    wl = W.make("farrep", W.GDN, B=4, T=3, H=2, HV=4, K=128, V=128,
                pool_size=8, seed=7790, separate_write=True)
    d = wl.to(DEV)
    fac = torch.full((wl.B, wl.T, wl.HV, 2 * wl.K + wl.V), float("nan"),
                     device=DEV)
    lad.gdn_decode_mtp(d.q, d.k, d.v, d.g, d.beta, d.backing.clone(),
                       d.read_idx, None, factors=fac, l2norm_qk=True,
                       beta_logit=True)
    ntok = torch.tensor([3, 1, 0, 2], dtype=torch.int32, device=DEV)
    near = d.backing.clone()
    lad.replay(fac, near, d.read_idx, d.write_idx, ntok)
    buf, far = _far_pool(wl)
    lad.replay(fac, far, d.read_idx, d.write_idx, ntok)
    torch.cuda.synchronize()
    assert torch.equal(_bits(near), _bits(far.contiguous()))
    del buf, far


# ------------------------------------------- random feature combinations


def _combo(i):
    """Configuration i of the combination sweep: a fixed draw over variant,
    tile shape, T, head grouping, dtypes, flags, gate form, varlen, paged
    slots, records, cache, strided pool, separate and skipped writes and a
    padded request."""
    import random
    rng = random.Random(8000 + i)
    variant = rng.choice([W.LIGHTNING, W.GDN, W.KDA])
    K, V = rng.choice(SHAPES)
    T = rng.choice([1, 2, 3, 5, 9])
    HV = rng.choice([2, 4])
    H = rng.choice([h for h in (1, 2, 4) if HV % h == 0])
    B = rng.randint(1, 6)
    paged = rng.random() < 0.25
    sep = not paged and rng.random() < 0.5
    cfg = dict(variant=variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
               act_dtype=rng.choice([torch.float32, torch.bfloat16]),
               out_dtype=rng.choice([torch.float32, torch.bfloat16]),
               state_dtype=rng.choice([torch.float32, torch.bfloat16]),
               l2norm=rng.random() < 0.7, beta_logit=rng.random() < 0.7,
               stride_mult=rng.choice([1, 1, 2]),
               inter=rng.random() < 0.4, paged=paged, separate_write=sep,
               write_skip=0.3 if sep and rng.random() < 0.5 else 0.0,
               varlen_min=(rng.choice([0, 1]) if rng.random() < 0.3
                           else None),
               pool_size=B * T + 3 if paged else (2 * B + 3 if sep
                                                   else B + 3))
    gate = None
    if variant != W.LIGHTNING and rng.random() < 0.35:
        gate = rng.choice([None, -5.0])  # softplus form, or bounded
        gate = ("lb", gate) if gate is not None else ("softplus", None)
    records = rng.random() < 0.35
    pad = None if paged or rng.random() < 0.7 else rng.randrange(B)
    return cfg, gate, records, pad


def _unit_keys(wl):
    """Keys scaled to unit length on the host for a delta-rule call with
    the l2norm flag off (the host-normalised reading of the flag-off path).
    Raw N(0,1) keys have |k|^2 near K, and the delta rule then multiplies
    rounding error by |1 - beta |k|^2| at every token: over 9 tokens one
    fp32 ulp of a key moved the fp64 outputs (up to 9e4) by 0.09, so no
    fixed tolerance separates right from wrong there."""
    if not wl.l2norm and wl.variant != W.LIGHTNING:
        k = wl.k.double()
        wl.k = (k / k.norm(dim=-1, keepdim=True)).to(wl.k.dtype)


def _combo_compare(kind, tol, got, ref, state_bf16, what):
    """NaN where the oracle wrote nothing, the tolerance elsewhere (plus one
    bf16 step for values stored in bf16)."""
    got = got.double()
    ref = torch.as_tensor(np.asarray(ref, dtype=np.float64))
    blank = torch.isnan(ref)
    assert bool(torch.isnan(got[blank]).all()), what + ": wrote a blank row"
    g, r = got[~blank], ref[~blank]
    assert bool(torch.isfinite(g).all()), what + ": non-finite value"
    if g.numel() == 0:
        return 0.0
    diff = (g - r).abs()
    if state_bf16:
        diff = (diff - r.abs() * 2.0 ** -7).clamp(min=0.0)
    e = float(diff.max())
    if kind == "rel":
        e /= max(float(r.abs().max()), 1e-30)
    assert e <= tol, (what, e)
    return e


@pytest.mark.parametrize("i", range(48))
def test_random_feature_combinations(i):
    """48 fixed draws from the whole feature space, each run through the C
    ABI and compared with the oracle: outputs, per-token cache, update
    records, every pool slot (slots the oracle leaves unchanged must keep
    their bits) and the gaps of strided pools."""
    _run_combo("combo%d" % i, 8100 + i, 8200 + i, *_combo(i))


def _combo_medium(i):
    """Draw 100 + i of the sweep moved to a medium grid, past the small-grid
    instance (up to 2048 tiles): the 32-row instances with every feature
    (the one-token kernel where a plain fp32 token takes it)."""
    import random
    cfg, gate, records, pad = _combo(100 + i)
    rng = random.Random(77000 + i)
    HV = rng.choice([16, 24, 32])
    H = rng.choice([h for h in (HV // 2, HV) if HV % h == 0])
    lo = 4096 * 16 // cfg["V"] + 1
    B = rng.randint(-(-lo // HV), 2048 // HV)
    cfg.update(B=B, H=H, HV=HV)
    T, paged, sep = cfg["T"], cfg["paged"], cfg["separate_write"]
    cfg["pool_size"] = B * T + 3 if paged else (2 * B + 3 if sep else B + 3)
    pad = None if paged or rng.random() < 0.7 else rng.randrange(B)
    return cfg, gate, records, pad


def _combo_one_token(i):
    """Draw 200 + i of the sweep as a one-token call on a large grid
    (1100-4096 tiles, 8-64 value heads): the one-token and packed kernels,
    and the general kernel for the shapes that keep it."""
    import random
    cfg, gate, _, _ = _combo(200 + i)
    rng = random.Random(88000 + i)
    HV = rng.choice([8, 16, 24, 32, 48, 64])
    H = rng.choice([h for h in (HV // 2, HV) if HV % h == 0])
    B = rng.randint(max(1, 1100 // HV), 4096 // HV)
    sep = rng.random() < 0.5
    cfg.update(B=B, H=H, HV=HV, T=1, inter=False, paged=False,
               varlen_min=None, separate_write=sep,
               write_skip=0.3 if sep and rng.random() < 0.5 else 0.0,
               pool_size=2 * B + 3 if sep else B + 3)
    pad = None if rng.random() < 0.5 else rng.randrange(B)
    return cfg, gate, False, pad


def _combo_long(i):
    """Draw 300 + i of the sweep as a call of 12-64 tokens (many LDS
    rounds), without the per-token cache or paged slots."""
    import random
    cfg, gate, records, pad = _combo(300 + i)
    rng = random.Random(99000 + i)
    T = rng.choice([12, 17, 33, 64])
    HV = rng.choice([4, 16, 24, 32])
    H = rng.choice([h for h in (HV // 2, HV) if HV % h == 0])
    B = rng.randint(1, max(1, 1536 // HV))
    sep = rng.random() < 0.5
    cfg.update(B=B, H=H, HV=HV, T=T, inter=False, paged=False,
               separate_write=sep,
               write_skip=0.3 if sep and rng.random() < 0.5 else 0.0,
               pool_size=2 * B + 3 if sep else B + 3)
    if records and B * HV * T > 40000:
        records = False
    return cfg, gate, records, pad if pad is None or pad < B else None


@pytest.mark.parametrize("i", range(12))
def test_random_feature_combinations_medium_grids(i):
    """12 draws of the whole feature space on medium grids (paged slots,
    varlen, records, the gate chain and the cache on the 32-row
    instances), checked as the sweep checks its draws."""
    _run_combo("combo_medium%d" % i, 8600 + i, 8700 + i, *_combo_medium(i))


@pytest.mark.parametrize("i", range(8))
def test_random_one_token_calls_on_large_grids(i):
    """8 one-token draws on grids of 1100-4096 tiles (dtypes, tile shapes,
    head grouping, gate chain, strided pools, separate, skipped and padded
    requests), checked as the sweep checks its draws."""
    _run_combo("combo_one%d" % i, 8800 + i, 8900 + i, *_combo_one_token(i))


@pytest.mark.parametrize("i", range(6))
def test_random_long_calls(i):
    """6 draws of 12-64 tokens per call, checked as the sweep checks its
    draws."""
    _run_combo("combo_long%d" % i, 9000 + i, 9100 + i, *_combo_long(i))


def _run_combo(name, seed, gate_seed, cfg, gate, records, pad):
    """Run one sweep draw through the C ABI and compare it with the oracle:
    outputs, cache, records, every pool slot and the stride gaps."""
    variant = cfg.pop("variant")
    wl = W.make(name, variant, seed=seed, **cfg)
    _unit_keys(wl)
    if pad is not None:
        wl.read_idx[pad] = -1
    lad = _lad()
    d = wl.to(DEV)
    m = wl.stride_mult
    pool = d.backing[::m]
    varlen = wl.cu_seqlens is not None
    paged = wl.token_slots is not None
    lead = (wl.q.shape[0],) if varlen else (wl.B, wl.T)
    out = torch.full(lead + (wl.HV, wl.V), float("nan"), dtype=wl.out_dtype,
                     device=DEV)
    inter = (torch.full(lead + (wl.HV, wl.V, wl.K), float("nan"),
                        dtype=wl.backing.dtype, device=DEV)
             if wl.inter else None)
    fac = (torch.full(lead + (wl.HV, 2 * wl.K + wl.V), float("nan"),
                      device=DEV) if records else None)
    kw = dict(out=out, inter=inter, factors=fac, token_slots=d.token_slots,
              num_accepted=d.num_accepted, out_dtype=wl.out_dtype)
    okw = dict(token_slots=wl.token_slots, num_accepted=wl.num_accepted)
    if varlen:
        kw.update(cu_seqlens=d.cu_seqlens, max_tokens=wl.T)
        okw.update(cu_seqlens=wl.cu_seqlens, max_tokens=wl.T)
    if gate is not None:
        a_log, dt = _gate_inputs(variant, wl.HV, wl.K, gate_seed)
        kw.update(A_log=a_log.to(DEV), dt_bias=dt.to(DEV),
                  lower_bound=gate[1])
        okw.update(A_log=a_log, dt_bias=dt, lower_bound=gate[1])
    ridx = None if paged else d.read_idx
    widx = None if paged else d.write_idx
    if variant == W.LIGHTNING:
        lad.la_decode(d.q, d.k, d.v, pool, ridx, widx, lam=d.g, **kw)
    else:
        fn = lad.gdn_decode_mtp if variant == W.GDN else lad.kda_decode_mtp
        fn(d.q, d.k, d.v, d.g, d.beta, pool, ridx, widx,
           l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit, **kw)
    torch.cuda.synchronize()
    ref = oracle.decode(VARIANT_CODE[variant], wl.q, wl.k, wl.v, wl.g,
                        wl.beta, wl.pool(), None if paged else wl.read_idx,
                        None if paged else wl.write_idx, flags=_flags(wl),
                        inter=wl.inter, factors=records, **okw)
    kind, tol_out, tol_state = _tol(wl)
    sb = wl.backing.dtype == torch.bfloat16
    ob = wl.out_dtype == torch.bfloat16
    _combo_compare(kind, tol_out, out.cpu(), ref["out"], ob, "out")
    if wl.inter:
        _combo_compare(kind, tol_state, inter.cpu(), ref["inter"], sb,
                       "inter")
    if records:
        _combo_compare(kind, tol_state, fac.cpu(), ref["factors"], False,
                       "records")
    before = wl.backing
    after = d.backing.cpu()
    logical_in = wl.pool().double().numpy()
    for s in range(wl.pool_size):
        if np.array_equal(ref["pool"][s], logical_in[s]):
            assert torch.equal(_bits(after[m * s]), _bits(before[m * s])), \
                "slot %d changed" % s
        else:
            _combo_compare(kind, tol_state, after[m * s], ref["pool"][s], sb,
                           "slot %d" % s)
    if m > 1:
        gaps = [j for j in range(before.shape[0]) if j % m]
        assert torch.equal(_bits(after[gaps]), _bits(before[gaps])), \
            "a stride gap changed"


# ------------------------------------------- sharding by head and by request


@pytest.mark.parametrize("variant,B,HV,H", [(W.GDN, 64, 32, 16),
                                            (W.LIGHTNING, 33, 64, 64),
                                            (W.KDA, 16, 24, 24)],
                         ids=["gdn_gva", "lightning", "kda"])
def test_head_and_request_shards_equal_the_full_call(variant, B, HV, H):
    """The decode shards with no exchange: running it on head slices (the
    pool's heads, the matching value heads and their q/k heads) or on
    request subsets gives the full call's bits. For the GDN and Lightning
    shapes the full call runs the one-token kernel and the shards the
    general one."""
    lad = _lad()
    wl = W.make("shard", variant, B=B, T=1, H=H, HV=HV, K=128, V=128,
                pool_size=2 * B, seed=7800 + HV, separate_write=True,
                l2norm=variant != W.LIGHTNING)
    d = wl.to(DEV)
    group = HV // H

    def run(pool, sl_b, h0, h1):
        q0, q1 = h0 // group, h1 // group
        q = d.q[sl_b, :, q0:q1]
        k = d.k[sl_b, :, q0:q1]
        v = d.v[sl_b, :, h0:h1]
        sub = pool[:, h0:h1]
        if variant == W.LIGHTNING:
            lam = d.g[h0:h1].contiguous() if d.g is not None else None
            if lam is None:  # the built-in schedule depends on HV: pass it
                hh = torch.arange(HV, dtype=torch.float64)
                lam = torch.exp(-torch.exp2(-8.0 * (hh + 1) / HV)).float()[
                    h0:h1].to(DEV)
            o, _ = lad.la_decode(q, k, v, sub, d.read_idx[sl_b],
                                 d.write_idx[sl_b], lam=lam)
        else:
            fn = lad.gdn_decode_mtp if variant == W.GDN else \
                lad.kda_decode_mtp
            o, _ = fn(q, k, v, d.g[sl_b, :, h0:h1], d.beta[sl_b, :, h0:h1],
                      sub, d.read_idx[sl_b], d.write_idx[sl_b],
                      l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)
        return o

    full_pool = d.backing.clone()
    full = run(full_pool, slice(0, B), 0, HV)
    # four head shards, each keeping whole q/k groups
    hs = HV // 4
    heads_pool = d.backing.clone()
    outs = [run(heads_pool, slice(0, B), i * hs, (i + 1) * hs)
            for i in range(4)]
    # two request shards
    req_pool = d.backing.clone()
    routs = [run(req_pool, slice(0, B // 2), 0, HV),
             run(req_pool, slice(B // 2, B), 0, HV)]
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch.cat(outs, dim=2)), _bits(full))
    assert torch.equal(_bits(heads_pool), _bits(full_pool))
    assert torch.equal(_bits(torch.cat(routs, dim=0)), _bits(full))
    assert torch.equal(_bits(req_pool), _bits(full_pool))


def _medium_combo(i):
    """Draw i of the medium-grid sweep: a grid that runs the general kernel
    at 32 rows per wave (more than one small-grid round of tiles, and no
    one-token or packed kernel)."""
    import random
    rng = random.Random(9700 + i)
    variant = rng.choice([W.LIGHTNING, W.GDN, W.KDA])
    K, V = rng.choice(SHAPES)
    HV = rng.choice([16, 24, 32])
    H = rng.choice([h for h in (HV // 2, HV) if HV % h == 0])
    state = rng.choice([torch.float32, torch.bfloat16])
    T = rng.choice([1, 2, 3, 4]) if state == torch.float32 else \
        rng.choice([2, 3, 4])
    lo = 4096 * 16 // V + 1   # first grid beyond the small-grid instance
    # one token on an fp32 pool at K = V = 128 takes the one-token kernel
    # beyond 1024 tiles
    hi = 1024 if (T == 1 and state == torch.float32 and K == V == 128) \
        else 2047
    B = rng.randint(-(-lo // HV), hi // HV)
    return dict(variant=variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
                pool_size=2 * B + 3, state_dtype=state,
                act_dtype=rng.choice([torch.float32, torch.bfloat16]),
                out_dtype=rng.choice([torch.float32, torch.bfloat16]),
                stride_mult=rng.choice([1, 2]),
                separate_write=rng.random() < 0.5, write_skip=0.1,
                inter=rng.random() < 0.4,
                l2norm=variant != W.LIGHTNING and rng.random() < 0.8)


@pytest.mark.parametrize("i", range(12))
def test_random_medium_grids_general_kernel(i):
    """12 fixed draws of medium grids (the 32-row general kernel): variant,
    tile shape, head count, dtypes, strided pools, separate and skipped
    writes, the per-token cache and a padded request; every request
    against the oracle, every untouched byte of the pool checked."""
    cfg = _medium_combo(i)
    variant = cfg.pop("variant")
    wl = W.make("medium%d" % i, variant, seed=9800 + i, **cfg)
    _unit_keys(wl)
    wl.read_idx[wl.B // 3] = -1
    assert _kernel_name(wl) == "decode_kernel"
    lad = _lad()
    d = wl.to(DEV)
    kw = {}
    if variant != W.LIGHTNING:
        kw = dict(l2norm_qk=wl.l2norm, beta_logit=wl.beta_logit)
    info = lad.kernel_info(variant, d.q, d.k, d.v, d.g, d.beta, d.pool(),
                           d.read_idx, d.write_idx, **kw)
    assert info["block_threads"] == (wl.V // 32) * 64, info
    run_and_check(wl)
