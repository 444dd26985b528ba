"""ctypes binding of libla_decode.so (argument marshalling only).

Every function here reads pointers, strides and dtypes off torch tensors,
fills the C argument struct of include/la_decode.h and calls the library on
the current HIP stream. No step of the decode runs in Python, and there is
no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libla_decode.so")

# la_status
LA_OK = 0
STATUS_NAMES = {0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE",
                3: "LA_ERR_STRIDE", 4: "LA_ERR_ALIGN", 5: "LA_ERR_DTYPE",
                6: "LA_ERR_ARG", 7: "LA_ERR_UNSUPPORTED", 8: "LA_ERR_LAUNCH"}
# la_dtype
LA_F32, LA_BF16 = 0, 1
# flags
LA_F_L2NORM_QK, LA_F_BETA_LOGIT = 0x1, 0x2
LA_F_GATE, LA_F_GATE_LOWER_BOUND = 0x4, 0x8

ENTRY_POINTS = ("la_decode", "gdn_decode_mtp", "kda_decode_mtp")


class ActStrides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("t", ctypes.c_int64),
                ("h", ctypes.c_int64)]


class PoolStrides(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int64), ("head", ctypes.c_int64),
                ("row", ctypes.c_int64)]


class DecodeArgs(ctypes.Structure):
    """Mirror of la_decode_args."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("pool_size", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("qkv_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("state_dtype", ctypes.c_int),
        ("q", ctypes.c_void_p), ("sq", ActStrides),
        ("k", ctypes.c_void_p), ("sk", ActStrides),
        ("v", ctypes.c_void_p), ("sv", ActStrides),
        ("g", ctypes.c_void_p), ("sg", ActStrides),
        ("beta", ctypes.c_void_p), ("sbeta", ActStrides),
        ("pool", ctypes.c_void_p), ("sp", PoolStrides),
        ("read_idx", ctypes.c_void_p), ("write_idx", ctypes.c_void_p),
        ("inter", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("so", ActStrides),
        ("token_slots", ctypes.c_void_p),
        ("token_slots_stride", ctypes.c_int64),
        ("num_accepted", ctypes.c_void_p),
        ("factors", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("total_tokens", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("lower_bound", ctypes.c_float), ("reserved2", ctypes.c_int32),
    ]


class KernelInfo(ctypes.Structure):
    """la_kernel_info: the kernel a decode call selects."""
    _fields_ = [("kernel", ctypes.c_char_p),
                ("grid_blocks", ctypes.c_int32),
                ("block_threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32),
                ("vgprs", ctypes.c_int32),
                ("scratch_bytes", ctypes.c_int32),
                ("blocks_per_cu", ctypes.c_int32),
                ("waves_per_simd", ctypes.c_int32),
                ("tokens_per_round", ctypes.c_int32)]


VARIANT_CODES = {"lightning": 0, "gdn": 1, "kda": 2}


class ReplayArgs(ctypes.Structure):
    """Mirror of la_replay_args."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("HV", ctypes.c_int32),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("pool_size", ctypes.c_int32), ("state_dtype", ctypes.c_int),
        ("factors", ctypes.c_void_p), ("pool", ctypes.c_void_p),
        ("sp", PoolStrides), ("read_idx", ctypes.c_void_p),
        ("write_idx", ctypes.c_void_p), ("num_tokens", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("total_tokens", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class LaDecodeError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS_NAMES.get(status, status),
                                          status_string(status)))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libla_decode.so is not built (expected at %s); run "
                "__graft_entry__.build() or python -m "
                "linear_attention_recurrent_slot_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name in ENTRY_POINTS:
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
        L.la_replay.restype = ctypes.c_int
        L.la_replay.argtypes = [ctypes.POINTER(ReplayArgs), ctypes.c_void_p]
        L.la_check_indices.restype = ctypes.c_int
        L.la_check_indices.argtypes = [ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
        L.la_check_token_slots.restype = ctypes.c_int
        L.la_check_token_slots.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.la_check_cu_seqlens.restype = ctypes.c_int
        L.la_check_cu_seqlens.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        L.la_status_string.restype = ctypes.c_char_p
        L.la_status_string.argtypes = [ctypes.c_int]
        L.la_version.restype = ctypes.c_int32
        L.la_version.argtypes = []
        L.la_decode_kernel_info.restype = ctypes.c_int
        L.la_decode_kernel_info.argtypes = [
            ctypes.c_int32, ctypes.POINTER(DecodeArgs),
            ctypes.POINTER(KernelInfo)]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().la_status_string(status).decode()


def call(entry: str, args: DecodeArgs, stream=None) -> int:
    """Raw C-ABI call; returns the la_status code."""
    return getattr(lib(), entry)(ctypes.byref(args), _stream_handle(stream))


def _stream_handle(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError("%s must be float32 or bfloat16, got %s" % (what, t.dtype))


def _act(t: torch.Tensor, ndim: int, what: str, packed: bool = False):
    """Pointer and (b, t, h) strides of a per-token tensor: [B, T, ...], or
    token-packed [total, ...] (packed=True: one dimension fewer, no b
    stride)."""
    nd = ndim - 1 if packed else ndim
    if t.dim() != nd:
        raise ValueError("%s must have %d dims, got %s" % (what, nd,
                                                           tuple(t.shape)))
    if ndim == 4 and t.stride(nd - 1) != 1:
        raise ValueError("%s: innermost stride must be 1" % what)
    s = t.stride()
    if packed:
        return ctypes.c_void_p(t.data_ptr()), ActStrides(
            0, s[0], s[1] if nd > 1 else 0)
    return ctypes.c_void_p(t.data_ptr()), ActStrides(s[0], s[1], s[2])


def _idx(t):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.dim() != 1 or t.stride(0) != 1:
        raise ValueError("slot indices must be contiguous 1-D int32")
    return ctypes.c_void_p(t.data_ptr())


def _slot_table(t, B, T):
    """[B, >=T] int32 table with unit inner stride -> (pointer, row stride)."""
    if t.dtype != torch.int32 or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("token_slots must be a 2-D int32 [B, >=T] table "
                         "with unit inner stride")
    if t.shape[0] != B or t.shape[1] < T:
        raise ValueError("token_slots shape %s does not cover [%d, %d]"
                         % (tuple(t.shape), B, T))
    stride = t.stride(0) if B > 1 else max(t.stride(0), t.shape[1])
    return ctypes.c_void_p(t.data_ptr()), stride


def _factors(f, shape, dev):
    if f is None:
        return None
    if (f.dtype != torch.float32 or not f.is_contiguous()
            or tuple(f.shape) != shape or f.device != dev):
        raise ValueError("factors must be a contiguous float32 %s tensor on "
                         "%s" % (shape, dev))
    return ctypes.c_void_p(f.data_ptr())


def _cu(cu_seqlens, max_tokens, dev):
    """(B, T, total pointer args) of a varlen batch."""
    if (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or cu_seqlens.stride(0) != 1 or cu_seqlens.shape[0] < 1):
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 [B + 1] "
                         "tensor")
    if cu_seqlens.device != dev:
        raise ValueError("cu_seqlens is on %s, pool on %s"
                         % (cu_seqlens.device, dev))
    B = cu_seqlens.shape[0] - 1
    if max_tokens is None:  # reads the offsets back: a device sync
        max_tokens = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) \
            if B > 0 else 1
    return B, max(1, int(max_tokens))


def _gate_inputs(a, variant, A_log, dt_bias, lower_bound, HV, K, dev):
    """Fill the gate-chain fields; returns the extra flag bits."""
    if A_log is None and dt_bias is None and lower_bound is None:
        return 0
    if variant == "lightning":
        raise ValueError("the gate chain applies to gdn and kda only")
    if A_log is None or dt_bias is None:
        raise ValueError("the gate chain needs both A_log and dt_bias")
    want = (HV,) if variant == "gdn" else (HV, K)
    for name, t, shape in (("A_log", A_log, (HV,)),
                           ("dt_bias", dt_bias, want)):
        if (t.dtype != torch.float32 or not t.is_contiguous()
                or tuple(t.shape) != shape or t.device != dev):
            raise ValueError("%s must be a contiguous float32 %s tensor on %s"
                             % (name, shape, dev))
    a.A_log = ctypes.c_void_p(A_log.data_ptr())
    a.dt_bias = ctypes.c_void_p(dt_bias.data_ptr())
    if lower_bound is None:
        return LA_F_GATE
    a.lower_bound = float(lower_bound)
    return LA_F_GATE | LA_F_GATE_LOWER_BOUND


def build_args(variant: str, q, k, v, g, beta, pool, read_idx, write_idx,
               out, inter, flags: int, token_slots=None,
               num_accepted=None, factors=None, cu_seqlens=None,
               max_tokens=None, A_log=None, dt_bias=None,
               lower_bound=None) -> DecodeArgs:
    vl = cu_seqlens is not None
    if vl:
        # token-packed: q, k [total, H, K], v [total, HV, V], ...
        if q.dim() != 3 or v.dim() != 3:
            raise ValueError("with cu_seqlens q must be [total,H,K] and v "
                             "[total,HV,V]")
        total, H, K = q.shape
        HV, V = v.shape[1], v.shape[2]
        B, T = _cu(cu_seqlens, max_tokens, pool.device)
        lead = (total,)
    else:
        if q.dim() != 4 or v.dim() != 4:
            raise ValueError("q must be [B,T,H,K] and v [B,T,HV,V]")
        B, T, H, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        total = 0
        lead = (B, T)
    if (pool.dim() != 4 or pool.dtype not in (torch.float32, torch.bfloat16)
            or pool.stride(3) != 1):
        raise ValueError("pool must be a float32 or bfloat16 "
                         "[pool_size, HV, V, K] tensor with unit innermost "
                         "stride")
    # The library sees raw pointers: every extent it will index is checked
    # here against the tensors that back it.
    want = {"k": (k, lead + (H, K)), "v": (v, lead + (HV, V)),
            "out": (out, lead + (HV, V))}
    if read_idx is not None:
        want["read_idx"] = (read_idx, (B,))
    if num_accepted is not None:
        want["num_accepted"] = (num_accepted, (B,))
    if tuple(pool.shape[1:]) != (HV, V, K):
        raise ValueError("pool shape %s does not match [*, %d, %d, %d]"
                         % (tuple(pool.shape), HV, V, K))
    if write_idx is not None:
        want["write_idx"] = (write_idx, (B,))
    if beta is not None:
        want["beta"] = (beta, lead + (HV,))
    if g is not None:
        want["g"] = (g, {"lightning": (HV,), "gdn": lead + (HV,),
                         "kda": lead + (HV, K)}[variant])
    if inter is not None:
        want["inter"] = (inter, lead + (HV, V, K))
    dev = pool.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape:
            raise ValueError("%s shape %s != %s" % (name, tuple(t.shape), shape))
        if t.device != dev:
            raise ValueError("%s is on %s, pool on %s" % (name, t.device, dev))
    if q.device != dev:
        raise ValueError("q is on %s, pool on %s" % (q.device, dev))
    a = DecodeArgs()
    a.B, a.T, a.H, a.HV, a.K, a.V = B, T, H, HV, K, V
    a.pool_size = pool.shape[0]
    a.flags = flags
    a.qkv_dtype = _dtype_code(q, "q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    a.out_dtype = _dtype_code(out, "out")
    a.state_dtype = _dtype_code(pool, "pool")
    a.q, a.sq = _act(q, 4, "q", vl)
    a.k, a.sk = _act(k, 4, "k", vl)
    a.v, a.sv = _act(v, 4, "v", vl)
    if g is not None:
        if g.dtype != torch.float32:
            raise TypeError("g must be float32")
        if variant == "lightning":
            if g.dim() != 1 or g.stride(0) != 1:
                raise ValueError("lambda must be a contiguous [HV] tensor")
            a.g = ctypes.c_void_p(g.data_ptr())
        elif variant == "gdn":
            a.g, a.sg = _act(g, 3, "gdn g", vl)
        else:
            a.g, a.sg = _act(g, 4, "g", vl)
    if beta is not None:
        if beta.dtype != torch.float32:
            raise ValueError("beta must be float32")
        a.beta, a.sbeta = _act(beta, 3, "beta", vl)
    a.pool = ctypes.c_void_p(pool.data_ptr())
    a.sp = PoolStrides(*pool.stride()[:3])
    a.read_idx = _idx(read_idx)
    a.write_idx = _idx(write_idx)
    if inter is not None:
        if (inter.dtype != pool.dtype or not inter.is_contiguous()
                or tuple(inter.shape) != lead + (HV, V, K)):
            raise ValueError("inter must be a contiguous %s tensor of the "
                             "pool's dtype" % (lead + (HV, V, K),))
        a.inter = ctypes.c_void_p(inter.data_ptr())
    a.out, a.so = _act(out, 4, "out", vl)
    if token_slots is not None:
        if token_slots.device != dev:
            raise ValueError("token_slots is on %s, pool on %s"
                             % (token_slots.device, dev))
        a.token_slots, a.token_slots_stride = _slot_table(token_slots, B, T)
    a.num_accepted = _idx(num_accepted)
    a.factors = _factors(factors, lead + (HV, 2 * K + V), dev)
    if vl:
        a.cu_seqlens = ctypes.c_void_p(cu_seqlens.data_ptr())
        a.total_tokens = total
    a.flags = flags | _gate_inputs(a, variant, A_log, dt_bias, lower_bound,
                                   HV, K, dev)
    return a


def _run(variant, entry, q, k, v, g, beta, pool, read_idx, write_idx, out,
         inter, flags, out_dtype, stream, token_slots=None,
         num_accepted=None, factors=None, cu_seqlens=None, max_tokens=None,
         A_log=None, dt_bias=None, lower_bound=None):
    lead = tuple(q.shape[:-2])  # (B, T), or (total,) with cu_seqlens
    HV, V, K = v.shape[-2], v.shape[-1], q.shape[-1]
    if out is None:
        out = torch.empty(lead + (HV, V), dtype=out_dtype, device=q.device)
    if inter is True:
        inter = torch.empty(lead + (HV, V, K), dtype=pool.dtype,
                            device=q.device)
    elif inter is False:
        inter = None
    args = build_args(variant, q, k, v, g, beta, pool, read_idx, write_idx,
                      out, inter, flags, token_slots, num_accepted, factors,
                      cu_seqlens, max_tokens, A_log, dt_bias, lower_bound)
    st = call(entry, args, stream)
    if st != LA_OK:
        raise LaDecodeError(st, entry)
    return out, inter


# Every decode entry point takes either read_idx (+ optional write_idx) or,
# for paged speculative decoding, token_slots ([B, >=T] int32 table) and
# num_accepted ([B] int32) with read_idx=None. `factors` is an optional
# caller-allocated float32 [B, T, HV, 2K + V] tensor that receives the
# per-token update records (see replay()). With cu_seqlens (int32 [B + 1]
# offsets) the batch is variable-length: every per-token tensor is
# token-packed ([total, ...] in place of [B, T, ...]) and max_tokens bounds
# the tokens of one request (None: read back from the offsets, a sync).
# gdn_decode_mtp / kda_decode_mtp: A_log ([HV]) and dt_bias ([HV] for GDN,
# [HV, K] for KDA), float32, switch the in-kernel gate chain on (g is then
# the raw gate); lower_bound selects its bounded form.

def la_decode(q, k, v, pool, read_idx=None, write_idx=None, *, lam=None,
              out=None, inter=None, out_dtype=torch.float32, stream=None,
              token_slots=None, num_accepted=None, factors=None,
              cu_seqlens=None, max_tokens=None):
    """Lightning decode. lam: optional float32 [HV] decay factors (default:
    exp(-2^(-8(h+1)/HV)) per value head). Returns (out, inter)."""
    return _run("lightning", "la_decode", q, k, v, lam, None, pool, read_idx,
                write_idx, out, inter, 0, out_dtype, stream, token_slots,
                num_accepted, factors, cu_seqlens, max_tokens)


def gdn_decode_mtp(q, k, v, g, beta, pool, read_idx=None, write_idx=None, *,
                   out=None, inter=None, l2norm_qk=False, beta_logit=False,
                   out_dtype=torch.float32, stream=None, token_slots=None,
                   num_accepted=None, factors=None, cu_seqlens=None,
                   max_tokens=None, A_log=None, dt_bias=None,
                   lower_bound=None):
    """Gated delta rule decode over T tokens. g: [B,T,HV] log-decay (the
    raw gate with A_log/dt_bias); beta: [B,T,HV] (logits if beta_logit).
    Returns (out, inter)."""
    flags = (LA_F_L2NORM_QK if l2norm_qk else 0) | \
        (LA_F_BETA_LOGIT if beta_logit else 0)
    return _run("gdn", "gdn_decode_mtp", q, k, v, g, beta, pool, read_idx,
                write_idx, out, inter, flags, out_dtype, stream, token_slots,
                num_accepted, factors, cu_seqlens, max_tokens, A_log,
                dt_bias, lower_bound)


def kda_decode_mtp(q, k, v, g, beta, pool, read_idx=None, write_idx=None, *,
                   out=None, inter=None, l2norm_qk=False, beta_logit=False,
                   out_dtype=torch.float32, stream=None, token_slots=None,
                   num_accepted=None, factors=None, cu_seqlens=None,
                   max_tokens=None, A_log=None, dt_bias=None,
                   lower_bound=None):
    """KDA decode over T tokens. g: [B,T,HV,K] per-key-channel log-decay
    (the raw gate with A_log/dt_bias). Returns (out, inter)."""
    flags = (LA_F_L2NORM_QK if l2norm_qk else 0) | \
        (LA_F_BETA_LOGIT if beta_logit else 0)
    return _run("kda", "kda_decode_mtp", q, k, v, g, beta, pool, read_idx,
                write_idx, out, inter, flags, out_dtype, stream, token_slots,
                num_accepted, factors, cu_seqlens, max_tokens, A_log,
                dt_bias, lower_bound)


def kernel_info_of(variant: str, args: DecodeArgs) -> dict:
    """la_decode_kernel_info for a prepared argument struct."""
    info = KernelInfo()
    st = lib().la_decode_kernel_info(VARIANT_CODES[variant],
                                     ctypes.byref(args), ctypes.byref(info))
    if st != LA_OK:
        raise LaDecodeError(st, "la_decode_kernel_info")
    return {"kernel": info.kernel.decode(), "grid_blocks": info.grid_blocks,
            "block_threads": info.block_threads,
            "lds_bytes": info.lds_bytes, "vgprs": info.vgprs,
            "scratch_bytes": info.scratch_bytes,
            "blocks_per_cu": info.blocks_per_cu,
            "waves_per_simd": info.waves_per_simd,
            "tokens_per_round": info.tokens_per_round}


def kernel_info(variant, q, k, v, g, beta, pool, read_idx=None,
                write_idx=None, *, out=None, inter=None, l2norm_qk=False,
                beta_logit=False, out_dtype=torch.float32, token_slots=None,
                num_accepted=None, factors=None, cu_seqlens=None,
                max_tokens=None, A_log=None, dt_bias=None, lower_bound=None):
    """Which kernel the decode call with these arguments would run, with its
    launch shape, VGPRs and occupancy; launches nothing. variant:
    "lightning" (g = lam, beta = None), "gdn" or "kda"; the other arguments
    are those of the matching decode function (out and an inter=True cache
    are allocated when not given, as the call would)."""
    flags = 0
    if variant != "lightning":
        flags = (LA_F_L2NORM_QK if l2norm_qk else 0) | \
            (LA_F_BETA_LOGIT if beta_logit else 0)
    lead = tuple(q.shape[:-2])
    HV, V, K = v.shape[-2], v.shape[-1], q.shape[-1]
    if out is None:
        out = torch.empty(lead + (HV, V), dtype=out_dtype, device=q.device)
    if inter is True:
        inter = torch.empty(lead + (HV, V, K), dtype=pool.dtype,
                            device=q.device)
    elif inter is False:
        inter = None
    args = build_args(variant, q, k, v, g, beta, pool, read_idx, write_idx,
                      out, inter, flags, token_slots, num_accepted, factors,
                      cu_seqlens, max_tokens, A_log, dt_bias, lower_bound)
    return kernel_info_of(variant, args)


def check_indices(read_idx, write_idx, pool_size, result=None, stream=None):
    """Launch the index validator; returns the device int32 result tensor
    (bits: 1 read out of range, 2 write out of range, 4 duplicate write,
    8 write into another request's read slot)."""
    if result is None:
        result = torch.empty((1,), dtype=torch.int32, device=read_idx.device)
    st = lib().la_check_indices(read_idx.shape[0], pool_size, _idx(read_idx),
                                _idx(write_idx),
                                ctypes.c_void_p(result.data_ptr()),
                                _stream_handle(stream))
    if st != LA_OK:
        raise LaDecodeError(st, "la_check_indices")
    return result


def check_token_slots(token_slots, num_accepted, pool_size, T, result=None,
                      stream=None):
    """Launch the paged slot-table validator; returns the device int32 result
    (bits: 1 seed out of range, 2 entry out of range, 4 slot written by two
    requests, 8 slot written over another request's seed, 16 accepted count
    outside [1, T])."""
    B = num_accepted.shape[0]
    ptr, stride = _slot_table(token_slots, B, T)
    if result is None:
        result = torch.empty((1,), dtype=torch.int32,
                             device=num_accepted.device)
    st = lib().la_check_token_slots(B, T, pool_size, ptr, stride,
                                    _idx(num_accepted),
                                    ctypes.c_void_p(result.data_ptr()),
                                    _stream_handle(stream))
    if st != LA_OK:
        raise LaDecodeError(st, "la_check_token_slots")
    return result


def check_cu_seqlens(cu_seqlens, max_tokens, total_tokens, result=None,
                     stream=None):
    """Launch the varlen offset validator; returns the device int32 result
    (bits: 1 an offset outside [0, total_tokens], 2 a request with a negative
    count or more than max_tokens tokens)."""
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D int32")
    if result is None:
        result = torch.empty((1,), dtype=torch.int32,
                             device=cu_seqlens.device)
    st = lib().la_check_cu_seqlens(cu_seqlens.shape[0] - 1, max_tokens,
                                   total_tokens, _idx(cu_seqlens),
                                   ctypes.c_void_p(result.data_ptr()),
                                   _stream_handle(stream))
    if st != LA_OK:
        raise LaDecodeError(st, "la_check_cu_seqlens")
    return result


def build_replay_args(factors, pool, read_idx, write_idx,
                      num_tokens, cu_seqlens=None,
                      max_tokens=None) -> ReplayArgs:
    if cu_seqlens is not None:
        if factors.dim() != 3:
            raise ValueError("with cu_seqlens factors must be "
                             "[total, HV, 2K + V]")
        total, HV, R = factors.shape
        B, T = _cu(cu_seqlens, max_tokens, pool.device)
        lead = (total,)
    else:
        if factors.dim() != 4:
            raise ValueError("factors must be [B, T, HV, 2K + V]")
        B, T, HV, R = factors.shape
        lead = (B, T)
    if (pool.dim() != 4 or pool.dtype not in (torch.float32, torch.bfloat16)
            or pool.stride(3) != 1):
        raise ValueError("pool must be a float32 or bfloat16 "
                         "[pool_size, HV, V, K] tensor with unit innermost "
                         "stride")
    V, K = pool.shape[2], pool.shape[3]
    if pool.shape[1] != HV or R != 2 * K + V:
        raise ValueError("factors %s do not match pool %s"
                         % (tuple(factors.shape), tuple(pool.shape)))
    dev = pool.device
    for name, t in (("read_idx", read_idx), ("write_idx", write_idx),
                    ("num_tokens", num_tokens)):
        if t is not None and (tuple(t.shape) != (B,) or t.device != dev):
            raise ValueError("%s must be [%d] on %s" % (name, B, dev))
    a = ReplayArgs()
    a.B, a.T, a.HV, a.K, a.V = B, T, HV, K, V
    a.pool_size = pool.shape[0]
    a.state_dtype = _dtype_code(pool, "pool")
    a.factors = _factors(factors, lead + (HV, R), dev)
    a.pool = ctypes.c_void_p(pool.data_ptr())
    a.sp = PoolStrides(*pool.stride()[:3])
    a.read_idx = _idx(read_idx)
    a.write_idx = _idx(write_idx)
    a.num_tokens = _idx(num_tokens)
    if cu_seqlens is not None:
        a.cu_seqlens = ctypes.c_void_p(cu_seqlens.data_ptr())
        a.total_tokens = lead[0]
    return a


def replay(factors, pool, read_idx, write_idx, num_tokens, stream=None, *,
           cu_seqlens=None, max_tokens=None):
    """Rebuild states from per-token update records (written by a decode call
    with factors=...): request b starts from pool[read_idx[b]], applies its
    first num_tokens[b] records and stores the result in write_idx[b]
    (None: the read slot; negative: skip)."""
    args = build_replay_args(factors, pool, read_idx, write_idx, num_tokens,
                             cu_seqlens, max_tokens)
    st = lib().la_replay(ctypes.byref(args), _stream_handle(stream))
    if st != LA_OK:
        raise LaDecodeError(st, "la_replay")
