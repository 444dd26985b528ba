"""Seeded synthetic inputs for pool-indexed recurrent-state decode.

This module draws random inputs and builds index tables. It holds none of the
decode method's arithmetic; the GPU library and the CPU oracle each consume
what it returns. Every tensor is drawn on the CPU from a
``torch.Generator().manual_seed(seed)`` in a fixed order: pool, q, k, v, g,
beta logit, indices.

Shapes and distributions follow the workloads the source pages describe
(cuLA "fix: wire h0_indices into Lightning Attention decode for state-pool
indexing", Tests; FlashInfer "fp32 sibling of #3268", Tests; aiter "Fused
Gluon KDA decode path (950/1250)", review): pools larger than the batch with
random distinct slots, multi-token verify with separate write slots and
negative entries, strided pools cut from an oversized buffer, per-key-channel
gates.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

LIGHTNING, GDN, KDA = "lightning", "gdn", "kda"


@dataclasses.dataclass
class Workload:
    name: str
    variant: str
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    pool_size: int
    l2norm: bool
    beta_logit: bool
    q: torch.Tensor            # [B,T,H,K]
    k: torch.Tensor            # [B,T,H,K]
    v: torch.Tensor            # [B,T,HV,V]
    g: Optional[torch.Tensor]  # lightning [HV] decay factors or None;
    #                            gdn [B,T,HV]; kda [B,T,HV,K] (log-decay)
    beta: Optional[torch.Tensor]  # [B,T,HV] (logits when beta_logit)
    backing: torch.Tensor      # [stride_mult*pool_size, HV, V, K], fp32 or
    #                            bf16 (the state dtype)
    stride_mult: int
    read_idx: torch.Tensor     # int32 [B]
    write_idx: Optional[torch.Tensor]  # int32 [B] or None (= read_idx)
    inter: bool                # cache the state after every token
    out_dtype: torch.dtype = torch.float32
    # paged per-token slots: [B, T] table and [B] accepted counts; when set
    # the call uses them instead of read_idx/write_idx
    token_slots: Optional[torch.Tensor] = None
    num_accepted: Optional[torch.Tensor] = None
    # speculative step with update records: the decode reads the read slots,
    # writes no state and records every token; then the first
    # replay_tokens[b] records are replayed into write slot b
    replay_tokens: Optional[torch.Tensor] = None
    # variable-length batch: int32 [B + 1] token offsets; q, k, v, g, beta
    # are then token-packed ([total, ...]) and T is the longest request
    cu_seqlens: Optional[torch.Tensor] = None

    @property
    def record_floats(self) -> int:
        return 2 * self.K + self.V

    def counts(self) -> list:
        """Tokens of each request."""
        if self.cu_seqlens is None:
            return [self.T] * self.B
        cu = self.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(self.B)]

    def pool(self, backing: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The logical pool [pool_size, HV, V, K]: every stride_mult-th slot
        of the backing buffer (a strided view when stride_mult > 1)."""
        b = self.backing if backing is None else backing
        return b[:: self.stride_mult]

    @property
    def tokens(self) -> int:
        return sum(self.counts())

    def to(self, device) -> "Workload":
        """A copy with every tensor moved to ``device``."""
        moved = {}
        for f in dataclasses.fields(self):
            val = getattr(self, f.name)
            moved[f.name] = val.to(device) if isinstance(val, torch.Tensor) else val
        return Workload(**moved)

    def state_bytes(self) -> int:
        """Algorithmic state bytes one call must move: one read and one
        write per active (request, value head) tile, plus one cache write
        per token when intermediate states are kept."""
        tile = self.V * self.K * self.backing.element_size()
        if self.replay_tokens is not None:
            ridx = self.read_idx.tolist()
            widx = self.write_idx.tolist()
            n = self.replay_tokens.tolist()
            active = sum(1 for r in ridx if r >= 0)
            replayed = sum(1 for r, w, c in zip(ridx, widx, n)
                           if r >= 0 and w >= 0 and 0 <= c <= self.T)
            # decode reads every active tile; replay reads and writes again
            return (active + 2 * replayed) * self.HV * tile
        counts = self.counts()
        if self.token_slots is not None:
            reads = writes = cached = 0
            for row, na, n in zip(self.token_slots.tolist(),
                                  self.num_accepted.tolist(), counts):
                if 1 <= na <= n and row[na - 1] >= 0:
                    reads += 1
                    writes += sum(1 for s in row[:n] if s >= 0)
                    cached += n
            total = (reads + writes) * self.HV * tile
            if self.inter:
                total += cached * self.HV * tile
            return total
        ridx = self.read_idx.tolist()
        widx = self.write_idx.tolist() if self.write_idx is not None else ridx
        reads = sum(1 for r in ridx if r >= 0)
        writes = sum(1 for r, w in zip(ridx, widx) if r >= 0 and w >= 0)
        total = (reads + writes) * self.HV * tile
        if self.inter:
            total += sum(n for r, n in zip(ridx, counts) if r >= 0) * \
                self.HV * tile
        return total

    def io_bytes(self) -> int:
        """Algorithmic bytes of everything except the state: q, k, v, gates,
        beta, indices and outputs."""
        act = self.q.element_size()
        B, T, H, HV, K, V = self.B, self.T, self.H, self.HV, self.K, self.V
        N = self.tokens  # B T, or the packed token count
        n = 2 * N * H * K * act + N * HV * V * act
        if self.variant == GDN:
            n += N * HV * 4
        elif self.variant == KDA:
            n += N * HV * K * 4
        elif self.g is not None:
            n += HV * 4
        if self.beta is not None:
            n += N * HV * 4
        if self.token_slots is not None:
            n += B * T * 4 + B * 4
        else:
            n += B * 4 * (2 if self.write_idx is not None else 1)
        if self.cu_seqlens is not None:
            n += (B + 1) * 4
        out_size = torch.empty((), dtype=self.out_dtype).element_size()
        n += N * HV * V * out_size
        if self.replay_tokens is not None:
            rec = self.record_floats * 4 * HV
            n += B * T * rec  # records written by the decode
            n += sum(c for c in self.replay_tokens.tolist()
                     if 0 <= c <= T) * rec  # and read back by the replay
            n += B * 4 * 2  # replay's read slots and token counts
        return n


def _randperm(n, gen):
    return torch.randperm(n, generator=gen)


def _packed(wl, gen, varlen_min):
    """Turn the dense draws of ``wl`` into a variable-length batch."""
    if varlen_min is None:
        return wl
    lengths = torch.randint(varlen_min, wl.T + 1, (wl.B,), generator=gen,
                            dtype=torch.int32)
    cu = torch.zeros((wl.B + 1,), dtype=torch.int32)
    cu[1:] = torch.cumsum(lengths, 0)

    def pack(x):
        return torch.cat([x[b, :n] for b, n in enumerate(lengths.tolist())],
                         0).contiguous()

    wl.q, wl.k, wl.v = pack(wl.q), pack(wl.k), pack(wl.v)
    if wl.variant != LIGHTNING:
        wl.g, wl.beta = pack(wl.g), pack(wl.beta)
    wl.cu_seqlens = cu
    return wl


def make(name, variant, B, T, H, HV, K, V, pool_size, *, seed,
         act_dtype=torch.bfloat16, pool_std=0.05, g_low=-1.0, g_high=0.0,
         l2norm=True, beta_logit=True, stride_mult=1, read_idx=None,
         write_idx=None, separate_write=False, write_skip=0.0,
         inter=False, lightning_decay=None, out_dtype=torch.float32,
         paged=False, state_dtype=torch.float32, spec_replay=False,
         varlen_min=None):
    """Draw one workload.

    paged: draw a [B, T] per-token slot table of distinct slots and accepted
    counts uniform in [1, T] (needs pool_size >= B*T); read_idx/write_idx
    then hold the seed slots and -1 (informational only).
    spec_replay: a verify step with update records followed by a replay of
    replay_tokens[b] ~U{1..T} records into the (separate) write slots.

    varlen_min: draw a variable-length batch, request b holding T_b ~
    U{varlen_min..T} tokens (drawn last); the per-token tensors are then
    token-packed and ``cu_seqlens`` holds the offsets.

    read_idx: explicit list, or None for ``randperm(pool_size)[:B]``.
    write_idx: explicit list, or None: equal to read_idx unless
    ``separate_write`` (then B slots drawn from the slots no request reads,
    and a ``write_skip`` fraction of them set to -1).
    """
    gen = torch.Generator().manual_seed(seed)
    backing = (torch.randn((stride_mult * pool_size, HV, V, K),
                           generator=gen, dtype=torch.float32)
               * pool_std).to(state_dtype)
    q = torch.randn((B, T, H, K), generator=gen).to(act_dtype)
    k = torch.randn((B, T, H, K), generator=gen).to(act_dtype)
    v = torch.randn((B, T, HV, V), generator=gen).to(act_dtype)
    if variant == LIGHTNING:
        g = lightning_decay
        beta = None
    else:
        gshape = (B, T, HV) if variant == GDN else (B, T, HV, K)
        g = g_low + (g_high - g_low) * torch.rand(gshape, generator=gen)
        beta = torch.randn((B, T, HV), generator=gen)
    perm = _randperm(pool_size, gen)
    if paged:
        if pool_size < B * T:
            raise ValueError("need pool_size >= B*T for a paged table")
        table = perm[: B * T].view(B, T).to(torch.int32).contiguous()
        accepted = torch.randint(1, T + 1, (B,), generator=gen,
                                 dtype=torch.int32)
        seeds = table[torch.arange(B), accepted.long() - 1]
        return _packed(Workload(
            name=name, variant=variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
            pool_size=pool_size,
            l2norm=l2norm if variant != LIGHTNING else False,
            beta_logit=beta_logit if variant != LIGHTNING else False,
            q=q, k=k, v=v, g=g, beta=beta, backing=backing,
            stride_mult=stride_mult, read_idx=seeds.contiguous(),
            write_idx=torch.full((B,), -1, dtype=torch.int32),
            inter=inter, out_dtype=out_dtype, token_slots=table,
            num_accepted=accepted), gen, varlen_min)
    if read_idx is None:
        if B > pool_size:
            raise ValueError("need pool_size >= B for distinct slots")
        ridx = perm[:B].to(torch.int32)
    else:
        ridx = torch.tensor(read_idx, dtype=torch.int32)
    if write_idx is not None:
        widx = torch.tensor(write_idx, dtype=torch.int32)
    elif separate_write:
        used = set(ridx.tolist())
        free = [s for s in perm.tolist() if s not in used]
        if len(free) < B:
            raise ValueError("not enough free slots for separate writes")
        widx = torch.tensor(free[:B], dtype=torch.int32)
        n_skip = int(round(write_skip * B))
        if n_skip:
            drop = _randperm(B, gen)[:n_skip]
            widx[drop] = -1
    else:
        widx = None
    replay_tokens = None
    if spec_replay:
        if widx is None:
            raise ValueError("spec_replay needs separate write slots")
        replay_tokens = torch.randint(1, T + 1, (B,), generator=gen,
                                      dtype=torch.int32)
    return _packed(Workload(
        name=name, variant=variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
        pool_size=pool_size,
        l2norm=l2norm if variant != LIGHTNING else False,
        beta_logit=beta_logit if variant != LIGHTNING else False,
        q=q, k=k, v=v, g=g, beta=beta, backing=backing,
        stride_mult=stride_mult, read_idx=ridx, write_idx=widx,
        inter=inter, out_dtype=out_dtype,
        replay_tokens=replay_tokens), gen, varlen_min)


def head_shard(wl: Workload, n: int) -> Workload:
    """One GPU's share of ``wl`` when n GPUs split the heads: value heads
    [0, HV/n) with their pool heads, and the q/k heads [0, H/n) that serve
    exactly those value heads (each group of HV/H value heads stays on one
    GPU). Requests and slots are unchanged. The pool becomes a contiguous
    buffer of the shard's heads, as a GPU holding only its heads would
    allocate it. A Lightning workload without explicit decays keeps none, so
    the kernel's built-in schedule is that of HV/n heads: other values, the
    same cost."""
    if n < 1 or wl.HV % n or wl.H % n:
        raise ValueError("H=%d and HV=%d must both be multiples of %d"
                         % (wl.H, wl.HV, n))
    h, hv = wl.H // n, wl.HV // n

    def heads(t, dim, m):
        return None if t is None else t.narrow(dim, 0, m).contiguous()

    if wl.variant == GDN:
        g = heads(wl.g, -1, hv)
    elif wl.variant == KDA:
        g = heads(wl.g, -2, hv)
    else:
        g = heads(wl.g, 0, hv)
    return dataclasses.replace(
        wl, name="%s_hs%d" % (wl.name, n), H=h, HV=hv,
        q=heads(wl.q, -2, h), k=heads(wl.k, -2, h), v=heads(wl.v, -2, hv),
        g=g, beta=heads(wl.beta, -1, hv), backing=heads(wl.backing, 1, hv))


# The named workloads. Each is the shape, distribution and index structure of
# one decode setting; the seed is fixed per workload.

def gdn_small_k64(seed=1):
    """GDN single-token decode, fp32 throughout: B=4 requests in a pool of 6
    at slots [2,0,5,1] (the cuLA pool test's non-identity offsets), H=HV=2,
    K=V=64, pool ~N(0,0.1), g ~U(-1,0), beta logit ~N(0,1), q/k
    l2-normalised in the kernel."""
    return make("gdn_small_k64", GDN, B=4, T=1, H=2, HV=2, K=64, V=64,
                pool_size=6, seed=seed, act_dtype=torch.float32,
                pool_std=0.1, g_low=-1.0, g_high=0.0, read_idx=[2, 0, 5, 1])


def head_decays(HV: int) -> torch.Tensor:
    """The per-head decay input lambda_h = exp(-2^(-8 (h + 1) / HV)),
    h = 0..HV-1 (the slope schedule of the Lightning setting), evaluated in
    fp64 and rounded once to fp32, so that every consumer is handed the same
    fp32 values."""
    h = torch.arange(HV, dtype=torch.float64)
    return torch.exp(-torch.exp2(-8.0 * (h + 1) / HV)).float()


def lightning_b33_h64(seed=2):
    """Lightning decode: B=33 requests at random distinct slots of a pool of
    40 (the cuLA big-batch pool test), H=64, K=V=128, T=1, bf16 q/k/v
    ~N(0,1) unnormalised, pool ~N(0,0.05), per-head decays given as the
    fp32 array head_decays(64)."""
    return make("lightning_b33_h64", LIGHTNING, B=33, T=1, H=64, HV=64,
                K=128, V=128, pool_size=40, seed=seed, l2norm=False,
                lightning_decay=head_decays(64))


def gdn_gva_b64(seed=3):
    """GDN grouped-value decode: B=64, 16 q/k heads, 32 value heads,
    K=V=128, T=1, pool of 128 with random distinct slots, bf16 q/k/v,
    in-kernel l2norm, beta logit ~N(0,1), g ~U(-0.5,0), pool ~N(0,0.05)."""
    return make("gdn_gva_b64", GDN, B=64, T=1, H=16, HV=32, K=128, V=128,
                pool_size=128, seed=seed, g_low=-0.5, g_high=0.0)


def gdn_mtp_b32_t4(seed=4):
    """GDN multi-token verify: B=32, T=4, H=16, HV=32, K=V=128; the pool of
    96 slots is every second slot of a [192,32,128,128] buffer; write slots
    are disjoint from read slots, 25% of them -1; every token's state is
    cached to a [B,T,HV,V,K] buffer."""
    return make("gdn_mtp_b32_t4", GDN, B=32, T=4, H=16, HV=32, K=128, V=128,
                pool_size=96, seed=seed, g_low=-0.5, g_high=0.0,
                stride_mult=2, separate_write=True, write_skip=0.25,
                inter=True)


def kda_b256(T, seed=5):
    """KDA decode with a per-key-channel gate: B=256, H=HV=24, K=V=128,
    g in R^K per (token, head) ~U(-1,0), in-kernel l2norm and beta sigmoid,
    pool of 512 with random distinct slots, bf16 q/k/v."""
    return make("kda_b256_t%d" % T, KDA, B=256, T=T, H=24, HV=24, K=128,
                V=128, pool_size=512, seed=seed, g_low=-1.0, g_high=0.0)


def gdn_paged_b64_t4(seed=6):
    """GDN speculative verify with paged per-token state slots: B=64, T=4,
    H=16, HV=32, K=V=128; each request owns 4 slots of a 256-slot pool, its
    seed is the slot of its last accepted token (accepted ~U{1..4}) and the
    state after every token is written to that token's slot."""
    return make("gdn_paged_b64_t4", GDN, B=64, T=4, H=16, HV=32, K=128,
                V=128, pool_size=256, seed=seed, g_low=-0.5, g_high=0.0,
                paged=True)


def kda_spec_b64_t4(seed=7):
    """KDA speculative step with update records: B=64 requests verify T=4
    tokens (H=HV=24, K=V=128) reading their state but writing only a
    [a | k | err] record per token; then the records of the accepted tokens
    (~U{1..4}) are replayed into a separate write slot (pool of 160)."""
    return make("kda_spec_b64_t4", KDA, B=64, T=4, H=24, HV=24, K=128,
                V=128, pool_size=160, seed=seed, separate_write=True,
                spec_replay=True)


def gdn_gva_b64_bf16_state(seed=3):
    """The grouped-value GDN decode (B=64, 16 q/k heads, 32 value heads,
    K=V=128, T=1, pool 128) with the state pool stored in bf16."""
    return make("gdn_gva_b64_bf16_state", GDN, B=64, T=1, H=16, HV=32, K=128,
                V=128, pool_size=128, seed=seed, g_low=-0.5, g_high=0.0,
                state_dtype=torch.bfloat16)


def gdn_varlen_b64_t4(seed=8):
    """GDN multi-token verify over a variable-length batch: B=64 requests
    with T_b ~ U{1..4} tokens each (token-packed q/k/v/g/beta), H=16, HV=32,
    K=V=128, pool of 128 with random distinct slots, every token's state
    cached to a token-packed [total, HV, V, K] buffer."""
    return make("gdn_varlen_b64_t4", GDN, B=64, T=4, H=16, HV=32, K=128,
                V=128, pool_size=128, seed=seed, g_low=-0.5, g_high=0.0,
                inter=True, varlen_min=1)


NAMED = {
    "gdn_small_k64": gdn_small_k64,
    "lightning_b33_h64": lightning_b33_h64,
    "gdn_gva_b64": gdn_gva_b64,
    "gdn_mtp_b32_t4": gdn_mtp_b32_t4,
    "kda_b256_t1": lambda seed=5: kda_b256(1, seed),
    "kda_b256_t8": lambda seed=5: kda_b256(8, seed),
    "gdn_paged_b64_t4": gdn_paged_b64_t4,
    "gdn_gva_b64_bf16_state": gdn_gva_b64_bf16_state,
    "kda_spec_b64_t4": kda_spec_b64_t4,
    "gdn_varlen_b64_t4": gdn_varlen_b64_t4,
}


def named(name: str, seed: Optional[int] = None) -> Workload:
    fn = NAMED[name]
    return fn() if seed is None else fn(seed=seed)
