"""Pool-indexed recurrent-state decode for linear attention on MI355X.

Hand-written gfx950 HIP kernels behind a C ABI (include/la_decode.h), with a
thin ctypes binding. Entry points: la_decode (Lightning), gdn_decode_mtp
(gated delta rule), kda_decode_mtp (Kimi delta attention), replay (rebuild
states from per-token update records), the validators check_indices,
check_token_slots and check_cu_seqlens, and kernel_info (which kernel a call
would run, with its occupancy).
"""
from ._binding import (DecodeArgs, KernelInfo, LaDecodeError, ReplayArgs,
                       check_cu_seqlens, check_indices, check_token_slots,
                       gdn_decode_mtp, kda_decode_mtp, kernel_info, la_decode,
                       lib, replay)

__all__ = ["DecodeArgs", "KernelInfo", "LaDecodeError", "ReplayArgs",
           "check_cu_seqlens", "check_indices", "check_token_slots",
           "gdn_decode_mtp", "kda_decode_mtp", "kernel_info", "la_decode",
           "lib", "replay"]
