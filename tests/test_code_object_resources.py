"""Register and private-memory budget of the built library (CPU only).

Every kernel is meant to keep its state tile in VGPRs: a spill to private
(scratch) memory would add HBM traffic on the hot path, and the one-token
kernel's layout is chosen for 8 waves per SIMD, which needs at most 64 VGPRs.
The general kernel at 32 rows per wave needs at most 128 for 4 waves per
SIMD.
This test reads the AMDGPU metadata notes of the gfx950 code object in
libla_decode.so (our own build) and checks those budgets for every kernel.
"""
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from linear_attention_recurrent_slot_amd import _binding as bnd  # noqa: E402

LLVM = "/opt/rocm/llvm/bin"


def _kernels():
    objdump = os.path.join(LLVM, "llvm-objdump")
    readelf = os.path.join(LLVM, "llvm-readelf")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("llvm tools not found under %s" % LLVM)
    if not os.path.exists(bnd.LIB_PATH):
        from linear_attention_recurrent_slot_amd import build
        build.build()
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "lib.so")
        shutil.copy(bnd.LIB_PATH, so)
        subprocess.run([objdump, "--offloading", so], cwd=d, check=True,
                       capture_output=True)
        objs = [f for f in os.listdir(d) if f.endswith("gfx950")]
        assert len(objs) == 1, os.listdir(d)
        notes = subprocess.run([readelf, "--notes", os.path.join(d, objs[0])],
                               check=True, capture_output=True,
                               text=True).stdout
    # one list entry per kernel; its own keys sit at the entry's first
    # indentation level, its argument list deeper
    kernels = []
    for entry in re.split(r"\n(?=  - \.agpr_count:)", notes)[1:]:
        fields = dict(re.findall(r"^(?:  - |    )\.([a-z_]+):\s+(\S+)\s*$",
                                 entry, re.M))
        kernels.append(fields)
    return kernels


def test_no_kernel_spills_or_uses_accumulation_registers():
    kernels = _kernels()
    assert len(kernels) > 100
    for k in kernels:
        assert int(k["private_segment_fixed_size"]) == 0, k["name"]
        assert int(k["vgpr_spill_count"]) == 0, k["name"]
        # a few GDN instances run out of SGPRs by one or two; with no
        # private segment those go to VGPR lanes, not to memory
        assert int(k["sgpr_spill_count"]) <= 2, k["name"]
        assert int(k["agpr_count"]) == 0, k["name"]


def test_register_budgets_of_the_decode_kernels():
    kernels = _kernels()
    families = {"decode1_kernel": 64, "decode_kernel": 128,
                "decode_packed_kernel": 256, "replay_kernel": 128}
    seen = set()
    for k in kernels:
        for fam, limit in families.items():
            if re.search(r"\d%s" % fam, k["name"]):
                seen.add(fam)
                assert int(k["vgpr_count"]) <= limit, (k["name"],
                                                        k["vgpr_count"])
    assert seen == set(families)
