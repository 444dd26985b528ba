"""Machine-code check of the built library (CPU only).

A vector-memory store of more than 64 bits may read its data VGPRs after it
issues, so a VALU instruction that overwrites those VGPRs must not follow it
directly (one wait state is required in between). The compiler guards this
for buffer stores only when their soffset operand is not an SGPR; the
kernels keep soffset at the constant 0 for that reason. This test
disassembles the gfx950 code object of libla_decode.so and checks every wide
store, so that a later change that brings the unguarded form back fails here
instead of corrupting stored states now and then on the GPU.
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

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
WIDE_STORE = re.compile(r"(buffer|global|flat)_store_(dwordx3|dwordx4|b96|b128)")


def _vregs(op):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", op)
    return {int(m.group(1))} if m else set()


def _disassemble():
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not found at %s" % OBJDUMP)
    if not os.path.exists(bnd.LIB_PATH):
        from linear_attention_recurrent_slot_amd import build
        build.build()
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "lib.so")
        shutil.copy(bnd.LIB_PATH, so)
        subprocess.run([OBJDUMP, "--offloading", so], cwd=d, check=True,
                       capture_output=True)
        objs = [f for f in os.listdir(d) if f.endswith("gfx950")]
        assert len(objs) == 1, os.listdir(d)
        out = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn",
                              os.path.join(d, objs[0])], check=True,
                             capture_output=True, text=True).stdout
    return out


def _scan(text):
    """(function, store, next instruction) for every wide store whose next
    instruction is a VALU write to one of the store's data VGPRs; plus the
    number of wide stores seen."""
    fn, pending, hits, n = None, None, [], 0
    for raw in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", raw)
        if m:
            fn, pending = m.group(1), None
            continue
        line = raw.split("//")[0].strip()
        if not line or line.endswith(":"):
            continue
        parts = line.replace(",", " ").split()
        op = parts[0]
        if pending is not None:
            if op.startswith("v_") and len(parts) > 1 and \
                    _vregs(parts[1]) & pending[0]:
                hits.append((fn, pending[1], line))
            pending = None
        if WIDE_STORE.match(op):
            n += 1
            # buffer: vdata first; global/flat: vaddr, then vdata
            data = parts[1] if op.startswith("buffer") else parts[2]
            pending = (_vregs(data), line)
    return hits, n


def test_scanner_flags_the_unguarded_pattern():
    text = """0000000000001000 <k>:
\tbuffer_store_dwordx4 v[82:85], v111, s[12:15], s4 offen nt
\tv_lshlrev_b32_e32 v82, 16, v74
\tbuffer_store_dwordx4 v[2:5], v1, s[12:15], 0 offen nt
\ts_nop 0
\tv_lshlrev_b32_e32 v2, 16, v74
\tbuffer_store_dwordx2 v[6:7], v1, s[12:15], s4 offen
\tv_mov_b32_e32 v6, 0
"""
    hits, n = _scan(text)
    assert n == 2
    assert len(hits) == 1 and "v82" in hits[0][2]


def test_no_wide_store_is_followed_by_a_write_of_its_data():
    hits, n = _scan(_disassemble())
    assert n > 0, "no wide stores found: the disassembly was not parsed"
    assert not hits, "%d unguarded wide stores, e.g. %s" % (len(hits), hits[:3])
