"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/la_decode.h declares,
agree with the ctypes mirror on the argument struct layout, and reject bad
arguments on the host before anything is launched (the pointers used here
are fake and never dereferenced).
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_decode.h")

from linear_attention_recurrent_slot_amd import _binding as bnd  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bnd.LIB_PATH):
        from linear_attention_recurrent_slot_amd import build
        build.build()
    return bnd.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("la_decode", "gdn_decode_mtp", "kda_decode_mtp", "la_replay",
              "la_check_indices", "la_check_token_slots",
              "la_check_cu_seqlens", "la_decode_kernel_info",
              "la_status_string", "la_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bnd.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_struct_layout_matches_ctypes(tmp_path):
    """Compile a C program against the header and compare sizeof/offsetof
    of every la_decode_args field with the ctypes mirror."""
    fields = [f for f, _ in bnd.DecodeArgs._fields_]
    body = "\n".join(
        '  printf("%s %%zu\\n", offsetof(la_decode_args, %s));' % (f, f)
        for f in fields)
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"la_decode.h\"\n"
        "int main(void){\n  printf(\"size %%zu\\n\", sizeof(la_decode_args));\n"
        "%s\n  return 0;\n}\n" % body)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in
               subprocess.run([str(exe)], capture_output=True, text=True,
                              check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(bnd.DecodeArgs)
    for f in fields:
        assert int(got[f]) == getattr(bnd.DecodeArgs, f).offset, f


@pytest.mark.parametrize("ctype,cstruct", [("KernelInfo", "la_kernel_info"),
                                           ("ReplayArgs", "la_replay_args")])
def test_other_struct_layouts_match_ctypes(tmp_path, ctype, cstruct):
    """sizeof/offsetof of the other C structs against their ctypes mirrors."""
    cls = getattr(bnd, ctype)
    fields = [f for f, _ in cls._fields_]
    body = "\n".join(
        '  printf("%s %%zu\\n", offsetof(%s, %s));' % (f, cstruct, f)
        for f in fields)
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"la_decode.h\"\n"
        "int main(void){\n  printf(\"size %%zu\\n\", sizeof(%s));\n"
        "%s\n  return 0;\n}\n" % (cstruct, body))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in
               subprocess.run([str(exe)], capture_output=True, text=True,
                              check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(cls)
    for f in fields:
        assert int(got[f]) == getattr(cls, f).offset, f


def test_status_strings_and_version(lib):
    for code in range(0, 9):
        s = bnd.status_string(code)
        assert s and s != "unknown status"
    assert bnd.status_string(99) == "unknown status"
    assert lib.la_version() >= 100


FAKE = 0x7f0000000000  # 16-byte aligned, never dereferenced


def _valid_args(variant="gdn", B=4, T=2, H=2, HV=4, K=128, V=128,
                pool_size=8, bf16=True):
    a = bnd.DecodeArgs()
    a.B, a.T, a.H, a.HV, a.K, a.V, a.pool_size = B, T, H, HV, K, V, pool_size
    a.flags = 0 if variant == "lightning" else 3
    a.qkv_dtype = bnd.LA_BF16 if bf16 else bnd.LA_F32
    a.out_dtype = bnd.LA_F32
    a.q = FAKE
    a.sq = bnd.ActStrides(T * H * K, H * K, K)
    a.k = FAKE + 0x100000
    a.sk = bnd.ActStrides(T * H * K, H * K, K)
    a.v = FAKE + 0x200000
    a.sv = bnd.ActStrides(T * HV * V, HV * V, V)
    if variant == "gdn":
        a.g = FAKE + 0x300000
        a.sg = bnd.ActStrides(T * HV, HV, 1)
    elif variant == "kda":
        a.g = FAKE + 0x300000
        a.sg = bnd.ActStrides(T * HV * K, HV * K, K)
    if variant != "lightning":
        a.beta = FAKE + 0x400000
        a.sbeta = bnd.ActStrides(T * HV, HV, 1)
    a.pool = FAKE + 0x1000000
    a.sp = bnd.PoolStrides(HV * V * K, V * K, K)
    a.read_idx = FAKE + 0x500000
    a.write_idx = FAKE + 0x500100
    a.out = FAKE + 0x600000
    a.so = bnd.ActStrides(T * HV * V, HV * V, V)
    return a


ENTRY = {"lightning": "la_decode", "gdn": "gdn_decode_mtp",
         "kda": "kda_decode_mtp"}


def _status(variant, a):
    return getattr(bnd.lib(), ENTRY[variant])(ctypes.byref(a), None)


def _mut(**kw):
    def f(a):
        for key, val in kw.items():
            setattr(a, key, val)
    return f


REJECT = [
    ("null_args", None, "gdn", 1),
    ("null_q", _mut(q=None), "gdn", 1),
    ("null_pool", _mut(pool=None), "kda", 1),
    ("null_read_idx", _mut(read_idx=None), "lightning", 1),
    ("null_out", _mut(out=None), "gdn", 1),
    ("null_beta_gdn", _mut(beta=None), "gdn", 1),
    ("null_g_kda", _mut(g=None), "kda", 1),
    ("T_zero", _mut(T=0), "gdn", 2),
    ("B_negative", _mut(B=-1), "gdn", 2),
    ("H_not_dividing_HV", _mut(H=3), "gdn", 2),
    ("pool_size_zero", _mut(pool_size=0), "gdn", 2),
    ("grid_too_large", _mut(B=2 ** 30, HV=4), "gdn", 2),
    ("K_96", _mut(K=96), "gdn", 7),
    ("V_256", _mut(V=256), "kda", 7),
    ("dtype_code", _mut(qkv_dtype=7), "gdn", 5),
    ("out_dtype_code", _mut(out_dtype=3), "lightning", 5),
    ("beta_for_lightning", _mut(beta=FAKE), "lightning", 6),
    ("flags_for_lightning", _mut(flags=1), "lightning", 6),
    ("unknown_flag_bit", _mut(flags=16), "gdn", 6),
    ("negative_q_stride", _mut(sq=bnd.ActStrides(-1, 0, 0)), "gdn", 3),
    ("negative_pool_stride", _mut(sp=bnd.PoolStrides(-4, 0, 128)), "gdn", 3),
    ("pool_rows_overlap", _mut(sp=bnd.PoolStrides(4 * 128 * 128 * 4,
                                                  128 * 128, 64)), "gdn", 3),
    ("pool_heads_overlap", _mut(sp=bnd.PoolStrides(4 * 128 * 128, 64 * 128,
                                                   128)), "gdn", 3),
    ("pool_slots_overlap", _mut(sp=bnd.PoolStrides(128 * 128, 128 * 128 * 2,
                                                   128)), "gdn", 3),
    ("out_rows_overlap", _mut(so=bnd.ActStrides(2 * 4 * 128, 4 * 128, 64)),
     "gdn", 3),
    ("tile_rows_span_2GiB", _mut(sp=bnd.PoolStrides(2 ** 30, 2 ** 26, 2 ** 22)),
     "gdn", 3),
    ("pool_misaligned", _mut(pool=FAKE + 0x1000004), "gdn", 4),
    ("pool_row_stride_misaligned",
     _mut(sp=bnd.PoolStrides(4 * 130 * 128, 130 * 128, 130)), "gdn", 4),
    ("inter_misaligned", _mut(inter=FAKE + 0x2000008), "kda", 4),
    ("bf16_q_odd_address", _mut(q=FAKE + 1), "gdn", 4),
    ("read_idx_misaligned", _mut(read_idx=FAKE + 0x500002), "gdn", 4),
    ("state_dtype_code", _mut(state_dtype=9), "kda", 5),
    ("bf16_pool_misaligned", _mut(state_dtype=1, pool=FAKE + 0x1000004),
     "gdn", 4),
    ("bf16_inter_misaligned", _mut(state_dtype=1, inter=FAKE + 0x2000008),
     "lightning", 4),
    ("bf16_pool_8B_aligned", _mut(state_dtype=1, pool=FAKE + 0x1000008),
     "kda", 4),
    ("bf16_row_stride_4_elements",
     _mut(state_dtype=1, sp=bnd.PoolStrides(4 * 132 * 128, 132 * 128, 132)),
     "gdn", 4),
    # paged per-token slots: the table replaces read/write slots, needs the
    # accepted counts and an explicit row stride covering T
    ("paged_with_read_idx", _mut(token_slots=FAKE + 0x700000,
                                 num_accepted=FAKE + 0x700100,
                                 token_slots_stride=2), "gdn", 6),
    ("paged_without_num_accepted", _mut(token_slots=FAKE + 0x700000,
                                        read_idx=None, write_idx=None,
                                        token_slots_stride=2), "kda", 1),
    ("paged_flat_table", _mut(token_slots=FAKE + 0x700000, read_idx=None,
                              write_idx=None, num_accepted=FAKE + 0x700100,
                              token_slots_stride=1), "kda", 3),
    ("paged_misaligned_table", _mut(token_slots=FAKE + 0x700002,
                                    read_idx=None, write_idx=None,
                                    num_accepted=FAKE + 0x700100,
                                    token_slots_stride=2), "lightning", 4),
    ("num_accepted_without_table", _mut(num_accepted=FAKE + 0x700100),
     "gdn", 6),
    # variable-length batches
    ("reserved_nonzero", _mut(reserved=1), "gdn", 6),
    ("varlen_negative_total", _mut(cu_seqlens=FAKE + 0x900000,
                                   total_tokens=-1), "kda", 2),
    ("varlen_misaligned_offsets", _mut(cu_seqlens=FAKE + 0x900002,
                                       total_tokens=8), "lightning", 4),
    # gate chain: inputs without the switch are refused, not ignored
    ("gate_inputs_without_flag", _mut(A_log=FAKE + 0xa00000), "kda", 6),
    ("dt_bias_without_flag", _mut(dt_bias=FAKE + 0xa00100), "gdn", 6),
    ("gate_flag_without_inputs", _mut(flags=3 | 4), "kda", 1),
    ("lower_bound_without_gate", _mut(flags=3 | 8), "gdn", 6),
    ("lower_bound_not_negative", _mut(flags=3 | 4 | 8, A_log=FAKE + 0xa00000,
                                      dt_bias=FAKE + 0xa00100,
                                      lower_bound=0.5), "kda", 6),
    ("gate_for_lightning", _mut(A_log=FAKE + 0xa00000,
                                dt_bias=FAKE + 0xa00100), "lightning", 6),
    ("gate_misaligned", _mut(flags=3 | 4, A_log=FAKE + 0xa00002,
                             dt_bias=FAKE + 0xa00100), "gdn", 4),
    ("reserved2_nonzero", _mut(reserved2=1), "gdn", 6),
    # packed outputs [total, HV, V]: rows of consecutive tokens overlap
    ("varlen_out_tokens_overlap", _mut(cu_seqlens=FAKE + 0x900000,
                                       total_tokens=8,
                                       so=bnd.ActStrides(0, 128, 128)),
     "gdn", 3),
]


@pytest.mark.parametrize("name,mutate,variant,code", REJECT,
                         ids=[r[0] for r in REJECT])
def test_host_validation_rejects(lib, name, mutate, variant, code):
    if mutate is None:
        st = getattr(lib, ENTRY[variant])(None, None)
    else:
        a = _valid_args(variant)
        mutate(a)
        st = _status(variant, a)
    assert st == code, (name, bnd.STATUS_NAMES.get(st))


def _info_status(variant, a):
    info = bnd.KernelInfo()
    st = bnd.lib().la_decode_kernel_info(
        bnd.VARIANT_CODES[variant], None if a is None else ctypes.byref(a),
        ctypes.byref(info))
    return st, info


@pytest.mark.parametrize("name,mutate,variant,code", REJECT,
                         ids=[r[0] for r in REJECT])
def test_kernel_info_returns_the_call_status(lib, name, mutate, variant,
                                             code):
    """The kernel query runs the entry point's host checks: every malformed
    call gets the status the call itself returns, and *info stays as it
    was."""
    if mutate is None:
        st, info = _info_status(variant, None)
    else:
        a = _valid_args(variant)
        mutate(a)
        st, info = _info_status(variant, a)
    assert st == code, (name, bnd.STATUS_NAMES.get(st))
    assert info.kernel is None and info.grid_blocks == 0


def test_kernel_info_own_errors_and_empty_batch(lib):
    a = _valid_args("gdn")
    info = bnd.KernelInfo()
    assert lib.la_decode_kernel_info(1, ctypes.byref(a), None) == 1
    assert lib.la_decode_kernel_info(3, ctypes.byref(a),
                                     ctypes.byref(info)) == 6
    assert lib.la_decode_kernel_info(-1, ctypes.byref(a),
                                     ctypes.byref(info)) == 6
    for variant in ("lightning", "gdn", "kda"):
        a = _valid_args(variant)
        a.B = 0
        st, info = _info_status(variant, a)
        assert st == 0 and info.kernel == b"none"
        assert info.grid_blocks == 0 and info.block_threads == 0


@pytest.mark.parametrize("variant", ["lightning", "gdn", "kda"])
def test_empty_batch_is_a_noop(lib, variant):
    a = _valid_args(variant)
    a.B = 0
    a.q = a.k = a.v = a.pool = a.out = a.read_idx = None
    assert _status(variant, a) == 0


def test_check_indices_host_rejections(lib):
    L = lib
    assert L.la_check_indices(-1, 4, FAKE, None, FAKE, None) == 2
    assert L.la_check_indices(4, 0, FAKE, None, FAKE, None) == 2
    assert L.la_check_indices(4, 4, FAKE, None, None, None) == 1
    assert L.la_check_indices(4, 4, None, None, FAKE, None) == 1
    assert L.la_check_indices(4, 4, FAKE, None, FAKE + 2, None) == 4


def test_check_cu_seqlens_host_rejections(lib):
    L = lib
    assert L.la_check_cu_seqlens(-1, 2, 4, FAKE, FAKE, None) == 2
    assert L.la_check_cu_seqlens(4, 0, 4, FAKE, FAKE, None) == 2
    assert L.la_check_cu_seqlens(4, 2, -1, FAKE, FAKE, None) == 2
    assert L.la_check_cu_seqlens(4, 2, 4, None, FAKE, None) == 1
    assert L.la_check_cu_seqlens(4, 2, 4, FAKE, None, None) == 1
    assert L.la_check_cu_seqlens(4, 2, 4, FAKE + 2, FAKE, None) == 4


def test_varlen_packed_outputs_accept_flat_token_strides(lib):
    """With cu_seqlens the b strides are ignored and outputs are
    [total, HV, V]: a packed output layout passes the overlap check. The
    offsets pointer is misaligned on purpose so that validation stops at the
    last host check (LA_ERR_ALIGN) and nothing is launched."""
    a = _valid_args("gdn")
    a.cu_seqlens = FAKE + 0x900002
    a.total_tokens = 8
    a.so = bnd.ActStrides(0, 4 * 128, 128)
    a.sq = bnd.ActStrides(0, 2 * 128, 128)
    assert _status("gdn", a) == 4
    a.so = bnd.ActStrides(0, 128, 128)  # token rows overlap: rejected first
    assert _status("gdn", a) == 3


@pytest.mark.parametrize("variant", ["lightning", "gdn", "kda"])
def test_varlen_without_tokens_needs_no_per_token_arrays(lib, variant):
    """A token-packed batch with total_tokens = 0 indexes no per-token
    array (empty tensors come with a NULL address), so q, k, v, g, beta and
    out may be NULL; with one token they are required. The offsets pointer
    is misaligned so that validation ends at its last host check
    (LA_ERR_ALIGN) and nothing is launched."""
    a = _valid_args(variant)
    a.cu_seqlens = FAKE + 0x900002
    a.total_tokens = 0
    a.q = a.k = a.v = a.g = a.beta = a.out = None
    assert _status(variant, a) == 4
    a.total_tokens = 1
    assert _status(variant, a) == 1


def test_replay_without_tokens_needs_no_records(lib):
    a = _valid_replay()
    a.cu_seqlens = FAKE + 0x900002
    a.total_tokens = 0
    a.factors = None
    assert lib.la_replay(ctypes.byref(a), None) == 4
    a.total_tokens = 1
    assert lib.la_replay(ctypes.byref(a), None) == 1


def test_check_token_slots_host_rejections(lib):
    L = lib
    assert L.la_check_token_slots(-1, 2, 4, FAKE, 2, FAKE, FAKE, None) == 2
    assert L.la_check_token_slots(4, 0, 4, FAKE, 2, FAKE, FAKE, None) == 2
    assert L.la_check_token_slots(4, 2, 4, FAKE, 1, FAKE, FAKE, None) == 3
    assert L.la_check_token_slots(4, 2, 4, None, 2, FAKE, FAKE, None) == 1
    assert L.la_check_token_slots(4, 2, 4, FAKE, 2, None, FAKE, None) == 1
    assert L.la_check_token_slots(4, 2, 4, FAKE, 2, FAKE, FAKE + 1, None) == 4


def test_valid_call_without_gpu_reports_launch_failure():
    """With no GPU the validated call reaches hipLaunchKernel, which fails;
    the library reports LA_ERR_LAUNCH instead of crashing. Run in a child
    process so the HIP runtime never initialises inside the test runner."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the launch would run")
    code = (
        "import sys, ctypes; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "from linear_attention_recurrent_slot_amd import _binding as b\n"
        "import test_boundary as tb\n"
        "a = tb._valid_args('gdn')\n"
        "print(b.lib().gdn_decode_mtp(ctypes.byref(a), None))\n"
        % (ROOT, os.path.join(ROOT, "tests")))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True,
                          text=True, timeout=120)
    assert proc.returncode == 0, proc.stderr
    assert proc.stdout.strip().splitlines()[-1] == "8"


# ------------------------------------------------------------ la_replay


def test_replay_struct_layout_matches_ctypes(tmp_path):
    fields = [f for f, _ in bnd.ReplayArgs._fields_]
    body = "\n".join(
        '  printf("%s %%zu\\n", offsetof(la_replay_args, %s));' % (f, f)
        for f in fields)
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"la_decode.h\"\n"
        "int main(void){\n  printf(\"size %%zu\\n\", sizeof(la_replay_args));\n"
        "%s\n  return 0;\n}\n" % body)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in
               subprocess.run([str(exe)], capture_output=True, text=True,
                              check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(bnd.ReplayArgs)
    for f in fields:
        assert int(got[f]) == getattr(bnd.ReplayArgs, f).offset, f


def _valid_replay(B=4, T=3, HV=4, K=128, V=128, pool_size=16):
    a = bnd.ReplayArgs()
    a.B, a.T, a.HV, a.K, a.V, a.pool_size = B, T, HV, K, V, pool_size
    a.state_dtype = bnd.LA_F32
    a.factors = FAKE + 0x800000
    a.pool = FAKE + 0x1000000
    a.sp = bnd.PoolStrides(HV * V * K, V * K, K)
    a.read_idx = FAKE + 0x500000
    a.write_idx = FAKE + 0x500100
    a.num_tokens = FAKE + 0x500200
    return a


REPLAY_REJECT = [
    ("T_zero", _mut(T=0), 2),
    ("B_negative", _mut(B=-1), 2),
    ("K_96", _mut(K=96), 7),
    ("state_dtype_code", _mut(state_dtype=4), 5),
    ("null_factors", _mut(factors=None), 1),
    ("null_pool", _mut(pool=None), 1),
    ("null_read_idx", _mut(read_idx=None), 1),
    ("null_num_tokens", _mut(num_tokens=None), 1),
    ("pool_heads_overlap", _mut(sp=bnd.PoolStrides(4 * 128 * 128, 64 * 128,
                                                   128)), 3),
    ("factors_misaligned", _mut(factors=FAKE + 0x800008), 4),
    ("pool_misaligned", _mut(pool=FAKE + 0x1000008), 4),
    ("num_tokens_misaligned", _mut(num_tokens=FAKE + 0x500202), 4),
    ("reserved_nonzero", _mut(reserved=3), 6),
    ("varlen_negative_total", _mut(cu_seqlens=FAKE + 0x900000,
                                   total_tokens=-2), 2),
    ("varlen_misaligned_offsets", _mut(cu_seqlens=FAKE + 0x900001,
                                       total_tokens=4), 4),
]


@pytest.mark.parametrize("name,mutate,code", REPLAY_REJECT,
                         ids=[r[0] for r in REPLAY_REJECT])
def test_replay_host_validation_rejects(lib, name, mutate, code):
    a = _valid_replay()
    mutate(a)
    assert lib.la_replay(ctypes.byref(a), None) == code, name


def test_replay_rejects_null_and_empty_is_noop(lib):
    assert lib.la_replay(None, None) == 1
    a = _valid_replay(B=0)
    a.factors = a.pool = a.read_idx = a.num_tokens = None
    assert lib.la_replay(ctypes.byref(a), None) == 0


def test_decode_factors_must_be_16_byte_aligned(lib):
    a = _valid_args("kda")
    a.factors = FAKE + 0x900008
    assert _status("kda", a) == 4
