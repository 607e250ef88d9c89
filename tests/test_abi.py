"""C ABI checks that need no GPU: the library loads, exports every function
include/gdn_replay.h and include/gdn_probe.h declare, and rejects malformed host arguments with the
documented status before any HIP call (vLLM RecoverSSM PR, Test Plan:
malformed-input rejection). Only calls that validation rejects are made."""
import ctypes as C
import os
import re

import pytest

import gated_deltanet_speculative_gdn_amd as g
from gated_deltanet_speculative_gdn_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN = 0, -1, -2, -3, -4


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return g.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTS)


def test_version_and_strings(lib):
    assert lib.gdn_abi_version() == 5
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.gdn_status_string(s), bytes)
    assert lib.gdn_status_string(-4).decode().startswith("a pointer or stride")


def test_record_stride():
    # delta[T][128] | k_hat[T][128] | gate[T] padded to 4 floats
    assert g.rec_stride(4) == 4 * 256 + 4
    assert g.rec_stride(16) == 16 * 256 + 16
    assert g.rec_stride(1) == 256 + 4
    assert g.rec_stride(5) == 5 * 256 + 8
    assert g.rec_stride(0) == 0


def test_payload_record_stride(lib):
    # k, v bf16 [T][128] each, gate and beta fp32 [T]: 520 bytes a token, padded to 16 bytes
    assert lib.gdn_record_stride(4, 1) == 4 * 520 // 4
    assert lib.gdn_record_stride(1, 1) == 528 // 4
    assert lib.gdn_record_stride(16, 1) == 16 * 520 // 4
    assert lib.gdn_record_stride(4, 0) == lib.gdn_rec_stride(4)
    # per-channel decay records: delta[T][128] | k_hat[T][128] | alpha[T][128]
    assert lib.gdn_record_stride(4, 2) == 4 * 384
    assert lib.gdn_record_stride(16, 2) == 16 * 384
    assert lib.gdn_record_stride(4, 3) == 0
    assert lib.gdn_record_stride(0, 1) == 0
    assert lib.gdn_record_stride(0, 2) == 0


def good_pools():
    p = B.gdn_pools()
    p.num_layers, p.num_v_heads, p.num_k_heads = 2, 4, 2
    p.head_k_dim = p.head_v_dim = 128
    p.state_dtype = 0
    p.num_state_slots, p.num_rec_slots, p.rec_tokens = 8, 8, 4
    for i in range(2):
        p.state[i] = 0x10000 + i * 0x100000   # never dereferenced: calls below are rejected
        p.rec[i] = 0x20000 + i * 0x100000
    return p


def good_io():
    io = B.gdn_verify_io()
    io.q, io.q_tok_stride, io.q_head_stride = 0x30000, 512, 128
    io.k, io.k_tok_stride, io.k_head_stride = 0x40000, 512, 128
    io.v, io.v_tok_stride, io.v_head_stride = 0x50000, 512, 128
    io.a, io.b, io.gate_tok_stride = 0x60000, 0x70000, 4
    io.out, io.out_tok_stride, io.out_head_stride = 0x80000, 512, 128
    io.num_tokens, io.scale = 16, 1.0
    return io


ROWS = C.c_void_p(0x90000)


def verify(lib, pools, io, layer=0, rows=4, slot=ROWS, rec=ROWS):
    return lib.gdn_verify(C.byref(pools) if pools is not None else None, layer, rows, slot, rec,
                          ROWS, ROWS, None, C.byref(io) if io is not None else None, None, None)


def test_verify_zero_rows_is_ok_without_launch(lib):
    assert verify(lib, good_pools(), good_io(), rows=0) == OK


@pytest.mark.parametrize("mutate,status", [
    (lambda p, io: None, None),
    (lambda p, io: setattr(p, "head_k_dim", 64), E_SHAPE),
    (lambda p, io: setattr(p, "head_v_dim", 256), E_SHAPE),
    (lambda p, io: setattr(p, "num_k_heads", 3), E_SHAPE),
    (lambda p, io: setattr(p, "num_layers", 0), E_SHAPE),
    (lambda p, io: setattr(p, "num_layers", 65), E_SHAPE),
    (lambda p, io: setattr(p, "rec_tokens", 0), E_SHAPE),
    (lambda p, io: setattr(p, "rec_tokens", 17), E_SHAPE),
    (lambda p, io: setattr(p, "num_state_slots", 0), E_SHAPE),
    (lambda p, io: setattr(p, "state_dtype", 2), E_DTYPE),
    (lambda p, io: setattr(p, "record_kind", 3), E_SHAPE),
    (lambda p, io: setattr(p, "record_kind", 2), E_SHAPE),    # channel records, scalar gates
    (lambda p, io: setattr(io, "gate_mode", 2), E_SHAPE),     # channel gates, scalar records
    (lambda p, io: setattr(io, "gate_mode", 3), E_SHAPE),
    (lambda p, io: p.state.__setitem__(0, 0), E_NULL),
    (lambda p, io: p.rec.__setitem__(0, 0), E_NULL),
    (lambda p, io: p.state.__setitem__(0, 0x10004), E_ALIGN),
    (lambda p, io: setattr(io, "q", None), E_NULL),
    (lambda p, io: setattr(io, "out", None), E_NULL),
    (lambda p, io: setattr(io, "q", 0x30008), E_ALIGN),
    (lambda p, io: setattr(io, "k_tok_stride", 516), E_ALIGN),
    (lambda p, io: setattr(io, "out_head_stride", 130), E_ALIGN),
    (lambda p, io: setattr(io, "a", 0x60002), E_ALIGN),
    (lambda p, io: setattr(io, "gate_mode", 2), E_SHAPE),
    (lambda p, io: setattr(io, "out_dtype", 2), E_DTYPE),
    (lambda p, io: setattr(io, "gate_mode", 1), E_NULL),                  # raw gates, no A_log
    (lambda p, io: (setattr(io, "gate_mode", 1), setattr(io, "A_log", 0x90000),
                    setattr(io, "dt_bias", 0x90102)), E_ALIGN),
    (lambda p, io: (setattr(io, "out_dtype", 1), setattr(io, "out", 0x80004)), E_ALIGN),
    (lambda p, io: setattr(io, "out", 0x80008), E_ALIGN),                 # fp32 out: 16-byte rule
    (lambda p, io: setattr(io, "num_tokens", -1), E_SHAPE),
    (lambda p, io: setattr(io, "v_head_stride", -8), E_SHAPE),
])
def test_verify_rejects_malformed(lib, mutate, status):
    p, io = good_pools(), good_io()
    mutate(p, io)
    if status is None:
        # the unmodified arguments are valid: only check with zero rows (no launch)
        assert verify(lib, p, io, rows=0) == OK
        return
    assert verify(lib, p, io) == status


def test_verify_accepts_raw_gates_and_bf16_out(lib):
    io = good_io()
    io.gate_mode, io.A_log, io.dt_bias = 1, 0x90000, 0x90100
    io.out_dtype, io.out = 1, 0x80008          # bf16 output: 8-byte pieces
    assert verify(lib, good_pools(), io, rows=0) == OK


def test_verify_channel_decays(lib):
    """Per-channel decays need the channel record kind, a 16-byte aligned a and
    a token stride of at least HV * 128 in multiples of 4."""
    p = good_pools()
    p.record_kind = 2
    io = good_io()
    io.gate_mode, io.decay_tok_stride = 2, 4 * 128
    assert verify(lib, p, io, rows=0) == OK
    io.decay_tok_stride = 4 * 128 - 4
    assert verify(lib, p, io) == E_SHAPE
    io.decay_tok_stride = 4 * 128 + 2
    assert verify(lib, p, io) == E_ALIGN
    io.decay_tok_stride, io.a = 4 * 128, 0x60004
    assert verify(lib, p, io) == E_ALIGN
    io.a, io.decay_tok_stride = 0x60000, -4
    assert verify(lib, p, io) == E_SHAPE


def test_payload_records_reject_a_ring_base(lib):
    p = good_pools()
    p.record_kind = 1
    assert lib.gdn_verify(C.byref(p), 0, 4, ROWS, ROWS, ROWS, ROWS, ROWS, C.byref(good_io()),
                          None, None) == E_SHAPE
    assert verify(lib, p, good_io(), rows=0) == OK


def test_verify_rejects_bad_layer_and_rows(lib):
    assert verify(lib, good_pools(), good_io(), layer=2) == E_SHAPE
    assert verify(lib, good_pools(), good_io(), layer=-1) == E_SHAPE
    assert verify(lib, good_pools(), good_io(), rows=-1) == E_SHAPE
    assert verify(lib, None, good_io()) == E_NULL
    assert verify(lib, good_pools(), None) == E_NULL
    assert verify(lib, good_pools(), good_io(), slot=None) == E_NULL


def commit(lib, pools, rows=4, bl=None, bs=None, src=ROWS):
    return lib.gdn_commit_all_layers(C.byref(pools), rows, src, ROWS, ROWS, ROWS, bl, bs, None,
                                     None)


def test_commit_rejects_malformed(lib):
    assert commit(lib, good_pools(), rows=0) == OK
    assert commit(lib, good_pools(), rows=-3) == E_SHAPE
    assert commit(lib, good_pools(), src=None) == E_NULL
    assert commit(lib, good_pools(), bl=ROWS, bs=None) == E_NULL
    p = good_pools()
    p.rec[1] = 0                      # every layer's pools must be present
    assert commit(lib, p) == E_NULL
    p = good_pools()
    p.state[1] = 0x10008
    assert commit(lib, p) == E_ALIGN
    p = good_pools()
    p.num_v_heads = 5
    assert commit(lib, p) == E_SHAPE


def test_launch_size_limits(lib):
    """A launch counts its work-items in 32 bits. Verify (and the native
    window) run 512 work-items per (row, value head): 2^32 / 512 = 8,388,608
    pairs is one too many. The commit splits its layers over several launches,
    but one layer (8 workgroups of 256 per head, plus 8 of padding) must fit:
    2,097,150 pairs is the most. The native accept copy is one workgroup per
    (layer, row, head). Rejected calls launch nothing (the pointers are fake)."""
    p = good_pools()
    p.num_v_heads, p.num_k_heads = 64, 64
    io = good_io()
    rows = 8_388_608 // 64
    assert verify(lib, p, io, rows=rows) == E_SHAPE
    assert lib.gdn_native_window(C.byref(p), 0, rows, ROWS, ROWS, ROWS, C.byref(io),
                                 C.c_void_p(0xA0000), None, None) == E_SHAPE
    rows = 2_097_152 // 64
    assert commit(lib, p, rows=rows) == E_SHAPE
    snaps = (C.c_void_p * 2)(0xB0000, 0xC0000)
    rows = 16_777_216 // (64 * 2)                      # two layers
    assert lib.gdn_native_accept(C.byref(p), snaps, rows, ROWS, ROWS, None, None) == E_SHAPE


def test_align_plan_rejects_malformed(lib):
    def plan(rows=4, stride=8, cols=8, block=64, max_n=16, table=ROWS):
        return lib.gdn_align_plan(rows, ROWS, ROWS, table, stride, cols, block, max_n,
                                  ROWS, ROWS, ROWS, ROWS, None, None)
    assert plan(rows=0) == OK
    assert plan(block=0) == E_SHAPE
    assert plan(max_n=-1) == E_SHAPE
    assert plan(cols=0) == E_SHAPE
    assert plan(stride=4, cols=8) == E_SHAPE
    assert plan(table=None) == E_NULL


def test_native_rejects_malformed(lib):
    p, io = good_pools(), good_io()
    assert lib.gdn_native_window(C.byref(p), 0, 4, ROWS, ROWS, ROWS, C.byref(io), None, None,
                                 None) == E_NULL
    assert lib.gdn_native_window(C.byref(p), 0, 4, ROWS, ROWS, ROWS, C.byref(io),
                                 C.c_void_p(0xA0004), None, None) == E_ALIGN
    snaps = (C.c_void_p * 2)(0xB0000, 0)
    assert lib.gdn_native_accept(C.byref(p), snaps, 4, ROWS, ROWS, None, None) == E_NULL
    snaps = (C.c_void_p * 2)(0xB0000, 0xC0000)
    assert lib.gdn_native_accept(C.byref(p), snaps, 0, ROWS, ROWS, None, None) == OK


def good_conv(layers=2):
    c = B.gdn_conv_pools()
    c.num_layers, c.channels, c.state_len, c.dtype, c.num_slots = layers, 8192, 3, 1, 8
    c.x_tok_stride, c.num_tokens = 8192, 64
    for i in range(layers):
        c.state[i] = 0xA0000 + i * 0x100000     # never dereferenced: calls below are rejected
        c.x[i] = 0xB0000 + i * 0x100000
    return c


def commit_conv(lib, pools, conv, rows=4, tok=ROWS, rec=ROWS):
    return lib.gdn_commit_all_layers_conv(C.byref(pools) if pools is not None else None,
                                          C.byref(conv) if conv is not None else None, rows,
                                          ROWS, ROWS, rec, ROWS, None, None, tok, None, None)


def test_commit_conv_validation(lib):
    assert commit_conv(lib, good_pools(), good_conv(), rows=0) == OK
    assert commit_conv(lib, None, good_conv(), rows=0, rec=None) == OK   # conv states only
    assert commit_conv(lib, good_pools(), None, rows=0) == OK             # plain commit
    assert commit_conv(lib, None, None) == E_NULL
    assert commit_conv(lib, good_pools(), good_conv(), tok=None) == E_NULL
    assert commit_conv(lib, good_pools(), good_conv(layers=3)) == E_SHAPE
    c = good_conv(); c.dtype = 2
    assert commit_conv(lib, None, c) == E_DTYPE
    c = good_conv(); c.state_len = 0
    assert commit_conv(lib, None, c) == E_SHAPE
    c = good_conv(); c.state_len = 1025
    assert commit_conv(lib, None, c) == E_SHAPE
    c = good_conv(); c.channels = 12; c.x_tok_stride = 16          # 24-byte bf16 rows
    assert commit_conv(lib, None, c) == E_ALIGN
    c = good_conv(); c.x_tok_stride = 8196                            # 16392-byte token stride
    assert commit_conv(lib, None, c) == E_ALIGN
    c = good_conv(); c.x_tok_stride = 4096                            # shorter than a row
    assert commit_conv(lib, None, c) == E_SHAPE
    c = good_conv(); c.x[1] = None
    assert commit_conv(lib, None, c) == E_NULL
    c = good_conv(); c.state[0] = 0xA0008
    assert commit_conv(lib, None, c) == E_ALIGN


def test_bandwidth_probe_rejects_bad_arguments(lib):
    fake = C.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced
    odd = C.c_void_p((1 << 20) + 8)
    chunk = B.GDN_PROBE_CHUNK
    assert lib.gdn_bandwidth_probe(3, fake, fake, chunk, None) == E_SHAPE
    assert lib.gdn_bandwidth_probe(-1, fake, fake, chunk, None) == E_SHAPE
    assert lib.gdn_bandwidth_probe(B.PROBE_COPY, fake, fake, 0, None) == E_SHAPE
    assert lib.gdn_bandwidth_probe(B.PROBE_COPY, fake, fake, chunk + 16, None) == E_SHAPE
    assert lib.gdn_bandwidth_probe(B.PROBE_COPY, fake, fake, chunk * (1 << 31), None) == E_SHAPE
    assert lib.gdn_bandwidth_probe(B.PROBE_COPY, None, fake, chunk, None) == E_NULL
    assert lib.gdn_bandwidth_probe(B.PROBE_READ, None, fake, chunk, None) == E_NULL
    assert lib.gdn_bandwidth_probe(B.PROBE_WRITE, None, None, chunk, None) == E_NULL
    assert lib.gdn_bandwidth_probe(B.PROBE_COPY, odd, fake, chunk, None) == E_ALIGN
    assert lib.gdn_bandwidth_probe(B.PROBE_WRITE, None, odd, chunk, None) == E_ALIGN


def test_check_slots_rejects_bad_arguments(lib):
    fake = C.c_void_p(1 << 20)
    assert lib.gdn_check_slots(-1, fake, fake, None, fake, None, None, fake, None) == E_SHAPE
    assert lib.gdn_check_slots(4, None, fake, None, fake, None, None, fake, None) == E_NULL
    assert lib.gdn_check_slots(4, fake, None, None, fake, None, None, fake, None) == E_NULL
    assert lib.gdn_check_slots(4, fake, fake, None, None, None, None, fake, None) == E_NULL
    assert lib.gdn_check_slots(4, fake, fake, None, fake, None, None, None, None) == E_NULL
    assert lib.gdn_check_slots(4, fake, fake, None, fake, fake, None, fake, None) == E_NULL
    assert lib.gdn_check_slots(0, fake, fake, None, fake, None, None, fake, None) == OK


def test_headers_are_plain_c_and_link_against_the_library(tmp_path, lib):
    """The public headers compile as strict C99 (no C++ or HIP headers needed),
    every declared function can be referenced from C, and a C program linked
    against the library gets the documented results of calls that need no GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    names = declared_functions()
    src = tmp_path / "abi.c"
    src.write_text(
        "#include <stdio.h>\n#include \"gdn_replay.h\"\n#include \"gdn_probe.h\"\n"
        "int main(void) {\n"
        "    typedef void (*fn_t)(void);\n"
        "    const fn_t fns[] = {" + ", ".join(f"(fn_t)&{n}" for n in names) + "};\n"
        "    unsigned i;\n"
        "    for (i = 0; i < sizeof fns / sizeof fns[0]; ++i) if (!fns[i]) return 10;\n"
        f"    if (gdn_abi_version() != {lib.gdn_abi_version()}) return 11;\n"
        "    if (gdn_verify(NULL, 0, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != GDN_ERR_NULL) return 12;\n"
        "    if (gdn_commit_all_layers(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != GDN_ERR_NULL) return 13;\n"
        "    printf(\"%s\\n\", gdn_status_string(GDN_ERR_ALIGN));\n"
        "    return 0;\n}\n")
    exe = tmp_path / "abi"
    libdir = os.path.dirname(B.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-lgdnreplay", f"-Wl,-rpath,{libdir}",
           "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.startswith("a pointer or stride")
