"""The C-ABI library loads on a machine without a GPU, exports every entry
point include/pic_stitch.h declares, and the binding's ctypes structs have
the C layout (checked against a C program compiled from the header)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import position_independent_kv_stitch_amd as pic
from position_independent_kv_stitch_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pic_stitch.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pic_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    lib = C.CDLL(pic.LIBRARY)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pic.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (pic_\w+)", out))
    assert set(names) <= exported


STRUCTS = {
    "pic_rope_config": B.RopeConfig, "pic_kv_shape": B.KvShape, "pic_chunk": B.ChunkC,
    "pic_entry": B.EntryC, "pic_request": B.RequestC, "pic_geom": B.Geom, "pic_attend_args": B.AttendArgs,
    "pic_kv_view": B.KvView, "pic_segment": B.SegmentC, "pic_page_segment": B.PageSegmentC,
    "pic_plan_info_t": B.PlanInfo,
    "pic_cdc_config": B.CdcConfig, "pic_match_t": B.MatchRecord,
    "pic_attend_latent_args": B.LatentArgs, "pic_attend_boundary_args": B.BoundaryArgs,
}


def test_struct_layout_matches_header(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "pic_stitch.h"',
             "int main(void) {"]
    for cname, cls in STRUCTS.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, cls in STRUCTS.items():
        assert got[(cname, "size")] == C.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_calls_fail_cleanly_without_device_work():
    """Invalid handles and views are refused before any device call."""
    lib = B.load_library()
    view = B.KvView(None, None, 0, 0, 0, 0, 0)
    assert lib.pic_stitch(None, C.byref(view), C.byref(view), 0, 1, None) == B.PIC_ERR_STATE
    assert b"plan" in lib.pic_last_error()
    info = B.PlanInfo()
    assert lib.pic_plan_info(None, C.byref(info)) == B.PIC_ERR_STATE
    lib.pic_plan_destroy(None)  # no-op


def test_last_error_is_thread_local():
    import threading
    lib = B.load_library()
    lib.pic_plan_info(None, None)
    seen = []

    def other():
        seen.append(lib.pic_last_error())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [b""]
    assert lib.pic_last_error() != b""


@pytest.mark.parametrize("mod", ["oracle", "oracle.ref"])
def test_product_does_not_import_oracle(mod):
    """The library's package never imports the oracle."""
    pkg = os.path.join(ROOT, "position_independent_kv_stitch_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text
                assert "pic_oracle" not in text and "orc_" not in text


def test_match_and_registry_errors_before_device_work():
    """pic_match and the registry calls refuse bad arguments before any
    device call (so these run without a GPU)."""
    lib = B.load_library()
    reg = C.c_void_p()
    assert lib.pic_registry_create(7, C.byref(reg)) == B.PIC_ERR_INVALID_ARG
    assert lib.pic_registry_create(B.FP_KINDS["sha256"], C.byref(reg)) == B.PIC_OK
    fp = (C.c_uint8 * 32)(*range(32))
    assert lib.pic_registry_add(reg, fp, 0, 1) == B.PIC_ERR_RANGE
    assert lib.pic_registry_add(reg, fp, 5, -1) == B.PIC_ERR_RANGE
    assert lib.pic_registry_add(reg, None, 5, 1) == B.PIC_ERR_INVALID_ARG
    assert lib.pic_registry_add(reg, fp, 5, 1) == B.PIC_OK
    assert lib.pic_registry_add(reg, fp, 5, 2) == B.PIC_ERR_OVERLAP
    assert lib.pic_registry_add(reg, fp, 6, 2) == B.PIC_OK
    assert lib.pic_registry_add(None, fp, 6, 2) == B.PIC_ERR_STATE

    tok, out, n_out = C.c_void_p(0x10000), C.c_void_p(0x20000), C.c_void_p(0x30000)

    def call(cfg, n=100, max_out=10, r=None, t=tok, o=out, no=n_out):
        return lib.pic_match(r, C.byref(cfg) if cfg is not None else None, t, n, o, max_out,
                             no, None)

    good = B.CdcConfig(1 << 56, 0, 0, B.FP_KINDS["xxh64"], 128)
    assert call(None) == B.PIC_ERR_INVALID_ARG
    assert call(B.CdcConfig(1 << 56, 0, 0, 9, 128)) == B.PIC_ERR_INVALID_ARG
    assert call(good, r=reg) == B.PIC_ERR_INVALID_ARG  # registry holds SHA-256 fingerprints
    assert b"fingerprint kind" in lib.pic_last_error()
    assert call(good, n=-1) == B.PIC_ERR_RANGE
    assert call(good, n=1 << 31) == B.PIC_ERR_RANGE
    assert call(B.CdcConfig(1 << 56, 0, 0, 0, -1)) == B.PIC_ERR_RANGE
    assert call(good, max_out=-1) == B.PIC_ERR_RANGE
    assert call(good, no=None) == B.PIC_ERR_INVALID_ARG
    assert call(good, t=None) == B.PIC_ERR_INVALID_ARG
    assert call(good, o=None) == B.PIC_ERR_INVALID_ARG
    assert call(good, t=C.c_void_p(0x10002)) == B.PIC_ERR_ALIGN
    assert call(good, o=C.c_void_p(0x20004)) == B.PIC_ERR_ALIGN
    assert call(good, no=C.c_void_p(0x30004)) == B.PIC_ERR_ALIGN
    lib.pic_registry_destroy(reg)
    lib.pic_registry_destroy(None)


# ------------------------------------------------- one HIP runtime per process

def _maps_line(path, addr="7f0000000000-7f0000100000"):
    return f"{addr} r-xp 00000000 08:01 1234 {path}\n"


def test_runtime_guard_accepts_one_runtime():
    """Several mappings of one runtime file (text, data, bss segments), plus
    other libraries and anonymous mappings, pass."""
    from position_independent_kv_stitch_amd import _binding as B
    lines = [_maps_line("/opt/rocm/lib/libamdhip64.so.7.2.0"),
             _maps_line("/opt/rocm/lib/libamdhip64.so.7.2.0", "7f0000100000-7f0000200000"),
             _maps_line("/usr/lib/libc.so.6"),
             "7ffd00000000-7ffd00021000 rw-p 00000000 00:00 0 [stack]\n",
             "7f0000300000-7f0000400000 rw-p 00000000 00:00 0\n"]
    B.check_single_runtime(lines, resolve=lambda p: p)
    assert B.hip_runtimes(lines, resolve=lambda p: p) == {"/opt/rocm/lib/libamdhip64.so.7.2.0"}
    B.check_single_runtime([], resolve=lambda p: p)  # no runtime mapped yet


def test_runtime_guard_refuses_two_runtimes():
    """torch's bundled runtime and ROCm's, both mapped: refused, naming both."""
    from position_independent_kv_stitch_amd import _binding as B
    torch_rt = "/usr/lib/python3/site-packages/torch/lib/libamdhip64.so"
    rocm_rt = "/opt/rocm/lib/libamdhip64.so.7"
    lines = [_maps_line(torch_rt), _maps_line(rocm_rt, "7f0000500000-7f0000600000")]
    with pytest.raises(ImportError) as e:
        B.check_single_runtime(lines, resolve=lambda p: p)
    assert torch_rt in str(e.value) and rocm_rt in str(e.value)


def test_runtime_guard_resolves_links_to_one_file():
    """Two names of one file (a soname link and its target) are one runtime."""
    from position_independent_kv_stitch_amd import _binding as B
    real = "/opt/rocm/lib/libamdhip64.so.7.2.0"
    links = {"/opt/rocm/lib/libamdhip64.so": real, real: real}
    lines = [_maps_line("/opt/rocm/lib/libamdhip64.so"), _maps_line(real)]
    B.check_single_runtime(lines, resolve=links.get)


def test_runtime_guard_on_this_process():
    """The package imported here (with torch) maps at most one runtime."""
    from position_independent_kv_stitch_amd import _binding as B
    assert len(B.hip_runtimes()) <= 1


def test_noalloc_refuses_metadata_beyond_its_array():
    """pic_rotate_inplace_noalloc checks the size of its staged metadata
    against its 4 MiB array before any device work: 140,000 one-token
    segments (32-byte tiles) need more, and are refused with PIC_ERR_RANGE
    (the view is a dummy: nothing is dereferenced)."""
    lib = B.load_library()
    shape, rope, keep = B._shape_and_rope("bf16", 1, 8, 128, 0, 128, "half", 1e6, False, None)
    n = 140_000
    segs = (B.SegmentC * n)()
    for i in range(n):
        segs[i] = B.SegmentC(2 * i, 1, 1, 0)
    view = B.KvView(0x10000, None, 0, 8 * 128, 128, 0, 0)
    st = lib.pic_rotate_inplace_noalloc(C.byref(shape), C.byref(rope), C.byref(view), 2 * n, segs,
                                        n, 0, 1, None)
    assert st == B.PIC_ERR_RANGE, lib.pic_last_error()
    assert b"static scratch" in lib.pic_last_error()
