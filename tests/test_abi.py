"""The C ABI library loads and exports what include/nf4.h declares; host-side
argument validation rejects bad arguments before anything is launched.  No
compute call is made here (these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import w4a16_gemv_amd as nf4
    if not os.path.exists(nf4.LIB_PATH):
        from w4a16_gemv_amd import build
        build.build()
    return nf4.load()


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn), encoding="utf-8").read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**((?:nf4|int4)_\w+)\s*\(", src,
                                flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("nf4_dequant", "nf4_gemv", "nf4_abi_version", "nf4_status_string",
                     "int4_dequant", "int4_gemv", "int4_quantize"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    import w4a16_gemv_amd as nf4
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(nf4.EXPORTED) >= set(declared_functions())


def test_abi_version_and_status_strings(lib):
    assert lib.nf4_abi_version() == 1
    for st in range(4):
        assert lib.nf4_status_string(st).decode().startswith("NF4_")
    assert b"unknown" in lib.nf4_status_string(99)


FAKE = C.c_void_p(0x1000)   # never dereferenced: validation fails first


def _dq(lib, n=16, bs=64, s2=256, dtype=0, packed=FAKE, out=FAKE):
    return lib.nf4_dequant(packed, FAKE, FAKE, FAKE, C.c_float(0.0), n, bs, s2, out, dtype, None)


def _gv(lib, N=4, K=64, bs=64, s2=256, batch=1, x=FAKE, y=FAKE, packed=FAKE):
    return lib.nf4_gemv(packed, FAKE, FAKE, FAKE, C.c_float(0.0), N, K, bs, s2, x, batch, y, None)


@pytest.mark.parametrize("kw", [dict(n=-1), dict(bs=0), dict(bs=48), dict(bs=-64),
                                dict(s2=0), dict(s2=3), dict(bs=3), dict(bs=2 ** 31 - 1),
                                dict(dtype=2), dict(dtype=-1), dict(packed=None), dict(out=None)])
def test_dequant_rejects_bad_arguments(lib, kw):
    assert _dq(lib, **kw) == 1


def test_dequant_empty_is_a_no_op(lib):
    assert lib.nf4_dequant(None, None, None, None, C.c_float(0.0), 0, 64, 256, None, 0, None) == 0


@pytest.mark.parametrize("kw", [dict(N=-1), dict(K=-2), dict(K=63), dict(batch=0), dict(batch=9),
                                dict(bs=24), dict(s2=0), dict(x=None), dict(y=None),
                                dict(packed=None)])
def test_gemv_rejects_bad_arguments(lib, kw):
    assert _gv(lib, **kw) == 1


def test_gemv_empty_is_a_no_op(lib):
    assert lib.nf4_gemv(None, None, None, None, C.c_float(0.0), 0, 64, 64, 256, None, 1, None,
                        None) == 0


def test_oversized_requests_are_unsupported(lib):
    assert _dq(lib, n=1 << 41) == 2
    assert _gv(lib, N=1 << 30, K=1 << 12) == 2


def test_code2_linear_table_matches_oracle(lib):
    """The library's host-side code2 table (independent code) equals the
    oracle's: fp16 nearest to -1 + 2 i / 255."""
    import numpy as np

    import oracle
    import w4a16_gemv_amd as nf4
    assert np.array_equal(nf4.nf4_code2_linear().numpy().view(np.uint16), oracle.code2_linear())


def test_quantize_workspace_size(lib):
    assert lib.nf4_quantize_workspace_size(0, 64) == 0
    ws = lib.nf4_quantize_workspace_size(1 << 20, 64)
    assert ws >= (1 << 14) * 4          # one fp32 absmax per block


@pytest.mark.parametrize("kw", [dict(n=-1), dict(bs=3), dict(s2=0), dict(w=None),
                                dict(ws_bytes=16), dict(ws=C.c_void_p(0x1010))])
def test_quantize_rejects_bad_arguments(lib, kw):
    n = kw.get("n", 4096)
    ws_bytes = kw.get("ws_bytes", 1 << 20)
    rc = lib.nf4_quantize(kw.get("w", FAKE), n, kw.get("bs", 64), kw.get("s2", 256), FAKE, FAKE,
                          FAKE, FAKE, FAKE, kw.get("ws", FAKE), ws_bytes, None)
    assert rc == 1


def test_gemv_sched_size(lib):
    assert lib.nf4_gemv_sched_size() >= 8 * 4


@pytest.mark.parametrize("kw", [dict(sched=C.c_void_p(0x1010)),            # misaligned
                                dict(sched_bytes=16),                       # too small
                                dict(K=63), dict(bs=3), dict(count=-1),
                                dict(descs=None), dict(code2=None)])
def test_gemv_grouped_rejects_bad_arguments(lib, kw):
    sched = kw.get("sched", C.c_void_p(0x1000))
    sched_bytes = kw.get("sched_bytes", lib.nf4_gemv_sched_size())
    rc = lib.nf4_gemv_grouped(kw.get("descs", FAKE), kw.get("count", 2), 100, kw.get("K", 64),
                              kw.get("bs", 64), 256, kw.get("code2", FAKE), 1, sched,
                              sched_bytes, None)
    assert rc == 1


def test_gemv_grouped_empty_is_a_no_op(lib):
    assert lib.nf4_gemv_grouped(None, 0, 0, 64, 64, 256, None, 1, None, 0, None) == 0


@pytest.mark.parametrize("fn", ["nf4_gemv_grouped_absmax32", "int4_gemv_grouped"])
@pytest.mark.parametrize("kw,expect", [
    (dict(sched=C.c_void_p(0x1010)), 1),        # misaligned workspace
    (dict(sched_bytes=16), 1),                   # too small
    (dict(K=63), 1), (dict(bs=3), 1), (dict(bs=0), 1), (dict(count=-1), 1),
    (dict(descs=None), 1), (dict(descs=C.c_void_p(0x1004)), 1),   # NULL / misaligned descs
    (dict(bs=16), 2), (dict(K=96 + 16), 2), (dict(batch=9), 2), (dict(count=1025), 2),
])
def test_grouped_formats_reject_bad_arguments(lib, fn, kw, expect):
    sched = kw.get("sched", C.c_void_p(0x1000))
    sched_bytes = kw.get("sched_bytes", lib.nf4_gemv_sched_size())
    rc = getattr(lib, fn)(kw.get("descs", FAKE), kw.get("count", 2), 100, kw.get("K", 64),
                          kw.get("bs", 64), kw.get("batch", 1), sched, sched_bytes, None)
    assert rc == expect


@pytest.mark.parametrize("fn", ["nf4_gemv_grouped_absmax32", "int4_gemv_grouped"])
def test_grouped_formats_empty_is_a_no_op(lib, fn):
    assert getattr(lib, fn)(None, 0, 0, 64, 64, 1, None, 0, None) == 0
    assert getattr(lib, fn)(None, 3, 0, 64, 64, 1, None, 0, None) == 0


def test_descriptor_layouts_match():
    """The three descriptor types have the same 64-byte layout (the binding
    writes all of them through one record type)."""
    import numpy as np

    from w4a16_gemv_amd._binding import _DESC_DTYPE
    assert np.dtype(_DESC_DTYPE).itemsize == 64
    src = open(os.path.join(ROOT, "include", "nf4.h"), encoding="utf-8").read()
    src += open(os.path.join(ROOT, "include", "int4.h"), encoding="utf-8").read()
    for name in ("nf4_gemv_desc", "nf4_absmax32_gemv_desc", "int4_gemv_desc"):
        body = re.search(r"typedef struct " + name + r" \{(.*?)\} " + name + ";", src, re.S)
        assert body, name
        fields = re.findall(r"^\s*([\w\s\*]+?)\s*(\w+);", re.sub(r"/\*.*?\*/", "", body.group(1)),
                            flags=re.M)
        assert len(fields) == 9, (name, fields)


def _dq32(lib, n=16, bs=64, dtype=0, packed=FAKE, absmax=FAKE, out=FAKE):
    return lib.nf4_dequant_absmax32(packed, absmax, n, bs, out, dtype, None)


def _gv32(lib, N=4, K=64, bs=64, batch=1, x=FAKE, y=FAKE, packed=FAKE, absmax=FAKE):
    return lib.nf4_gemv_absmax32(packed, absmax, N, K, bs, x, batch, y, None)


@pytest.mark.parametrize("kw", [dict(n=-1), dict(bs=0), dict(bs=48), dict(bs=2 ** 31 - 1),
                                dict(dtype=2), dict(packed=None), dict(absmax=None),
                                dict(out=None), dict(absmax=C.c_void_p(0x1002))])
def test_dequant_absmax32_rejects_bad_arguments(lib, kw):
    assert _dq32(lib, **kw) == 1


@pytest.mark.parametrize("kw", [dict(N=-1), dict(K=-2), dict(K=63), dict(batch=0), dict(batch=9),
                                dict(bs=24), dict(x=None), dict(y=None), dict(packed=None),
                                dict(absmax=None), dict(absmax=C.c_void_p(0x1001))])
def test_gemv_absmax32_rejects_bad_arguments(lib, kw):
    assert _gv32(lib, **kw) == 1


def test_absmax32_empty_and_oversized(lib):
    assert lib.nf4_dequant_absmax32(None, None, 0, 64, None, 0, None) == 0
    assert lib.nf4_gemv_absmax32(None, None, 0, 64, 64, None, 1, None, None) == 0
    assert _dq32(lib, n=1 << 41) == 2
    assert _gv32(lib, N=1 << 30, K=1 << 12) == 2


@pytest.mark.parametrize("kw", [dict(n=-1), dict(bs=3), dict(w=None), dict(packed=None),
                                dict(absmax=None), dict(absmax=C.c_void_p(0x1002))])
def test_quantize_absmax32_rejects_bad_arguments(lib, kw):
    rc = lib.nf4_quantize_absmax32(kw.get("w", FAKE), kw.get("n", 4096), kw.get("bs", 64),
                                   kw.get("packed", FAKE), kw.get("absmax", FAKE), None)
    assert rc == 1
    assert lib.nf4_quantize_absmax32(None, 0, 64, None, None, None) == 0


@pytest.mark.parametrize("kw", [dict(n=-1), dict(G=1), dict(G=48), dict(G=0), dict(dtype=2),
                                dict(packed=None), dict(scales=None), dict(zeros=None),
                                dict(out=None)])
def test_int4_dequant_rejects_bad_arguments(lib, kw):
    rc = lib.int4_dequant(kw.get("packed", FAKE), kw.get("scales", FAKE), kw.get("zeros", FAKE),
                          kw.get("n", 4096), kw.get("G", 128), kw.get("out", FAKE),
                          kw.get("dtype", 0), None)
    assert rc == 1


@pytest.mark.parametrize("kw", [dict(N=-1), dict(K=63), dict(batch=0), dict(batch=9), dict(G=3),
                                dict(x=None), dict(y=None), dict(packed=None), dict(zeros=None)])
def test_int4_gemv_rejects_bad_arguments(lib, kw):
    rc = lib.int4_gemv(kw.get("packed", FAKE), FAKE, kw.get("zeros", FAKE), kw.get("N", 4),
                       kw.get("K", 256), kw.get("G", 128), kw.get("x", FAKE), kw.get("batch", 1),
                       kw.get("y", FAKE), None)
    assert rc == 1


def test_int4_empty_oversized_and_quantize_validation(lib):
    assert lib.int4_dequant(None, None, None, 0, 128, None, 0, None) == 0
    assert lib.int4_gemv(None, None, None, 0, 256, 128, None, 1, None, None) == 0
    assert lib.int4_dequant(FAKE, FAKE, FAKE, 1 << 41, 128, FAKE, 0, None) == 2
    assert lib.int4_gemv(FAKE, FAKE, FAKE, 1 << 30, 1 << 12, 128, FAKE, 1, FAKE, None) == 2
    assert lib.int4_quantize(FAKE, 4096, 1, FAKE, FAKE, FAKE, None) == 1
    assert lib.int4_quantize(None, 4096, 128, FAKE, FAKE, FAKE, None) == 1
    assert lib.int4_quantize(None, 0, 128, None, None, None, None) == 0


def _gm(lib, M=16, N=4, K=64, bs=64, s2=256, x=FAKE, y=FAKE, packed=FAKE, ws=None):
    return lib.nf4_gemm(packed, FAKE, FAKE, FAKE, C.c_float(0.0), M, N, K, bs, s2, x, y, ws, 0,
                        None)


@pytest.mark.parametrize("kw", [dict(M=-1), dict(N=-1), dict(K=-2), dict(K=63), dict(bs=24),
                                dict(s2=0), dict(x=None), dict(y=None), dict(packed=None),
                                dict(ws=C.c_void_p(0x1008))])
def test_gemm_rejects_bad_arguments(lib, kw):
    assert _gm(lib, **kw) == 1


def test_gemm_empty_and_oversized(lib):
    assert lib.nf4_gemm(None, None, None, None, C.c_float(0.0), 0, 64, 64, 64, 256, None, None,
                        None, 0, None) == 0
    assert lib.nf4_gemm(None, None, None, None, C.c_float(0.0), 16, 0, 64, 64, 256, None, None,
                        None, 0, None) == 0
    assert _gm(lib, M=1 << 30) == 2
    assert _gm(lib, N=1 << 30, K=1 << 12) == 2


def test_probes_validate_arguments(lib):
    assert lib.nf4_probe_stream_read(None, 0, None, None) == 0
    assert lib.nf4_probe_stream_read(None, 64, FAKE, None) == 1
    assert lib.nf4_probe_stream_read(C.c_void_p(0x1008), 64, FAKE, None) == 1   # misaligned
    assert lib.nf4_probe_stream_read(FAKE, 40, FAKE, None) == 1                  # not 16 * k
    assert lib.nf4_probe_expand_copy(None, 0, None, None) == 0
    assert lib.nf4_probe_expand_copy(FAKE, 64, None, None) == 1
    assert lib.nf4_probe_expand_copy(FAKE, 64, C.c_void_p(0x1008), None) == 1   # dst misaligned
    assert lib.nf4_probe_expand_copy(FAKE, 6, FAKE, None) == 1                   # not 4 * k


@pytest.mark.parametrize("kw,expect", [
    (dict(K=63), 1), (dict(bs=3), 1), (dict(s2=0), 1), (dict(count=-1), 1),
    (dict(descs=None), 1), (dict(code2=None), 1), (dict(descs=C.c_void_p(0x1004)), 1),
    (dict(bs=16), 2), (dict(K=96 + 16), 2), (dict(batch=9), 2), (dict(count=1025), 2),
])
def test_gemv_grouped_noalloc_rejects_bad_arguments(lib, kw, expect):
    """Argument errors come back before any HIP call (and before the scratch
    is looked up)."""
    rc = lib.nf4_gemv_grouped_noalloc(kw.get("descs", FAKE), kw.get("count", 2), 100,
                                      kw.get("K", 64), kw.get("bs", 64), kw.get("s2", 256),
                                      kw.get("code2", FAKE), kw.get("batch", 1), None)
    assert rc == expect


def test_gemv_grouped_noalloc_empty_is_a_no_op(lib):
    assert lib.nf4_gemv_grouped_noalloc(None, 0, 0, 64, 64, 256, None, 1, None) == 0
    assert lib.nf4_gemv_grouped_noalloc(None, 3, 0, 64, 64, 256, None, 1, None) == 0


def _desc_table(Ns, K, align=16):
    """A host descriptor table with fake, suitably aligned pointers."""
    import numpy as np

    from w4a16_gemv_amd._binding import _DESC_DTYPE
    t = np.zeros(len(Ns), dtype=np.dtype(_DESC_DTYPE))
    row = 0
    for i, N in enumerate(Ns):
        base = 0x100000 * (i + 1)
        t[i] = (base, base + 0x40000, base + 0x80000, base + 0xC0000, base + 0xE0000, N, row,
                0.0, 0)
        row += N
    return t, row


def _check(lib, t, total, K, fmt=0):
    bad = C.c_int32(-7)
    rc = lib.nf4_gemv_desc_check(t.ctypes.data if t is not None else None,
                                 0 if t is None else len(t), total, K, fmt, C.byref(bad))
    return rc, bad.value


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_gemv_desc_check_accepts_a_good_table(lib, fmt):
    t, total = _desc_table([64, 3, 0, 4096], 4096)
    assert _check(lib, t, total, 4096, fmt) == (0, -1)


@pytest.mark.parametrize("field,value,fmt,index", [
    ("packed", 0x200008, 0, 1),      # packed not 16-byte aligned
    ("x", 0x2C0004, 0, 1),           # x not 16-byte aligned
    ("y", 0, 0, 1),                  # NULL y
    ("absmax2", 0, 0, 1),            # NULL second scale (formats 0 and 2)
    ("absmax2", 0, 2, 1),
    ("absmax2", 0x280001, 0, 1),     # fp16 absmax2 misaligned
    ("absmax_q", 0x240002, 1, 1),    # fp32 absmax not 4-byte aligned
    ("absmax_q", 0x240001, 2, 1),    # fp16 scales misaligned
    ("N", -1, 0, 1),
    ("row_begin", 63, 0, 1),         # not the running sum of N
    ("N", 1 << 20, 0, 1),            # N * K >= 2^31
])
def test_gemv_desc_check_finds_the_bad_descriptor(lib, field, value, fmt, index):
    t, total = _desc_table([64, 3, 5], 4096)
    t[index][field] = value
    if field == "N":
        total = int(t["N"].sum())
        t[2]["row_begin"] = int(t[0]["N"] + t[1]["N"])
    rc, bad = _check(lib, t, total, 4096, fmt)
    assert (rc, bad) == (1, index)


def test_gemv_desc_check_other_cases(lib):
    t, total = _desc_table([64, 3], 4096)
    assert _check(lib, t, total + 1, 4096) == (1, 2)        # N does not add up
    t1, total1 = _desc_table([64], 4096)
    t1[0]["absmax2"] = 0
    assert _check(lib, t1, total1, 4096, 1) == (0, -1)      # format 1: second slot unused
    assert _check(lib, t, total, 4096, 3)[0] == 1           # unknown format
    assert _check(lib, None, 0, 4096) == (0, -1)            # empty table
    assert lib.nf4_gemv_desc_check(None, 2, 10, 4096, 0, None) == 1


def test_hot_path_kernels_do_not_spill():
    """The build's resource table (from the compiler's kernel-resource-usage
    remarks) lists every hot-path instance with zero scratch; the build itself
    refuses a spilling one, so this checks the table is there and complete."""
    from w4a16_gemv_amd import build
    if not os.path.exists(build.RESOURCES):
        pytest.skip("kernel_resources.txt not written (library built elsewhere)")
    rows = {}
    with open(build.RESOURCES, encoding="utf-8") as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            vgpr, agpr, scratch, occ, lds, name = line.split(None, 5)
            rows[name.strip()] = int(scratch)
    for hot in build.NO_SPILL:
        hits = [n for n in rows if hot in n]
        assert hits, f"{hot} missing from the resource table"
        assert all(rows[n] == 0 for n in hits), f"{hot} spills"


def test_resource_remarks_are_parsed():
    from w4a16_gemv_amd import build
    text = ("x.hip:1:1: remark: Function Name: _Z3foov [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs: 108 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     LDS Size [bytes/block]: 95248 [-Rpass-analysis=kernel-resource-usage]\n")
    res = build.parse_resources(text)
    (name, r), = res.items()
    assert name in ("foo()", "_Z3foov")
    assert r == {"vgpr": 108, "agpr": 0, "scratch": 16, "occupancy": 4, "lds": 95248}
