"""CPU checks of the C ABI: the HIP library loads, exports every function include/growpage.h
declares, and rejects invalid arguments on the host before anything is launched (no GPU needed;
every call below returns during argument validation)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "growpage.h")


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_472_amd import growpage
    if not os.path.exists(growpage.LIB_PATH):
        from paged_kv_cache_472_amd.build import build
        build()
    return growpage.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gp_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_path_calls():
    names = declared_functions()
    for n in ("gp_paged_decode_attn", "gp_update_query_summaries", "gp_score_and_working_set",
              "gp_compact_or_grow", "gp_quantize_pages_int4"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from paged_kv_cache_472_amd import growpage
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(growpage.EXPORTED) == names
    dyn = subprocess.run(["nm", "-D", "--defined-only", growpage.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in dyn.splitlines() if ln.strip()}
    assert set(names) <= exported


def test_version_and_status_strings(lib):
    m = re.search(r"#define\s+GP_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.gp_version() == int(m.group(1))
    assert lib.gp_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4, -5):
        assert lib.gp_status_string(code) not in (b"ok", b"unknown status")
    assert lib.gp_status_string(7) == b"unknown status"


def test_workspace_sizes(lib):
    # a prefix of tile counts (B + 1 ints, 256-byte aligned) plus split partials that grow
    # with the longest context
    small = lib.gp_paged_decode_attn_workspace_size(2, 8, 2, 64, 16, 16)
    big = lib.gp_paged_decode_attn_workspace_size(64, 32, 8, 128, 16, 16384)
    assert small >= 3 * 4 and big > small
    header = ((64 + 1) * 4 + 255) // 256 * 256
    assert (big - header) % (64 * 32 * 130 * 4) == 0
    assert lib.gp_paged_decode_attn_workspace_size(-1, 32, 8, 128, 16, 16384) == 0
    s1 = lib.gp_score_and_working_set_workspace_size(4, 32, 8, 128, 16, 8192)
    s2 = lib.gp_score_and_working_set_workspace_size(8, 32, 8, 128, 16, 8192)
    assert 0 < s1 < s2
    c1 = lib.gp_compact_or_grow_workspace_size(4, 8, 1028, 16, 16384)
    assert c1 > 0 and lib.gp_compact_or_grow_workspace_size(0, 8, 1028, 16, 16384) == 0


def _kv(growpage, D=128, b=16, fake=True, dtype=1):
    p = ctypes.c_void_p(0x1000) if fake else None
    return growpage.GpKvCache(p, p, None, None, None, None, None, 100, b, 8, D, dtype)


def test_invalid_arguments_rejected_on_host(lib):
    from paged_kv_cache_472_amd import growpage
    fake = ctypes.c_void_p(0x1000)
    kv = _kv(growpage)
    # negative batch, null pointers, head_dim 96, page size 24, dtype mismatch, missing workspace
    assert lib.gp_paged_decode_attn(fake, 1, -1, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1,
                                    fake, None, None, 0, None) == -1
    assert lib.gp_paged_decode_attn(None, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1,
                                    fake, None, None, 0, None) == -1
    kv96 = _kv(growpage, D=96)
    assert lib.gp_paged_decode_attn(fake, 1, 4, 32, ctypes.byref(kv96), fake, 8, fake, 128, 0.1,
                                    fake, None, None, 0, None) == -2
    kvb = _kv(growpage, b=24)
    assert lib.gp_paged_decode_attn(fake, 1, 4, 32, ctypes.byref(kvb), fake, 8, fake, 128, 0.1,
                                    fake, None, None, 0, None) == -2
    assert lib.gp_paged_decode_attn(fake, 0, 4, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1,
                                    fake, None, None, 0, None) == -1
    assert lib.gp_paged_decode_attn(fake, 1, 64, 32, ctypes.byref(kv), fake, 1024, fake, 16384,
                                    0.1, fake, None, None, 0, None) == -3
    assert lib.gp_paged_decode_attn(fake, 1, 9000, 32, ctypes.byref(kv), fake, 1024, fake, 16384,
                                    0.1, fake, None, fake, 1 << 40, None) == -2
    # the allocation-free decode: a call whose partials exceed the static buffer is refused on
    # the host (4096 requests of up to 16384 tokens need about 1.2 GB of partials)
    assert lib.gp_paged_decode_attn_noalloc(fake, 1, 4096, 32, ctypes.byref(kv), fake, 1024, fake,
                                            16384, 0.1, fake, None, None, 0, None) == -5
    assert lib.gp_paged_decode_attn_noalloc(None, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 128,
                                            0.1, fake, None, None, 0, None) == -1
    # max_context beyond the block table's reach
    assert lib.gp_paged_decode_attn(fake, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 1000, 0.1,
                                    fake, None, None, 0, None) == -1
    # summaries: bad dtype, H_q * d not a multiple of 4
    assert lib.gp_update_query_summaries(fake, 7, 4, 32, 128, fake, fake, fake, 16, 0.9,
                                         0.999, None) == -1
    assert lib.gp_update_query_summaries(fake, 0, 4, 1, 3, fake, fake, fake, 16, 0.9,
                                         0.999, None) == -2
    # score: p outside (0, 1], C_max not a multiple of 4, missing workspace
    args = lambda p, cmax, ws, wsb: (fake, 1, 4, 32, fake, 16, fake, fake, 2, ctypes.byref(kv),  # noqa: E731
                                     fake, 8, fake, fake, 10000.0, p, 0.1, fake, fake, cmax, fake,
                                     fake, ws, wsb, None)
    assert lib.gp_score_and_working_set(*args(0.0, 128, fake, 1 << 30)) == -1
    assert lib.gp_score_and_working_set(*args(1.5, 128, fake, 1 << 30)) == -1
    assert lib.gp_score_and_working_set(*args(0.99, 126, fake, 1 << 30)) == -2
    assert lib.gp_score_and_working_set(*args(0.99, 128, None, 0)) == -3
    # compact: bad policy, NaN tau, unsupported page size, missing workspace
    cargs = lambda tau, pol, kvx, ws, wsb: (fake, 2, 4, fake, fake, 128, fake, fake, tau, 4, pol,  # noqa: E731
                                            None, ctypes.byref(kvx), fake, fake, 8, fake, fake,
                                            fake, fake, fake, fake, ws, wsb, None)
    assert lib.gp_compact_or_grow(*cargs(0.0, 9, kv, fake, 1 << 30)) == -1
    assert lib.gp_compact_or_grow(*cargs(float("nan"), 0, kv, fake, 1 << 30)) == -1
    for b in (48, 512):   # page sizes 16, 32, 64, 128 and 256 only
        assert lib.gp_compact_or_grow(*cargs(0.0, 0, _kv(growpage, b=b), fake, 1 << 30)) == -2
    # GrowPage-Shrink evicts up to two pages: not with 32-token pages
    assert lib.gp_compact_or_grow(*cargs(0.0, 4, _kv(growpage, b=32), fake, 1 << 30)) == -2
    # mixed-precision caches: bf16 with every pool, pages of 16 or 32 tokens
    assert lib.gp_compact_or_grow(*cargs(0.0, 0, _mixed_kv(growpage, int4=False), fake,
                                         1 << 30)) == -1
    assert lib.gp_compact_or_grow(*cargs(0.0, 0, _mixed_kv(growpage, dtype=0), fake,
                                         1 << 30)) == -2
    assert lib.gp_compact_or_grow(*cargs(0.0, 0, _mixed_kv(growpage, b=64), fake,
                                         1 << 30)) == -2
    assert lib.gp_compact_or_grow(*cargs(0.0, 0, kv, None, 0)) == -3
    # phased form: only PLAN (1), MOVE (2) or both (3)
    for bad in (0, 4, -1):
        assert lib.gp_compact_or_grow_phase(*cargs(0.0, 0, kv, fake, 1 << 30)[:-1], bad,
                                            None) == -1
    # R = 0 and B = 0 are no-ops that succeed without touching anything
    assert lib.gp_compact_or_grow(None, 0, 4, None, None, 128, None, None, 0.0, 4, 0, None,
                                  ctypes.byref(kv), None, None, 8, None, None, None, None, None,
                                  None, None, 0, None) == 0
    assert lib.gp_paged_decode_attn(None, 1, 0, 32, ctypes.byref(kv), None, 8, None, 128, 0.1,
                                    None, None, None, 0, None) == 0


def _mixed_kv(growpage, D=128, b=16, dtype=1, int4=True):
    f = ctypes.c_void_p(0x1000)
    i4 = f if int4 else None
    return growpage.GpKvCache(f, f, f, f, f, f, f, 100, b, 8, D, dtype, i4, i4, i4, i4)


def test_int4_arguments_rejected_on_host(lib):
    from paged_kv_cache_472_amd import growpage
    fake = ctypes.c_void_p(0x1000)
    # a mixed cache must carry the INT4 pools for decode
    kv = _mixed_kv(growpage, int4=False)
    assert lib.gp_paged_decode_attn(fake, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1,
                                    fake, None, fake, 1 << 30, None) == -1
    # quantizer: null cache, negative count, missing pools, fp32 pools, head_dim 96, page 24
    assert lib.gp_quantize_pages_int4(None, fake, 4, None) == -1
    good = _mixed_kv(growpage)
    assert lib.gp_quantize_pages_int4(ctypes.byref(good), fake, -1, None) == -1
    assert lib.gp_quantize_pages_int4(ctypes.byref(good), None, 4, None) == -1
    assert lib.gp_quantize_pages_int4(ctypes.byref(kv), fake, 4, None) == -1
    assert lib.gp_quantize_pages_int4(ctypes.byref(_mixed_kv(growpage, dtype=0)), fake, 4,
                                      None) == -1
    assert lib.gp_quantize_pages_int4(ctypes.byref(_mixed_kv(growpage, D=96)), fake, 4,
                                      None) == -2
    assert lib.gp_quantize_pages_int4(ctypes.byref(_mixed_kv(growpage, b=24)), fake, 4,
                                      None) == -2
    # no pages: a no-op that succeeds without launching
    assert lib.gp_quantize_pages_int4(ctypes.byref(good), None, 0, None) == 0


def test_fused_decode_arguments_rejected_on_host(lib):
    from paged_kv_cache_472_amd import growpage
    fake = ctypes.c_void_p(0x1000)
    kv = _kv(growpage)
    ex = lib.gp_paged_decode_attn_ex
    # negative grid cap; a summary update with no state pool; zero slots
    assert ex(fake, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1, fake, None, None, -1,
              fake, 1 << 30, None) == -1
    upd = growpage.GpSummaryUpdate(fake, fake, fake, None, 16, 0.9, 0.999)
    assert ex(fake, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1, fake, None,
              ctypes.byref(upd), 0, fake, 1 << 30, None) == -1
    upd = growpage.GpSummaryUpdate(fake, fake, fake, fake, 0, 0.9, 0.999)
    assert ex(fake, 1, 4, 32, ctypes.byref(kv), fake, 8, fake, 128, 0.1, fake, None,
              ctypes.byref(upd), 0, fake, 1 << 30, None) == -1
    # the checks of the plain call still apply (head_dim 96)
    kv96 = _kv(growpage, D=96)
    assert ex(fake, 1, 4, 32, ctypes.byref(kv96), fake, 8, fake, 128, 0.1, fake, None, None, 0,
              fake, 1 << 30, None) == -2
    # B = 0 succeeds without launching
    assert ex(None, 1, 0, 32, ctypes.byref(kv), None, 8, None, 128, 0.1, None, None, None, 0,
              None, 0, None) == 0


def test_mixed_boundary_arguments_rejected_on_host(lib):
    from paged_kv_cache_472_amd import growpage
    fake = ctypes.c_void_p(0x1000)
    # scores over a mixed cache: bf16 only, with the fp8 and INT4 key pools
    args = lambda kvx: (fake, kvx.dtype, 4, 32, fake, 16, fake, fake, 2, ctypes.byref(kvx),  # noqa: E731
                        fake, 8, fake, fake, 10000.0, 0.99, 0.1, fake, fake, 128, fake, fake,
                        fake, 1 << 30, None)
    assert lib.gp_score_and_working_set(*args(_mixed_kv(growpage, dtype=0))) == -2
    assert lib.gp_score_and_working_set(*args(_mixed_kv(growpage, int4=False))) == -1
    # compaction of mixed caches: one layer per call; the layers must all be mixed or all uniform
    two = (ctypes.POINTER(growpage.GpKvCache) * 2)()
    m0, m1, u1 = _mixed_kv(growpage), _mixed_kv(growpage), _kv(growpage)
    two[0], two[1] = ctypes.pointer(m0), ctypes.pointer(m1)
    largs = lambda arr: (fake, 2, 4, 2, fake, fake, 128, fake, fake, 0.0, 4, 0, None, arr,  # noqa: E731
                         fake, fake, 8, fake, fake, fake, fake, fake, fake, fake, 1 << 30, 3, None)
    assert lib.gp_compact_or_grow_layers(*largs(two)) == -2
    two[1] = ctypes.pointer(u1)
    assert lib.gp_compact_or_grow_layers(*largs(two)) == -1


def test_binding_structs_match_the_header_layout(tmp_path):
    """The ctypes mirrors of the header's argument structs (gp_kv_cache, gp_summary_update) have the
    header's fields in its order, at the offsets and total size a C compiler gives them: a field
    added on one side only (as tags_present once was) fails here instead of shifting every later
    argument of a call."""
    from paged_kv_cache_472_amd.growpage import GpKvCache, GpSummaryUpdate
    structs = {"gp_kv_cache": GpKvCache, "gp_summary_update": GpSummaryUpdate}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "growpage.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        struct, key, val = ln.split()
        got[(struct, key)] = int(val)
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, cls in structs.items():
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + name + r"\s*;", text).group(1)
        header_fields = re.findall(r"(\w+)\s*(?:,|;)", body)
        assert header_fields == [f for f, _ in cls._fields_], name
        assert ctypes.sizeof(cls) == got[(name, "size")], name
        for field, _ in cls._fields_:
            assert getattr(cls, field).offset == got[(name, field)], (name, field)
