"""The C ABI without a GPU: the library loads, exports what include/pa.h declares,
and rejects bad arguments on the host before launching anything.

Every call here fails validation (or is a documented no-op), so no kernel is
ever launched and no pointer is dereferenced; the fake addresses below are
never touched.
"""

import ctypes
import os
import re

import pytest

import paged_kv_cache_heads_amd as pa
from paged_kv_cache_heads_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("pa.h", "pa_blocks.h")]

PA_OK, NULLP, INVAL, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
A = 0x100000  # a 16-byte aligned fake address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_heads_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = ""
    for h in HEADERS:
        with open(h, encoding="utf-8") as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ["pa_store_kvcache", "pa_qk_norm_rope_store", "pa_decode", "pa_decode_workspace_size", "pa_prefill_varlen",
              "pa_status_string", "pa_last_error", "pa_bm_create", "pa_bm_allocate", "pa_bm_append_batch",
              "pa_bm_prefill_metadata", "pa_xxh64", "pa_store_decode_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"


def test_status_strings(lib):
    for s in range(0, 9):
        assert lib.pa_status_string(s)
    assert lib.pa_status_string(99) == b"unknown status"
    assert lib.pa_version() >= 100


def store(lib, **kw):
    args = dict(k=A, ks=1024, v=A, vs=1024, kc=A, vc=A, slot=A, T=4, hkv=8, d=128, nb=16, bs=256, stream=None)
    args.update(kw)
    return lib.pa_store_kvcache(args["k"], args["ks"], args["v"], args["vs"], args["kc"], args["vc"], args["slot"],
                                args["T"], args["hkv"], args["d"], args["nb"], args["bs"], args["stream"])


def test_store_validation(lib):
    assert store(lib, T=-1) == INVAL
    assert store(lib, k=None) == NULLP
    assert store(lib, slot=None) == NULLP
    assert store(lib, ks=512) == INVAL
    assert store(lib, k=A + 8) == ALIGN
    assert store(lib, vs=1028) == ALIGN
    assert store(lib, nb=0) == INVAL
    assert store(lib, hkv=3, d=5) == ALIGN
    assert store(lib, nb=1 << 24, bs=256) == UNSUP
    assert b"null" in lib.pa_last_error() or lib.pa_last_error()
    # zero tokens: a no-op that needs no pointers
    assert store(lib, T=0, k=None, v=None, kc=None, vc=None, slot=None) == PA_OK


def decode(lib, **kw):
    a = dict(out=A, q=A, qs=2048, kc=A, vc=A, bt=A, W=8, cl=A, B=4, hq=16, hkv=8, d=128, bs=256, maxL=2048,
             scale=0.088, part=0, ws=A, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["W"], a["cl"], a["B"], a["hq"],
                         a["hkv"], a["d"], a["bs"], a["maxL"], a["scale"], a["part"], a["ws"], a["wsb"], a["stream"])


def test_decode_validation(lib):
    assert decode(lib, hq=12) == INVAL           # 12 % 8
    assert decode(lib, hq=24) == UNSUP           # group 3
    assert decode(lib, hq=128) == UNSUP          # group 16
    assert decode(lib, d=64) == UNSUP
    assert decode(lib, bs=100) == UNSUP
    assert decode(lib, bs=0) == INVAL
    assert decode(lib, W=7) == INVAL             # 7 * 256 < 2048
    assert decode(lib, B=-1) == INVAL
    assert decode(lib, B=70000) == UNSUP
    assert decode(lib, part=-1) == INVAL
    assert decode(lib, scale=float("nan")) == INVAL
    assert decode(lib, q=None) == NULLP
    assert decode(lib, cl=None) == NULLP
    assert decode(lib, qs=1024) == INVAL
    assert decode(lib, out=A + 2) == ALIGN
    assert decode(lib, ws=None) == NULLP         # the workspace is always required
    assert decode(lib, wsb=16) == WS
    assert decode(lib, ws=A + 4) == ALIGN
    assert decode(lib, B=0, out=None, q=None, kc=None, vc=None, bt=None, cl=None) == PA_OK


def store_decode(lib, **kw):
    a = dict(out=A, q=A, qs=2048, kn=A, kns=1024, vn=A, vns=1024, kc=A, vc=A, bt=A, W=8, cl=A, B=4, hq=16, hkv=8,
             d=128, bs=256, maxL=2048, scale=0.088, part=0, ws=A, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.pa_store_decode(a["out"], a["q"], a["qs"], a["kn"], a["kns"], a["vn"], a["vns"], a["kc"], a["vc"],
                               a["bt"], a["W"], a["cl"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["maxL"],
                               a["scale"], a["part"], a["ws"], a["wsb"], a["stream"])


def test_store_decode_validation(lib):
    assert store_decode(lib, kn=None) == NULLP
    assert store_decode(lib, vn=None) == NULLP
    assert store_decode(lib, kns=512) == INVAL          # below num_kv_heads * head_dim
    assert store_decode(lib, vns=1028) == ALIGN          # not a multiple of 8 elements
    assert store_decode(lib, kn=A + 2) == ALIGN
    assert store_decode(lib, W=7) == INVAL               # the decode checks apply too
    assert store_decode(lib, ws=None) == NULLP
    assert store_decode(lib, B=0, out=None, q=None, kn=None, vn=None, kc=None, vc=None, bt=None, cl=None) == PA_OK


def store_decode_noalloc(lib, **kw):
    a = dict(out=A, q=A, qs=2048, kn=A, kns=1024, vn=A, vns=1024, kc=A, vc=A, bt=A, W=8, cl=A, B=4, hq=16, hkv=8,
             d=128, bs=256, maxL=2048, scale=0.088, part=0, stream=None)
    a.update(kw)
    return lib.pa_store_decode_noalloc(a["out"], a["q"], a["qs"], a["kn"], a["kns"], a["vn"], a["vns"], a["kc"],
                                       a["vc"], a["bt"], a["W"], a["cl"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"],
                                       a["maxL"], a["scale"], a["part"], a["stream"])


def test_store_decode_noalloc_validation(lib):
    # the pa_store_decode checks, before the static scratch is looked up
    assert store_decode_noalloc(lib, kn=None) == NULLP
    assert store_decode_noalloc(lib, kns=512) == INVAL
    assert store_decode_noalloc(lib, W=7) == INVAL
    assert store_decode_noalloc(lib, d=64) == UNSUP
    assert store_decode_noalloc(lib, B=0, out=None, q=None, kn=None, vn=None, kc=None, vc=None, bt=None,
                                cl=None) == PA_OK
    # a split larger than the static scratch (16.25 MiB) is refused with a clear message
    assert store_decode_noalloc(lib, hq=64, hkv=8, qs=8192, part=2049, B=512, maxL=32768, W=128) == WS
    assert "static scratch" in pa.pa_last_error()


def store_prefill(lib, **kw):
    a = dict(out=A, q=A, qs=2048, kn=A, kns=1024, vn=A, vns=1024, kc=A, vc=A, sl=A, cq=A, ck=A, S=4, maxq=1024,
             maxk=1024, hq=16, hkv=8, d=128, scale=0.088, causal=1, bt=None, W=0, bs=256, nb=16, stream=None)
    a.update(kw)
    return lib.pa_store_prefill_varlen(a["out"], a["q"], a["qs"], a["kn"], a["kns"], a["vn"], a["vns"], a["kc"],
                                       a["vc"], a["sl"], a["cq"], a["ck"], a["S"], a["maxq"], a["maxk"], a["hq"],
                                       a["hkv"], a["d"], a["scale"], a["causal"], a["bt"], a["W"], a["bs"], a["nb"],
                                       a["stream"])


def test_store_prefill_validation(lib):
    assert store_prefill(lib, sl=None) == NULLP
    assert store_prefill(lib, kc=None) == NULLP
    assert store_prefill(lib, kns=512) == INVAL        # below a row
    assert store_prefill(lib, vns=1028) == ALIGN       # not 16-byte aligned
    assert store_prefill(lib, kn=A + 2) == ALIGN
    assert store_prefill(lib, nb=0) == INVAL
    assert store_prefill(lib, nb=(1 << 23) + 1) == INVAL  # num_blocks * block_size > 2^31
    assert store_prefill(lib, bs=96) == UNSUP
    assert store_prefill(lib, hq=20) == INVAL           # the prefill checks apply too
    assert store_prefill(lib, bt=A, W=3, maxk=1024) == INVAL
    assert store_prefill(lib, S=0, out=None, q=None, kn=None, vn=None, kc=None, vc=None, sl=None, cq=None,
                         ck=None) == PA_OK


def test_decode_workspace_size(lib):
    # G = 2: 32-token chunks; 256 seqs x 8 kv heads x 64 chunks leave the default 2048 waves
    assert lib.pa_decode_split_waves(256, 16, 8, 2048, 0) == 2048
    assert lib.pa_decode_workspace_size(256, 16, 8, 128, 2048, 0) == 2048 * 2 * 2 * (128 + 2) * 4
    # fewer chunks than waves: one wave per chunk at most (4 x 8 x ceil(200/32) = 224)
    assert lib.pa_decode_split_waves(4, 16, 8, 200, 256) == 224
    assert lib.pa_decode_workspace_size(4, 16, 8, 128, 200, 256) == 224 * 2 * 2 * 130 * 4
    # G = 4: 16-token chunks; by default at least 4 chunks per wave by the length bound (1 x 8 x 7 = 56 -> 14)
    # 32-token chunks at every group size: 4 chunks x 8 kv heads, at least 4 chunks per wave
    assert lib.pa_decode_split_waves(1, 32, 8, 100, 0) == 8
    assert lib.pa_decode_split_waves(1, 64, 8, 100, 0) == 8
    # a small batch under the bound: 16 x 8 x 64 = 8192 chunks -> 2048 waves; 1 x 8 x 64 = 512 -> 128
    assert lib.pa_decode_split_waves(16, 16, 8, 2048, 0) == 2048
    assert lib.pa_decode_split_waves(1, 16, 8, 2048, 0) == 128
    # an explicit split is taken as given (clamped to one chunk per wave)
    assert lib.pa_decode_split_waves(1, 16, 8, 2048, 512) == 512
    assert lib.pa_decode_workspace_size(4, 16, 8, 64, 2048, 0) == 0    # unsupported head_dim
    assert lib.pa_decode_workspace_size(4, 16, 8, 128, 2048, -1) == 0  # bad split
    assert lib.pa_decode_split_waves(4, 16, 8, 2048, 100) == 100


def prefill(lib, **kw):
    a = dict(out=A, q=A, qs=2048, k=A, v=A, ks=3072, vs=3072, cq=A, ck=A, S=4, maxq=1024, maxk=1024, hq=16, hkv=8,
             d=128, scale=0.088, causal=1, bt=None, W=0, bs=0, stream=None)
    a.update(kw)
    return lib.pa_prefill_varlen(a["out"], a["q"], a["qs"], a["k"], a["v"], a["ks"], a["vs"], a["cq"], a["ck"],
                                 a["S"], a["maxq"], a["maxk"], a["hq"], a["hkv"], a["d"], a["scale"], a["causal"],
                                 a["bt"], a["W"], a["bs"], a["stream"])


def test_prefill_validation(lib):
    assert prefill(lib, hq=20) == INVAL
    assert prefill(lib, d=256) == UNSUP
    assert prefill(lib, S=-2) == INVAL
    assert prefill(lib, maxq=-1) == INVAL
    assert prefill(lib, maxk=-1) == INVAL
    assert prefill(lib, ks=512) == INVAL
    assert prefill(lib, vs=1028) == ALIGN
    assert prefill(lib, cq=None) == NULLP
    assert prefill(lib, qs=1000) == ALIGN or prefill(lib, qs=1000) == INVAL
    assert prefill(lib, q=A + 6) == ALIGN
    assert prefill(lib, bt=A, W=0, bs=256) == INVAL
    assert prefill(lib, bt=A, W=6, bs=96) == UNSUP
    # a table of 3 blocks of 256 tokens cannot address 1024 keys
    assert prefill(lib, bt=A, W=3, bs=256, maxk=1024) == INVAL
    assert prefill(lib, scale=float("inf")) == INVAL
    assert prefill(lib, S=0, out=None, q=None, k=None, v=None, cq=None, ck=None) == PA_OK


def test_python_binding_reports_errors(lib):
    with pytest.raises(pa.PAError) as e:
        pa._check("pa_decode", INVAL)
    assert "invalid argument" in str(e.value)


def norm_rope(lib, **kw):
    a = dict(qo=A, qos=2048, qkv=A, qkvs=4096, qw=A, kw=A, eps=1e-6, cs=A, maxp=4096, pos=A, kc=A, vc=A, slot=A,
             T=4, hq=16, hkv=8, d=128, nb=16, bs=256, stream=None)
    a.update(kw)
    return lib.pa_qk_norm_rope_store(a["qo"], a["qos"], a["qkv"], a["qkvs"], a["qw"], a["kw"], a["eps"], a["cs"],
                                     a["maxp"], a["pos"], a["kc"], a["vc"], a["slot"], a["T"], a["hq"], a["hkv"],
                                     a["d"], a["nb"], a["bs"], a["stream"])


def test_norm_rope_validation(lib):
    assert norm_rope(lib, T=-1) == INVAL
    assert norm_rope(lib, d=64) == UNSUP
    assert norm_rope(lib, hq=12) == INVAL
    assert norm_rope(lib, hq=24) == UNSUP
    assert norm_rope(lib, nb=0) == INVAL
    assert norm_rope(lib, nb=1 << 24) == UNSUP
    assert norm_rope(lib, eps=-1.0) == INVAL
    assert norm_rope(lib, eps=float("nan")) == INVAL
    assert norm_rope(lib, eps=float("inf")) == INVAL
    assert norm_rope(lib, maxp=0) == INVAL
    assert norm_rope(lib, qkvs=4088) == INVAL     # below 32 heads x 128
    assert norm_rope(lib, qos=1024) == INVAL      # below 16 heads x 128
    assert norm_rope(lib, T=1 << 27) == UNSUP     # items past 2^31
    assert norm_rope(lib, cs=None) == NULLP
    assert norm_rope(lib, pos=None) == NULLP
    assert norm_rope(lib, kw=None) == NULLP
    assert norm_rope(lib, qkv=A + 8) == ALIGN
    assert norm_rope(lib, cs=A + 4) == ALIGN
    assert norm_rope(lib, qkvs=4100) == ALIGN
    assert norm_rope(lib, T=0, qo=None, qkv=None, qw=None, kw=None, cs=None, pos=None, kc=None, vc=None,
                     slot=None) == PA_OK


def test_sampler_validation(lib):
    def smp(**kw):
        a = dict(tok=A, lg=A, ls=1024, t=A, B=4, V=1000, seed=1, off=0, ws=A, wsb=1 << 20, stream=None)
        a.update(kw)
        return lib.pa_sample_gumbel(a["tok"], a["lg"], a["ls"], a["t"], a["B"], a["V"], a["seed"], a["off"],
                                    a["ws"], a["wsb"], a["stream"])
    assert lib.pa_sample_workspace_size(4, 1000) == 4 * 1 * 8
    assert lib.pa_sample_workspace_size(2, 151936) == 2 * 13 * 8  # ceil(151936 / 12288) partials per row
    assert lib.pa_sample_workspace_size(2, 0) == 0
    assert smp(B=-1) == INVAL
    assert smp(V=0) == INVAL
    assert smp(ls=999) == INVAL
    assert smp(B=70000) == UNSUP
    assert smp(lg=None) == NULLP
    assert smp(ws=None) == NULLP
    assert smp(lg=A + 2) == ALIGN
    assert smp(ws=A + 4) == ALIGN
    assert smp(wsb=8) == WS
    assert smp(B=0, tok=None, lg=None, t=None, ws=None) == PA_OK


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++17")])
def test_headers_compile_and_link_from_c(lib, tmp_path, compiler, std):
    """A C (and a C++) program that includes both headers, takes the address of every declared
    entry point, links against the built library and calls two host-only functions."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    names = declared_functions()
    src = ['#include "pa.h"', '#include "pa_blocks.h"', "#include <stdio.h>", "#include <string.h>",
           "typedef void (*fn_t)(void);", "int main(void) {", "  fn_t fns[] = {"]
    src += [f"    (fn_t){n}," for n in names]
    src += ["  };",
            "  for (size_t i = 0; i < sizeof(fns) / sizeof(fns[0]); ++i)",
            "    if (!fns[i]) return 2;",
            "  if (pa_version() < 100) return 3;",
            "  /* a failing argument check: no GPU work, a status and a message */",
            "  if (pa_store_kvcache(0, 0, 0, 0, 0, 0, 0, -1, 8, 128, 16, 256, 0) != PA_ERR_INVALID_ARGUMENT) return 4;",
            "  if (strlen(pa_last_error()) == 0) return 5;",
            '  printf("%zu entry points\\n", sizeof(fns) / sizeof(fns[0]));',
            "  return 0;", "}"]
    ext = ".c" if compiler == "gcc" else ".cpp"
    c_file, exe = tmp_path / f"abi_user{ext}", tmp_path / "abi_user"
    c_file.write_text("\n".join(src) + "\n")
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [compiler, std, "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(c_file),
           "-L", libdir, "-lpa", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    if compiler == "gcc":
        cmd.insert(2, "-pedantic")
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == f"{len(names)} entry points"
