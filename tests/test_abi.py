"""C-ABI checks that need no GPU: the library loads, exports every function
include/kvrec.h declares, rejects every malformed call on the host before any
launch, and its kernels contain no fused multiply-add and no packed fp32 ops.

Pointers passed here are fake but aligned addresses: every call below either
fails validation or has nothing to launch (zero tokens), so the library never
dereferences them.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from quantized_paged_kv_rope_amd import binding as B
from quantized_paged_kv_rope_amd import build as KB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvrec.h")

OK, NULL, RECORD, BLOCK, STRIDE, ALIGN, SIZE, OPTION, OVERLAP = 0, -1, -2, -3, -4, -5, -6, -8, -9
FAKE = 0x10000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH) or os.path.getmtime(B.LIB_PATH) < max(
            os.path.getmtime(os.path.join(KB.CSRC, s)) for s in os.listdir(KB.CSRC)):
        KB.build()
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvrec_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(B.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_does_not_depend_on_the_oracle():
    needed = subprocess.run(["readelf", "-d", B.LIB_PATH], capture_output=True, text=True,
                            check=True).stdout
    assert "oracle" not in needed
    pkg = os.path.dirname(B.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), f
                assert "kvrec_oracle" not in src and "liboracle" not in src, f


def test_status_strings(lib):
    for code in (OK, NULL, RECORD, BLOCK, STRIDE, ALIGN, SIZE, -7, OPTION, OVERLAP, 12345):
        s = lib.kvrec_status_str(code)
        assert s and isinstance(s, bytes)
    assert lib.kvrec_status_str(OK) == b"ok"


@pytest.mark.parametrize("record,bs,want", [
    (528, 32, 16896), (528, 64, 33792), (528, 128, 67584), (528, 256, 135168),
    (584, 32, 19008), (584, 64, 37440), (584, 128, 74880), (584, 256, 149760),
    (528, 1, 1024), (528, 4, 2560), (584, 4, 2880), (584, 1, 1152),
    (1024, 1, 1024), (1024, 64, 65536), (512, 3, 1536), (512, 64, 32768)])
def test_page_stride(lib, record, bs, want):
    out = ctypes.c_int64(-1)
    assert lib.kvrec_page_stride(record, bs, ctypes.byref(out)) == OK
    assert out.value == want


def test_page_stride_errors(lib):
    out = ctypes.c_int64(-1)
    assert lib.kvrec_page_stride(528, 64, None) == NULL
    assert lib.kvrec_page_stride(513, 64, ctypes.byref(out)) == RECORD
    assert lib.kvrec_page_stride(576, 64, ctypes.byref(out)) == RECORD
    assert lib.kvrec_page_stride(528, 0, ctypes.byref(out)) == BLOCK
    # a page of 2^31 bytes or more would overflow the kernels' 32-bit offsets
    assert lib.kvrec_page_stride(1024, 2 ** 21, ctypes.byref(out)) == OK
    assert lib.kvrec_page_stride(1024, 2 ** 21 + 1, ctypes.byref(out)) == BLOCK
    assert lib.kvrec_page_stride(528, 2 ** 22, ctypes.byref(out)) == BLOCK
    out.value = -1
    assert out.value == -1


def cache(base=FAKE, nb=4, stride=33792, bs=64, rec=528):
    return B.kvrec_cache(base, nb, stride, bs, rec)


def ins(lib, c, n=8, kv=FAKE, slots=FAKE, pos=FAKE, cs=FAKE, max_pos=16, bs=64, rec=528):
    return lib.kvrec_insert(kv, n, ctypes.byref(c) if c is not None else None, slots, pos, cs,
                            max_pos, bs, rec, None)


def gat(lib, c, n=8, idx=FAKE, out=FAKE):
    return lib.kvrec_gather(ctypes.byref(c) if c is not None else None, idx, n, out, None)


def test_insert_validation(lib):
    good = cache()
    assert ins(lib, good, n=0) == OK                        # nothing to launch
    assert ins(lib, good, n=0, kv=None, slots=None, pos=None, cs=None) == OK
    assert ins(lib, None) == NULL
    assert ins(lib, cache(base=None)) == NULL
    assert ins(lib, good, kv=None) == NULL
    assert ins(lib, good, slots=None) == NULL
    assert ins(lib, good, pos=None) == NULL
    assert ins(lib, good, cs=None) == NULL
    assert ins(lib, good, rec=512) == RECORD
    assert ins(lib, good, rec=584) == RECORD                 # != cache record
    assert ins(lib, cache(rec=600, stride=38400), rec=600) == RECORD
    assert ins(lib, good, bs=32) == BLOCK                    # != cache block size
    assert ins(lib, cache(bs=0), bs=0) == BLOCK
    assert ins(lib, cache(stride=33792 - 512)) == STRIDE    # < block_size * record
    assert ins(lib, cache(stride=33792 + 64)) == STRIDE     # not a multiple of 512
    assert ins(lib, cache(stride=212160)) == STRIDE         # the pages' bad block stride
    assert ins(lib, cache(rec=584, stride=37440 + 512), rec=584) == STRIDE
    assert ins(lib, cache(nb=-1)) == SIZE
    assert ins(lib, cache(nb=2 ** 30 // 64 + 1)) == SIZE    # more than 2^30 slots
    assert ins(lib, cache(nb=2 ** 30 // 64), n=0) == OK
    assert ins(lib, good, n=-1) == SIZE
    assert ins(lib, good, n=2 ** 30 + 1) == SIZE
    assert ins(lib, good, max_pos=0) == SIZE
    assert ins(lib, cache(base=FAKE + 8)) == ALIGN
    assert ins(lib, good, kv=FAKE + 8) == ALIGN
    assert ins(lib, good, cs=FAKE + 4) == ALIGN
    assert ins(lib, good, slots=FAKE + 4) == ALIGN
    assert ins(lib, good, pos=FAKE + 4) == ALIGN


def test_gather_validation(lib):
    good = cache()
    assert gat(lib, good, n=0) == OK
    assert gat(lib, good, n=0, idx=None, out=None) == OK
    assert gat(lib, None) == NULL
    assert gat(lib, cache(base=None)) == NULL
    assert gat(lib, good, idx=None) == NULL
    assert gat(lib, good, out=None) == NULL
    assert gat(lib, cache(rec=512)) == RECORD
    assert gat(lib, cache(bs=0)) == BLOCK
    assert gat(lib, cache(stride=1000)) == STRIDE
    assert gat(lib, cache(rec=584, stride=37440 + 64)) == STRIDE
    assert gat(lib, good, n=-3) == SIZE
    assert gat(lib, good, out=FAKE + 8) == ALIGN
    assert gat(lib, good, idx=FAKE + 2) == ALIGN
    assert gat(lib, cache(base=FAKE + 1)) == ALIGN


def ins_ex(lib, c, opts, n=8, kv=FAKE, slots=FAKE, pos=FAKE, cs=FAKE, max_pos=16, bs=64, rec=528):
    return lib.kvrec_insert_ex(kv, n, ctypes.byref(c), slots, pos, cs, max_pos, bs, rec,
                               ctypes.byref(opts) if opts is not None else None, None)


def test_insert_options_validation(lib):
    good = cache()
    O = B.kvrec_insert_options
    assert ins_ex(lib, good, None, n=0) == OK
    assert ins_ex(lib, good, O(1, 4, 1e-4, 1), n=0) == OK
    assert ins_ex(lib, good, O(3, 1, 0.0, 0)) == OPTION       # unknown rotation
    assert ins_ex(lib, good, O(-1, 1, 0.0, 0)) == OPTION
    assert ins_ex(lib, good, O(1, 0, 0.0, 0)) == OPTION       # ratio < 1
    assert ins_ex(lib, good, O(1, 2 ** 30 + 1, 0.0, 0)) == OPTION
    assert ins_ex(lib, good, O(1, 1, -1e-4, 0)) == OPTION     # negative floor
    assert ins_ex(lib, good, O(1, 1, float("nan"), 0)) == OPTION
    assert ins_ex(lib, good, O(1, 1, float("inf"), 0)) == OPTION
    assert ins_ex(lib, good, O(1, 1, 0.0, 2)) == OPTION       # sanitize is 0 or 1
    # what may be NULL: the table without a rotation; positions too with ratio 1
    assert ins_ex(lib, good, O(0, 1, 0.0, 0), pos=None) == NULL
    assert ins_ex(lib, good, O(1, 1, 0.0, 0), cs=None) == NULL
    assert ins_ex(lib, good, O(2, 2, 0.0, 0), pos=None) == NULL  # the ratio gate needs them
    assert ins_ex(lib, good, O(2, 1, 0.0, 0), n=0, pos=None, cs=None) == OK
    assert ins_ex(lib, good, O(0, 1, 0.0, 0), max_pos=2 ** 30 + 1) == SIZE
    assert lib.kvrec_status_str(OPTION) == b"insert option out of range"


def test_page_size_limit(lib):
    # block_size * record above 2^31 is refused before anything else about the page
    big = 2 ** 22 * 528
    assert ins(lib, cache(nb=1, bs=2 ** 22, stride=big), bs=2 ** 22) == BLOCK
    assert gat(lib, cache(nb=1, bs=2 ** 22, stride=big)) == BLOCK
    ok_bs = 2 ** 31 // 528 // 512 * 512  # largest multiple of 512 slots under the limit
    assert ins(lib, cache(nb=1, bs=ok_bs, stride=ok_bs * 528), n=0, bs=ok_bs) == OK


def full(lib, c, n=8, kv=FAKE, slots=FAKE, pos=FAKE, cs=FAKE, max_pos=16, bs=64, rec=1024,
         scale=None):
    return lib.kvrec_insert_full(kv, n, ctypes.byref(c) if c is not None else None, slots, pos,
                                 cs, max_pos, bs, rec, scale, None)


def test_insert_full_validation(lib):
    bf = cache(rec=1024, stride=65536)
    f8 = cache(rec=512, stride=32768)
    assert full(lib, bf, n=0) == OK
    assert full(lib, f8, n=0, rec=512, scale=FAKE) == OK
    assert full(lib, bf, n=0, kv=None, slots=None, pos=None, cs=None) == OK
    assert full(lib, None) == NULL
    assert full(lib, cache(base=None, rec=1024, stride=65536)) == NULL
    assert full(lib, f8, rec=512) == NULL                        # the fp8 cache needs its scale
    assert full(lib, f8, rec=512, n=0) == NULL
    assert full(lib, bf, scale=FAKE) == OPTION                   # a bf16 cache takes none
    for arg in ("kv", "slots", "pos", "cs"):
        assert full(lib, bf, **{arg: None}) == NULL, arg
    assert full(lib, bf, rec=512) == RECORD                      # != cache record
    assert full(lib, cache(), rec=528) == RECORD                 # packed: not this call
    assert full(lib, cache(rec=584, stride=37440), rec=584) == RECORD
    assert full(lib, bf, bs=32) == BLOCK
    assert full(lib, cache(rec=1024, stride=65536 - 16)) == STRIDE
    assert full(lib, cache(rec=1024, stride=65536 + 8)) == STRIDE  # not a multiple of 16
    assert full(lib, cache(rec=1024, stride=65536 + 16), n=0) == OK
    assert full(lib, cache(rec=512, stride=32768 + 48), rec=512, scale=FAKE, n=0) == OK
    assert full(lib, bf, n=-1) == SIZE
    assert full(lib, bf, max_pos=0) == SIZE
    assert full(lib, bf, kv=FAKE + 8) == ALIGN
    assert full(lib, f8, rec=512, scale=FAKE + 2) == ALIGN
    # the packed calls refuse the non-packed records
    assert ins(lib, bf, rec=1024) == RECORD
    assert ins_ex(lib, f8, None, rec=512) == RECORD
    assert gat(lib, bf) == RECORD
    assert gat(lib, f8) == RECORD


def qkv(lib, c, q_in=FAKE * 64, q_out=FAKE * 64, heads=8, eps=1e-6, norm=1, n=8, kv=FAKE,
        slots=FAKE, pos=FAKE, cs=FAKE, max_pos=16, bs=64, rec=528):
    return lib.kvrec_qnorm_rope_insert(q_in, q_out, heads, eps, norm, kv, n,
                                       ctypes.byref(c) if c is not None else None, slots, pos,
                                       cs, max_pos, bs, rec, None)


def test_qnorm_rope_insert_validation(lib):
    good = cache()
    assert qkv(lib, good, n=0) == OK
    assert qkv(lib, good, n=0, q_in=None, q_out=None, kv=None, slots=None, pos=None,
               cs=None) == OK
    assert qkv(lib, None) == NULL
    for arg in ("q_in", "q_out", "kv", "slots", "pos", "cs"):
        assert qkv(lib, good, **{arg: None}) == NULL, arg
    assert qkv(lib, good, rec=584) == RECORD
    assert qkv(lib, cache(rec=1024, stride=65536), rec=1024) == RECORD  # packed only
    assert qkv(lib, good, bs=32) == BLOCK
    assert qkv(lib, good, heads=0) == SIZE
    assert qkv(lib, good, heads=1025) == SIZE
    assert qkv(lib, good, heads=1024, n=2 ** 20 + 1) == SIZE         # tokens * heads > 2^30
    assert qkv(lib, good, heads=1024, n=-1) == SIZE
    assert qkv(lib, good, norm=2) == OPTION
    assert qkv(lib, good, eps=0.0) == OPTION
    assert qkv(lib, good, eps=-1e-6) == OPTION
    assert qkv(lib, good, eps=float("inf")) == OPTION
    assert qkv(lib, good, eps=0.0, norm=0, n=0) == OK                # eps unused
    assert qkv(lib, good, max_pos=0) == SIZE
    assert qkv(lib, good, q_in=FAKE * 64 + 8) == ALIGN
    assert qkv(lib, good, q_out=FAKE * 64 + 8) == ALIGN
    # in place is fine; a partial overlap is not
    row = 8 * 512 * 2  # one token's q rows
    assert qkv(lib, good, q_out=FAKE * 64 + row, n=0) == OK
    assert qkv(lib, good, q_out=FAKE * 64 + row) == OVERLAP
    assert qkv(lib, good, q_out=FAKE * 64 - row) == OVERLAP


def expand(lib, rows=4, k=64, ratio=2, sbk=8, cand=FAKE, cs=None, ks=FAKE, kss=1, ke=FAKE,
           kes=1, out=FAKE, ss=None, end=FAKE, es=1):
    cs = k if cs is None else cs
    ss = k * ratio if ss is None else ss
    return lib.kvrec_expand_candidates(cand, cs, ks, kss, ke, kes, rows, k, ratio, sbk, out, ss,
                                       end, es, None)


def test_expand_candidates_validation(lib):
    assert expand(lib, rows=0) == OK
    assert expand(lib, rows=0, cand=None, ks=None, ke=None, out=None, end=None) == OK
    for arg in ("cand", "ks", "ke", "out", "end"):
        assert expand(lib, **{arg: None}) == NULL, arg
    for k in (0, 3, 48, 2048):
        assert expand(lib, k=k, ratio=1) == SIZE, k
    assert expand(lib, k=1024, ratio=2) == SIZE            # K * ratio > 1024
    assert expand(lib, k=1024, ratio=1, rows=0) == OK
    assert expand(lib, ratio=3) == OPTION
    assert expand(lib, ratio=0) == OPTION
    assert expand(lib, sbk=4) == OPTION
    assert expand(lib, sbk=32) == OPTION
    assert expand(lib, rows=-1) == SIZE
    assert expand(lib, rows=2 ** 30 + 1) == SIZE
    assert expand(lib, cs=63) == SIZE                      # row stride < K
    assert expand(lib, ss=127) == SIZE                     # row stride < K * ratio
    assert expand(lib, kss=0) == SIZE
    assert expand(lib, kes=0) == SIZE
    assert expand(lib, es=0) == SIZE
    assert expand(lib, cand=FAKE + 2) == ALIGN
    assert expand(lib, out=FAKE + 1) == ALIGN
    assert expand(lib, end=FAKE + 2) == ALIGN


def test_legacy_cache_accepted(lib):
    assert ins(lib, cache(rec=584, stride=37440), n=0, rec=584) == OK
    assert gat(lib, cache(rec=584, stride=37440), n=0) == OK
    assert gat(lib, cache(rec=584, stride=37440 + 576 * 3), n=0) == OK  # padded stride


def test_python_binding_rejects_cpu_tensors():
    import torch

    kv = torch.zeros(4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.kvrec_insert(kv, torch.zeros(1, 4, 528, dtype=torch.uint8), torch.zeros(4, dtype=torch.int64),
                       torch.zeros(4, dtype=torch.int64), torch.zeros(8, 64), 4)
    with pytest.raises(ValueError):
        B.kvrec_gather(torch.zeros(1, 4, 528, dtype=torch.uint8), torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        B.kvrec_insert_full(kv, torch.zeros(1, 4, 512, dtype=torch.bfloat16),
                            torch.zeros(4, dtype=torch.int64), torch.zeros(4, dtype=torch.int64),
                            torch.zeros(8, 64), 4)


def test_python_binding_rejects_cpu_tensors_widened_calls():
    import torch

    q = torch.zeros(4, 2, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on a GPU"):
        B.kvrec_qnorm_rope_insert(q, torch.zeros(4, 512, dtype=torch.bfloat16),
                                  torch.zeros(1, 4, 528, dtype=torch.uint8),
                                  torch.zeros(4, dtype=torch.int64), torch.zeros(4, dtype=torch.int64),
                                  torch.zeros(8, 64), 4)
    with pytest.raises(ValueError, match="on a GPU"):
        B.kvrec_expand_candidates(torch.zeros(2, 8, dtype=torch.int32),
                                  torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                                  2, 8)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no other
    path to fall back to."""
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        B.load_library(str(tmp_path / "libkvrec.so"))


def _kernel_bodies(asm: str) -> dict:
    bodies = {}
    for name in re.findall(r"^(_Z\S+):", asm, re.M):
        b = asm[asm.index(name + ":"):]
        b = b[:b.index(".Lfunc_end")]
        bodies[name] = [l.split()[0] for l in (x.strip() for x in b.splitlines())
                        if l and not l.startswith((";", ".", "_"))]
    return bodies


def test_kernels_have_no_fma_and_no_packed_fp32():
    """No contraction: the rotation's products and sums are rounded one by
    one. Fused multiply-adds appear only in the fp8 cache's insert, which
    divides by the per-tensor scale: five inside each IEEE division sequence
    (ending in v_div_fixup_f32) and four per element (32 per lane) in the
    reciprocal path's two Markstein corrections, per token of the wave
    (insert_kernel's third template argument). Every other kernel has none."""
    asm = KB.device_asm()
    code = "\n".join(l for l in asm.splitlines() if not l.lstrip().startswith((";", ".")))
    for op in ("v_mad_f32", "v_mac_f32", "v_fma_mix",
               "v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"):
        assert op not in code, op
    fp8_kernels = 0
    for name, ops in _kernel_bodies(asm).items():
        fma = sum(op.startswith(("v_fma_f32", "v_fmac_f32")) for op in ops)
        fixup = sum(op.startswith("v_div_fixup_f32") for op in ops)
        m = re.search(r"insert_kernelILi\d+ELi\d+ELi(\d+)ELi3E", name)  # the fp8 format
        if m:
            fp8_kernels += 1
            tokens = int(m.group(1))
            # one division for the reciprocal, eight per token on the other path
            assert fixup >= 8 * tokens + 1 and fma <= 5 * fixup + 32 * tokens, \
                (name, fma, fixup)
        else:
            assert fma == 0 and fixup == 0, (name, fma, fixup)
    assert fp8_kernels > 0
    # fp32 denormals preserved for every kernel (mode 3 = keep inputs and outputs)
    modes = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", asm)
    assert modes and set(modes) == {"3"}
    # the gfx950 scaled conversions, the bf16 conversion, and the NeoX partner
    # exchange (ds_swizzle xor 4)
    for needed in ("v_cvt_scalef32_pk_fp8_f32", "v_cvt_scalef32_pk_bf16_fp8", "v_cvt_pk_bf16_f32",
                   "ds_swizzle_b32"):
        assert needed in code, needed
