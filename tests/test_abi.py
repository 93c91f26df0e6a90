"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import fp8_fine_grained_amd as fp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8fg.h")

OK, ENULL, ESHAPE, EALIGN, EUNSUP = 0, -1, -2, -3, -4
P = ctypes.c_void_p(0x10000)          # a fake, 16-byte aligned "device" pointer (never dereferenced)
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)        # misaligned
NUL = ctypes.c_void_p(0)


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|int)\s+(\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = fp8.load_library()
    names = header_functions()
    assert set(names) == set(fp8.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    declared = int(re.search(r"#define FP8FG_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert fp8.abi_version() == fp8.ABI_VERSION == declared
    assert fp8.status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert fp8.status_string(code) not in ("ok", "unknown status")
    assert "128" not in fp8.status_string(-2)            # the size rules differ by call (16, 32, 64, 128, 256)
    assert fp8.status_string(7) == "unknown status"


def test_quant_argument_errors():
    lib = fp8.load_library()
    q = lib.fp8_quant_act_1x128
    assert q(NUL, 128, 128, 0, P, P2, NUL) == ENULL
    assert q(P, 128, 100, 0, P, P2, NUL) == ESHAPE          # K % 16
    assert q(P, 100, 128, 1, P, P2, NUL) == ESHAPE          # tokens % 16 when transposed
    assert q(P, -1, 128, 0, P, P2, NUL) == ESHAPE
    assert q(MIS, 128, 128, 0, P, P2, NUL) == EALIGN
    assert q(P, 128, 128, 2, P, P2, NUL) == EUNSUP
    assert q(P, 0, 128, 0, P, P2, NUL) == OK                # empty: no launch
    assert q(P, 128, 0, 1, P, P2, NUL) == OK
    assert q(NUL, 0, 128, 0, NUL, NUL, NUL) == OK          # empty arrays may be NULL
    w = lib.fp8_quant_weight_128x128
    assert w(P, 128, 72, 0, P, P2, NUL) == ESHAPE          # K % 16
    assert w(P, 72, 128, 0, P, P2, NUL) == ESHAPE          # N % 16
    assert w(P, 128, 128, 0, NUL, P2, NUL) == ENULL
    assert w(P, 128, 128, 0, P, MIS, NUL) == EALIGN
    assert w(P, 0, 128, 1, P, P2, NUL) == OK
    assert w(NUL, 128, 0, 0, NUL, NUL, NUL) == OK


def test_bf16_quant_argument_errors():
    lib = fp8.load_library()
    q = lib.fp8_quant_act_1x128_bf16
    assert q(NUL, 128, 128, 0, P, P2, NUL) == ENULL
    assert q(P, 128, 100, 0, P, P2, NUL) == ESHAPE
    assert q(P, 100, 128, 1, P, P2, NUL) == ESHAPE
    assert q(MIS, 128, 128, 1, P, P2, NUL) == EALIGN
    assert q(P, 128, 128, -1, P, P2, NUL) == EUNSUP
    assert q(P, 0, 128, 1, P, P2, NUL) == OK
    w = lib.fp8_quant_weight_128x128_bf16
    assert w(P, 128, 72, 1, P, P2, NUL) == ESHAPE
    assert w(P, 128, 128, 0, P, NUL, NUL) == ENULL
    assert w(MIS, 128, 128, 0, P, P2, NUL) == EALIGN
    assert w(P, 128, 128, 3, P, P2, NUL) == EUNSUP
    assert w(P, 128, 0, 0, P, P2, NUL) == OK


def test_fprop_operands_argument_errors():
    f = fp8.load_library().fp8_quant_fprop_operands
    #      x  xb  M    w  wb   N    K   qa  sa  qb  sb
    assert f(NUL, 0, 128, P, 0, 128, 128, P, P2, P, P2, NUL) == ENULL
    assert f(P, 0, 128, P, 0, 128, 128, P, P2, P, NUL, NUL) == ENULL
    assert f(P, 0, 128, P, 0, 128, 100, P, P2, P, P2, NUL) == ESHAPE     # K % 16
    assert f(P, 0, 128, P, 0, 72, 128, P, P2, P, P2, NUL) == ESHAPE      # N % 16
    assert f(P, 0, -1, P, 0, 128, 128, P, P2, P, P2, NUL) == ESHAPE
    assert f(P, 2, 128, P, 0, 128, 128, P, P2, P, P2, NUL) == EUNSUP     # x_bf16 not 0 / 1
    assert f(P, 0, 128, P, -1, 128, 128, P, P2, P, P2, NUL) == EUNSUP
    assert f(P, 0, 128, MIS, 0, 128, 128, P, P2, P, P2, NUL) == EALIGN
    assert f(P, 1, 128, P, 1, 128, 0, P, P2, P, P2, NUL) == OK          # K = 0: no launch
    assert f(P, 0, 0, P, 1, 0, 128, P, P2, P, P2, NUL) == OK            # M = N = 0: no launch
    assert f(NUL, 0, 0, NUL, 0, 0, 128, NUL, NUL, NUL, NUL, NUL) == OK  # empty operands may be NULL
    assert f(NUL, 0, 0, P, 0, 128, 128, NUL, NUL, NUL, P2, NUL) == ENULL  # the weight is not empty


def test_requant_argument_errors():
    r = fp8.load_library().fp8_requant_act_tokenwise
    assert r(NUL, P, 128, 128, P, P2, NUL) == ENULL
    assert r(P, P, 128, 128, P, NUL, NUL) == ENULL
    assert r(P, P, 100, 128, P, P2, NUL) == ESHAPE       # tokens % 16
    assert r(P, P, 128, 72, P, P2, NUL) == ESHAPE        # channels % 16
    assert r(P, P, -128, 128, P, P2, NUL) == ESHAPE
    assert r(P, MIS, 128, 128, P, P2, NUL) == EALIGN
    assert r(P, P, 0, 128, P, P2, NUL) == OK
    assert r(P, P, 128, 0, P, P2, NUL) == OK


def test_mx_argument_errors():
    lib = fp8.load_library()
    q = lib.fp8_quant_mx_1x32
    assert q(NUL, 4, 64, P, P2, NUL) == ENULL
    assert q(P, 4, 48, P, P2, NUL) == ESHAPE            # K % 32
    assert q(MIS, 4, 64, P, P2, NUL) == EALIGN
    assert q(P, 0, 64, P, P2, NUL) == OK
    t = lib.fp8_quant_mx_1x32_transposed
    assert t(NUL, 64, 8, P, P2, NUL) == ENULL
    assert t(P, 48, 8, P, P2, NUL) == ESHAPE             # M % 32 (the blocked axis)
    assert t(P, -32, 8, P, P2, NUL) == ESHAPE
    assert t(P, 64, 8, MIS, P2, NUL) == EALIGN
    assert t(P, 64, 64 * 65535 + 1, P, P2, NUL) == EUNSUP
    assert t(NUL, 0, 8, NUL, NUL, NUL) == OK             # empty: NULL allowed
    g = lib.fp8_gemm_mx
    assert g(P, P, P, NUL, P, 0, 4, 256, 64, NUL) == ENULL
    assert g(P, P, P, P, P, 0, 6, 256, 64, NUL) == ESHAPE     # M % 4
    assert g(P, P, P, P, P, 0, 4, 128, 64, NUL) == ESHAPE     # N % 256
    assert g(P, P, P, P, P, 0, 4, 256, 32, NUL) == ESHAPE     # K % 64
    assert g(P, P, P, P, P, 0, 4, 256, 0, NUL) == ESHAPE
    assert g(P, MIS, P, P, P, 0, 4, 256, 64, NUL) == EALIGN
    assert g(P, P, P, P, P, 7, 4, 256, 64, NUL) == EUNSUP
    assert g(P, P, P, P, P, 0, 0, 256, 64, NUL) == OK
    c = lib.fp8_grouped_gemm_contiguous_mx
    #        a  ea  b  eb off  G  M_total N   K   c  out
    assert c(P, P, P, P, NUL, 4, 512, 256, 64, P, 0, NUL) == ENULL
    assert c(P, P, P, P, P, 4, 500, 256, 64, P, 0, NUL) == ESHAPE      # M_total % 128
    assert c(P, P, P, P, P, 4, 512, 128, 64, P, 0, NUL) == ESHAPE      # N % 256
    assert c(P, P, P, P, P, 4, 512, 256, 96, P, 0, NUL) == ESHAPE      # K % 64
    assert c(P, P, P, P, P, 4, 512, 256, 0, P, 0, NUL) == ESHAPE       # K = 0 with work to do
    assert c(P, P, P, P, MIS, 4, 512, 256, 64, P, 0, NUL) == EALIGN
    assert c(P, P, P, P, P, 4, 512, 256, 64, P, 2, NUL) == EUNSUP      # output dtype
    assert c(P, P, P, P, P, 4, 512, 256, 1 << 24, P, 0, NUL) == EUNSUP
    assert c(P, P, P, P, P, 0, 512, 256, 64, P, 0, NUL) == OK          # G = 0
    m = lib.fp8_grouped_gemm_masked_mx
    assert m(P, P, P, NUL, P, 4, 128, 256, 64, P, 0, NUL) == ENULL
    assert m(P, P, P, P, P, 4, 126, 256, 64, P, 0, NUL) == ESHAPE      # M_max % 4
    assert m(P, P, P, P, P, 4, 128, 384, 64, P, 0, NUL) == ESHAPE      # N % 256
    assert m(P, P, P, P, P, 4, 128, 256, 32, P, 0, NUL) == ESHAPE      # K % 64
    assert m(P, P, P, P, P, -1, 128, 256, 64, P, 0, NUL) == ESHAPE
    assert m(P, MIS, P, P, P, 4, 128, 256, 64, P, 0, NUL) == EALIGN
    assert m(P, P, P, P, P, 4, 128, 256, 64, P, 5, NUL) == EUNSUP
    assert m(P, P, P, P, P, 4, 0, 256, 64, P, 0, NUL) == OK            # M_max = 0


@pytest.mark.parametrize("name", ["fp8_gemm_blockscaled", "fp8_gemm_blockscaled_fp8mfma"])
def test_gemm_argument_errors(name):
    g = getattr(fp8.load_library(), name)
    assert g(P, P, P, NUL, 0, P, 0, 1, 128, 128, NUL) == ENULL
    assert g(P, P, P, P, 0, P, 0, 1, 100, 128, NUL) == ESHAPE     # N % 16
    assert g(P, P, P, P, 0, P, 0, 1, 128, 100, NUL) == ESHAPE     # K % 16
    assert g(P, P, P, P, 0, P, 0, 1, 128, 0, NUL) == ESHAPE       # empty contraction
    assert g(P, P, MIS, P, 0, P, 0, 1, 128, 128, NUL) == EALIGN
    assert g(P, P, P, P, 5, P, 0, 1, 128, 128, NUL) == EUNSUP     # bscale kind
    assert g(P, P, P, P, 0, P, 9, 1, 128, 128, NUL) == EUNSUP     # out dtype
    assert g(P, P, P, P, 0, P, 0, 0, 128, 128, NUL) == OK          # M = 0
    assert g(P, P, P, P, 1, P, 1, 5, 0, 128, NUL) == OK            # N = 0


def test_fp8out_argument_errors():
    f = fp8.load_library().fp8_gemm_blockscaled_fp8out
    assert f(P, P, P, P, P, NUL, 4, 256, 128, NUL) == ENULL
    assert f(P, P, P, P, P, P2, 4, 128, 128, NUL) == ESHAPE     # N % 256
    assert f(P, P, P, P, P, P2, 4, 256, 72, NUL) == ESHAPE      # K % 16
    assert f(P, P, P, P, P, P2, 4, 256, 0, NUL) == ESHAPE
    assert f(P, P, P, P, MIS, P2, 4, 256, 128, NUL) == EALIGN
    assert f(P, P, P, P, P, P2, 4, 256, 92 * 128 + 16, NUL) == EUNSUP   # beyond 92 K-blocks (one accumulator)
    assert f(P, P, P, P, P, P2, 0, 256, 92 * 128, NUL) == OK


def test_grouped_argument_errors():
    lib = fp8.load_library()
    c = lib.fp8_grouped_gemm_contiguous
    assert c(P, P, P, P, NUL, 4, 512, 128, 128, P, 0, NUL) == ENULL
    assert c(P, P, P, P, P, 4, 500, 128, 128, P, 0, NUL) == ESHAPE   # M_total % 128
    assert c(P, P, P, P, MIS, 4, 512, 128, 128, P, 0, NUL) == EALIGN
    assert c(P, P, P, P, P, 4, 512, 128, 128, P, 3, NUL) == EUNSUP
    assert c(P, P, P, P, P, 0, 512, 128, 128, P, 0, NUL) == OK       # G = 0
    f = lib.fp8_grouped_gemm_contiguous_fp8out
    assert f(P, P, P, P, P, 4, 512, 256, 128, NUL, P, NUL) == ENULL
    assert f(P, P, P, P, P, 4, 512, 128, 128, P, P, NUL) == ESHAPE     # N % 256
    assert f(P, P, P, P, P, 4, 500, 256, 128, P, P, NUL) == ESHAPE     # M_total % 128
    assert f(P, P, P, P, P, 4, 512, 256, 0, P, P, NUL) == ESHAPE       # K = 0 with work to do
    assert f(P, P, P, P, P, 4, 512, 256, 128, MIS, P, NUL) == EALIGN
    assert f(P, P, P, P, P, 4, 512, 256, 92 * 128 + 16, P, P, NUL) == EUNSUP   # beyond 92 K-blocks
    assert f(P, P, P, P, P, 0, 512, 256, 128, P, P, NUL) == OK         # G = 0
    m = lib.fp8_grouped_gemm_masked
    assert m(P, P, P, P, NUL, 4, 128, 128, 128, P, 0, NUL) == ENULL
    assert m(P, P, P, P, P, 4, 128, 128, 130, P, 0, NUL) == ESHAPE
    assert m(P, P, P, P, P, -1, 128, 128, 128, P, 0, NUL) == ESHAPE
    assert m(P, P, P, P, P, 4, 0, 128, 128, P, 0, NUL) == OK


def test_decode_tiled_argument_errors():
    lib = fp8.load_library()
    t = lib.fp8_tile_weights_decode
    assert t(NUL, 2, 512, 128, P, NUL) == ENULL
    assert t(P, 2, 384, 128, P2, NUL) == ESHAPE       # N % 256
    assert t(P, 2, 512, 96, P2, NUL) == ESHAPE        # K % 64
    assert t(P, -1, 512, 128, P2, NUL) == ESHAPE
    assert t(MIS, 2, 512, 128, P2, NUL) == EALIGN
    assert t(P, 2, 512, 1 << 24, P2, NUL) == EUNSUP
    assert t(NUL, 0, 512, 128, NUL, NUL) == OK         # empty: NULL allowed
    m = lib.fp8_grouped_gemm_masked_tiled
    assert m(P, P, P, P, NUL, 4, 128, 256, 128, P, 0, NUL) == ENULL
    assert m(P, P, P, P, P, 4, 128, 128, 128, P, 0, NUL) == ESHAPE   # N % 256
    assert m(P, P, P, P, P, 4, 128, 256, 96, P, 0, NUL) == ESHAPE    # K % 64
    assert m(P, P, P, P, P, 4, 128, 256, 0, P, 0, NUL) == ESHAPE     # K = 0 with work to do
    assert m(P, P, P, P, P, 4, 128, 256, 92 * 128 + 64, P, 0, NUL) == EUNSUP   # beyond 92 K-blocks
    assert m(P, P, P, P, P, 2049, 128, 256, 128, P, 0, NUL) == EUNSUP    # 4098 (expert, 64-row) pairs
    assert m(P, P, P, P, P, 4097, 64, 256, 128, P, 0, NUL) == EUNSUP     # 4097 pairs
    assert m(P, P, MIS, P, P, 4, 128, 256, 128, P, 0, NUL) == EALIGN
    assert m(P, P, P, P, P, 4, 128, 256, 128, P, 2, NUL) == EUNSUP   # output dtype
    assert m(P, P, P, P, P, 4, 129, 256, 128, P, 0, NUL) == EUNSUP   # M_max > 128
    assert m(P, P, P, P, P, 0, 128, 256, 128, P, 0, NUL) == OK       # G = 0
    assert m(P, P, P, P, P, 4, 0, 256, 128, P, 0, NUL) == OK         # M_max = 0
    x = lib.fp8_grouped_gemm_masked_tiled_mx
    assert x(P, P, P, NUL, P, 4, 128, 256, 128, P, 0, NUL) == ENULL
    assert x(P, P, P, P, P, 4, 126, 256, 128, P, 0, NUL) == ESHAPE    # M_max % 4
    assert x(P, P, P, P, P, 4, 128, 128, 128, P, 0, NUL) == ESHAPE    # N % 256
    assert x(P, P, P, P, P, 4, 128, 256, 96, P, 0, NUL) == ESHAPE     # K % 64
    assert x(P, P, P, P, P, 4, 128, 256, 0, P, 0, NUL) == ESHAPE      # K = 0 with work to do
    assert x(P, MIS, P, P, P, 4, 128, 256, 128, P, 0, NUL) == EALIGN
    assert x(P, P, P, P, P, 4, 128, 256, 128, P, 2, NUL) == EUNSUP    # output dtype
    assert x(P, P, P, P, P, 4, 132, 256, 128, P, 0, NUL) == EUNSUP    # M_max > 128
    assert x(P, P, P, P, P, 4097, 64, 256, 128, P, 0, NUL) == EUNSUP  # 4097 (expert, 64-row) pairs
    assert x(P, P, P, P, P, 0, 128, 256, 128, P, 0, NUL) == OK        # G = 0
    f = lib.fp8_grouped_gemm_masked_tiled_fp8out
    #        a  sa  b  sb  mm  G  M_max N    K    q  s
    assert f(P, P, P, P, P, 4, 128, 256, 128, P, NUL, NUL) == ENULL
    assert f(P, P, P, P, P, 4, 128, 128, 128, P, P2, NUL) == ESHAPE     # N % 256
    assert f(P, P, P, P, P, 4, 128, 256, 96, P, P2, NUL) == ESHAPE      # K % 64
    assert f(P, P, P, P, P, 4, 128, 256, 0, P, P2, NUL) == ESHAPE       # K = 0 with work to do
    assert f(P, P, P, P, P, 4, 128, 256, 128, P, MIS, NUL) == EALIGN
    assert f(P, P, P, P, P, 4, 129, 256, 128, P, P2, NUL) == EUNSUP     # M_max > 128
    assert f(P, P, P, P, P, 4, 128, 256, 92 * 128 + 64, P, P2, NUL) == EUNSUP   # beyond 92 K-blocks
    assert f(P, P, P, P, P, 0, 128, 256, 128, P, P2, NUL) == OK         # G = 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        fp8.fp8_quant_act_1x128(torch.zeros(4, 128))
    with pytest.raises(ValueError):
        fp8.fp8_quant_act_1x128_bf16(torch.zeros(4, 128, dtype=torch.bfloat16))


def test_plain_c_program_links_and_runs(tmp_path):
    """The header is valid C99 and a C program links libfp8fg.so directly:
    it reads the ABI version and gets host-side argument errors (no GPU work)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_fp8fg.c"
    src.write_text(r"""
#include <stdio.h>
#include "fp8fg.h"
int main(void) {
    int v = fp8fg_abi_version();
    int e1 = fp8_quant_act_1x128((const float*)0, 128, 128, 0, (uint8_t*)0, (float*)0, (void*)0);
    int e2 = fp8_gemm_blockscaled((const uint8_t*)16, (const float*)16, (const uint8_t*)16, (const float*)16,
                                  FP8FG_BSCALE_128x128, (void*)16, FP8FG_OUT_BF16, 4, 100, 128, (void*)0);
    int e3 = fp8_gemm_blockscaled_fp8mfma((const uint8_t*)16, (const float*)16, (const uint8_t*)16,
                                          (const float*)0, FP8FG_BSCALE_1x128, (void*)16, FP8FG_OUT_FP32,
                                          4, 128, 128, (void*)0);
    int e4 = fp8_grouped_gemm_contiguous_fp8out((const uint8_t*)16, (const float*)16, (const uint8_t*)16,
                                                (const float*)16, (const int32_t*)16, 4, 512, 128, 128,
                                                (uint8_t*)16, (float*)16, (void*)0);
    int e5 = fp8_grouped_gemm_masked_mx((const uint8_t*)16, (const uint8_t*)16, (const uint8_t*)16,
                                        (const uint8_t*)16, (const int32_t*)16, 4, 128, 256, 96, (void*)16,
                                        FP8FG_OUT_BF16, (void*)0);
    printf("%d %d %d %d %d %d %s\n", v, e1, e2, e3, e4, e5, fp8fg_status_string(e2));
    return v == FP8FG_ABI_VERSION && e1 == FP8FG_ERR_NULL && e2 == FP8FG_ERR_SHAPE && e3 == FP8FG_ERR_NULL &&
           e4 == FP8FG_ERR_SHAPE && e5 == FP8FG_ERR_SHAPE ? 0 : 1;
}
""")
    libdir = os.path.dirname(fp8.LIB_PATH)
    exe = tmp_path / "use_fp8fg"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", libdir, "-lfp8fg", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.split()[0] == str(fp8.ABI_VERSION)
