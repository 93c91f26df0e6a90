"""Python binding of libfp8fg.so: fine-grained FP8 quantization and block-scaled
FP8 GEMM for AMD MI355X (gfx950).

The functions below carry the names of the C entry points declared in
include/fp8fg.h and only marshal arguments: they take torch tensors that live
on the GPU, check dtypes and shapes, pass raw device pointers and the current
HIP stream to the library, and raise Fp8fgError on a non-zero status.  Every
step of the computation runs in the library's HIP kernels; there is no other
implementation behind these names.  Outputs are allocated here with torch
unless the caller passes them in (``out=``/``q=``/``s=``).
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8fg.so")

BSCALE_128x128 = 0
BSCALE_1x128 = 1
OUT_BF16 = 0
OUT_FP32 = 1

ABI_VERSION = 14
EXPORTS = ("fp8_quant_act_1x128", "fp8_quant_weight_128x128", "fp8_gemm_blockscaled",
           "fp8_grouped_gemm_contiguous", "fp8_grouped_gemm_masked",
           "fp8_quant_act_1x128_bf16", "fp8_quant_weight_128x128_bf16", "fp8_requant_act_tokenwise",
           "fp8_quant_mx_1x32", "fp8_gemm_mx", "fp8_gemm_blockscaled_fp8out", "fp8_quant_fprop_operands",
           "fp8_tile_weights_decode", "fp8_grouped_gemm_masked_tiled", "fp8_gemm_blockscaled_fp8mfma",
           "fp8_grouped_gemm_contiguous_fp8out", "fp8_grouped_gemm_contiguous_mx", "fp8_grouped_gemm_masked_mx",
           "fp8_quant_mx_1x32_transposed", "fp8_grouped_gemm_masked_tiled_fp8out",
           "fp8_grouped_gemm_masked_tiled_mx", "fp8fg_status_string", "fp8fg_abi_version")
_COMPUTE = EXPORTS[:21]


class Fp8fgError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


_lib = None


def load_library(path=LIB_PATH):
    """Load (once) and return the ctypes handle of libfp8fg.so; raise if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python fp8_fine_grained_amd/build.py`")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.fp8_quant_act_1x128.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.fp8_quant_weight_128x128.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.fp8_gemm_blockscaled.argtypes = [vp, vp, vp, vp, i32, vp, i32, i64, i64, i64, vp]
    lib.fp8_gemm_blockscaled_fp8mfma.argtypes = [vp, vp, vp, vp, i32, vp, i32, i64, i64, i64, vp]
    lib.fp8_grouped_gemm_contiguous.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    lib.fp8_grouped_gemm_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    lib.fp8_quant_act_1x128_bf16.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.fp8_quant_weight_128x128_bf16.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.fp8_requant_act_tokenwise.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.fp8_quant_mx_1x32.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.fp8_quant_mx_1x32_transposed.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.fp8_gemm_mx.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    lib.fp8_gemm_blockscaled_fp8out.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_quant_fprop_operands.argtypes = [vp, i32, i64, vp, i32, i64, i64, vp, vp, vp, vp, vp]
    lib.fp8_tile_weights_decode.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.fp8_grouped_gemm_masked_tiled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    lib.fp8_grouped_gemm_contiguous_fp8out.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.fp8_grouped_gemm_masked_tiled_fp8out.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.fp8_grouped_gemm_masked_tiled_mx.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    lib.fp8_grouped_gemm_contiguous_mx.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    lib.fp8_grouped_gemm_masked_mx.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    for name in _COMPUTE:
        getattr(lib, name).restype = ctypes.c_int
    lib.fp8fg_status_string.argtypes = [ctypes.c_int]
    lib.fp8fg_status_string.restype = ctypes.c_char_p
    lib.fp8fg_abi_version.argtypes = []
    lib.fp8fg_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status):
    return load_library().fp8fg_status_string(int(status)).decode()


def abi_version():
    return load_library().fp8fg_abi_version()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn, status):
    if status != 0:
        raise Fp8fgError(fn, status)


def _need(t, dtype, shape, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nb(n):
    """Number of 128-wide groups along an axis of length n (a last partial group counts)."""
    return (n + 127) // 128


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _quant_act(fn, x, dtype, transpose_out, q, s):
    M, K = x.shape
    _need(x, dtype, (M, K), "x")
    qs = (K, M) if transpose_out else (M, K)
    ss = (_nb(M), K) if transpose_out else (_nb(K), M)
    q = _empty(qs, torch.uint8, x) if q is None else q
    s = _empty(ss, torch.float32, x) if s is None else s
    _need(q, torch.uint8, qs, "q")
    _need(s, torch.float32, ss, "s")
    _check(fn, getattr(load_library(), fn)(_ptr(x), M, K, int(bool(transpose_out)), _ptr(q), _ptr(s), _stream(x)))
    return q, s


def _quant_weight(fn, w, dtype, transpose_out, q, s):
    N, K = w.shape
    _need(w, dtype, (N, K), "w")
    qs = (K, N) if transpose_out else (N, K)
    ss = (_nb(K), _nb(N)) if transpose_out else (_nb(N), _nb(K))
    q = _empty(qs, torch.uint8, w) if q is None else q
    s = _empty(ss, torch.float32, w) if s is None else s
    _need(q, torch.uint8, qs, "q")
    _need(s, torch.float32, ss, "s")
    _check(fn, getattr(load_library(), fn)(_ptr(w), N, K, int(bool(transpose_out)), _ptr(q), _ptr(s), _stream(w)))
    return q, s


def fp8_quant_act_1x128(x, transpose_out=False, q=None, s=None):
    """1x128 activation quantization of x f32 [M][K].
    transpose_out=False -> (q u8 [M][K], s f32 [K/128][M]);
    transpose_out=True  -> (q u8 [K][M], s f32 [M/128][K]) (tiles along M)."""
    return _quant_act("fp8_quant_act_1x128", x, torch.float32, transpose_out, q, s)


def fp8_quant_act_1x128_bf16(x, transpose_out=False, q=None, s=None):
    """fp8_quant_act_1x128 for x bf16 [M][K] (quantizes the exactly widened values)."""
    return _quant_act("fp8_quant_act_1x128_bf16", x, torch.bfloat16, transpose_out, q, s)


def fp8_quant_weight_128x128(w, transpose_out=False, q=None, s=None):
    """128x128 weight quantization of w f32 [N][K] -> (q u8 [N][K], s f32 [N/128][K/128]),
    or the transposed codes and scales when transpose_out=True."""
    return _quant_weight("fp8_quant_weight_128x128", w, torch.float32, transpose_out, q, s)


def fp8_quant_weight_128x128_bf16(w, transpose_out=False, q=None, s=None):
    """fp8_quant_weight_128x128 for w bf16 [N][K] (quantizes the exactly widened values)."""
    return _quant_weight("fp8_quant_weight_128x128_bf16", w, torch.bfloat16, transpose_out, q, s)


def fp8_quant_fprop_operands(x, w, qa=None, sa=None, qb=None, sb=None):
    """Both Fprop operands in one launch: x f32 or bf16 [M][K], w f32 or bf16
    [N][K] -> (qa u8 [M][K], sa f32 [K/128][M], qb u8 [N][K], sb f32
    [N/128][K/128]), exactly fp8_quant_act_1x128(x) and
    fp8_quant_weight_128x128(w) (or their bf16 forms)."""
    M, K = x.shape
    N = w.shape[0]
    if x.dtype not in (torch.float32, torch.bfloat16) or w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x and w must be float32 or bfloat16")
    _need(x, x.dtype, (M, K), "x")
    _need(w, w.dtype, (N, K), "w")
    qa = _empty((M, K), torch.uint8, x) if qa is None else qa
    sa = _empty((_nb(K), M), torch.float32, x) if sa is None else sa
    qb = _empty((N, K), torch.uint8, w) if qb is None else qb
    sb = _empty((_nb(N), _nb(K)), torch.float32, w) if sb is None else sb
    _need(qa, torch.uint8, (M, K), "qa")
    _need(sa, torch.float32, (_nb(K), M), "sa")
    _need(qb, torch.uint8, (N, K), "qb")
    _need(sb, torch.float32, (_nb(N), _nb(K)), "sb")
    _check("fp8_quant_fprop_operands", load_library().fp8_quant_fprop_operands(
        _ptr(x), int(x.dtype == torch.bfloat16), M, _ptr(w), int(w.dtype == torch.bfloat16), N, K,
        _ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), _stream(x)))
    return qa, sa, qb, sb


def fp8_requant_act_tokenwise(q, s, qt=None, st=None):
    """Rowwise FP8 cache (q u8 [M][K], s f32 [K/128][M]) -> the token-wise
    operand (qt u8 [K][M], st f32 [M/128][K]) of RN32(decode(q) * s)."""
    M, K = q.shape
    _need(q, torch.uint8, (M, K), "q")
    _need(s, torch.float32, (_nb(K), M), "s")
    qt = _empty((K, M), torch.uint8, q) if qt is None else qt
    st = _empty((_nb(M), K), torch.float32, q) if st is None else st
    _need(qt, torch.uint8, (K, M), "qt")
    _need(st, torch.float32, (_nb(M), K), "st")
    _check("fp8_requant_act_tokenwise",
           load_library().fp8_requant_act_tokenwise(_ptr(q), _ptr(s), M, K, _ptr(qt), _ptr(st), _stream(q)))
    return qt, st


def fp8_quant_mx_1x32(x, q=None, e=None):
    """MX quantization of x f32 [R][K]: (codes u8 [R][K], E8M0 scale bytes u8 [K/32][R])."""
    R, K = x.shape
    _need(x, torch.float32, (R, K), "x")
    q = _empty((R, K), torch.uint8, x) if q is None else q
    e = _empty((K // 32, R), torch.uint8, x) if e is None else e
    _need(q, torch.uint8, (R, K), "q")
    _need(e, torch.uint8, (K // 32, R), "e")
    _check("fp8_quant_mx_1x32", load_library().fp8_quant_mx_1x32(_ptr(x), R, K, _ptr(q), _ptr(e), _stream(x)))
    return q, e


def fp8_quant_mx_1x32_transposed(x, q=None, e=None):
    """MX quantization of x f32 [M][K] in blocks of 32 rows, transposed:
    (codes u8 [K][M], E8M0 scale bytes u8 [M/32][K]) = fp8_quant_mx_1x32(x^T)."""
    M, K = x.shape
    _need(x, torch.float32, (M, K), "x")
    q = _empty((K, M), torch.uint8, x) if q is None else q
    e = _empty((M // 32, K), torch.uint8, x) if e is None else e
    _need(q, torch.uint8, (K, M), "q")
    _need(e, torch.uint8, (M // 32, K), "e")
    _check("fp8_quant_mx_1x32_transposed", load_library().fp8_quant_mx_1x32_transposed(
        _ptr(x), M, K, _ptr(q), _ptr(e), _stream(x)))
    return q, e


def fp8_gemm_mx(a, ea, b, eb, out_dtype=torch.bfloat16, out=None):
    """C = A . B^T of MX operands: a u8 [M][K] / ea u8 [K/32][M], b u8 [N][K] / eb u8 [K/32][N]."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(ea, torch.uint8, (K // 32, M), "ea")
    _need(b, torch.uint8, (N, K), "b")
    _need(eb, torch.uint8, (K // 32, N), "eb")
    out = _empty((M, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (M, N), "out")
    _check("fp8_gemm_mx", load_library().fp8_gemm_mx(_ptr(a), _ptr(ea), _ptr(b), _ptr(eb), _ptr(out),
                                                      _out_dtype(out_dtype), M, N, K, _stream(a)))
    return out


def fp8_grouped_gemm_contiguous_mx(a, ea, b, eb, group_offsets, out_dtype=torch.bfloat16, out=None):
    """fp8_grouped_gemm_contiguous on MX operands: a u8 [M_total][K] / ea u8
    [K/32][M_total], b u8 [G][N][K] / eb u8 [G][K/32][N]; off device int32 [G+1]."""
    M_total, K = a.shape
    G, N, _ = b.shape
    _need(a, torch.uint8, (M_total, K), "a")
    _need(ea, torch.uint8, (K // 32, M_total), "ea")
    _need(b, torch.uint8, (G, N, K), "b")
    _need(eb, torch.uint8, (G, K // 32, N), "eb")
    _need(group_offsets, torch.int32, (G + 1,), "group_offsets")
    out = _empty((M_total, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (M_total, N), "out")
    _check("fp8_grouped_gemm_contiguous_mx", load_library().fp8_grouped_gemm_contiguous_mx(
        _ptr(a), _ptr(ea), _ptr(b), _ptr(eb), _ptr(group_offsets), G, M_total, N, K, _ptr(out),
        _out_dtype(out_dtype), _stream(a)))
    return out


def fp8_grouped_gemm_masked_mx(a, ea, b, eb, masked_m, out_dtype=torch.bfloat16, out=None):
    """fp8_grouped_gemm_masked on MX operands: a u8 [G][M_max][K] / ea u8
    [G][K/32][M_max], b u8 [G][N][K] / eb u8 [G][K/32][N]; rows >= masked_m[g]
    of out are not written."""
    G, M_max, K = a.shape
    N = b.shape[1]
    _need(a, torch.uint8, (G, M_max, K), "a")
    _need(ea, torch.uint8, (G, K // 32, M_max), "ea")
    _need(b, torch.uint8, (G, N, K), "b")
    _need(eb, torch.uint8, (G, K // 32, N), "eb")
    _need(masked_m, torch.int32, (G,), "masked_m")
    out = _empty((G, M_max, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (G, M_max, N), "out")
    _check("fp8_grouped_gemm_masked_mx", load_library().fp8_grouped_gemm_masked_mx(
        _ptr(a), _ptr(ea), _ptr(b), _ptr(eb), _ptr(masked_m), G, M_max, N, K, _ptr(out),
        _out_dtype(out_dtype), _stream(a)))
    return out


def _out_dtype(out_dtype):
    return {torch.bfloat16: OUT_BF16, torch.float32: OUT_FP32}[out_dtype]


def _gemm_dense(fn, a, sa, b, sb, bscale_kind, out_dtype, out):
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(sa, torch.float32, (_nb(K), M), "sa")
    _need(b, torch.uint8, (N, K), "b")
    _need(sb, torch.float32, (_nb(N), _nb(K)) if bscale_kind == BSCALE_128x128 else (_nb(K), N), "sb")
    out = _empty((M, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (M, N), "out")
    _check(fn, getattr(load_library(), fn)(
        _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), int(bscale_kind), _ptr(out), _out_dtype(out_dtype),
        M, N, K, _stream(a)))
    return out


def fp8_gemm_blockscaled(a, sa, b, sb, bscale_kind=BSCALE_128x128, out_dtype=torch.bfloat16, out=None):
    """C[M][N] = A[M][K] . B[N][K]^T with 1x128 A scales and 128x128 (or 1x128) B scales."""
    return _gemm_dense("fp8_gemm_blockscaled", a, sa, b, sb, bscale_kind, out_dtype, out)


def fp8_gemm_blockscaled_fp8mfma(a, sa, b, sb, bscale_kind=BSCALE_128x128, out_dtype=torch.bfloat16, out=None):
    """fp8_gemm_blockscaled on the FP8 matrix cores: same operands and layouts,
    accuracy contract 2^-9 * sum|a b| instead of 2^-14 (see fp8fg.h)."""
    return _gemm_dense("fp8_gemm_blockscaled_fp8mfma", a, sa, b, sb, bscale_kind, out_dtype, out)


def fp8_gemm_blockscaled_fp8out(a, sa, b, sb, q=None, s=None):
    """C = A . B^T (128x128 B scales) quantized 1x128 along N in the epilogue:
    returns (q u8 [M][N], s f32 [N/128][M]) -- the next layer's A operand."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(sa, torch.float32, (_nb(K), M), "sa")
    _need(b, torch.uint8, (N, K), "b")
    _need(sb, torch.float32, (N // 128, _nb(K)), "sb")
    q = _empty((M, N), torch.uint8, a) if q is None else q
    s = _empty((N // 128, M), torch.float32, a) if s is None else s
    _need(q, torch.uint8, (M, N), "q")
    _need(s, torch.float32, (N // 128, M), "s")
    _check("fp8_gemm_blockscaled_fp8out", load_library().fp8_gemm_blockscaled_fp8out(
        _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(q), _ptr(s), M, N, K, _stream(a)))
    return q, s


def fp8_grouped_gemm_contiguous_fp8out(a, sa, b, sb, group_offsets, q=None, s=None):
    """Contiguous MoE layout with the output quantized 1x128 along N in the
    epilogue: returns (q u8 [M_total][N], s f32 [N/128][M_total]); rows in no
    expert's range are left as they were (zeros when q, s are allocated here)."""
    M_total, K = a.shape
    G, N, _ = b.shape
    _need(a, torch.uint8, (M_total, K), "a")
    _need(sa, torch.float32, (_nb(K), M_total), "sa")
    _need(b, torch.uint8, (G, N, K), "b")
    _need(sb, torch.float32, (G, _nb(N), _nb(K)), "sb")
    _need(group_offsets, torch.int32, (G + 1,), "group_offsets")
    q = torch.zeros((M_total, N), dtype=torch.uint8, device=a.device) if q is None else q
    s = torch.zeros((N // 128, M_total), dtype=torch.float32, device=a.device) if s is None else s
    _need(q, torch.uint8, (M_total, N), "q")
    _need(s, torch.float32, (N // 128, M_total), "s")
    _check("fp8_grouped_gemm_contiguous_fp8out", load_library().fp8_grouped_gemm_contiguous_fp8out(
        _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(group_offsets), G, M_total, N, K, _ptr(q), _ptr(s), _stream(a)))
    return q, s


def fp8_grouped_gemm_contiguous(a, sa, b, sb, group_offsets, out_dtype=torch.bfloat16, out=None):
    """Contiguous MoE layout: expert g owns rows [off[g], off[g+1]) of a; off is device int32 [G+1]."""
    M_total, K = a.shape
    G, N, _ = b.shape
    _need(a, torch.uint8, (M_total, K), "a")
    _need(sa, torch.float32, (_nb(K), M_total), "sa")
    _need(b, torch.uint8, (G, N, K), "b")
    _need(sb, torch.float32, (G, _nb(N), _nb(K)), "sb")
    _need(group_offsets, torch.int32, (G + 1,), "group_offsets")
    out = _empty((M_total, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (M_total, N), "out")
    _check("fp8_grouped_gemm_contiguous", load_library().fp8_grouped_gemm_contiguous(
        _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(group_offsets), G, M_total, N, K, _ptr(out),
        _out_dtype(out_dtype), _stream(a)))
    return out


def fp8_grouped_gemm_masked(a, sa, b, sb, masked_m, out_dtype=torch.bfloat16, out=None):
    """Masked MoE layout: a u8 [G][M_max][K]; rows >= masked_m[g] of out are not written."""
    G, M_max, K = a.shape
    N = b.shape[1]
    _need(a, torch.uint8, (G, M_max, K), "a")
    _need(sa, torch.float32, (G, _nb(K), M_max), "sa")
    _need(b, torch.uint8, (G, N, K), "b")
    _need(sb, torch.float32, (G, _nb(N), _nb(K)), "sb")
    _need(masked_m, torch.int32, (G,), "masked_m")
    out = _empty((G, M_max, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (G, M_max, N), "out")
    _check("fp8_grouped_gemm_masked", load_library().fp8_grouped_gemm_masked(
        _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(masked_m), G, M_max, N, K, _ptr(out),
        _out_dtype(out_dtype), _stream(a)))
    return out


def fp8_grouped_gemm_masked_tiled_mx(a, ea, b_tiled, eb, masked_m, out_dtype=torch.bfloat16, out=None):
    """fp8_grouped_gemm_masked_mx with the experts' codes in the decode-tiled
    layout (b_tiled u8 [G][N/256][K/64][16384], from fp8_tile_weights_decode)."""
    G, M_max, K = a.shape
    N = b_tiled.shape[1] * 256
    _need(a, torch.uint8, (G, M_max, K), "a")
    _need(ea, torch.uint8, (G, K // 32, M_max), "ea")
    _need(b_tiled, torch.uint8, (G, N // 256, K // 64, 16384), "b_tiled")
    _need(eb, torch.uint8, (G, K // 32, N), "eb")
    _need(masked_m, torch.int32, (G,), "masked_m")
    out = _empty((G, M_max, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (G, M_max, N), "out")
    _check("fp8_grouped_gemm_masked_tiled_mx", load_library().fp8_grouped_gemm_masked_tiled_mx(
        _ptr(a), _ptr(ea), _ptr(b_tiled), _ptr(eb), _ptr(masked_m), G, M_max, N, K, _ptr(out),
        _out_dtype(out_dtype), _stream(a)))
    return out


def fp8_grouped_gemm_masked_tiled_fp8out(a, sa, b_tiled, sb, masked_m, q=None, s=None):
    """fp8_grouped_gemm_masked_tiled with the output quantized 1x128 along N in
    the epilogue: returns (q u8 [G][M_max][N], s f32 [G][N/128][M_max]); rows
    past masked_m[g] are left as they were (zeros when q, s are allocated here)."""
    G, M_max, K = a.shape
    N = b_tiled.shape[1] * 256
    _need(a, torch.uint8, (G, M_max, K), "a")
    _need(sa, torch.float32, (G, _nb(K), M_max), "sa")
    _need(b_tiled, torch.uint8, (G, N // 256, K // 64, 16384), "b_tiled")
    _need(sb, torch.float32, (G, _nb(N), _nb(K)), "sb")
    _need(masked_m, torch.int32, (G,), "masked_m")
    q = torch.zeros((G, M_max, N), dtype=torch.uint8, device=a.device) if q is None else q
    s = torch.zeros((G, N // 128, M_max), dtype=torch.float32, device=a.device) if s is None else s
    _need(q, torch.uint8, (G, M_max, N), "q")
    _need(s, torch.float32, (G, N // 128, M_max), "s")
    _check("fp8_grouped_gemm_masked_tiled_fp8out", load_library().fp8_grouped_gemm_masked_tiled_fp8out(
        _ptr(a), _ptr(sa), _ptr(b_tiled), _ptr(sb), _ptr(masked_m), G, M_max, N, K, _ptr(q), _ptr(s), _stream(a)))
    return q, s


def fp8_tile_weights_decode(q, out=None):
    """Experts' codes u8 [G][N][K] -> the decode-tiled layout, returned as u8
    [G][N/256][K/64][16384]: one 16 KB block per (expert, 256-row n-tile,
    64-byte K piece), in the order fp8fg.h defines."""
    G, N, K = q.shape
    _need(q, torch.uint8, (G, N, K), "q")
    shape = (G, N // 256, K // 64, 16384)
    out = _empty(shape, torch.uint8, q) if out is None else out
    _need(out, torch.uint8, shape, "out")
    _check("fp8_tile_weights_decode", load_library().fp8_tile_weights_decode(
        _ptr(q), G, N, K, _ptr(out), _stream(q)))
    return out


def fp8_grouped_gemm_masked_tiled(a, sa, b_tiled, sb, masked_m, out_dtype=torch.bfloat16, out=None):
    """fp8_grouped_gemm_masked with the experts' codes in the decode-tiled
    layout (b_tiled u8 [G][N/256][K/64][16384], from fp8_tile_weights_decode)."""
    G, M_max, K = a.shape
    N = b_tiled.shape[1] * 256
    _need(a, torch.uint8, (G, M_max, K), "a")
    _need(sa, torch.float32, (G, _nb(K), M_max), "sa")
    _need(b_tiled, torch.uint8, (G, N // 256, K // 64, 16384), "b_tiled")
    _need(sb, torch.float32, (G, _nb(N), _nb(K)), "sb")
    _need(masked_m, torch.int32, (G,), "masked_m")
    out = _empty((G, M_max, N), out_dtype, a) if out is None else out
    _need(out, out_dtype, (G, M_max, N), "out")
    _check("fp8_grouped_gemm_masked_tiled", load_library().fp8_grouped_gemm_masked_tiled(
        _ptr(a), _ptr(sa), _ptr(b_tiled), _ptr(sb), _ptr(masked_m), G, M_max, N, K, _ptr(out),
        _out_dtype(out_dtype), _stream(a)))
    return out
