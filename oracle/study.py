"""Format and granularity study on one Linear layer (test infrastructure only).

DeepSeek-V3 FP8 knowledge-base page (codingmall.com), section on unified
E4M3: where earlier FP8 training mixed formats (E4M3 forward, E5M2 for
gradients), the method uses E4M3 for every tensor, which the fine-grained
scaling makes possible; "The Insider Secrets Of Deepseek Discovered", opening
passage: per-tensor max-abs scaling is sensitive to activation outliers.

This module measures, on the linear-layer workload (X [T][7168] with outlier
channels, W [2048][7168], dY [T][2048]; the first T tokens), the relative
error that quantization alone puts into the three GEMMs of the layer --
Fprop Y = X W^T, Dgrad dX = dY W, Wgrad dW = dY^T X -- under five schemes:

  fine_e4m3     the method: 1x128 tiles for X and dY (along channels for
                Fprop / Dgrad, along tokens for Wgrad), 128x128 blocks for W,
                E4M3 everywhere
  fine_hybrid   the same groups, dY in E5M2 (scale amax / 57344)
  tensor_e4m3   one max-abs scale per tensor, E4M3 everywhere
  tensor_hybrid one scale per tensor, X and W in E4M3, dY in E5M2 (the
                earlier practice)
  mx_e4m3       microscaling (oracle/mx.py): blocks of 32 along each GEMM's
                contraction axis with power-of-two (E8M0) scales, E4M3

Each GEMM is computed exactly (float64) on the dequantized operands and
compared with the float64 GEMM of the unquantized operands, so the numbers
isolate quantization error; accumulation error is the subject of accum.py.
Run ``python -m oracle.study`` for the table.
"""

import numpy as np

from . import e4m3, e5m2, mx, quant

SCHEMES = ("fine_e4m3", "fine_hybrid", "tensor_e4m3", "tensor_hybrid", "mx_e4m3")
GEMMS = ("fprop", "dgrad", "wgrad")


def _groups_e5m2(x):
    """1x128 E5M2 quantize-dequantize along the last axis (same steps as the
    E4M3 quantizer: s = RN32(amax / 57344), code = E5M2(RN32(x / s)))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    t = x.reshape(R, K // 128, 128)
    amax = np.max(np.abs(t), axis=2, keepdims=True)
    s = (amax / np.float32(e5m2.MAX_FINITE)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(s == 0, t, (t / s).astype(np.float32))
    return (e5m2.decode(e5m2.encode(y)) * s.astype(np.float64)).reshape(R, K)


def _tensor(x, codec):
    """Per-tensor max-abs quantize-dequantize in E4M3 or E5M2."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    s = np.float32(amax / np.float32(codec.MAX_FINITE))
    if s == 0:
        return x.astype(np.float64)
    return codec.decode(codec.encode((x / s).astype(np.float32))) * np.float64(s)


def _fine_act_rows(x, fmt):
    if fmt == "e4m3":
        return quant.dequant_act(*quant.quant_act_1x128(x))
    return _groups_e5m2(x)


def _fine_act_tokens(x, fmt):
    """1x128 along tokens: the rowwise scheme applied to x^T, returned as x's layout."""
    return _fine_act_rows(np.ascontiguousarray(np.asarray(x, np.float32).T), fmt).T


def _mx_rows(x):
    """MX quantize-dequantize of each row (blocks of 32 along the last axis)."""
    return mx.dequant_mx(*mx.quant_mx_1x32(np.ascontiguousarray(x, dtype=np.float32)))


def operands(x, w, dy, scheme):
    """Dequantized float64 operands (A, B) of each GEMM, C = A . B^T."""
    if scheme == "mx_e4m3":
        x32, w32, d32 = (np.asarray(v, np.float32) for v in (x, w, dy))
        return {
            "fprop": (_mx_rows(x32), _mx_rows(w32)),
            "dgrad": (_mx_rows(d32), _mx_rows(w32.T)),
            "wgrad": (_mx_rows(d32.T), _mx_rows(x32.T)),
        }
    if scheme.startswith("fine"):
        g = "e5m2" if scheme == "fine_hybrid" else "e4m3"
        wq = quant.dequant_weight(*quant.quant_weight_128x128(w))
        return {
            "fprop": (_fine_act_rows(x, "e4m3"), wq),
            "dgrad": (_fine_act_rows(dy, g), np.ascontiguousarray(wq.T)),
            "wgrad": (np.ascontiguousarray(_fine_act_tokens(dy, g).T),
                      np.ascontiguousarray(_fine_act_tokens(x, "e4m3").T)),
        }
    gc = e5m2 if scheme == "tensor_hybrid" else e4m3
    xq, wq, dq = _tensor(x, e4m3), _tensor(w, e4m3), _tensor(dy, gc)
    return {"fprop": (xq, wq), "dgrad": (dq, np.ascontiguousarray(wq.T)),
            "wgrad": (np.ascontiguousarray(dq.T), np.ascontiguousarray(xq.T))}


def exact_operands(x, w, dy):
    x, w, dy = (np.asarray(v, np.float64) for v in (x, w, dy))
    return {"fprop": (x, w), "dgrad": (dy, np.ascontiguousarray(w.T)),
            "wgrad": (np.ascontiguousarray(dy.T), np.ascontiguousarray(x.T))}


def rel_error(c, c_ref):
    """Relative Frobenius error ||C - C_ref|| / ||C_ref||."""
    return float(np.linalg.norm(c - c_ref) / np.linalg.norm(c_ref))


def run(x, w, dy, schemes=SCHEMES):
    """{scheme: {gemm: relative error}} on the given tensors."""
    ref = {k: a @ b.T for k, (a, b) in exact_operands(x, w, dy).items()}
    out = {}
    for sc in schemes:
        ops = operands(x, w, dy, sc)
        out[sc] = {k: rel_error(a @ b.T, ref[k]) for k, (a, b) in ops.items()}
    return out


def main(tokens=1024):
    import workloads
    x, w, dy = workloads.linear_trio()
    x, dy = x[:tokens], dy[:tokens]
    res = run(x, w, dy)
    print(f"relative Frobenius error of each GEMM from quantization alone, first {tokens} tokens")
    print("| scheme | " + " | ".join(GEMMS) + " |")
    print("|---|" + "---|" * len(GEMMS))
    for sc in SCHEMES:
        print(f"| {sc} | " + " | ".join(f"{res[sc][g]:.3e}" for g in GEMMS) + " |")


if __name__ == "__main__":
    main()
