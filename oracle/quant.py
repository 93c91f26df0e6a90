"""Online fine-grained FP8 quantization (test infrastructure only).

Method: "The Insider Secrets Of Deepseek Discovered", passage on Figure 7(a):
activations are grouped and scaled per 1x128 tile (one token, 128 channels),
weights per 128x128 block (128 input x 128 output channels).  The usual
per-tensor practice of mapping the tensor's max-abs onto the FP8 maximum is
named there as the outlier-sensitive baseline; the fine-grained scheme applies
the same max-abs mapping per group.  DeepSeek-V3 FP8 knowledge-base page
(codingmall.com), section on online quantization: each scale is computed from
the current tile or block, not from a history of past maxima.

Steps per group g (all float32, IEEE round-to-nearest):
    amax_g = max |x|                        (exact)
    s_g    = RN32(amax_g / 448)             stored dequantization multiplier
    y      = RN32(x / s_g)                  IEEE division, not x * (1/s)
    q      = E4M3_RNE_SAT(y)
Readings where the pages are silent: s is the multiplier that dequantizes
(value ~ dec(q) * s), not its inverse; a group whose amax is 0 keeps s = 0
and its codes are signed zeros.

Scale layouts (shared with the library's C interface):
    1x128, tiles along K : q [R][K],  s [K/128][R]       ("kb-major")
    1x128, tiles along R : q [K][R],  s [R/128][K]       (token-wise, transposed out)
    128x128              : q [N][K],  s [N/128][K/128]   (or q^T, s^T)

Partial tiles (reading; the pages only use whole groups): when the grouped
axis is not a multiple of 128 the last group is shorter, and it is treated as
the group zero-padded to 128 -- its max-abs runs over the elements that exist,
the padding's codes are dropped.  Scale counts round up: K/128 above means
ceil(K/128).  Computed exactly that way here: pad with zeros, quantize, slice.
"""


def _ceil128(n):
    return -(-n // 128) * 128

import numpy as np

from . import e4m3

_F448 = np.float32(448.0)


def _scale_and_cast(groups, amax):
    """groups: float32 array whose trailing axes hold one group each, with
    ``amax`` broadcastable against it.  Returns codes (same shape) and s."""
    amax = amax.astype(np.float32)
    s = (amax / _F448).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (groups / s).astype(np.float32)
    y = np.where(s == 0, groups, y)          # all-zero group: keep the signed zeros
    return e4m3.encode(y), s


def quant_act_1x128(x):
    """1x128 tiles along K.  x float32 [R][K] -> (q u8 [R][K], s f32 [ceil(K/128)][R])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    if K % 128:
        q, s = quant_act_1x128(np.pad(x, ((0, 0), (0, _ceil128(K) - K))))
        return np.ascontiguousarray(q[:, :K]), s
    t = x.reshape(R, K // 128, 128)
    amax = np.max(np.abs(t), axis=2, keepdims=True) if R else np.zeros((0, K // 128, 1), np.float32)
    q, s = _scale_and_cast(t, amax)
    return q.reshape(R, K), np.ascontiguousarray(s[:, :, 0].T)


def quant_act_1x128_tokenwise(x):
    """1x128 tiles along the token axis R, transposed output.

    x float32 [R][K] -> (q u8 [K][R], s f32 [R/128][K]).  A tile is 128
    consecutive tokens of one channel: exactly the 1x128 rowwise quantization
    of x^T, which is how it is computed here.
    """
    x = np.asarray(x, dtype=np.float32)
    return quant_act_1x128(np.ascontiguousarray(x.T))


def quant_weight_128x128(w, transpose_out=False):
    """128x128 blocks.  w float32 [N][K] ->
    (q u8 [N][K], s f32 [N/128][K/128]), or (q^T [K][N], s^T [K/128][N/128])
    (block counts rounded up)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if N % 128 or K % 128:
        q, s = quant_weight_128x128(np.pad(w, ((0, _ceil128(N) - N), (0, _ceil128(K) - K))))
        q = np.ascontiguousarray(q[:N, :K])
        if transpose_out:
            return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)
        return q, s
    t = w.reshape(N // 128, 128, K // 128, 128)
    amax = np.max(np.abs(t), axis=(1, 3), keepdims=True)
    q, s = _scale_and_cast(t, amax)
    q = q.reshape(N, K)
    s = s[:, 0, :, 0]
    if transpose_out:
        return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)
    return q, np.ascontiguousarray(s)


def quant_per_tensor(x):
    """Per-tensor max-abs scaling (the baseline the fine-grained scheme replaces).
    Used only by the outlier demonstration.  Returns (q, s) with a scalar s."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x)).reshape(1)
    q, s = _scale_and_cast(x, amax)
    return q, s[0]


def dequant_act(q, s):
    """Exact float64 values of 1x128-quantized rows: q u8 [R][K], s [ceil(K/128)][R]."""
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    K = np.asarray(q).shape[1]
    return e4m3.decode(q) * np.repeat(s.T, 128, axis=1)[:, :K]


def dequant_weight(q, s):
    """Exact float64 values of 128x128-quantized blocks: q u8 [N][K], s [ceil(N/128)][ceil(K/128)]."""
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    N, K = np.asarray(q).shape
    return e4m3.decode(q) * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:N, :K]


def dequant32(q, s_full):
    """RN32(dec(q) * s) with s already expanded per element (for idempotence checks)."""
    return (e4m3.decode(q).astype(np.float32) * np.asarray(s_full, np.float32)).astype(np.float32)


def requant_act_tokenwise(q, s):
    """FP8 activation cache for backward.

    "The Insider Secrets Of Deepseek Discovered", passage on Figure 6: with
    Wgrad in FP8, a Linear's input can be kept in FP8 for the backward pass.
    The Fprop operand is cached as rowwise 1x128 codes q u8 [R][K] with scales
    s f32 [K/128][R]; the Wgrad operand is 1x128 along tokens.  Steps:
        x'[r][k] = RN32(dec(q[r][k]) * s[k/128][r])   (fp32 dequantization)
        (qt, st) = 1x128 quantization of x' along tokens, transposed out
    Returns (qt u8 [K][R], st f32 [ceil(R/128)][K]).
    """
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    R, K = q.shape
    assert s.shape == (-(-K // 128), R)
    x = dequant32(q, np.repeat(s.T, 128, axis=1)[:, :K])
    return quant_act_1x128_tokenwise(x)
