"""MXFP4 expert weights oracle (test infrastructure only; see the package docstring).

The vLLM PR #45457 report's gpt-oss path runs its experts with MXFP4 weights
(the ``OAITritonMxfp4ExpertsMonolithic`` forward named in "key source
snippets") and bf16 activations; the pages name the format only.  The
definition followed here is the public OCP Microscaling (MX) one for MXFP4:

* every 32 consecutive weights along K share one E8M0 scale 2^X (stored as the
  byte X + 127);
* X = floor(log2(max |w| of the block)) - 2, the 2 being the largest exponent
  of the element format, so the block's largest value lands in [4, 8);
* each weight is w / 2^X rounded to the nearest FP4 E2M1 value (magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the code whose lowest bit is 0,
  magnitudes above 6 saturating to 6; the sign is kept (a negative weight that
  rounds to zero gets the negative-zero code 8);
* an all-zero block gets X = -127 (scale byte 0) and zero codes.

Codes pack two to a byte along K, the even element in the low nibble.  The
value of code c is (-1)^(c >> 3) * E2M1[c & 7] * 2^X.
"""
from __future__ import annotations

import numpy as np

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 32


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (uint8 0..15) of values already divided by the block scale."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # nearest magnitude; on a tie keep the lower index if it is even, else the higher
    d = np.abs(a[..., None] - E2M1)                  # [..., 8]
    best = np.argmin(d, axis=-1)                     # first minimum: the lower magnitude
    dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
    up = np.minimum(best + 1, 7)
    tie = (np.take_along_axis(d, up[..., None], -1)[..., 0] == dmin) & (up != best)
    best = np.where(tie & (best % 2 == 1), up, best)
    best = np.where(a > 6.0, 7, best)                # saturate
    sign = (np.signbit(v) & ~np.isnan(v)).astype(np.uint8) << 3
    return (best.astype(np.uint8) | sign).astype(np.uint8)


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    mag = E2M1[c & 7]
    return np.where(c & 8, -mag, mag)


def quantize_mxfp4(w) -> tuple[np.ndarray, np.ndarray]:
    """``w [..., K]`` (K a multiple of 32) -> packed codes ``q [..., K/2]`` uint8 and
    scale bytes ``s [..., K/32]`` uint8 (the block-major layout the kernels take is
    a transpose of ``s``, made by the caller)."""
    try:
        import torch
        if isinstance(w, torch.Tensor):
            w = w.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    w = np.asarray(w, dtype=np.float64)
    k = w.shape[-1]
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = w.reshape(*w.shape[:-1], k // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        x = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    x = np.clip(x, -127, 127)
    codes = e2m1_encode(blocks / np.exp2(x)[..., None])
    codes = codes.reshape(*w.shape[:-1], k)
    q = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    s = (x + 127).astype(np.uint8)
    return q, s


def dequantize_mxfp4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Float64 weights ``[..., K]`` from packed codes and scale bytes."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    k = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(*q.shape[:-1], k // BLOCK, BLOCK)
    scale = np.exp2(s.astype(np.float64) - 127.0)
    return (vals * scale[..., None]).reshape(*q.shape[:-1], k)
