"""Symmetric absmax KV quantiser (oracle, test-only).

"KV Cache Engineering for LLM Serving", section 8 "Quantization": one scale
for a group of values, ``scale = max|x| / largest_code`` with
``largest_code = 2^(bits-1) - 1``; codes are ``x / scale`` rounded half to even
and clipped to ``[-largest_code, largest_code]``; the restored value is
``code * scale``.  The page's example uses bits = 4 (codes -7..7), which is
also the INT4 cache's rule (two codes per byte, ``codecs.i4_pack``); the
INT8 cache uses bits = 8 (largest code 127).  "Chapter 18", section "KV-Cache
Quantization", lists INT8 storage at one byte per value.

FP8 storage follows the same rule with the format's largest finite magnitude
as the largest code (448 for E4M3, 57344 for E5M2) and FP8
round-to-nearest-even in place of integer rounding.  ("Chapter 18", section
"vLLM with PagedAttention + KV Quantization", names an ``fp8_e5m2`` cache
without saying how it is scaled; this takes the same per-tile absmax scale
as the other formats.)

Group: one scale per (physical block, KV head) over the ``[block_size, d_k]``
tile, separately for K and V.

Grouped scales (section 8's KIVI paragraph: keys grouped by channel, values
by token, smaller groups fitting their own ranges): here a group stays
inside one block tile, so K gets one scale per (block, KV head, channel)
over the block's rows and V one per (block, KV head, token row) over the
channels (``quantize_grouped``).  The tile's largest channel scale is kept
beside the channel scales; it equals the tile scale of the one-scale rule
(rounding a quotient by the same positive divisor is monotonic).

Appending to a quantised cache (the pages do not say how): a sequence keeps
the source values of its partial last block (its "tail"); each new token is
added to the tail and the whole block is quantised again from the tail, with
the rows not yet written taken as zeros.  Zeros change neither the absmax
nor any other code, so the block holds, at every step, the codes of its
written rows, and once full exactly the codes of quantising the block at
once.

Precision: the page's example runs in float64; here every step is a single
IEEE float32 operation (absmax is exact, then one fp32 division for the scale,
one fp32 division per element, one rounding to the code grid), which is what
a GPU kernel computes.  The page's 4-bit example gives the same codes either
way.  An all-zero group has scale 0 and all codes 0.
"""

import numpy as np

from . import codecs

INT8_QMAX = 127
INT4_QMAX = 7
FP8E4M3_QMAX = 448.0
FP8E5M2_QMAX = 57344.0
CODE_DTYPES = ("i8", "i4", "fp8e4m3", "fp8e5m2")


def largest_code(bits):
    """``2^(bits-1) - 1``: 7 for 4-bit, 127 for 8-bit codes."""
    return 2 ** (bits - 1) - 1


def absmax_scale(x, qmax):
    """fp32(max|x| / qmax) for one group (x float32)."""
    a = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    return np.float32(a / np.float32(qmax))


def quantize_int(x, bits):
    """Integer codes and scale for one group (float32 arithmetic).

    Returns (codes int array, scale float32).  Half-to-even rounding is
    ``np.rint``.
    """
    x = np.asarray(x, dtype=np.float32)
    qmax = largest_code(bits)
    sc = absmax_scale(x, qmax)
    if sc == 0:
        return np.zeros(x.shape, dtype=np.int32), np.float32(0)
    y = (x / sc).astype(np.float32)
    codes = np.clip(np.rint(y), -qmax, qmax).astype(np.int32)
    return codes, sc


def quantize_fp8(x, fmt="e4m3"):
    """FP8 codes (``fmt`` "e4m3" or "e5m2") and scale for one group
    (float32 arithmetic)."""
    x = np.asarray(x, dtype=np.float32)
    qmax, encode = (FP8E4M3_QMAX, codecs.e4m3_encode) if fmt == "e4m3" else (FP8E5M2_QMAX, codecs.e5m2_encode)
    sc = absmax_scale(x, qmax)
    if sc == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0)
    y = (x / sc).astype(np.float32)
    return encode(y), sc


def dequantize(code_values, scale):
    """Restored value ``fp32(code * scale)``: one float32 multiply, rounded to
    nearest even.  ``code_values`` are the codes' own values (float32)."""
    return (np.asarray(code_values, dtype=np.float32) * np.asarray(scale, dtype=np.float32)).astype(np.float32)


def quantize_cache_blocks(cache_vals, code_dtype, block_ids=None):
    """Quantise whole blocks of a decoded float32 cache.

    ``cache_vals``: [NB, BS, Hkv, D] float32 values.  For every block in
    ``block_ids`` (all blocks if None) and every KV head, the
    ``[BS, D]`` tile gets its own scale.  Returns (codes, scales) where
    ``codes`` has the cache's shape (int8 for "i8", uint8 for "fp8e4m3" and
    "fp8e5m2", packed uint8 with D / 2 bytes per row for "i4") and
    ``scales`` is [NB, Hkv] float32; blocks not listed keep code 0 / scale 0.
    """
    NB, BS, Hkv, D = cache_vals.shape
    ids = range(NB) if block_ids is None else [int(b) for b in block_ids]
    if code_dtype == "i8":
        codes = np.zeros(cache_vals.shape, dtype=np.int8)
    elif code_dtype == "i4":
        codes = np.zeros(cache_vals.shape[:-1] + (D // 2,), dtype=np.uint8)
    elif code_dtype in ("fp8e4m3", "fp8e5m2"):
        codes = np.zeros(cache_vals.shape, dtype=np.uint8)
    else:
        raise ValueError(code_dtype)
    scales = np.zeros((NB, Hkv), dtype=np.float32)
    for b in ids:
        for h in range(Hkv):
            tile = cache_vals[b, :, h, :]
            if code_dtype == "i8":
                c, sc = quantize_int(tile, 8)
                codes[b, :, h, :] = c.astype(np.int8)
            elif code_dtype == "i4":
                c, sc = quantize_int(tile, 4)
                codes[b, :, h, :] = codecs.i4_pack(c)
            else:
                c, sc = quantize_fp8(tile, code_dtype[3:])
                codes[b, :, h, :] = c
            scales[b, h] = sc
    return codes, scales


def requantize_tail(tail_vals, rows, code_dtype):
    """Codes and scales of a block quantised from its first ``rows`` written
    rows, the others taken as zeros.

    ``tail_vals``: [BS, Hkv, D] float32 source values (rows >= ``rows`` are
    ignored).  Returns (codes of one block as ``quantize_cache_blocks``
    stores them, and scales [Hkv] float32)."""
    t = np.array(tail_vals, dtype=np.float32)
    t[rows:] = 0.0
    codes, scales = quantize_cache_blocks(t[None], code_dtype)
    return codes[0], scales[0]


def quantize_group_rows(tile, code_dtype):
    """Codes and scales of a [n, m] array quantised row by row: each row is
    one group with its own absmax scale.  Returns (codes [n, m] - packed to
    [n, m / 2] bytes for "i4" -, scales [n] float32)."""
    t = np.asarray(tile, dtype=np.float32)
    n, m = t.shape
    out = quantize_cache_blocks(t.reshape(n, 1, 1, m), code_dtype)
    return out[0][:, 0, 0, :], out[1][:, 0]


def quantize_grouped(tile, code_dtype, group):
    """One block tile [BS, D] quantised with grouped scales.

    ``group`` "channel": one scale per column (a channel across the block's
    tokens); "token": one scale per row.  Returns (codes [BS, D] as
    ``quantize_cache_blocks`` stores them, scales [D] or [BS] float32)."""
    t = np.asarray(tile, dtype=np.float32)
    if group == "token":
        return quantize_group_rows(t, code_dtype)
    if group != "channel":
        raise ValueError(group)
    if code_dtype == "i4":
        # quantise the columns as rows (integer codes), then pack the rows
        c, sc = quantize_group_rows(t.T, "i4")
        vals = codecs.decode(c, "i4").astype(np.int64)            # [D, BS] code values
        return codecs.i4_pack(vals.T), sc
    c, sc = quantize_group_rows(t.T, code_dtype)
    return np.ascontiguousarray(c.T), sc


def quantize_cache_blocks_grouped(cache_vals, code_dtype, group, block_ids=None):
    """Grouped-scale quantisation of whole blocks of a decoded cache
    [NB, BS, Hkv, D] float32.  Returns (codes in the cache's layout, group
    scales [NB, Hkv, D] for "channel" or [NB, Hkv, BS] for "token", tile
    scales [NB, Hkv] = the largest group scale of each tile).  Blocks not
    listed keep code 0 and scales 0."""
    NB, BS, Hkv, D = cache_vals.shape
    ids = range(NB) if block_ids is None else [int(b) for b in block_ids]
    codes, _ = quantize_cache_blocks(np.zeros((NB, BS, Hkv, D), np.float32), code_dtype, [])
    gs = np.zeros((NB, Hkv, D if group == "channel" else BS), dtype=np.float32)
    ts = np.zeros((NB, Hkv), dtype=np.float32)
    for b in ids:
        for h in range(Hkv):
            c, sc = quantize_grouped(cache_vals[b, :, h, :], code_dtype, group)
            codes[b, :, h, :] = c
            gs[b, h] = sc
            ts[b, h] = sc.max() if sc.size else 0
    return codes, gs, ts


def dequantize_grouped(code_values, scales, group):
    """Restored tile ``fp32(code * scale)`` for a [BS, D] tile of code values
    (float32) and its group scales ([D] for "channel", [BS] for "token")."""
    cv = np.asarray(code_values, dtype=np.float32)
    sc = np.asarray(scales, dtype=np.float32)
    return dequantize(cv, sc[None, :] if group == "channel" else sc[:, None])


def requantize_tail_grouped(tail_vals, rows, code_dtype, group):
    """``requantize_tail`` with grouped scales: the block quantised from its
    first ``rows`` written rows (the others taken as zeros) with one scale
    per channel ("channel") or per token row ("token").  Returns (codes of
    one block, group scales [Hkv, D] or [Hkv, BS], tile scales [Hkv])."""
    t = np.array(tail_vals, dtype=np.float32)
    t[rows:] = 0.0
    codes, gs, ts = quantize_cache_blocks_grouped(t[None], code_dtype, group)
    return codes[0], gs[0], ts[0]
