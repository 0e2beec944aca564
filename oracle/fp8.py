"""fp8 payload for dispatch and combine (oracle, test infrastructure only).

TensorRT-LLM PR #13888 (opt-in gate commit message) lists an fp8
low-precision combine among the cases its dispatch / combine checks cover.
The pages fix no format or scale convention; the reading taken here:

  * format: OCP 8-bit floating point E4M3 -- 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest
    finite value 448 (S.1111.110), subnormals m * 2^-9;
  * scaling: every row is cut into blocks of 128 elements (the last block may
    be shorter); each block has one power-of-two scale 2^e, the smallest
    with amax(|block|) <= 448 * 2^e (e = 0 for an all-zero block, and for a
    block holding an infinity or a NaN, whose codes are then unspecified;
    e kept in [-126, 127]).  Dividing by a power of two is exact, so the only rounding
    is the code choice;
  * code choice: round to the nearest representable E4M3 value, ties to the
    even code (last mantissa bit 0), saturating at +-448; NaN stays NaN;
  * dispatch quantizes each token row once and sends the codes and block
    scales to its k receive rows (with node deduplication: once per
    destination node to a staging row, then fanned out); combine decodes
    (code value * 2^e, exact), and forms the same weighted sum as the bf16
    combine.
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f32

BLOCK = 128
MAX_FINITE = 448.0


def e4m3_values() -> np.ndarray:
    """Value of every code 0..255 (float64); NaN for the two NaN codes."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * man * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


_VALS = e4m3_values()
_POS_CODES = np.arange(0, 0x7F)          # 0x00 .. 0x7E: the finite non-negative codes
_POS_VALS = _VALS[_POS_CODES]            # ascending


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each float (ties to the even code), saturating at +-448."""
    a = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(a), MAX_FINITE)
    hi = np.clip(np.searchsorted(_POS_VALS, mag, side="left"), 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    d_lo = np.abs(mag - _POS_VALS[lo])
    d_hi = np.abs(_POS_VALS[hi] - mag)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(a), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(a), np.uint8(0x7F) | (np.signbit(a) * np.uint8(0x80)), code).astype(np.uint8)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return _VALS[np.asarray(codes, dtype=np.uint8)]


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest e with amax <= 448 * 2^e, by comparing against the powers of two.

    e = 0 for an all-zero block, and for a block whose largest magnitude is
    not finite (an infinity or a NaN in the block); such a block's codes are
    left unspecified (reading: the pages give no rule for non-finite inputs).
    """
    a = np.asarray(amax, dtype=np.float64)
    ok = np.isfinite(a) & (a > 0)
    s = np.where(ok, a, 1.0)
    e = np.ceil(np.log2(s / MAX_FINITE)).astype(np.int64)
    # settle the borderline cases exactly: 448*2^(e-1) < amax <= 448*2^e
    e = np.where(s > MAX_FINITE * np.ldexp(1.0, e), e + 1, e)
    e = np.where(s <= MAX_FINITE * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.where(ok, e, 0)
    return np.clip(e, -126, 127)


def quantize_rows(rows_bits: np.ndarray):
    """bf16 rows [n, H] -> (codes uint8 [n, H], block exponents int [n, nb])."""
    v = bf16_to_f32(rows_bits).astype(np.float64)
    n, H = v.shape
    nb = (H + BLOCK - 1) // BLOCK
    exps = np.zeros((n, nb), dtype=np.int64)
    codes = np.zeros((n, H), dtype=np.uint8)
    for b in range(nb):
        blk = v[:, b * BLOCK:(b + 1) * BLOCK]
        e = block_exponent(np.max(np.abs(blk), axis=1)) if blk.size else np.zeros(n, np.int64)
        exps[:, b] = e
        codes[:, b * BLOCK:(b + 1) * BLOCK] = encode_e4m3(blk * np.ldexp(1.0, -e)[:, None])
    return codes, exps


def dequantize_rows(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    n, H = c.shape
    scale = np.repeat(np.ldexp(1.0, np.asarray(exps, dtype=np.int64)), BLOCK, axis=1)[:, :H]
    return decode_e4m3(c) * scale


def dispatch_fp8(x_bits: np.ndarray, plan: dict):
    """fp8 dispatch: (codes [T*k, H], block exponents [T*k, nb]) of recv rows."""
    codes, exps = quantize_rows(x_bits)
    return codes[plan["row_src"]], exps[plan["row_src"]]


def dedup_dispatch_fp8(x_bits: np.ndarray, plan: dict):
    """Node-deduplicated fp8 dispatch (FUSCO article, "load balancing and
    cross-node deduplication", with the fp8 payload above): each token is
    quantized once; hop 1 writes one staging row of codes and block exponents
    per distinct (token, node), hop 2 fans each staging row out to the
    token's receive rows on that node.

    Returns (staging codes [D, H], staging exponents [D, nb], receive codes
    [T*k, H], receive exponents [T*k, nb]).
    """
    codes, exps = quantize_rows(x_bits)
    sc, se = codes[plan["stage_src"]], exps[plan["stage_src"]]
    slots, stages = plan["slot_of"].ravel(), plan["stage_of"].ravel()
    rc = np.empty((slots.size, codes.shape[1]), dtype=np.uint8)
    re = np.empty((slots.size, exps.shape[1]), dtype=np.int64)
    rc[slots] = sc[stages]
    re[slots] = se[stages]
    return sc, se, rc, re


def combine_fp8(codes: np.ndarray, exps: np.ndarray, w: np.ndarray, plan: dict,
                chunk: int = 1024) -> np.ndarray:
    """out[t] = sum_j w[t, j] * decode(y[slot_of[t, j]]), float64, ascending j."""
    wa = np.asarray(w, dtype=np.float32).astype(np.float64)
    slot_of = plan["slot_of"]
    T, k = slot_of.shape
    H = codes.shape[1] if codes.ndim == 2 else 0
    out = np.zeros((T, H), dtype=np.float64)
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        acc = np.zeros((e - s, H), dtype=np.float64)
        for j in range(k):
            rows = slot_of[s:e, j]
            acc += wa[s:e, j:j + 1] * dequantize_rows(codes[rows], exps[rows])
        out[s:e] = acc
    return out
