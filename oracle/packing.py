"""Canonical packed layout of quantized key and value streams.

Test infrastructure (see ``oracle/__init__``).

The pages only say the indices are stored compactly and that attention is
computed straight from them (P3 "How it works", closing paragraph; "How to
implement", item 1, which mentions uint8 indices).  The bit layout is this
implementation's choice, fixed here so that GPU parity is byte-for-byte.
All words are little-endian uint32; bit k of a word is (word >> k) & 1.

Key stream (one record per token, coordinates along the word):
  codes[s, t, w, p]  bit k = bit p of idx[s, t, 32*w + k]     shape [S, T, ceil(d/32), b]
  signs[s, t, w]     bit k = sign bit of z[s, t, 32*w + k]    shape [S, T, ceil(m/32)]
  (when d or m is not a multiple of 32 the last word is padded with 0 bits:
  the search workload of the pages runs at d = 200)
Value stream (blocks of 32 tokens; one record of b words per coordinate):
  codes[s, B, j, :]  the 32 b-bit indices idx[s, 32*B + k, j], k = 0..31,
                     packed in token order: index k occupies bits
                     [b*k, b*k + b) of the record read as one little-endian
                     32b-bit integer (word 0 holds the lowest bits; a field
                     may straddle two words).       shape [S, ceil(T/32), d, b]
  fields of tokens past T in the last block are 0.
Norms are one value per token, [S, T], stored as float32 or as float16
(round to nearest even).
"""

import numpy as np


def pack_key_codes(idx, bits):
    """idx [..., d] -> words [..., ceil(d/32), bits]; the bits of the padding
    coordinates d .. 32 ceil(d/32) - 1 are 0."""
    idx = np.asarray(idx, dtype=np.int64)
    *lead, d = idx.shape
    words = np.zeros((*lead, (d + 31) // 32, bits), dtype=np.uint64)
    for j in range(d):
        w, k = divmod(j, 32)
        for p in range(bits):
            words[..., w, p] |= ((idx[..., j] >> p) & 1).astype(np.uint64) << np.uint64(k)
    return words.astype(np.uint32)


def unpack_key_codes(words, d):
    words = np.asarray(words, dtype=np.uint32).astype(np.int64)
    *lead, nw, bits = words.shape
    idx = np.zeros((*lead, d), dtype=np.int64)
    for j in range(d):
        w, k = divmod(j, 32)
        for p in range(bits):
            idx[..., j] |= ((words[..., w, p] >> k) & 1) << p
    return idx


def pack_signs(signs):
    """signs [..., m] -> words [..., ceil(m/32)]; padding rows' bits are 0."""
    signs = np.asarray(signs, dtype=bool)
    *lead, m = signs.shape
    words = np.zeros((*lead, (m + 31) // 32), dtype=np.uint64)
    for i in range(m):
        w, k = divmod(i, 32)
        words[..., w] |= signs[..., i].astype(np.uint64) << np.uint64(k)
    return words.astype(np.uint32)


def unpack_signs(words, m):
    words = np.asarray(words, dtype=np.uint32).astype(np.int64)
    *lead, nw = words.shape
    out = np.zeros((*lead, m), dtype=bool)
    for i in range(m):
        w, k = divmod(i, 32)
        out[..., i] = ((words[..., w] >> k) & 1) == 1
    return out


def pack_value_codes(idx, bits):
    """idx: [S, T, d] -> words [S, ceil(T/32), d, bits] (token-order fields)."""
    idx = np.asarray(idx, dtype=np.int64)
    S, T, d = idx.shape
    nb = (T + 31) // 32
    padded = np.zeros((S, nb * 32, d), dtype=np.int64)
    padded[:, :T] = idx
    blocks = padded.reshape(S, nb, 32, d)            # [S, block, k, j]
    words = np.zeros((S, nb, d, bits), dtype=np.uint64)
    for k in range(32):
        for p in range(bits):
            pos = bits * k + p                       # bit position in the record
            w, sh = divmod(pos, 32)
            words[:, :, :, w] |= ((blocks[:, :, k, :] >> p) & 1).astype(np.uint64) << np.uint64(sh)
    return words.astype(np.uint32)


def unpack_value_codes(words, T):
    words = np.asarray(words, dtype=np.uint32).astype(np.int64)
    S, nb, d, bits = words.shape
    blocks = np.zeros((S, nb, 32, d), dtype=np.int64)
    for k in range(32):
        for p in range(bits):
            w, sh = divmod(bits * k + p, 32)
            blocks[:, :, k, :] |= ((words[:, :, :, w] >> sh) & 1) << p
    return blocks.reshape(S, nb * 32, d)[:, :T]


def round_norms(x, dtype):
    """Round fp64 norms to the storage type ('f32' or 'f16', nearest even).

    Returns the stored array (numpy float32 / float16)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    raise ValueError(dtype)


# ------------------------------------------------ split (fractional) widths
# A fractional width gives the leading coordinates one bit more than the
# rest (codebook.split_codebook).  The records keep the layouts above, with
# each 32-coordinate word (keys) or each coordinate (values) taking its own
# number of planes / bits, concatenated in coordinate order:
#   keys    record[..., sum(word_bits)]: word w's word_bits[w] planes,
#           word after word (bit k of plane p of word w = bit p of
#           idx[32 w + k]);
#   values  record[S, block, sum(coord_bits)]: coordinate j's coord_bits[j]
#           words at offset sum(coord_bits[:j]), its 32 tokens' fields in
#           token order as in pack_value_codes.
# With equal widths these are exactly the uniform layouts.

def pack_key_codes_split(idx, word_bits):
    idx = np.asarray(idx, dtype=np.int64)
    *lead, d = idx.shape
    if d != 32 * len(word_bits):
        raise ValueError("one width per 32-coordinate word")
    out = np.zeros((*lead, int(np.sum(word_bits))), dtype=np.uint64)
    o = 0
    for w, nb in enumerate(word_bits):
        for p in range(nb):
            for k in range(32):
                out[..., o] |= ((idx[..., 32 * w + k] >> p) & 1).astype(np.uint64) << np.uint64(k)
            o += 1
    return out.astype(np.uint32)


def unpack_key_codes_split(words, d, word_bits):
    words = np.asarray(words, dtype=np.uint32).astype(np.int64)
    *lead, nwords = words.shape
    if nwords != int(np.sum(word_bits)) or d != 32 * len(word_bits):
        raise ValueError("record size does not match the widths")
    idx = np.zeros((*lead, d), dtype=np.int64)
    o = 0
    for w, nb in enumerate(word_bits):
        for p in range(nb):
            for k in range(32):
                idx[..., 32 * w + k] |= ((words[..., o] >> k) & 1) << p
            o += 1
    return idx


def pack_value_codes_split(idx, coord_bits):
    """idx [S, T, d] -> records [S, ceil(T/32), sum(coord_bits)]."""
    idx = np.asarray(idx, dtype=np.int64)
    S, T, d = idx.shape
    nb = (T + 31) // 32
    padded = np.zeros((S, nb * 32, d), dtype=np.int64)
    padded[:, :T] = idx
    blocks = padded.reshape(S, nb, 32, d)
    out = np.zeros((S, nb, int(np.sum(coord_bits))), dtype=np.uint64)
    o = 0
    for j in range(d):
        b = int(coord_bits[j])
        for k in range(32):
            for p in range(b):
                w, sh = divmod(b * k + p, 32)
                out[:, :, o + w] |= ((blocks[:, :, k, j] >> p) & 1).astype(np.uint64) << np.uint64(sh)
        o += b
    return out.astype(np.uint32)


def unpack_value_codes_split(words, T, coord_bits):
    words = np.asarray(words, dtype=np.uint32).astype(np.int64)
    S, nb, nwords = words.shape
    d = len(coord_bits)
    if nwords != int(np.sum(coord_bits)):
        raise ValueError("record size does not match the widths")
    blocks = np.zeros((S, nb, 32, d), dtype=np.int64)
    o = 0
    for j in range(d):
        b = int(coord_bits[j])
        for k in range(32):
            for p in range(b):
                w, sh = divmod(b * k + p, 32)
                blocks[:, :, k, j] |= ((words[:, :, o + w] >> sh) & 1) << p
        o += b
    return blocks.reshape(S, nb * 32, d)[:, :T]
