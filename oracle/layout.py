"""Byte layout of the packed cache (test infrastructure only).

The pages fix what a code *is* but store it in formats made for other
hardware (TurboQuant spec page, "Step 3: Packing": 4 two-bit values per byte,
2 four-bit values per byte).  This package follows the storage format the HIP
library documents in ``include/kvq.h``; it is written here from that text, not
from the library.  The format keeps the pages' bits-per-value and packing
density and changes only which bit a code lands in:

* **Word-interleaved packing.**  A little-endian 32-bit word holds n = 32/b
  codes of b bits.  Code k of the word sits at bit 16*(k%2) + b*(k//2): even
  codes fill the low 16 bits, odd codes the high 16 bits, each half from the
  least significant bit up.

* **K codes: token rows.**  Inside a 32-token block record, row t (token
  base+t) occupies bytes [t*D*b/8, (t+1)*D*b/8) and holds its D channel codes
  in channel order, word-interleaved.

* **V codes: channel tiles.**  The V codes of a 32-token block are 64 chunks
  of D*b/16 bytes.  Chunk q = 16*kg + i (kg in 0..3, i in 0..15) holds, in
  order k = 8*mu + e (mu in 0..D/16-1, e in 0..7), the code of channel
  16*mu + i of token T(kg, e) = 16*(e//4) + 4*kg + e%4, word-interleaved.

* **Block record** = [K codes | V codes | K meta | V meta] with

  ====== ======================================= ===================================
  format K meta                                  V meta
  ====== ======================================= ===================================
  KIVI   scale fp16 [D], then zero fp16 [D]      scale fp16 [16][D/32][2], then zero
  q2k    rms fp16 [D]                            scale fp16 [16][D/32][2]
  TQ     K norm fp32 [32] (per token)            V norm fp32 [32] (per token)
  ====== ======================================= ===================================

  The V scale (and zero) of token t and 32-channel group g sits at index
  [t // 2][g][t % 2]: the two tokens of a pair are adjacent for every group.

* **3-bit TurboQuant codes** use the page's per-byte packing, two codes per
  byte with two bits unused ("Step 3: Packing"): they are stored in 4-bit
  slots, b = 4 above.  With the dense option (the page's "8 values into 3
  bytes") they are a plain little-endian bit stream instead: code i of a
  section's sequence (K: row-major token rows; V: the 64 chunks above, one
  after another) occupies bits [3i, 3i + 3), least significant bit first.
"""

import numpy as np

G = 32  # token-block length and V channel-group length


def t_of(kg, e):
    """Token (0..31) of element e of token group kg in the V tile order."""
    return 16 * (e // 4) + 4 * kg + (e % 4)


def pack_words(codes, bits):
    """Pack codes (last axis, length a multiple of 32/bits) word-interleaved; returns uint8 [..., n*bits/8]."""
    per = 32 // bits
    c = np.asarray(codes, dtype=np.uint32)
    lead = c.shape[:-1]
    c = c.reshape(lead + (-1, per))
    assert np.all(c < (1 << bits)), "code out of range"
    k = np.arange(per, dtype=np.uint32)
    shift = 16 * (k % 2) + bits * (k // 2)
    words = np.ascontiguousarray(np.bitwise_or.reduce(c << shift, axis=-1).astype("<u4"))
    return words.view(np.uint8).reshape(lead + (-1,))


def unpack_words(data, bits):
    """Inverse of pack_words: uint8 [..., nbytes] -> codes uint8 [..., nbytes*8/bits]."""
    per = 32 // bits
    d = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    lead = d.shape[:-1]
    words = d.reshape(lead + (-1, 4)).view("<u4")[..., 0].astype(np.uint32)
    k = np.arange(per, dtype=np.uint32)
    shift = 16 * (k % 2) + bits * (k // 2)
    codes = (words[..., None] >> shift) & np.uint32((1 << bits) - 1)
    return codes.reshape(lead + (-1,)).astype(np.uint8)


def pack_k_rows(codes, bits):
    """K codes [..., 32, D] -> bytes [..., 32*D*bits/8] (token rows; bits = 3: the dense stream)."""
    c = np.asarray(codes)
    if bits == 3:
        return pack_bits3(c.reshape(c.shape[:-2] + (-1,)))
    packed = pack_words(c, bits)  # [..., 32, D*bits/8]
    return packed.reshape(c.shape[:-2] + (-1,))


def unpack_k_rows(data, D, bits):
    d = np.asarray(data)
    if bits == 3:
        return unpack_bits3(d, G * D).reshape(d.shape[:-1] + (G, D))
    rows = d.reshape(d.shape[:-1] + (G, D * bits // 8))
    return unpack_words(rows, bits)


def _v_tile_order(D):
    """(token, channel) index arrays of the V tile sequence, shape [64, D/2] each."""
    nmu = D // 16
    q = np.arange(64)
    kg, i = q // 16, q % 16
    k = np.arange(8 * nmu)
    mu, e = k // 8, k % 8
    tok = t_of(kg[:, None], e[None, :])
    ch = 16 * mu[None, :] + i[:, None]
    return tok, ch


def pack_v_tiles(codes, bits):
    """V codes [..., 32, D] -> bytes [..., 32*D*bits/8] (channel tiles)."""
    c = np.asarray(codes)
    D = c.shape[-1]
    tok, ch = _v_tile_order(D)
    seq = c[..., tok, ch]  # [..., 64, D/2]
    if bits == 3:
        return pack_bits3(seq.reshape(seq.shape[:-2] + (-1,)))
    packed = pack_words(seq, bits)  # [..., 64, D*bits/16]
    return packed.reshape(c.shape[:-2] + (-1,))


def unpack_v_tiles(data, D, bits):
    d = np.asarray(data)
    if bits == 3:
        seq = unpack_bits3(d, 64 * D // 2).reshape(d.shape[:-1] + (64, D // 2))
    else:
        chunks = d.reshape(d.shape[:-1] + (64, D * bits // 16))
        seq = unpack_words(chunks, bits)  # [..., 64, D/2]
    tok, ch = _v_tile_order(D)
    out = np.zeros(d.shape[:-1] + (G, D), dtype=np.uint8)
    out[..., tok, ch] = seq
    return out


def pack_v_meta(meta):
    """V metadata [..., 32, D/32] (token, group) -> [..., 32*D/32] in [t // 2][g][t % 2] order."""
    m = np.asarray(meta)
    ng = m.shape[-1]
    pairs = m.reshape(m.shape[:-2] + (G // 2, 2, ng))
    return np.swapaxes(pairs, -1, -2).reshape(m.shape[:-2] + (G * ng,))


def unpack_v_meta(flat, ng):
    """Inverse of pack_v_meta."""
    f = np.asarray(flat)
    pairs = f.reshape(f.shape[:-1] + (G // 2, ng, 2))
    return np.swapaxes(pairs, -1, -2).reshape(f.shape[:-1] + (G, ng))


def slot_bits(bits, dense3=False):
    """Bits a code occupies in storage (3-bit codes: two per byte with two bits unused, or 3 when dense)."""
    if bits == 3:
        return 3 if dense3 else 4
    return bits


def pack_bits3(codes):
    """Dense 3-bit stream of codes [..., n] (3n a multiple of 8): code i at bits [3i, 3i+3), LSB first."""
    c = np.asarray(codes, dtype=np.uint8)
    assert np.all(c < 8), "code out of range"
    bits = ((c[..., :, None] >> np.arange(3, dtype=np.uint8)) & 1).reshape(c.shape[:-1] + (-1,))
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_bits3(data, n):
    """Inverse of pack_bits3: the first n codes of a dense 3-bit stream."""
    bits = np.unpackbits(np.asarray(data, dtype=np.uint8), axis=-1, bitorder="little")
    b = bits[..., : 3 * n].reshape(bits.shape[:-1] + (n, 3)).astype(np.uint8)
    return b[..., 0] | (b[..., 1] << 1) | (b[..., 2] << 2)


def record_sections(fmt, D, k_bits, v_bits, dense3=False):
    """Byte sizes of the four sections of one block record, and their offsets."""
    kc = G * D * slot_bits(k_bits, dense3) // 8
    vc = G * D * slot_bits(v_bits, dense3) // 8
    if fmt == "kivi":
        km, vm = 2 * 2 * D, 2 * 2 * G * (D // 32)
    elif fmt == "q2k":
        km, vm = 2 * D, 2 * G * (D // 32)
    elif fmt == "tq":
        km, vm = 4 * G, 4 * G
    else:
        raise ValueError(fmt)
    off = {"k_codes": 0, "v_codes": kc, "k_meta": kc + vc, "v_meta": kc + vc + km}
    size = {"k_codes": kc, "v_codes": vc, "k_meta": km, "v_meta": vm}
    return off, size, kc + vc + km + vm
