"""The packed byte layout of the quantized weights, written twice: bit by bit and vectorised.

Test infrastructure only (see the package docstring for who may import it).

The FP6-LLM news page (m.zhengruan.com), section "重新设计内核方案", says that 6-bit
weights fit a memory system built on 32/64-bit accesses badly, and that they are
therefore re-packed before inference into aligned blocks, in the order in which the
kernel consumes them. It gives no concrete layout. The layout used here is:

* Rows are stored one after another (output row n first). Row n holds K codes, cut
  into units of 32 consecutive K (unit u covers k = 32u .. 32u+31). Units follow one
  another with no padding, so a row is exactly K*bits/8 bytes and the whole array is
  exactly N*K*bits/8 bytes.
* Inside a unit, for code j (k = 32u + j):
    - W8 (32 bytes): byte j holds q_j + 128 (offset binary; q in -127..127).
    - W4 (16 bytes): four little-endian 32-bit words. Word d holds codes 8d .. 8d+7.
      Code 8d+2t sits in nibble t and code 8d+2t+1 in nibble t+4 (t = 0..3), nibble p
      being bits 4p .. 4p+3 of the word.
    - W6 (24 bytes): one 192-bit little-endian number; code j sits in bits 6j .. 6j+5.
      These 24 bytes are not stored in one piece (see below).
    - FP4 (16 bytes): one 128-bit little-endian number; code j sits in bits 4j .. 4j+3,
      so byte p holds code 2p in its low nibble and code 2p+1 in its high nibble (the
      order in which gfx950's packed FP4 convert takes a byte).
    - FP5 (20 bytes): one 160-bit little-endian number. Bits 0..127 hold the low four
      bits of every code (e1 e0 m1 m0), placed as the W4 codes are: word d holds codes
      8d .. 8d+7, code 8d+2t in nibble t and code 8d+2t+1 in nibble t+4. Bits 128..159
      hold the signs: the sign of code 2p in bit 128+p and of code 2p+1 in bit 144+p
      (p = 0..15), so that one shift puts the signs of a pair at bits 15 and 31.
    - W3 (12 bytes): three little-endian 32-bit words. Codes 2p and 2p+1 form pair p
      (p = 0..15); the even code sits in the low 16 bits of a word and the odd code in the
      high 16 bits at the same offset, so that one mask takes both. Pairs 0..14: pair p sits
      in word p // 5 at offset o = (0, 3, 6, 10, 13)[p % 5], code 2p in bits o .. o+2 and
      code 2p+1 in bits 16+o .. 18+o. Pair 15 fills the two bits left in each word: bit b of
      code 30 in bit 9 of word b and bit b of code 31 in bit 25 of word b (b = 0, 1, 2).
    - W6 split 2+4 ("P24", 24 bytes; the same e3m2 codes as W6, the two-plus-four split of
      the FP6-LLM news page): bytes 0..15 hold the low four bits of every code, placed as
      the W4 codes; bytes 16..19 a little-endian word holding bit 4 of code 2p in bit p and
      bit 4 of code 2p+1 in bit 16+p (p = 0..15); bytes 20..23 the same for bit 5, the sign.
    - F16 (64 bytes, the unquantized baseline): bytes 2j, 2j+1 hold the fp16 bits of
      weight j, little-endian.
    - BF16 (64 bytes, the unquantized baseline for bfloat16 activations): the same with
      bfloat16 bits.
* W6, P24 and FP5 only, split by planes: the units of a row are taken 64 at a time ("chunks";
  the last chunk of a row may hold fewer, Uc units). In a chunk, bytes 0..15 of its units
  come first, unit after unit (16*Uc bytes), then bytes 16.. of its units (8*Uc bytes for
  W6 and P24, 4*Uc for FP5). A chunk with one unit is therefore stored exactly as that unit. (A
  device lane reads one unit, so each of the two loads of a wave reads one contiguous block.)
* Metadata stays in logical order: W8/W6/P24/FP4/FP5 scales [N]; W4 and W3 scales and zeros
  [N][K/32], row-major (group g of row n covers the same 32 K as unit g).

Codes given to and returned by these functions are the logical codes: int8 q for W8,
0..15 for W4 and FP4, 0..63 for W6 and P24, 0..31 for FP5, 0..7 for W3, uint16 fp16 bits
for F16, uint16 bfloat16 bits for BF16.
"""

import numpy as np

FMT_F16 = 0
FMT_W8 = 1
FMT_W4G32 = 2
FMT_W6E3M2 = 3
FMT_W4E2M1 = 4
FMT_BF16 = 5
FMT_W5E2M2 = 6
FMT_W3G32 = 7
FMT_W6E3M2_P24 = 8

_BITS = {FMT_F16: 16, FMT_W8: 8, FMT_W4G32: 4, FMT_W6E3M2: 6, FMT_W4E2M1: 4, FMT_BF16: 16, FMT_W5E2M2: 5,
         FMT_W3G32: 3, FMT_W6E3M2_P24: 6}
UNIT = 32
CHUNK = 64          # units per W6 / P24 / FP5 plane chunk
_PLANED = (FMT_W6E3M2, FMT_W5E2M2, FMT_W6E3M2_P24)
_GROUPED = (FMT_W4G32, FMT_W3G32)   # a scale and a zero point per group of 32 K
_W3_OFFSETS = (0, 3, 6, 10, 13)     # W3: bit offset of pair p (p < 15) inside word p // 5


def _bits(fmt):
    if fmt not in _BITS:
        raise ValueError("unknown format %r" % fmt)
    return _BITS[fmt]


def unit_bytes(fmt):
    return UNIT * _bits(fmt) // 8


def packed_bytes(fmt, n, k):
    return n * k * _bits(fmt) // 8


def scales_count(fmt, n, k):
    """Number of fp16 scales."""
    _bits(fmt)
    if fmt in (FMT_F16, FMT_BF16):
        return 0
    return n * (k // 32) if fmt in _GROUPED else n


def zeros_count(fmt, n, k):
    """Number of fp16 zero points."""
    _bits(fmt)
    return n * (k // 32) if fmt in _GROUPED else 0


def code_fields(fmt, j):
    """[(first bit, width, shift)] of code j inside its unit, counting bits little-endian from the
    unit's first byte: bits shift .. shift+width-1 of the code's stored value go to bits
    first .. first+width-1 (one field for every format but FP5 and P24, whose high bits sit
    apart, and the last pair of W3, whose bits are spread over the three words)."""
    if fmt == FMT_W5E2M2:
        nib_first, _ = code_field(FMT_W4G32, j)
        p, odd = divmod(j, 2)
        return [(nib_first, 4, 0), (128 + 16 * odd + p, 1, 4)]
    if fmt == FMT_W6E3M2_P24:
        nib_first, _ = code_field(FMT_W4G32, j)
        p, odd = divmod(j, 2)
        return [(nib_first, 4, 0), (128 + 16 * odd + p, 1, 4), (160 + 16 * odd + p, 1, 5)]
    if fmt == FMT_W3G32:
        p, odd = divmod(j, 2)
        if p < 15:
            word, f = divmod(p, 5)
            return [(32 * word + 16 * odd + _W3_OFFSETS[f], 3, 0)]
        return [(32 * b + 16 * odd + 9, 1, b) for b in range(3)]
    first, width = code_field(fmt, j)
    return [(first, width, 0)]


def code_field(fmt, j):
    """(first bit, width) of code j inside its unit, for the formats stored as one field per code."""
    if fmt == FMT_W8:
        return 8 * j, 8
    if fmt == FMT_W4G32:
        d, i = divmod(j, 8)
        t, odd = divmod(i, 2)
        nibble = t + 4 * odd
        return 32 * d + 4 * nibble, 4
    if fmt == FMT_W6E3M2:
        return 6 * j, 6
    if fmt == FMT_W4E2M1:
        return 4 * j, 4
    if fmt in (FMT_F16, FMT_BF16):
        return 16 * j, 16
    raise ValueError("unknown format %r" % fmt)


def _stored(fmt, code):
    """The unsigned field value stored for one logical code."""
    code = int(code)
    if fmt == FMT_W8:
        if not -127 <= code <= 127:
            raise ValueError("int8 code out of range")
        return code + 128
    limit = {FMT_W4G32: 16, FMT_W6E3M2: 64, FMT_W4E2M1: 16, FMT_W5E2M2: 32, FMT_F16: 65536, FMT_BF16: 65536,
             FMT_W3G32: 8, FMT_W6E3M2_P24: 64}[fmt]
    if not 0 <= code < limit:
        raise ValueError("code out of range")
    return code


def _logical(fmt, field):
    return field - 128 if fmt == FMT_W8 else field


def _check_shape(codes, k):
    if k % UNIT:
        raise ValueError("K must be a multiple of 32")
    return codes


def pack_scalar(fmt, codes):
    """Bit-writer: pack logical codes [N,K] one code at a time. Slow; for small arrays."""
    codes = np.asarray(codes)
    n, k = codes.shape
    _check_shape(codes, k)
    ub = unit_bytes(fmt)
    out = bytearray(packed_bytes(fmt, n, k))
    for r in range(n):
        for u in range(k // UNIT):
            acc = 0
            for j in range(UNIT):
                v = _stored(fmt, codes[r, UNIT * u + j])
                for first, width, shift in code_fields(fmt, j):
                    for b in range(width):
                        if (v >> (shift + b)) & 1:
                            acc |= 1 << (first + b)
            unit = acc.to_bytes(ub, "little")
            for i in range(ub):
                out[_byte_home(fmt, r, u, i, k)] = unit[i]
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def _byte_home(fmt, r, u, i, k):
    """Offset in the packed array of byte i of unit u of row r."""
    ub = unit_bytes(fmt)
    units = k // UNIT
    if fmt not in _PLANED:
        return (r * units + u) * ub + i
    c, j = divmod(u, CHUNK)
    uc = min(CHUNK, units - c * CHUNK)
    base = (r * units + c * CHUNK) * ub
    return base + 16 * j + i if i < 16 else base + 16 * uc + (ub - 16) * j + (i - 16)


def unpack_scalar(fmt, packed, n, k):
    """Bit-reader: the inverse of pack_scalar."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    if packed.size != packed_bytes(fmt, n, k):
        raise ValueError("packed size mismatch")
    ub = unit_bytes(fmt)
    dtype = {FMT_W8: np.int8, FMT_F16: np.uint16, FMT_BF16: np.uint16}.get(fmt, np.uint8)
    codes = np.zeros((n, k), dtype=dtype)
    for r in range(n):
        for u in range(k // UNIT):
            unit = bytes(int(packed[_byte_home(fmt, r, u, i, k)]) for i in range(ub))
            acc = int.from_bytes(unit, "little")
            for j in range(UNIT):
                v = 0
                for first, width, shift in code_fields(fmt, j):
                    v |= ((acc >> first) & ((1 << width) - 1)) << shift
                codes[r, UNIT * u + j] = _logical(fmt, v)
    return codes


# ---- vectorised packer / unpacker: the same layout, computed with whole-array ops ----
# W4: slot p of a 32-bit word holds code order[p]; W6: every 4 codes fill 3 whole bytes.
_W4_ORDER = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def pack_vectorized(fmt, codes):
    codes = np.asarray(codes)
    n, k = codes.shape
    _check_shape(codes, k)
    if fmt == FMT_W8:
        c = codes.astype(np.int16)
        if c.min(initial=0) < -127 or c.max(initial=0) > 127:
            raise ValueError("int8 code out of range")
        return (c + 128).astype(np.uint8).reshape(-1)
    if fmt == FMT_W4G32:
        c = codes.astype(np.uint32)
        if c.max(initial=0) > 15:
            raise ValueError("int4 code out of range")
        c = c.reshape(n, k // 8, 8)[:, :, _W4_ORDER]          # slot p <- code order[p]
        words = np.zeros((n, k // 8), dtype=np.uint32)
        for p in range(8):
            words |= c[:, :, p] << np.uint32(4 * p)
        return words.astype("<u4").view(np.uint8).reshape(-1)
    if fmt == FMT_W6E3M2:
        c = codes.astype(np.uint32)
        if c.max(initial=0) > 63:
            raise ValueError("fp6 code out of range")
        c = c.reshape(n, k // 4, 4)
        v = c[:, :, 0] | (c[:, :, 1] << 6) | (c[:, :, 2] << 12) | (c[:, :, 3] << 18)
        b = np.stack([v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF], axis=-1).astype(np.uint8)
        return _to_planes(b.reshape(n, k // UNIT, 24)).reshape(-1)
    if fmt == FMT_W4E2M1:
        c = codes.astype(np.uint8)
        if c.max(initial=0) > 15:
            raise ValueError("fp4 code out of range")
        c = c.reshape(n, k // 2, 2)
        return (c[:, :, 0] | (c[:, :, 1] << 4)).astype(np.uint8).reshape(-1)
    if fmt == FMT_W5E2M2:
        c = codes.astype(np.uint32)
        if c.max(initial=0) > 31:
            raise ValueError("fp5 code out of range")
        mag = (c & 0xF).reshape(n, k // 8, 8)[:, :, _W4_ORDER]
        words = np.zeros((n, k // 8), dtype=np.uint32)
        for p in range(8):
            words |= mag[:, :, p] << np.uint32(4 * p)
        sgn = (c >> 4).reshape(n, k // UNIT, 16, 2)            # [.., p, odd]
        sw = np.zeros((n, k // UNIT), dtype=np.uint32)
        for p in range(16):
            sw |= (sgn[:, :, p, 0] << np.uint32(p)) | (sgn[:, :, p, 1] << np.uint32(16 + p))
        units = np.concatenate([words.reshape(n, k // UNIT, 4), sw.reshape(n, k // UNIT, 1)], axis=2)
        return _to_planes(units.astype("<u4").view(np.uint8).reshape(n, k // UNIT, 20)).reshape(-1)
    if fmt == FMT_W6E3M2_P24:
        c = codes.astype(np.uint32)
        if c.max(initial=0) > 63:
            raise ValueError("fp6 code out of range")
        mag = (c & 0xF).reshape(n, k // 8, 8)[:, :, _W4_ORDER]
        words = np.zeros((n, k // 8), dtype=np.uint32)
        for p in range(8):
            words |= mag[:, :, p] << np.uint32(4 * p)
        planes = []
        for bit in (4, 5):                                     # bit 4 (e2), then bit 5 (sign)
            b = ((c >> np.uint32(bit)) & 1).reshape(n, k // UNIT, 16, 2)   # [.., p, odd]
            pw = np.zeros((n, k // UNIT), dtype=np.uint32)
            for p in range(16):
                pw |= (b[:, :, p, 0] << np.uint32(p)) | (b[:, :, p, 1] << np.uint32(16 + p))
            planes.append(pw.reshape(n, k // UNIT, 1))
        units = np.concatenate([words.reshape(n, k // UNIT, 4)] + planes, axis=2)
        return _to_planes(units.astype("<u4").view(np.uint8).reshape(n, k // UNIT, 24)).reshape(-1)
    if fmt == FMT_W3G32:
        c = codes.astype(np.uint32)
        if c.max(initial=0) > 7:
            raise ValueError("int3 code out of range")
        c = c.reshape(n, k // UNIT, 16, 2)                    # [.., pair, odd]
        words = np.zeros((n, k // UNIT, 3), dtype=np.uint32)
        for p in range(15):
            word, f = divmod(p, 5)
            o = _W3_OFFSETS[f]
            words[:, :, word] |= (c[:, :, p, 0] << np.uint32(o)) | (c[:, :, p, 1] << np.uint32(16 + o))
        for b in range(3):
            words[:, :, b] |= (((c[:, :, 15, 0] >> np.uint32(b)) & 1) << np.uint32(9)) | \
                              (((c[:, :, 15, 1] >> np.uint32(b)) & 1) << np.uint32(25))
        return words.astype("<u4").view(np.uint8).reshape(-1)
    if fmt in (FMT_F16, FMT_BF16):
        return codes.astype(np.uint16).astype("<u2").view(np.uint8).reshape(-1)
    raise ValueError("unknown format %r" % fmt)


def unpack_vectorized(fmt, packed, n, k):
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    if packed.size != packed_bytes(fmt, n, k):
        raise ValueError("packed size mismatch")
    if fmt == FMT_W8:
        return (packed.astype(np.int16) - 128).astype(np.int8).reshape(n, k)
    if fmt == FMT_W4G32:
        words = packed.view("<u4").reshape(n, k // 8)
        out = np.zeros((n, k // 8, 8), dtype=np.uint8)
        for p in range(8):
            out[:, :, _W4_ORDER[p]] = (words >> np.uint32(4 * p)) & 0xF
        return out.reshape(n, k)
    if fmt == FMT_W6E3M2:
        b = _from_planes(packed.reshape(n, -1), k // UNIT, 24).reshape(n, k // 4, 3).astype(np.uint32)
        v = b[:, :, 0] | (b[:, :, 1] << 8) | (b[:, :, 2] << 16)
        out = np.stack([(v >> s) & 0x3F for s in (0, 6, 12, 18)], axis=-1).astype(np.uint8)
        return out.reshape(n, k)
    if fmt == FMT_W4E2M1:
        b = packed.reshape(n, k // 2)
        return np.stack([b & 0xF, b >> 4], axis=-1).astype(np.uint8).reshape(n, k)
    if fmt == FMT_W5E2M2:
        units = _from_planes(packed.reshape(n, -1), k // UNIT, 20).copy().view("<u4").reshape(n, k // UNIT, 5)
        words = units[:, :, :4].reshape(n, k // 8)
        mag = np.zeros((n, k // 8, 8), dtype=np.uint8)
        for p in range(8):
            mag[:, :, _W4_ORDER[p]] = (words >> np.uint32(4 * p)) & 0xF
        sw = units[:, :, 4]
        sgn = np.zeros((n, k // UNIT, 16, 2), dtype=np.uint8)
        for p in range(16):
            sgn[:, :, p, 0] = (sw >> np.uint32(p)) & 1
            sgn[:, :, p, 1] = (sw >> np.uint32(16 + p)) & 1
        return (mag.reshape(n, k) | (sgn.reshape(n, k) << 4)).astype(np.uint8)
    if fmt == FMT_W6E3M2_P24:
        units = _from_planes(packed.reshape(n, -1), k // UNIT, 24).copy().view("<u4").reshape(n, k // UNIT, 6)
        words = units[:, :, :4].reshape(n, k // 8)
        out = np.zeros((n, k // 8, 8), dtype=np.uint8)
        for p in range(8):
            out[:, :, _W4_ORDER[p]] = (words >> np.uint32(4 * p)) & 0xF
        out = out.reshape(n, k // UNIT, 16, 2)
        for bit, plane in ((4, 4), (5, 5)):
            pw = units[:, :, plane]
            for p in range(16):
                out[:, :, p, 0] |= (((pw >> np.uint32(p)) & 1) << bit).astype(np.uint8)
                out[:, :, p, 1] |= (((pw >> np.uint32(16 + p)) & 1) << bit).astype(np.uint8)
        return out.reshape(n, k)
    if fmt == FMT_W3G32:
        words = packed.view("<u4").reshape(n, k // UNIT, 3)
        out = np.zeros((n, k // UNIT, 16, 2), dtype=np.uint8)
        for p in range(15):
            word, f = divmod(p, 5)
            o = _W3_OFFSETS[f]
            out[:, :, p, 0] = (words[:, :, word] >> np.uint32(o)) & 7
            out[:, :, p, 1] = (words[:, :, word] >> np.uint32(16 + o)) & 7
        for b in range(3):
            out[:, :, 15, 0] |= (((words[:, :, b] >> np.uint32(9)) & 1) << b).astype(np.uint8)
            out[:, :, 15, 1] |= (((words[:, :, b] >> np.uint32(25)) & 1) << b).astype(np.uint8)
        return out.reshape(n, k)
    if fmt in (FMT_F16, FMT_BF16):
        return packed.view("<u2").reshape(n, k).astype(np.uint16)
    raise ValueError("unknown format %r" % fmt)


def _to_planes(units):
    """[N, U, B] unit-contiguous bytes -> [N, U*B] with every chunk of 64 units split into planes
    (bytes 0..15 of its units, then bytes 16..B-1)."""
    n, u, _ = units.shape
    parts = []
    for c0 in range(0, u, CHUNK):
        blk = units[:, c0:c0 + CHUNK, :]
        parts.append(blk[:, :, :16].reshape(n, -1))
        parts.append(blk[:, :, 16:].reshape(n, -1))
    return np.concatenate(parts, axis=1)


def _from_planes(rows, u, ub):
    """Inverse of _to_planes: [N, U*ub] -> [N, U, ub]."""
    n = rows.shape[0]
    out = np.empty((n, u, ub), dtype=np.uint8)
    pos = 0
    for c0 in range(0, u, CHUNK):
        uc = min(CHUNK, u - c0)
        out[:, c0:c0 + uc, :16] = rows[:, pos:pos + 16 * uc].reshape(n, uc, 16)
        pos += 16 * uc
        out[:, c0:c0 + uc, 16:] = rows[:, pos:pos + (ub - 16) * uc].reshape(n, uc, ub - 16)
        pos += (ub - 16) * uc
    return out
