"""Every address of the plain-load paths stays inside its tile or buffer.

Buffer-resource loads are bounds-checked by the hardware (a lane past the
resource reads zero).  Two paths use plain addresses and must stay in bounds
on their own:

* the prefill ring (pa_prefill.hip): each step's K and V are copied from the
  pool into an LDS stage by global-to-LDS loads, one 16-byte piece per lane
  at a per-lane offset inside one block's tile of the KV head, and read back
  by fragment loads at fixed LDS offsets (FP8 pools: raw codes, widened to
  bf16 fragments by the lanes that loaded them);
* the paired 8-token decode tiles (pa_decode.hip, load_pair8);
* the 16-row decode tiles of 16-bit pools with 16- and 32-token blocks
  (pa_decode.hip, load_tile16), whose out-of-pool and past-the-end tiles
  address block 0 of the pool.

This test re-derives those lane offsets, written as in the kernels, for every
supported block size and head dim, and checks them against the tile sizes of
the pool layout in include/pa.h (a 16-bit tile of b tokens holds b * head_dim
* 2 bytes of K and the same of V) and against the LDS ring.  It also checks
that a step's loads copy every byte of its 32 keys exactly once and that the
LDS fragment reads see each key's data where the matrix-core layout expects
it.  Runs on the CPU.
"""
import pytest

WAVES = 4


def ring_dma(b, D):
    """Per (wave, lane, instruction): (quarter qi, byte offset in the block's
    tile, LDS byte offset in the stage) of the 16-byte piece it loads."""
    R = min(b, 16)
    r_shift = 3 if R == 8 else 4
    sub_bytes = R * D * 2
    chunks = D // 32
    kbytes = 2 * chunks * 1024
    out = []
    for wave in range(WAVES):
        for lane in range(64):
            qi = 2 * wave + ((lane >> 3) & 1) if wave < 2 else (lane >> 4) & 3
            in_blk = (8 * qi) & (b - 1)
            row_q = in_blk & (R - 1)
            if wave < 2:
                off = (in_blk >> r_shift) * sub_bytes + (row_q + (lane & 7)) * 64 + (lane >> 4) * 16
                for m in range(chunks):
                    out.append((wave, lane, qi, off + m * R * 64, (wave * chunks + m) * 1024 + lane * 16))
            else:
                off = ((in_blk >> r_shift) * sub_bytes
                       + ((row_q >> 2) + ((lane >> 3) & 1)) * D * 8 + (lane & 7) * 16)
                n0 = (wave - 2) * chunks
                for i in range(chunks):
                    out.append((wave, lane, qi, off + (n0 + i) * 128, kbytes + (n0 + i) * 1024 + lane * 16))
    return out


def k_elem(b, D, t, d):
    """Byte offset of K element (token t of the block, dim d) in a 16-bit tile."""
    R = min(b, 16)
    s, tl = divmod(t, R)
    return (s * R * D + (d >> 5) * (R * 32) + tl * 32 + (d & 31)) * 2


def v_elem(b, D, t, d):
    R = min(b, 16)
    s, tl = divmod(t, R)
    return (s * R * D + (tl >> 2) * D * 4 + d * 4 + (tl & 3)) * 2


@pytest.mark.parametrize("b", [8, 16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_ring_loads_in_bounds(b, D):
    tile = b * D * 2
    step = 2 * (D // 32) * 1024 + (D // 16) * 1024
    for wave, lane, qi, off, lds in ring_dma(b, D):
        assert 0 <= off and off + 16 <= tile, (wave, lane, off)
        assert 0 <= lds and lds + 16 <= step
    # the instructions per wavefront are what the kernel's wait counts assume
    per_wave = {}
    for wave, lane, *_ in ring_dma(b, D):
        per_wave[wave] = per_wave.get(wave, 0) + 1
    assert all(n == 64 * (D // 32) for n in per_wave.values())


@pytest.mark.parametrize("b", [8, 16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_ring_copies_each_key_once(b, D):
    """Build the step's 32 keys from (quarter, offset) pieces and check that
    the LDS stage holds K row t / V token t of the step exactly where the
    fragment reads look for them."""
    # element id = (kind, key in step, dim); the pool block of a key is fixed
    # by its quarter (8 keys), its position inside the block by the offset.
    src = {}
    for qi in range(4):
        for kk in range(8):
            key = 8 * qi + kk
            t = ((8 * qi) & (b - 1)) + kk             # token inside its block
            for d in range(D):
                src[(qi, "K", k_elem(b, D, t, d))] = ("K", key, d)
                src[(qi, "V", v_elem(b, D, t, d))] = ("V", key, d)
    stage = {}
    for wave, lane, qi, off, lds in ring_dma(b, D):
        kind = "K" if wave < 2 else "V"
        for e in range(8):                            # 8 two-byte elements per piece
            item = src[(qi, kind, off + 2 * e)]
            assert (lds + 2 * e) not in stage
            stage[lds + 2 * e] = item
    assert len(stage) == 2 * 32 * D                   # K and V of 32 keys, each once
    chunks = D // 32
    kbytes = 2 * chunks * 1024
    # K fragment: chunk (h, m), lane (t, g) reads 8 dims 32m + 8g.. of row 16h + t
    for h in range(2):
        for m in range(chunks):
            for lane in range(64):
                t, g = lane & 15, lane >> 4
                for e in range(8):
                    assert stage[(h * chunks + m) * 1024 + lane * 16 + 2 * e] == ("K", 16 * h + t, 32 * m + 8 * g + e)
    # V fragment: chunk n, tile h, lane (d, tg) reads tokens 4tg..4tg+3 of dim 16n + d
    for n in range(D // 16):
        for h in range(2):
            for lane in range(64):
                d, tg = lane & 15, lane >> 4
                for e in range(4):
                    assert stage[kbytes + n * 1024 + h * 512 + lane * 8 + 2 * e] == ("V", 16 * h + 4 * tg + e, 16 * n + d)


def decode_pair8_offsets(D):
    """(block, offset) pairs: block 0 is the pair's first 8-token block, 1 the second."""
    k, v = [], []
    for lane in range(64):
        kb = 0 if (lane & 15) < 8 else 1
        for m in range(D // 32):
            k.append((kb, (lane & 7) * 64 + (lane >> 4) * 16 + m * 8 * 64))
        vb = 0 if (lane >> 4) < 2 else 1
        for n in range(D // 16):
            v.append((vb, ((lane >> 4) & 1) * (D * 8) + (lane & 15) * 8 + n * 128))
    return k, v


@pytest.mark.parametrize("D", [64, 128])
def test_decode_pair8_loads_in_bounds(D):
    block_bytes = 8 * D * 2
    k, v = decode_pair8_offsets(D)
    for blk, o in k:
        assert 0 <= o and o + 16 <= block_bytes
    for blk, o in v:
        assert 0 <= o and o + 8 <= block_bytes
    for pieces, w in ((k, 16), (v, 8)):
        for blk in (0, 1):
            assert len({o + i for b, o in pieces if b == blk for i in range(w)}) == block_bytes


def decode_tile16_offsets(D):
    """(byte offset, width) of every lane's K and V pieces in one 16-row
    sub-tile, as load_tile16 forms them (K and V offsets relative to the
    sub-tile's K and V starts)."""
    k, v = [], []
    for lane in range(64):
        for m in range(D // 32):
            k.append((lane & 15) * 64 + (lane >> 4) * 16 + m * 16 * 64)
        for n in range(D // 16):
            v.append((lane >> 4) * (D * 8) + (lane & 15) * 8 + n * 128)
    return k, v


@pytest.mark.parametrize("b", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_tile16_loads_in_bounds(b, D):
    """Each piece lies inside its 16-row sub-tile, the pieces cover the
    sub-tile's bytes exactly once, and every sub-tile of the block (the
    sub-tile offset of open_table, (j mod b/16) * sub-tile bytes) lies inside
    the block's tile of the KV head -- so any block in the pool, block 0
    included, is a safe address."""
    sub_bytes = 16 * D * 2
    tile_bytes = b * D * 2
    k, v = decode_tile16_offsets(D)
    for pieces, w in ((k, 16), (v, 8)):
        for o in pieces:
            assert 0 <= o and o + w <= sub_bytes
        covered = [o + i for o in pieces for i in range(w)]
        assert len(covered) == len(set(covered)) == sub_bytes
    for j in range(b // 16):
        assert 0 <= j * sub_bytes and (j + 1) * sub_bytes <= tile_bytes


def ring_dma_fp8(b, D):
    """FP8 pools: per (wave, lane, instruction): (quarter, byte offset in the
    block's tile, LDS byte offset in the raw stage)."""
    R = min(b, 16)
    r_shift = 3 if R == 8 else 4
    sub_bytes = R * D
    pieces = D // 64
    out = []
    for wave in range(WAVES):
        for lane in range(64):
            qi = 2 * wave + ((lane >> 3) & 1) if wave < 2 else 2 * (wave - 2) + (lane >> 5)
            in_blk = (8 * qi) & (b - 1)
            row_q = in_blk & (R - 1)
            off = (in_blk >> r_shift) * sub_bytes
            if wave < 2:
                off += (row_q + (lane & 7)) * 16 + (lane >> 4) * (R * D // 4)
                stride = R * 16
            else:
                off += ((row_q >> 2) + ((lane >> 4) & 1)) * 4 * D + (lane & 15) * 16
                stride = 256
            for i in range(pieces):
                out.append((wave, lane, qi, off + i * stride, (wave * pieces + i) * 1024 + lane * 16))
    return out


def k8_elem(b, D, t, d):
    """Byte of FP8 K element (token t of the block, dim d), include/pa.h."""
    R = min(b, 16)
    s, r = divmod(t, R)
    return s * R * D + (d // (D // 4)) * R * D // 4 + ((d % (D // 4)) // 16) * R * 16 + r * 16 + d % 16


def v8_elem(b, D, t, d):
    R = min(b, 16)
    s, r = divmod(t, R)
    return (s * R * D + (r // 4) * 4 * D + ((d % (D // 16)) // 4) * 256 + (d // (D // 16)) * 16
            + (d % 4) * 4 + r % 4)


@pytest.mark.parametrize("b", [8, 16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_ring_fp8_loads_and_widening(b, D):
    """FP8 ring: loads stay inside the tile and the raw stage, copy each key's
    codes once, and the widening pass (each lane its own pieces) leaves the
    bf16 slot holding the fragments of the FP8 lane roles: K chunk (h, m),
    lane (t, g) = dims g*D/4 + 8m .. of row 16h + t; V chunk n, tile h, lane
    (r, tg) = tokens 4tg .. of dim r*D/16 + n."""
    tile = b * D
    pieces = D // 64
    raw_step = 2 * 2 * pieces * 1024
    src = {}
    for qi in range(4):
        for kk in range(8):
            key = 8 * qi + kk
            t = ((8 * qi) & (b - 1)) + kk
            for d in range(D):
                src[(qi, "K", k8_elem(b, D, t, d))] = ("K", key, d)
                src[(qi, "V", v8_elem(b, D, t, d))] = ("V", key, d)
    raw = {}
    for wave, lane, qi, off, lds in ring_dma_fp8(b, D):
        assert 0 <= off and off + 16 <= tile
        assert 0 <= lds and lds + 16 <= raw_step
        kind = "K" if wave < 2 else "V"
        for e in range(16):
            assert lds + e not in raw
            raw[lds + e] = src[(qi, kind, off + e)]
    assert len(raw) == 2 * 32 * D
    # widening, as in the kernel's landing pass
    chunks = D // 32
    kbytes = 2 * chunks * 1024
    slot = {}
    for wave in range(WAVES):
        for lane in range(64):
            for pc in range(pieces):
                base = (wave * pieces + pc) * 1024 + lane * 16
                if wave < 2:
                    for u in range(2):
                        for e in range(8):
                            slot[(wave * chunks + 2 * pc + u) * 1024 + lane * 16 + 2 * e] = raw[base + 8 * u + e]
                else:
                    h = wave - 2
                    for e4 in range(4):
                        for tok in range(4):
                            slot[kbytes + (4 * pc + e4) * 1024 + h * 512 + lane * 8 + 2 * tok] = raw[base + 4 * e4 + tok]
    for h in range(2):
        for m in range(chunks):
            for lane in range(64):
                t, g = lane & 15, lane >> 4
                for e in range(8):
                    assert slot[(h * chunks + m) * 1024 + lane * 16 + 2 * e] == ("K", 16 * h + t, g * (D // 4) + 8 * m + e)
    for n in range(D // 16):
        for h in range(2):
            for lane in range(64):
                r, tg = lane & 15, lane >> 4
                for e in range(4):
                    assert slot[kbytes + n * 1024 + h * 512 + lane * 8 + 2 * e] == ("V", 16 * h + 4 * tg + e, r * (D // 16) + n)
