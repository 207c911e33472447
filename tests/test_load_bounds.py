"""Every address of the two global-load paths stays inside its tile.

Buffer-resource loads are bounds-checked by the hardware (a lane past the
resource reads zero); the 16-bit prefill fragments and the paired 8-token
decode tiles use plain global loads from a uniform tile base plus a lane
offset, so their offsets must stay within the tile on their own.  This test
enumerates those lane offsets, written as in pa_prefill.hip (FragPair loads,
kro/vro) and pa_decode.hip (load_pair8), for every supported sub-tile height
and head dim, and checks them against the tile sizes of the pool layout in
include/pa.h: a 16-bit sub-tile of R rows holds R * head_dim * 2 bytes of K
and the same of V.  Runs on the CPU.
"""
import pytest


def prefill_offsets(rows, D):
    k, v = [], []
    for lane in range(64):
        for m in range(D // 32):
            k.append(((lane & 15) & (rows - 1)) * 64 + (lane >> 4) * 16 + m * rows * 64)
        for n in range(D // 16):
            v.append(((lane >> 4) & (rows // 4 - 1)) * (D * 8) + (lane & 15) * 8 + n * 128)
    return k, v


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


@pytest.mark.parametrize("rows", [8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_fragment_loads_in_bounds(rows, D):
    sub_bytes = rows * D * 2
    k, v = prefill_offsets(rows, D)
    assert min(k) >= 0 and max(k) + 16 <= sub_bytes     # 16-byte K pieces
    assert min(v) >= 0 and max(v) + 8 <= sub_bytes      # 8-byte V pieces
    # every byte of the sub-tile is read (nothing of the tile is skipped)
    assert len({o + i for o in k for i in range(16)}) == sub_bytes
    assert len({o + i for o in v for i in range(8)}) == sub_bytes


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
