"""The parity tests read the library's code bytes through
parity_util.unpack_gpu_codes, which maps the library's layout to codes (the
oracle keeps one record per token for K and V alike).  Here that mapping is
checked against bytes packed bit by bit from the layout's definition: K one
record per token (channel d at bit n*d); V 32-token tiles of 32-bit words,
word w of channel d at byte (w*D + d)*4 of the tile, token k of a word at
bit n*k."""
import numpy as np
import pytest

from parity_util import unpack_gpu_codes


def _pack_bits(nbytes, placements):
    out = np.zeros(nbytes, np.uint8)
    for bit, width, val in placements:
        for i in range(width):
            if (val >> i) & 1:
                b = bit + i
                out[b // 8] |= np.uint8(1 << (b % 8))
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_unpack_gpu_codes_against_definition(bits):
    rng = np.random.default_rng(7 + bits)
    U, T, D = 2, 64, 16
    codes = rng.integers(0, 1 << bits, size=(U, T, D))
    rec = D * bits // 8
    k_packed = np.stack([
        _pack_bits(T * rec, [((t * rec) * 8 + d * bits, bits, int(codes[u, t, d]))
                             for t in range(T) for d in range(D)]) for u in range(U)])
    per_word = 32 // bits
    tile_bytes = 32 * D * bits // 8
    v_pl = []
    for t in range(T):
        tile, i = divmod(t, 32)
        w, k = divmod(i, per_word)
        for d in range(D):
            v_pl.append((tile * tile_bytes * 8 + (w * D + d) * 32 + k * bits, bits, d))
    v_packed = np.stack([
        _pack_bits(T * rec, [(bit, wd, int(codes[u, t, d]))
                             for (bit, wd, d), t in zip(v_pl, np.repeat(np.arange(T), D))])
        for u in range(U)])
    assert np.array_equal(unpack_gpu_codes(k_packed, 0, T, D, bits), codes)
    assert np.array_equal(unpack_gpu_codes(v_packed, 1, T, D, bits), codes)
    # a ragged T reads only the first T tokens
    assert np.array_equal(unpack_gpu_codes(v_packed, 1, 40, D, bits), codes[:, :40])
