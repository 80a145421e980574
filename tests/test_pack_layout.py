"""CPU check of the test-side readers of the workspace pack layouts
(tests/gpu_util.py) against a direct packer written from the layout text in
include/oc_attn.h."""
import numpy as np

from gpu_util import unpack_k, unpack_v


def operand_offset(r, col):
    """The layout text: the 16-byte chunk holding columns 32g+16h..+16 of row r
    (lane l = 16g + r%16 of the MFMA operand for row block r//16) is chunk
    (2*(r//16) + h)*64 + l."""
    c = col // 16
    g, h = c // 2, c % 2
    lane = 16 * g + r % 16
    return ((2 * (r // 16) + h) * 64 + lane) * 16 + col % 16


def pack_k(codes):
    S = codes.shape[0]
    nT = -(-S // 128)
    out = np.zeros((nT, 16384), np.uint8)
    for j in range(S):
        t, r = divmod(j, 128)
        for ch in range(128):
            out[t, operand_offset(r, ch)] = codes[j, ch]
    return out.reshape(-1)


def pack_v(codes):
    S = codes.shape[0]
    nT = -(-S // 128)
    out = np.zeros((nT, 16384), np.uint8)
    for j in range(S):
        t, jj = divmod(j, 128)
        kk = 32 * ((jj >> 2) & 3) + 4 * (jj >> 4) + (jj & 3)
        for d in range(128):
            out[t, operand_offset(d, kk)] = codes[j, d]
    return out.reshape(-1)


def test_unpack_inverts_pack():
    rng = np.random.default_rng(0)
    for S in (1, 77, 128, 300):
        codes = rng.integers(0, 256, (S, 128), dtype=np.uint8)
        assert np.array_equal(unpack_k(pack_k(codes), S), codes)
        assert np.array_equal(unpack_v(pack_v(codes), S), codes)


def test_v_column_order_matches_score_layout():
    """Lane group g of a 16x16 MFMA output holds keys 16t + 4g + r; those 32
    keys must occupy the contiguous columns 32g..32g+31 of a V row."""
    for g in range(4):
        keys = [16 * t + 4 * g + r for t in range(8) for r in range(4)]
        cols = [32 * ((j >> 2) & 3) + 4 * (j >> 4) + (j & 3) for j in keys]
        assert cols == list(range(32 * g, 32 * g + 32))
