"""The oracle's storage-layout module (CPU only): the 256-k panel layouts of
the MXFP4 and NVFP4 scale bytes, checked against loops written from the C
header's definitions (MXFP4: panel p = blocks 8p.., rows of min(8, blocks
left) bytes, the even blocks' bytes before the odd ones'; NVFP4: panel p =
blocks 16p.., rows of 16 bytes in a fixed block order), the canonical
two's-complement nibbles and the group-major INT4 scales."""
import numpy as np
import pytest


def panels_by_definition(e_rows):
    rows, nb = e_rows.shape
    out = np.full(rows * nb, 255, np.uint8)
    pos = 0
    for p in range(0, nb, 8):
        w = min(8, nb - p)
        order = list(range(0, w, 2)) + list(range(1, w, 2))    # even blocks first
        for r in range(rows):
            for j in order:
                out[pos] = e_rows[r, p + j]
                pos += 1
    assert pos == rows * nb
    return out


def nv_panels_by_definition(s_rows):
    """The NVFP4 scale panel layout written out with loops from its definition:
    panel p = blocks 16p..16p+15, rows of 16 bytes, the blocks in the order
    0,1,4,5,8,9,12,13,2,3,6,7,10,11,14,15."""
    rows, nb = s_rows.shape
    order = [0, 1, 4, 5, 8, 9, 12, 13, 2, 3, 6, 7, 10, 11, 14, 15]
    out = []
    for p in range(nb // 16):
        for r in range(rows):
            for j in order:
                out.append(s_rows[r, 16 * p + j])
    return np.array(out, dtype=s_rows.dtype)


# ------------------------------------------------ the oracle's layout module
import oracle  # noqa: E402


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 384), (4, 2048)])
def test_e8m0_offsets_are_a_permutation(rows, K):
    offs = oracle.e8m0_panel_offsets(rows, K)
    assert sorted(offs.reshape(-1).tolist()) == list(range(rows * (K // 32)))


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 384), (5, 256), (2, 96), (7, 1152)])
def test_oracle_e8m0_panels_match_definition(rows, K):
    rng = np.random.default_rng(7 * rows + K)
    e_rows = rng.integers(0, 255, size=(rows, K // 32), dtype=np.uint8)
    offs = oracle.e8m0_panel_offsets(rows, K)
    assert np.array_equal(oracle.to_panels(e_rows, offs), panels_by_definition(e_rows))
    assert np.array_equal(oracle.from_panels(oracle.to_panels(e_rows, offs), offs), e_rows)


@pytest.mark.parametrize("rows,K", [(1, 256), (5, 512), (3, 3584)])
def test_oracle_e4m3_panels_match_definition(rows, K):
    rng = np.random.default_rng(rows * 3 + K)
    s_rows = rng.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    offs = oracle.e4m3_panel_offsets(rows, K)
    assert np.array_equal(oracle.to_panels(s_rows, offs), nv_panels_by_definition(s_rows))


def test_twos_complement_nibbles():
    """Canonical INT4 storage: byte = (c[2i] & 0xF) | (c[2i+1] & 0xF) << 4,
    worked by hand for codes (-8, 7), (-1, 0), (3, -4)."""
    c = np.array([[-8, 7, -1, 0, 3, -4]], np.int8)
    assert oracle.pack_int4_twos(c).tolist() == [[0x78, 0x0F, 0xC3]]
    assert np.array_equal(oracle.unpack_int4_twos(oracle.pack_int4_twos(c)), c)
    every = np.arange(-8, 8, dtype=np.int8).reshape(1, 16)
    assert np.array_equal(oracle.unpack_int4_twos(oracle.pack_int4_twos(every)), every)
    with pytest.raises(ValueError):
        oracle.pack_int4_twos(np.array([[8, 0]], np.int16))


def test_group_major_is_transpose():
    s = np.arange(12, dtype=np.float32).reshape(3, 4)      # [rows=3][groups=4]
    gm = oracle.group_major(s)
    assert gm.shape == (4, 3) and gm.flags["C_CONTIGUOUS"]
    assert gm[2, 1] == s[1, 2]
