"""Host RoPE table builder (package code, CPU): worked values and structure."""
import math

import numpy as np
import pytest

from transformer_attention_attn_amd.rope import grid_positions, rope_tables


def test_grid_positions_row_major_with_prefix():
    pos, rot = grid_positions(2, 3, prefix_tokens=2)
    assert pos.shape == (8, 2) and rot.tolist() == [False, False] + [True] * 6
    assert pos[2:].tolist() == [[0, 0], [0, 1], [0, 2], [1, 0], [1, 1], [1, 2]]


def test_1d_tables_worked_values():
    # D=8: 4 pairs, one axis, base 100: pair i turns by pos * 100^(-i/4)
    c, s = rope_tables(np.arange(5), 8, base=100.0)
    assert c.shape == (5, 4) and c.dtype == np.float32
    for p in (0, 3, 4):
        for i in range(4):
            ang = p * 100.0 ** (-i / 4)
            assert abs(c[p, i] - math.cos(ang)) < 1e-7 and abs(s[p, i] - math.sin(ang)) < 1e-7
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)


def test_3d_tables_split_pairs_per_axis_and_leave_the_rest():
    # D=64: 32 pairs over 3 axes -> 10 per axis, pairs 30 and 31 unrotated
    pos, _ = grid_positions(8, 16, 16)
    c, s = rope_tables(pos, 64)
    tok = 3 * 256 + 5 * 16 + 7  # frame 3, row 5, column 7
    for a, coord in enumerate((3, 5, 7)):
        for i in (0, 4, 9):
            ang = coord * 10000.0 ** (-i / 10)
            assert abs(c[tok, 10 * a + i] - math.cos(ang)) < 1e-6
            assert abs(s[tok, 10 * a + i] - math.sin(ang)) < 1e-6
    assert np.all(c[:, 30:] == 1.0) and np.all(s[:, 30:] == 0.0)


def test_prefix_tokens_are_identity():
    pos, rot = grid_positions(28, 28, prefix_tokens=5)  # DINOv3 at 448 px: class + 4 registers + 28x28
    c, s = rope_tables(pos, 64, rotate=rot)
    assert c.shape == (789, 32)
    assert np.all(c[:5] == 1.0) and np.all(s[:5] == 0.0)
    assert not np.all(c[5:] == 1.0)


def test_ntk_factor_rescales_the_base():
    # one axis, P = 4 pairs: base' = base * f^(4/3)
    c1, s1 = rope_tables([7.0], 8, base=500.0, ntk_factor=2.0)
    c2, s2 = rope_tables([7.0], 8, base=500.0 * 2.0 ** (4 / 3))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("bad", [dict(head_dim=7), dict(base=1.0), dict(ntk_factor=0.0)])
def test_rejects_bad_arguments(bad):
    kw = dict(positions=np.arange(4), head_dim=8)
    kw.update(bad)
    with pytest.raises(ValueError):
        rope_tables(**kw)
