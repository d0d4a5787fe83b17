"""CPU checks of the comparison helpers the GPU parity tests use."""
import numpy as np
import pytest

from tests.parity import assert_parity, rel_l2, stream_errors, token_block_errors, worst_local


def test_one_wrong_chunk_passes_the_whole_tensor_bar_but_not_the_block_bar():
    # the training shape's o: 8 x 4096 x 6 x 128; one 64-token chunk of one stream
    # entirely wrong moves the whole-tensor figure by only ~1/sqrt(3072)
    r = np.random.default_rng(0)
    ref = r.standard_normal((8, 4096, 6, 16))
    x = ref.copy()
    x[3, 640:704, 2] = -ref[3, 640:704, 2]          # chunk 10 of stream (3, 2)
    assert rel_l2(x, ref) < 2e-2 * 3                   # small against the whole tensor
    w, at = worst_local("o", x, ref)
    assert at == (3, 10, 2) and abs(w - 2.0) < 1e-12  # -y against y: relative L2 = 2
    with pytest.raises(AssertionError):
        assert_parity("planted", {"o": (x, ref)}, 0.1)


def test_block_errors_cover_a_ragged_tail_and_zero_blocks():
    ref = np.zeros((1, 70, 2, 3))
    ref[0, :64, 0] = 1.0
    ref[0, 64:, 1] = 2.0
    x = ref.copy()
    x[0, 69, 1, 0] += 0.5                              # the 6-token tail of head 1
    e = token_block_errors(x, ref)
    assert e.shape == (1, 2, 2)
    assert e[0, 0, 0] == 0 and e[0, 0, 1] == 0         # zero reference, zero GPU block
    assert e[0, 1, 0] == 0
    assert abs(e[0, 1, 1] - 0.5 / np.sqrt(6 * 3 * 4.0)) < 1e-15
    x[0, 0, 1, 0] = 1e-3                               # zero reference block: absolute norm
    assert abs(token_block_errors(x, ref)[0, 0, 1] - 1e-3) < 1e-15


def test_stream_errors_for_states_and_gates():
    r = np.random.default_rng(1)
    s = r.standard_normal((2, 3, 4, 5))
    s2 = s.copy()
    s2[1, 2] *= 1.01
    e = stream_errors(s2, s, "state")
    assert e.shape == (2, 3) and abs(e[1, 2] - 0.01) < 1e-12 and e.sum() == e[1, 2]
    g = r.standard_normal((2, 50, 3))
    g2 = g.copy()
    g2[0, :, 1] *= 0.9
    e = stream_errors(g2, g, "gate")
    assert e.shape == (2, 3) and abs(e[0, 1] - 0.1) < 1e-12
