"""Host-side logic of the layer composites that needs no GPU: the decode
state's capacity guard refuses a step before anything is launched."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_amd import layer


def _state(B=3, capacity=5, m=4):
    return layer.DecodeState(B, capacity, m, 8, 4, torch.float32, "cpu")


def test_capacity_guard_accepts_the_last_token_that_fits():
    st = _state()
    st.t_host[:] = [0, 7, st.capacity * st.m - 1]
    st.check_room()  # token capacity*m - 1 still belongs to block capacity - 1


def test_capacity_guard_refuses_a_full_sequence():
    st = _state()
    st.t_host[:] = [3, st.capacity * st.m, 2]
    with pytest.raises(ValueError, match="sequence 1"):
        st.check_room()


def test_decode_step_refuses_before_any_launch():
    """decode_step checks the room first: with a full sequence it raises before reaching the library
    (which a CPU-only test could not call)."""
    st = _state(B=2)
    st.t_host[:] = [0, st.capacity * st.m]
    W = {"c": 8, "cI": 4, "dc": 16}
    H_new = torch.zeros(2, 32)
    with pytest.raises(ValueError, match="sequence 1"):
        layer.decode_step(H_new, W, st, st.m, k=4, nh=2, nhI=2)
    with pytest.raises(ValueError, match="one row per sequence"):
        layer.decode_step(torch.zeros(3, 32), W, st, st.m, k=4, nh=2, nhI=2)
    assert np.all(st.t.numpy() == 0)  # nothing advanced


def test_positions_follow_a_prefill_hand_off():
    """load_prefill sets both position mirrors; a prefill longer than the cache is refused."""
    st = _state(B=2, capacity=3, m=2)

    class Buf:  # the fields of a prefill's buffers that the hand-off reads
        def __init__(self, L):
            self.Y_H = torch.zeros(L, 4 * 8 + 4 * 4 + 16)
            self.Ccomp = torch.zeros(L // 2, 8)
            self.KIcomp = torch.zeros(L // 2, 4)

    st.load_prefill(1, Buf(5), 8, 4)
    assert st.t_host.tolist() == [0, 5] and st.t.tolist() == [0, 5]
    with pytest.raises(ValueError):
        st.load_prefill(0, Buf(8), 8, 4)
