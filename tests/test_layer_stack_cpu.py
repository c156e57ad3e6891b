"""Host logic of the layer stack (CodecLayerStack) on CPU tensors, with no
library call: per-layer views are the right slices of one allocation, the
capacity doubling keeps every layer's archived blocks, and stack-wide calls
refuse layers at different lengths and tensors whose (layer, batch) axes do
not fold, before anything is enqueued."""

import pytest
import torch

from compressed_domain_attention_amd import binding as bd


def make(L=3, B=2, H=2, D=64, R=8, S=2, fmt="i8"):
    return bd.CodecLayerStack(L, B, H, D, R, S, k_fmt=fmt, device="cpu")


def test_views_are_slices_of_one_allocation():
    st = make()
    cap = st.capacity
    for l in range(st.L):
        kl, vl = st.layer(l)
        assert kl.rows.shape == (2, 2, cap, 2, 64) and kl.scales.shape == (2, 2, cap, 2)
        assert kl.tail.shape == (2, 2, 8, 64)
        assert kl.rows.data_ptr() == st.k.rows.data_ptr() + l * 2 * 2 * cap * 2 * 64
        assert vl.tail.data_ptr() == st.v.tail.data_ptr() + l * 2 * 2 * 8 * 64 * 2
        d = kl._desc()
        assert (d.batch, d.heads, d.capacity) == (2, 2, cap)


def test_growth_keeps_every_layer():
    st = make()
    for l in range(st.L):
        kl, vl = st.layer(l)
        kl.n_blocks = vl.n_blocks = l + 1
        kl.rows[:, :, :l + 1] = l + 1
        kl.scales[:, :, :l + 1] = 0.5 * (l + 1)
    st._grow(40)
    assert st.capacity == 64 and st.k.rows.shape[2] == 64
    for l in range(st.L):
        kl, _ = st.layer(l)
        assert kl.rows.shape[2] == 64
        assert torch.all(kl.rows[:, :, :l + 1] == l + 1)
        assert torch.all(kl.scales[:, :, :l + 1] == 0.5 * (l + 1))


def test_stack_calls_need_equal_lengths():
    st = make()
    st.layer(1)[0].n_tail = 3
    st.layer(1)[1].n_tail = 3
    q = torch.zeros((3, 2, 4, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="same length"):
        st.decode(q)
    with pytest.raises(ValueError, match="same length"):
        st.crop(0)


def test_stack_tensor_shapes():
    st = make()
    with pytest.raises(ValueError):
        st._flat(torch.zeros((2, 2, 4, 1, 64)), "q")        # wrong layer count
    with pytest.raises(ValueError):
        st._flat(torch.zeros((3, 2, 4, 64)), "q")           # not 5-D
    t = torch.zeros((2, 3, 4, 1, 64)).transpose(0, 1)       # (3, 2, ...) whose axes do not fold
    with pytest.raises(ValueError, match="fold"):
        st._flat(t, "q")
    assert st._flat(torch.zeros((3, 2, 4, 1, 64)), "q").shape == (6, 4, 1, 64)


def test_layer_views_refuse_their_own_beam_reorder():
    st = make()
    with pytest.raises(ValueError):
        st.layer(0)[0].select_batch([1, 0])
    with pytest.raises(ValueError):
        bd.select_batch(st.layer(0)[1], [1, 0])
    with pytest.raises(ValueError):
        st.select_batch([0, 2])                               # row 2 out of range for B = 2
    with pytest.raises(ValueError):
        st.select_batch([])
