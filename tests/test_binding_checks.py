"""The binding's checks of caller-supplied outputs, without a GPU.

The C ABI takes bare pointers and leading dimensions, so it cannot know how
large an output buffer is: a buffer with fewer rows than the result would be
written past its end.  The binding therefore checks every enabled output's
shape, dtype and device before any call into the library.  These checks run
on CPU tensors here (the device is a parameter of the check).
"""
import pytest
import torch

from swiglu_activation_cast_amd import _binding as b


def outs(M, W, layout, **override):
    o = dict(zip(("q_row", "q_col", "s_row", "s_col"), b.alloc_outputs(M, W, layout, "cpu")))
    o.update(override)
    return (o["q_row"], o["q_col"], o["s_row"], o["s_col"])


@pytest.mark.parametrize("layout", [1, 2, 3])
def test_matching_outputs_pass(layout):
    args = b._out_args(outs(64, 96, layout), layout, 64, 96, "cpu")
    assert len(args) == 8
    for ptr, on in zip(args[0::2], (layout & 1, layout & 1, layout & 2, layout & 2)):
        assert (ptr is not None) == bool(on)


def test_padded_row_stride_passes():
    big = torch.empty((64, 128), dtype=torch.uint8)
    args = b._out_args(outs(64, 96, 1, q_row=big[:, :96]), 1, 64, 96, "cpu")
    assert args[1] == 128


@pytest.mark.parametrize("name,shape", [("q_row", (32, 96)), ("s_row", (32, 3)), ("q_col", (96, 32)),
                                        ("s_col", (96, 1)), ("q_row", (64, 64)), ("s_col", (48, 2))])
def test_undersized_output_raises(name, shape):
    bad = torch.empty(shape, dtype=torch.uint8)
    with pytest.raises(ValueError, match=name):
        b._out_args(outs(64, 96, 3, **{name: bad}), 3, 64, 96, "cpu")


def test_wrong_dtype_device_and_stride_raise():
    with pytest.raises(ValueError):
        b._out_args(outs(64, 96, 1, q_row=torch.empty((64, 96), dtype=torch.int8)), 1, 64, 96, "cpu")
    with pytest.raises(ValueError, match="unit column stride"):
        b._out_args(outs(64, 96, 2, q_col=torch.empty((64, 96), dtype=torch.uint8).t()), 2, 64, 96, "cpu")
    with pytest.raises(ValueError, match="is on"):
        b._out_args(outs(64, 96, 1), 1, 64, 96, "meta")
    with pytest.raises(ValueError):
        b._out_args(outs(64, 96, 1)[:3], 1, 64, 96, "cpu")


def test_disabled_layout_is_ignored():
    # colwise-only: the rowwise slots may hold anything
    o = outs(64, 96, 2, q_row=torch.empty(0, dtype=torch.uint8), s_row=None)
    args = b._out_args(o, 2, 64, 96, "cpu")
    assert args[0] is None and args[2] is None
