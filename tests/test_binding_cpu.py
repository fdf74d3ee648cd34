"""The Python binding's checks of caller-supplied tensors (no GPU needed: the
helpers run before anything reaches the library)."""
import torch
import pytest

from block_sparse_attention_softmax_amd import binding as S


def test_buffer_check_accepts_the_exact_tensor():
    t = torch.zeros((1, 2, 3, 4), dtype=torch.int32)
    assert S._buf(t, "x", torch.int32, (1, 2, 3, 4), t.device) is t


@pytest.mark.parametrize("t", [
    torch.zeros((1, 2, 3, 5), dtype=torch.int32),             # wrong shape
    torch.zeros((1, 2, 3, 4), dtype=torch.int64),             # wrong dtype
    torch.zeros((1, 2, 4, 3), dtype=torch.int32).transpose(2, 3),  # not contiguous
    [0, 1, 2],                                                 # not a tensor
])
def test_buffer_check_rejects(t):
    with pytest.raises(ValueError):
        S._buf(t, "x", torch.int32, (1, 2, 3, 4), torch.device("cpu"))


def test_buffer_check_rejects_another_device():
    t = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError):
        S._buf(t, "x", torch.int32, (2,), torch.device("cuda:0"))


def test_block_counts():
    assert S._blocks(32760, 128, 64) == (256, 512)
    assert S._blocks(1, 128, 64) == (1, 1)
    assert S._blocks(100, 0, 64) == (0, 2)  # left for the library to reject


def test_workspace_size_counts_bytes_of_any_dtype():
    ws = torch.zeros(10, dtype=torch.float32)
    t, n = S._workspace(ws, 0, ws.device)
    assert t is ws and n == 40
    with pytest.raises(ValueError):
        S._workspace(torch.zeros((4, 4))[:, 0], 0, torch.device("cpu"))
    with pytest.raises(ValueError):
        S._workspace(ws, 0, torch.device("cuda:0"))
