"""The guard-band checks of the GPU tests, on CPU tensors: a stray byte
written just past either end of the middle, anywhere in a guard, or a word of
the middle left unwritten is detected; a middle written in full with the
edges untouched passes."""
import torch

from helpers import GUARD, all_written, edges_intact, guarded


def test_untouched_edges_and_full_middle_pass():
    full, mid = guarded(64, device="cpu")
    mid.view(torch.float32).copy_(torch.arange(16, dtype=torch.float32))
    assert edges_intact(full, 64)
    assert all_written(mid)


def test_stray_writes_are_caught():
    for pos in (GUARD - 1, GUARD + 64, 0, 2 * GUARD + 63):
        full, mid = guarded(64, device="cpu")
        mid.fill_(0)
        full[pos] = 0
        assert not edges_intact(full, 64), pos


def test_unwritten_word_is_caught():
    full, mid = guarded(64, device="cpu")
    w = mid.view(torch.float32)
    w.copy_(torch.ones(16))
    w[7] = float(torch.tensor([0xA5A5A5A5 - (1 << 32)], dtype=torch.int64).to(torch.int32).view(torch.float32)[0])
    assert not all_written(mid)
    assert edges_intact(full, 64)


def test_wrong_middle_size_is_caught():
    full, _ = guarded(64, device="cpu")
    assert not edges_intact(full, 60)
