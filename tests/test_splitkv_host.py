"""Host logic of the split-KV path: the split-count heuristic."""
import pytest

from exact_attention_forward_05_amd.api import _SPLIT_CHOICES, choose_splits


def test_full_machine_non_causal_is_not_split():
    # 1024 workgroups of equal work on 256 CUs: nothing to gain
    assert choose_splits(1, 8, 16384, 64, False) == 1
    assert choose_splits(4, 32, 4096, 128, False) == 1


def test_underfilled_machine_is_split():
    # 128 workgroups on 256 CUs
    assert choose_splits(1, 1, 16384, 64, False) >= 2
    # causal 4k: the longest query tiles set the time of a one-wave grid
    assert choose_splits(1, 8, 4096, 64, True) >= 2


@pytest.mark.parametrize("shape", [(1, 4, 128, 64, False), (1, 1, 1, 64, True),
                                   (2, 3, 300, 128, True), (1, 8, 4096, 64, True)])
def test_choice_is_valid(shape):
    s = choose_splits(*shape)
    assert s in _SPLIT_CHOICES
    B, H, S, D, causal = shape
    assert s <= max(1, -(-S // 128))  # never more runs than the longest tile has pairs
