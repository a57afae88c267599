"""Host-side checks of the harness's greedy token choice (CPU torch)."""
import pytest
import torch

from persistent_interpreter_amd.harness import _chunks, greedy_tokens


@pytest.mark.parametrize("V", [128256, 151936, 1024, 1000, 17])
def test_greedy_tokens_equal_torch_argmax_with_ties(V):
    g = torch.Generator().manual_seed(V)
    for trial in range(10):
        x = torch.randn(3, V, generator=g)
        if trial % 2:
            # several copies of the maximum: the first index must win
            m = x.max() + 1
            idx = torch.randint(0, V, (3, 4), generator=g)
            for b in range(3):
                x[b, idx[b]] = m
        assert torch.equal(greedy_tokens(x), torch.argmax(x, dim=-1).to(torch.int32))


def test_chunk_count_divides_vocab():
    for V in (128256, 151936, 1024, 1000):
        C = _chunks(V)
        assert V % C == 0 and 16 <= C and V // C >= 16
    assert _chunks(17) == 1
