"""The round-trip smoke check (every entry point family once, against the oracle) runs
as a GPU test too, so a change that breaks it shows up with the other parity tests."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__
    __graft_entry__.smoke()
