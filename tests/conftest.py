"""Shared fixtures. GPU tests are marked ``gpu``; everything else runs on the CPU."""

from __future__ import annotations

import pytest


@pytest.fixture(scope="session")
def cuda():
    """The GPU device; GPU tests fail (not skip) when no GPU or library is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import paged_attention_decode_amd as pa
    pa.load_library()
    return torch.device("cuda:0")
