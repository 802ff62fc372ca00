"""The Python binding's marshalling checks run before anything reaches the
library (CPU only: every call here is rejected on the host)."""

import pytest
import torch

from hybrid_recurrent_serving_amd import kda as K


def test_same_dtype_accepts_none_and_rejects_mismatch():
    x = torch.zeros(2, dtype=torch.bfloat16)
    K._same_dtype(x, a=None, b=torch.zeros(1, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        K._same_dtype(x, a=torch.zeros(1))


def test_host_tensors_are_rejected():
    q = torch.zeros(2, 1, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_decode(q, q, q, q, torch.zeros(2, 1), q, torch.zeros(2, 1, 16, 16),
                     torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32))


def test_shape_mismatch_is_rejected():
    q = torch.zeros(2, 1, 16)
    with pytest.raises(ValueError, match="leading shape"):
        K.kda_decode(q, q, torch.zeros(3, 1, 16), q, torch.zeros(2, 1), q,
                     torch.zeros(2, 1, 16, 16), torch.zeros(2, dtype=torch.int32),
                     torch.zeros(2, dtype=torch.int32))
    x = torch.zeros(4, 16)
    with pytest.raises(ValueError, match="conv_pool"):
        K.kda_conv_short(x, torch.zeros(16, 4), torch.tensor([0, 4], dtype=torch.int32),
                         torch.zeros(1, 16, 2), torch.zeros(1, dtype=torch.int32),
                         torch.zeros(1, dtype=torch.int32))
