"""Host-side checks of the torch wrappers (no GPU): tensors the kernels read or write
beside q, k and v must sit on the inputs' device, be contiguous and have the stated dtype
and shape, and per-head parameters must hold one value per head, before any pointer
reaches the library."""
import numpy as np
import pytest
import torch

from long_context_lm_amd import polar

GPU = torch.device("cuda:0")


def test_host_tensor_for_a_gpu_call_is_refused():
    table = torch.zeros(2, 8, dtype=torch.int32)               # host memory
    with pytest.raises(ValueError, match="must be on cuda:0"):
        polar._check_aux(table, "page_table", GPU, torch.int32)


def test_strided_table_is_refused():
    table = torch.zeros(2, 16, dtype=torch.int32)[:, :8]       # row stride 16, not 8
    assert not table.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        polar._check_aux(table, "page_table", table.device, torch.int32)


def test_dtype_shape_and_type_are_checked():
    t = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="int32"):
        polar._check_aux(t, "seq_lens", t.device, torch.int32)
    t = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="shape"):
        polar._check_aux(t, "seq_lens", t.device, torch.int32, (4,))
    with pytest.raises(ValueError, match="torch tensor"):
        polar._check_aux(np.zeros(4, np.int32), "seq_lens", t.device, torch.int32)
    with pytest.raises(ValueError, match="torch tensor"):
        polar._check_aux(None, "fwd['u_norm']", t.device, torch.float32)
    polar._check_aux(torch.zeros(4, dtype=torch.int32), "seq_lens", t.device, torch.int32, (4,))


def test_per_head_parameters_hold_one_value_per_head():
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="beta must hold 16"):
        polar._head_params(np.ones(4, np.float32), None, None, 16, 64, cpu)
    with pytest.raises(ValueError, match="count_vec must hold 1024"):
        polar._head_params(None, None, np.ones((16, 32), np.float32), 16, 64, cpu)
    b, nb, w = polar._head_params(np.ones(16), np.zeros(16), np.ones((16, 64)), 16, 64, cpu)
    assert b.dtype == torch.float32 and w.is_contiguous() and w.numel() == 1024

