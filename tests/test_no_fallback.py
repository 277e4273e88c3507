"""The binding has no CPU path: a missing library or host tensors raise errors, never a
result computed another way."""
import pytest
import torch

import paged_kv_cache_409_amd as pkv
from paged_kv_cache_409_amd import _lib


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libpkv.so"))
    with pytest.raises(RuntimeError, match="missing"):
        pkv.partition_tokens(8, 32, 8, 4096)


def test_host_tensors_are_refused():
    S, H, D, NB = 2, 8, 128, 4
    q = torch.zeros(S, H, D, dtype=torch.bfloat16)
    kc = torch.zeros(NB, 1, 16, D, dtype=torch.bfloat16)
    bt = torch.zeros(S, 2, dtype=torch.int32)
    cl = torch.ones(S, dtype=torch.int32)
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="device tensors"):
        pkv.paged_attention_decode(out, q, kc, kc.clone(), bt, cl, 0.088, 32)


def test_host_or_strided_workspace_is_refused():
    # A caller's workspace is written by the kernels, so the binding takes only a
    # contiguous uint8 device tensor (checked before any library call; no GPU here, so
    # every tensor below is refused).
    from paged_kv_cache_409_amd import ops
    with pytest.raises(ValueError, match="device tensors"):
        ops._workspace(torch.zeros(1024, dtype=torch.uint8), 512, "cpu")
    with pytest.raises(ValueError, match="device tensors"):
        ops._workspace(torch.zeros(256, dtype=torch.float32), 512, "cpu")
    assert ops._workspace(None, 0, "cpu") == (None, 0)


def test_host_copy_on_write_sources_are_refused():
    # cow_src is read by the kernels: the binding takes only an int32 [num_seqs] device
    # tensor (checked before any library call; no GPU here, so a host tensor is refused).
    from paged_kv_cache_409_amd import ops
    assert ops._cow_ptr(None, 4) is None
    with pytest.raises(ValueError, match="device tensors"):
        ops._cow_ptr(torch.full((4,), -1, dtype=torch.int32), 4)
