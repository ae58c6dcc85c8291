"""The Python binding has no CPU fallback: a missing library is an error, and
tensors that do not live on a GPU are refused instead of computed."""
import pytest
import torch

from partial_context_patch_amd import npa


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(npa, "LIB_PATH", str(tmp_path / "libnpa.so"))
    monkeypatch.setattr(npa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        npa.load(build_if_missing=False)


def test_cpu_tensors_are_refused():
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        npa.attn_fwd(q, q.clone(), q.clone(), map_hw=(8, 8), tile=(4, 4), halo=(1, 1))
    x = torch.zeros(1, 4, 8, 8)
    with pytest.raises(ValueError, match="GPU"):
        npa.sg_blend(x, x.clone(), 0.5, 4.0)
    with pytest.raises(ValueError, match="GPU"):
        npa.asg_blend(x, x.clone(), x.clone(), 0.5)


def test_shape_and_dtype_mismatches_are_refused():
    q = torch.zeros(1, 64, 2, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        npa.attn_fwd(q, q, q, map_hw=(8, 8), tile=(4, 4), halo=(1, 1))
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="do not match"):
        npa.attn_fwd(q, q, q, map_hw=(8, 9), tile=(4, 4), halo=(1, 1))
