"""The Python binding refuses tensors the C ABI cannot check (CPU tensors,
wrong dtypes) before any call into the library.  The library handle is
replaced by a tripwire, so a check that let a call through would fail the
test instead of passing a host pointer to a kernel.  Shape checks need GPU
tensors and are covered in tests/test_gpu_binding.py."""

import pytest

torch = pytest.importorskip("torch")
binding = pytest.importorskip("depth_wise_attention_amd.binding")


class _Tripwire:
    def __getattr__(self, name):
        raise AssertionError(f"the library was called ({name}) although the arguments are invalid")


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    monkeypatch.setattr(binding, "_lib", _Tripwire())
    monkeypatch.setattr(binding, "lib", lambda: _Tripwire())


def cpu(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_cpu_tensors_are_refused():
    reps, parts, w = cpu(8, 4, 64), cpu(3, 4, 64), cpu(4, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        binding.mhar_fwd(reps, parts, w)
    with pytest.raises(ValueError, match="GPU"):
        binding.attnres_block_phase1(reps, w)
    with pytest.raises(ValueError, match="GPU"):
        binding.attnres_bwd(reps, parts, w, cpu(4, 4, 64))
    with pytest.raises(ValueError, match="GPU"):
        binding.attnres_full_fwd(cpu(8, 4, 64), cpu(8, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        binding.attnres_full_bwd(cpu(8, 4, 64), cpu(8, 64, dtype=torch.float32), cpu(8, 4, 64))
    with pytest.raises(ValueError, match="GPU"):
        binding.attnres_block_phase2_merge(cpu(4, 64, dtype=torch.float32), cpu(1, 4, dtype=torch.float32),
                                           cpu(4, 64), cpu(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        binding.attnres_msar_fwd(cpu(3, 4, 512), cpu(1, 4, 512, dtype=torch.float32),
                                 cpu(24, 512, dtype=torch.float32), cpu(1, 2048, 4, dtype=torch.float32))


def test_activation_dtypes_are_checked():
    w = cpu(4, 64, dtype=torch.float32)
    for bad in (torch.float16, torch.float64, torch.int16):
        with pytest.raises(TypeError, match="float32 or bfloat16"):
            binding.mhar_fwd(cpu(8, 4, 64, dtype=bad), cpu(3, 4, 64, dtype=bad), w)
        with pytest.raises(TypeError, match="float32 or bfloat16"):
            binding.attnres_full_fwd(cpu(8, 4, 64, dtype=bad), cpu(8, 64, dtype=torch.float32))


def test_non_tensors_are_refused():
    with pytest.raises(TypeError):
        binding.mhar_fwd([[1.0]], None, None)


def test_binding_has_no_library_override():
    """The product binding loads the library built next to it and nothing else
    (no environment variable can redirect it to another build)."""
    import inspect
    import os

    assert binding.LIB_PATH == os.path.join(os.path.dirname(os.path.abspath(binding.__file__)), "libattnres.so")
    assert "environ" not in inspect.getsource(binding)
