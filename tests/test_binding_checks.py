"""The Python binding rejects, before any call into the library, every tensor the C ABI could
not check itself (it receives bare pointers): a CPU tensor where device memory is expected,
a wrong shape or dtype, a non-contiguous tensor.  These run without a GPU: a CPU tensor
fails the first check of every entry point."""
import pytest

torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402


def cpu(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


CASES = {
    "la_fwd": lambda: la.la_fwd(cpu(1, 2, 8, 16), cpu(1, 2, 8, 16), cpu(1, 2, 8, 16), [0.5, 0.5]),
    "la_bwd": lambda: la.la_bwd(*(cpu(1, 2, 8, 16) for _ in range(4)), [0.5, 0.5]),
    "la_dlam": lambda: la.la_dlam(*(cpu(1, 2, 8, 16) for _ in range(4)), [0.5, 0.5]),
    "la_fwd_varlen": lambda: la.la_fwd_varlen(cpu(8, 2, 128), cpu(8, 2, 128), cpu(8, 2, 128), [0.5, 0.5],
                                              [0, 3, 8]),
    "la_decode_step": lambda: la.la_decode_step(cpu(1, 2, 16, 16, dtype=torch.float32), cpu(1, 2, 16),
                                                cpu(1, 2, 16), cpu(1, 2, 16), [0.5, 0.5]),
    "la_decode_step_paged": lambda: la.la_decode_step_paged(
        cpu(4, 2, 16, 16, dtype=torch.float32), torch.zeros(1, dtype=torch.int32), cpu(1, 2, 16),
        cpu(1, 2, 16), cpu(1, 2, 16), [0.5, 0.5]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_cpu_tensors_rejected(name):
    with pytest.raises(ValueError, match="GPU tensor"):
        CASES[name]()


def test_wrong_rank_and_dtype_rejected():
    with pytest.raises(ValueError, match="dimensions"):
        la.la_fwd(cpu(2, 8, 16), cpu(2, 8, 16), cpu(2, 8, 16), [0.5, 0.5])
    with pytest.raises(TypeError):
        la.la_fwd("q", "k", "v", [0.5])
    with pytest.raises(ValueError):
        la.la_decode_step_paged(cpu(4, 2, 16), torch.zeros(1, dtype=torch.int32), cpu(1, 2, 16),
                                cpu(1, 2, 16), cpu(1, 2, 16), [0.5, 0.5])
