"""The Python binding refuses, on the host, device buffers that are shorter
than what the call touches, or scalar buffers of the wrong dtype, before
anything reaches the library: a short buffer would otherwise be overrun by
the kernels.  No GPU is needed: the stand-in tensors below carry only what
the checks read, and every case raises before the library is called."""
import pytest

torch = pytest.importorskip("torch")

import zero_sharded_mixed_partition_amd as Z  # noqa: E402


class FakeDev:
    """A device tensor as far as the binding's checks can tell."""
    is_cuda = True

    def __init__(self, numel, dtype, addr=1 << 40):
        self.dtype, self._n, self._addr = dtype, numel, addr

    def is_contiguous(self):
        return True

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def data_ptr(self):
        return self._addr


class FakeState:
    def ptr(self):
        return 1 << 41


N = 1000
F16, BF16, F32, F64, I32 = torch.float16, torch.bfloat16, torch.float32, torch.float64, torch.int32


def shard(n=N, gdt=F16):
    return FakeDev(n, F32), FakeDev(n, F32), FakeDev(n, F32), FakeDev(n, gdt), FakeDev(n, gdt)


def ws():
    return FakeDev(Z.zero_norm_workspace_bytes(N), torch.uint8)


def coef():
    return FakeDev(Z.zero_adam_coef_bytes(), torch.uint8)


def test_norm_pass_checks():
    with pytest.raises(ValueError, match="grad"):
        Z.zero_shard_unscale_norm_overflow(FakeDev(N - 1, F16), 1.0, FakeDev(1, F64), FakeDev(1, I32), ws(),
                                           n=N, stream=0)
    with pytest.raises(ValueError, match="sqnorm"):
        Z.zero_shard_unscale_norm_overflow(FakeDev(N, F16), 1.0, FakeDev(1, F32), FakeDev(1, I32), ws(), stream=0)
    with pytest.raises(ValueError, match="overflow"):
        Z.zero_shard_unscale_norm_overflow(FakeDev(N, F16), 1.0, FakeDev(1, F64), FakeDev(1, torch.int64), ws(),
                                           stream=0)
    with pytest.raises(ValueError, match="sqnorm"):
        Z.zero_shard_unscale_norm_overflow_dev(FakeDev(N, F16), FakeState(), FakeDev(0, F64), FakeDev(1, I32),
                                               ws(), stream=0)


@pytest.mark.parametrize("short", ["master", "exp_avg", "exp_avg_sq", "grad", "param_out"])
def test_update_checks_every_stream(short):
    bufs = dict(zip(["master", "exp_avg", "exp_avg_sq", "grad", "param_out"], shard()))
    bufs[short] = FakeDev(N - 1, bufs[short].dtype)
    hp = Z.AdamHyper(max_grad_norm=1.0)
    # the state-in-device-memory update takes n from master and checks the rest
    if short != "master":
        with pytest.raises(ValueError, match=short):
            Z.zero_shard_adam_step_dev(*bufs.values(), hp, FakeState(), FakeDev(1, F64), FakeDev(1, I32), coef(),
                                       stream=0)
    # the by-value update also insists on equal lengths
    with pytest.raises(ValueError, match="differ"):
        Z.zero_shard_adam_step(*bufs.values(), hp, FakeDev(1, F64), FakeDev(1, I32), stream=0)
    with pytest.raises(ValueError, match=short):
        Z.zero_shard_adam_step_coef(*bufs.values(), coef(), FakeDev(1, F64), FakeDev(1, I32),
                                    n=N, stream=0)


def test_update_checks_scalars_and_coefficients():
    hp = Z.AdamHyper(max_grad_norm=1.0)
    with pytest.raises(ValueError, match="global_sqnorm"):
        Z.zero_shard_adam_step(*shard(), hp, FakeDev(1, F32), FakeDev(1, I32), stream=0)
    with pytest.raises(ValueError, match="global_overflow"):
        Z.zero_shard_adam_step(*shard(), hp, FakeDev(1, F64), FakeDev(1, torch.uint8), stream=0)
    with pytest.raises(ValueError, match="d_coef"):
        Z.zero_shard_adam_step_dev(*shard(), hp, FakeState(), FakeDev(1, F64), FakeDev(1, I32),
                                   FakeDev(Z.zero_adam_coef_bytes() - 1, torch.uint8), stream=0)
    with pytest.raises(ValueError, match="d_coef"):
        Z.zero_step_decide_dev(hp, Z.ZERO_F16, FakeState(), FakeDev(1, I32), FakeDev(8, torch.uint8), stream=0)
    with pytest.raises(ValueError, match="d_coef"):
        Z.zero_shard_norm_decide_dev(FakeDev(N, F16), hp, FakeState(), FakeDev(1, F64), FakeDev(1, I32),
                                     FakeDev(8, torch.uint8), ws(), stream=0)


def test_accumulate_and_reduce_checks():
    with pytest.raises(ValueError, match="acc"):
        Z.zero_shard_grad_accumulate(FakeDev(N, F32), FakeDev(N + 1, BF16), 1.0, True, n=N + 1, stream=0)
    with pytest.raises(ValueError, match="grad"):
        Z.zero_shard_grad_accumulate_dev(FakeDev(N, F32), FakeDev(N - 1, BF16), FakeState(), True, stream=0)
    slices = [FakeDev(N, F16), FakeDev(N - 1, F16), FakeDev(N, F16)]
    with pytest.raises(ValueError, match=r"slices\[1\]"):
        Z.zero_shard_grad_reduce(FakeDev(N, F32), slices, 1.0, stream=0)
    with pytest.raises(ValueError, match=r"slices\[1\]"):
        Z.zero_shard_grad_reduce_dev(FakeDev(N, F32), slices, FakeState(), stream=0)
    # an fp32 slice is read as 4 bytes per element
    with pytest.raises(ValueError, match=r"slices\[0\]"):
        Z.zero_shard_grad_sum_norm(FakeDev(N, F32), [FakeDev(N, F16)], False, 1.0, FakeDev(1, F64),
                                   FakeDev(1, I32), ws(), grad_dtype=Z.ZERO_F32, stream=0)
    with pytest.raises(ValueError, match="overflow"):
        Z.zero_shard_grad_sum_norm_dev(FakeDev(N, F32), [FakeDev(N, F16)], False, FakeState(), FakeDev(1, F64),
                                       FakeDev(1, F32), ws(), stream=0)


def test_combine_and_copy_checks():
    with pytest.raises(ValueError, match="slot_sqnorm"):
        Z.zero_norm_combine_ranks(FakeDev(8, F32), FakeDev(8, I32), FakeDev(1, F64), FakeDev(1, I32), stream=0)
    with pytest.raises(ValueError, match="global_overflow"):
        Z.zero_norm_combine_ranks(FakeDev(8, F64), FakeDev(8, I32), FakeDev(1, F64), FakeDev(0, I32), stream=0)
    with pytest.raises(ValueError, match="dst"):
        Z.zero_copy_reference(FakeDev(100, torch.uint8), FakeDev(200, torch.uint8), stream=0)


def test_recorded_steps_check_their_buffers():
    m, e, v, g, p = shard()
    with pytest.raises(ValueError, match="param_out"):
        Z.StepGraph(m, e, v, g, FakeDev(N - 1, F16), 1.0, FakeDev(1, F64), FakeDev(1, I32), ws())
    with pytest.raises(ValueError, match="sqnorm"):
        Z.StepGraphDev(m, e, v, g, p, Z.AdamHyper(), FakeState(), FakeDev(1, F32), FakeDev(1, I32), coef(), ws())
