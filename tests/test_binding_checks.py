"""The Python binding's checks of caller-supplied buffers, on the CPU.

The C-ABI sees only addresses, so the binding is the one place where a wrong buffer
(host memory, another GPU, too small, wrong dtype or layout) can be caught before a
kernel would read or write out of bounds.  These tests feed the checks stand-in
objects that look like GPU tensors; nothing is launched.
"""
import pytest

torch = pytest.importorskip("torch")

from flashattention_tiling_online_amd import binding  # noqa: E402


class FakeGpuTensor:
    """Just the attributes the checks read."""

    def __init__(self, shape, dtype=torch.bfloat16, device="cuda:0", contiguous=True,
                 cuda=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device) if cuda else torch.device("cpu")
        self.is_cuda = cuda
        self._contig = contiguous

    def is_contiguous(self):
        return self._contig

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()


DEV = torch.device("cuda:0")


def test_buffer_accepts_matching_tensor():
    t = FakeGpuTensor((2, 3, 5, 64))
    assert binding._check_buf("o", t, (2, 3, 5, 64), torch.bfloat16, DEV) is t


@pytest.mark.parametrize("kw,exc", [
    (dict(cuda=False), ValueError),                      # host memory
    (dict(device="cuda:1"), ValueError),                 # another GPU
    (dict(contiguous=False), ValueError),                # strided view
    (dict(dtype=torch.float16), TypeError),              # wrong element type
    (dict(shape=(2, 3, 4, 64)), ValueError),             # too few rows
    (dict(shape=(2, 3, 5, 128)), ValueError),            # wrong head size
])
def test_buffer_rejects(kw, exc):
    args = dict(shape=(2, 3, 5, 64))
    args.update(kw)
    t = FakeGpuTensor(args.pop("shape"), **args)
    with pytest.raises(exc):
        binding._check_buf("o", t, (2, 3, 5, 64), torch.bfloat16, DEV)


def test_lse_must_be_fp32():
    with pytest.raises(TypeError):
        binding._check_buf("lse", FakeGpuTensor((2, 3, 5), dtype=torch.bfloat16), (2, 3, 5),
                           torch.float32, DEV)


def test_workspace_size_and_placement():
    ok = FakeGpuTensor((4096,), dtype=torch.uint8)
    assert binding._check_workspace(ok, 4096, DEV) is ok
    with pytest.raises(ValueError):
        binding._check_workspace(FakeGpuTensor((4095,), dtype=torch.uint8), 4096, DEV)
    with pytest.raises(ValueError):
        binding._check_workspace(FakeGpuTensor((4096,), dtype=torch.uint8, cuda=False), 16, DEV)
    with pytest.raises(ValueError):
        binding._check_workspace(FakeGpuTensor((4096,), dtype=torch.uint8, contiguous=False),
                                 16, DEV)
    # a float32 workspace counts bytes, not elements
    assert binding._check_workspace(FakeGpuTensor((1024,), dtype=torch.float32), 4096, DEV)


def test_qkv_checks_reject_host_and_mixed_devices():
    q = FakeGpuTensor((1, 2, 8, 64))
    k = FakeGpuTensor((1, 2, 8, 64))
    with pytest.raises(ValueError):
        binding._check_qkv(q, k, FakeGpuTensor((1, 2, 8, 64), cuda=False))
    with pytest.raises(ValueError):
        binding._check_qkv(q, k, FakeGpuTensor((1, 2, 8, 64), device="cuda:1"))
    with pytest.raises(ValueError):
        binding._check_qkv(q, k, FakeGpuTensor((1, 2, 9, 64)))
    assert binding._check_qkv(q, k, FakeGpuTensor((1, 2, 8, 64))) == (1, 2, 8, 8, 64)


def test_public_calls_reject_before_launch():
    """fa_bwd with a host-memory lse raises in the binding (no library call is made)."""
    q = FakeGpuTensor((1, 2, 8, 64))
    with pytest.raises(ValueError):
        binding._bwd_buffers(q, q, q, q, FakeGpuTensor((1, 2, 8), dtype=torch.float32, cuda=False),
                             q, None, None, None, None, None)
    with pytest.raises(ValueError):
        binding._bwd_buffers(q, q, q, FakeGpuTensor((1, 2, 7, 64)),
                             FakeGpuTensor((1, 2, 8), dtype=torch.float32), q, None, None, None,
                             None, None)
