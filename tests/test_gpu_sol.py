"""The speed-of-light reference kernels (sv_sol_read, sv_sol_read_write) do
what their declarations say: the read writes its sink only for the marker
value, the read-write stores a - b in fp32 for every element, tails
included.  Their figures are only meaningful if they move the stated bytes."""
import numpy as np
import pytest

from parity import to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import speculative_decoding_verification_amd as sv

    sv.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("nbytes", [16, 8192, 8192 * 3 + 48, 41_326_592])
def test_sol_read_leaves_sink_for_ordinary_data(dev, nbytes):
    import torch

    import speculative_decoding_verification_amd as sv

    print("sol_read bytes", nbytes, flush=True)
    data = torch.full((nbytes // 4,), 0x3c003c00, dtype=torch.int32, device=dev)
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    sv.sol_read(data, sink)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


def test_sol_read_reaches_every_slab(dev):
    """A marker slab anywhere in the buffer (here the ragged last one) sets
    the sink: the loads are issued over the whole range."""
    import torch

    import speculative_decoding_verification_amd as sv

    n_words = (8192 * 5 + 64) // 4
    host = np.zeros(n_words, dtype=np.uint32)
    host[-4] = 0x9E3779B9  # the XOR of the words the last lane with data loads
    data = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    sv.sol_read(data, sink)
    torch.cuda.synchronize()
    assert np.uint32(sink.cpu().numpy()[0]) == np.uint32(0x9E3779B9)


@pytest.mark.parametrize("dtype,n", [("f32", 4), ("f32", 2048 * 5 + 12), ("bf16", 8), ("bf16", 4096 * 3 + 72),
                                     ("bf16", 151936 * 7)])
def test_sol_read_write_is_a_minus_b(dev, dtype, n):
    import torch

    import speculative_decoding_verification_amd as sv
    import workloads

    print("sol_read_write", dtype, n, flush=True)
    rng = np.random.default_rng(n)
    a = rng.standard_normal(n).astype(np.float32) * 4
    b = rng.standard_normal(n).astype(np.float32) * 4
    if dtype == "bf16":
        a = workloads.round_to_bf16_bits(a)
        b = workloads.round_to_bf16_bits(b)
        want = workloads.bf16_bits_to_f32(a).astype(np.float64) - workloads.bf16_bits_to_f32(b)
    else:
        want = a.astype(np.float64) - b
    out = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    sv.sol_read_write(to_torch(a, dev), to_torch(b, dev), out)
    torch.cuda.synchronize()
    # one fp32 subtraction of exactly representable operands: correctly rounded
    assert np.array_equal(out.cpu().numpy(), want.astype(np.float32))
