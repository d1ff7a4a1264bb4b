"""The torch wrappers reject operands they cannot describe to the C ABI, on
the host, before anything is launched: an operand whose rows overlap (row
stride below the row length, e.g. an expanded view with row stride 0), an
`out` of the wrong shape, and tensors on different devices.  A rejected
call leaves `out` untouched."""

from __future__ import annotations

import pytest

import dense_fp32_tiled_amd as dft

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu(gemm_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _wrappers(torch):
    f32 = (torch.float32, lambda a, b, out: dft.matmul(a, b, out=out))
    sk = (torch.float32, lambda a, b, out: dft.matmul_splitk(a, b, out=out, splits=2))
    bf = (torch.bfloat16, lambda a, b, out: dft.matmul_mixed(a, b, out=out))
    return {"matmul": f32, "matmul_splitk": sk, "matmul_mixed": bf}


@pytest.mark.parametrize("which", ["matmul", "matmul_splitk", "matmul_mixed"])
def test_overlapping_rows_are_rejected(torch_gpu, which):
    torch = torch_gpu
    dtype, fn = _wrappers(torch)[which]
    row = torch.ones((1, 64), dtype=dtype, device="cuda")
    b = torch.ones((64, 32), dtype=dtype, device="cuda")
    expanded = row.expand(48, 64)  # row stride 0
    assert expanded.stride(0) == 0
    out = torch.full((48, 32), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="overlapping rows"):
        fn(expanded, b, out)
    a = torch.ones((48, 64), dtype=dtype, device="cuda")
    with pytest.raises(ValueError, match="overlapping rows"):
        fn(a, torch.ones((1, 32), dtype=dtype, device="cuda").expand(64, 32), out)
    # rows that overlap partly: a strided view with row stride 16 < 64 columns
    base = torch.ones(48 * 16 + 64, dtype=dtype, device="cuda")
    partly = base.as_strided((48, 64), (16, 1))
    with pytest.raises(ValueError, match="overlapping rows"):
        fn(partly, b, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("which", ["matmul", "matmul_splitk", "matmul_mixed"])
def test_out_of_the_wrong_shape_is_rejected(torch_gpu, which):
    torch = torch_gpu
    dtype, fn = _wrappers(torch)[which]
    a = torch.ones((48, 64), dtype=dtype, device="cuda")
    b = torch.ones((64, 32), dtype=dtype, device="cuda")
    for shape in [(1, 64), (48, 16), (96, 32), (32, 48)]:
        out = torch.full(shape, 7.0, dtype=torch.float32, device="cuda")
        with pytest.raises(ValueError, match="out has shape"):
            fn(a, b, out)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())


@pytest.mark.parametrize("which", ["matmul", "matmul_splitk", "matmul_mixed"])
def test_operands_off_the_gpu_are_rejected(torch_gpu, which):
    torch = torch_gpu
    dtype, fn = _wrappers(torch)[which]
    a = torch.ones((48, 64), dtype=dtype, device="cuda")
    b = torch.ones((64, 32), dtype=dtype, device="cuda")
    with pytest.raises(ValueError, match="GPU device"):
        fn(a, b.cpu(), None)
    with pytest.raises(ValueError, match="GPU device"):
        fn(a, b, torch.empty((48, 32), dtype=torch.float32))


def test_row_pitch_above_the_width_is_accepted(torch_gpu):
    """A column slice keeps its parent's row pitch; the wrappers pass it on."""
    import oracle
    import workloads

    torch = torch_gpu
    a_np, b_np = workloads.make_operands(48, 40, 80, "uniform", 5)
    big_a = torch.from_numpy(a_np).cuda()
    big_b = torch.from_numpy(b_np).cuda()
    a, b = big_a[:, :64], big_b[:64, :32]
    assert a.stride(0) == 80 and b.stride(0) == 40
    c = dft.matmul(a, b)
    torch.cuda.synchronize()
    cref, den = oracle.reference(a_np[:, :64].copy(), b_np[:64, :32].copy())
    assert oracle.normalised_error(c.cpu().numpy(), cref, den) <= 1e-5
