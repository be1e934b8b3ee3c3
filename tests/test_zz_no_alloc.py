"""The quantization entry point that allocates nothing
(rtv_quant_fp8_per_tensor_static, its workspace in the library's static device
array) against the one with a caller workspace, through the C ABI: codes and
scale bit-identical on two calls in a row, the second with a smaller input
(the array keeps the first call's words, which the second must not use)."""
import numpy as np
import pytest
import torch

from workloads.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _run_both(abi, x_bits: np.ndarray):
    n = x_bits.size
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    stream = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(abi.lib.rtv_quant_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    codes_ref = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    scale_ref = torch.empty(1, dtype=torch.float32, device="cuda")
    abi.rtv_quant_fp8_per_tensor(x.data_ptr(), n, codes_ref.data_ptr(), scale_ref.data_ptr(), ws.data_ptr(), stream)
    codes = torch.full((max(n, 1),), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    abi.rtv_quant_fp8_per_tensor_static(x.data_ptr(), n, codes.data_ptr(), scale.data_ptr(), stream)
    torch.cuda.synchronize()
    return (codes_ref[:n].cpu().numpy(), scale_ref.cpu().numpy(), codes[:n].cpu().numpy(), scale.cpu().numpy())


def test_static_workspace_quantization_matches(rtv_lib):
    abi = rtv_lib.abi
    rng = np.random.default_rng(41)
    # first a large input with a large amax (fills every partial word), then a
    # smaller one whose amax is far below the first's: a stale word would move
    # its scale
    big = rng.standard_normal(4_000_003).astype(np.float32) * np.float32(50.0)
    small = rng.standard_normal(70_001).astype(np.float32)
    for label, x in (("large", big), ("smaller", small)):
        bits = f32_to_bf16_bits(x)
        cr, sr, c, s = _run_both(abi, bits)
        print(f"no-alloc quantization {label}: n={bits.size} scale={s[0]!r} ref={sr[0]!r}", flush=True)
        assert s.view(np.uint32)[0] == sr.view(np.uint32)[0]
        assert np.array_equal(c, cr)
    with pytest.raises(rtv_lib.RtvError) as e:
        abi.rtv_quant_fp8_per_tensor_static(0, -1, 0, 0, 0)
    assert e.value.status == abi.RTV_ERR_INVALID_ARG
