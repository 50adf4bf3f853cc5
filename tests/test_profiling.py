"""Host logic of the profile summaries: demangled kernel names map to the
library's timing names, with and without the chain kernels' wave count."""

import pytest

from gated_delta_rule_54_amd import profiling


@pytest.mark.parametrize("name,want", [
    ("void chain16_kernel<64, unsigned short, true, false>(K16)", "chunk_fwd"),
    ("void chain16_kernel<64, unsigned short, true, false, 4>(K16)", "chunk_fwd"),
    ("void chain16_kernel<64, float, true, true, 2>(K16)", "chunk_fwd_save"),
    ("void chain16_kernel<32, unsigned short, false, true, 1>(K16)", "chunk_states"),
    ("void cwchain16_kernel<64, unsigned short, true, false, 1>(K16)", "chunk_fwd_cw"),
    ("void cwchain16_kernel<64, unsigned short, false, true, 4>(K16)", "chunk_states_cw"),
    ("void dh16_kernel<64, unsigned short, 4>(K16)", "chunk_dh"),
    ("void cwdh16_kernel<64, unsigned short, 2>(K16)", "chunk_dh_cw"),
    ("void grad16_kernel<64, unsigned short, 2>(K16)", "chunk_grad"),
    ("void cwgrad16_kernel<64, unsigned short>(K16)", "chunk_grad_cw"),
    ("void prep16_kernel<64>(K16)", "chunk_prep"),
    ("void cwprep16_kernel<64>(K16)", "chunk_prep_cw"),
    ("void decode_kernel<unsigned short, unsigned short, false, 2, 32>(Dims, gdr::SeqFwdArgs)", "decode"),
    ("void calib_copy_kernel(float4 const*, float4*, long)", "copy"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", None),
])
def test_label(name, want):
    assert profiling.label(name) == want
