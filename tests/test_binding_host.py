"""Host-side checks of the Python binding that need no GPU: host tensors,
wrong dtypes and malformed output tuples are rejected with ValueError before
the library is asked to launch anything (a host pointer reaching a kernel
would fault the device)."""
import pytest
import torch

import mx9_dual_axis_amd as mxq


def _raises_value_error(fn):
    with pytest.raises(ValueError) as e:
        fn()
    assert not isinstance(e.value, mxq.MXError)


def test_host_inputs_rejected():
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    _raises_value_error(lambda: mxq.mx_quantize_2d_dual(x))
    _raises_value_error(lambda: mxq.mx_quantize_grouped(x, torch.zeros(1, dtype=torch.int32)))
    _raises_value_error(lambda: mxq.mx9_pack(torch.zeros((4, 16))))
    _raises_value_error(lambda: mxq.mx9_pack_axis(torch.zeros((4, 16)), 0))
    _raises_value_error(lambda: mxq.mx9_pack_records(torch.zeros((4, 16))))
    q = torch.zeros((4, 16), dtype=torch.int8)
    e = torch.zeros(4, dtype=torch.uint8)
    _raises_value_error(lambda: mxq.mx9_unpack(q, e, e, 4, 16))
    _raises_value_error(lambda: mxq.mx9_unpack_axis(q, e, e, (4, 16), 0))
    _raises_value_error(lambda: mxq.mx9_unpack_records(torch.zeros((4, 18), dtype=torch.uint8), (4, 16)))
    a = torch.zeros((128, 128), dtype=torch.uint8)
    s = torch.zeros((128, 4), dtype=torch.uint8)
    _raises_value_error(lambda: mxq.mx_gemm_nt(a, s, a, s))
    _raises_value_error(lambda: mxq.scales_to_mfma(s))


def test_output_check_helper():
    dev = torch.device("cuda:0")
    host = torch.zeros((4, 16), dtype=torch.int8)
    # a host tensor is never accepted as an output of a device call
    _raises_value_error(lambda: mxq._check_out(host, "q", (4, 16), torch.int8, dev))
    _raises_value_error(lambda: mxq._out_tuple((host, host), 3, "q, max_exp, prime"))
    _raises_value_error(lambda: mxq._out_tuple(host, 3, "q, max_exp, prime"))
