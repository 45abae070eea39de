"""mmf_layer_decode_step_noalloc through the C ABI against mmf_layer_decode_step, which it
must reproduce bit for bit (same kernels, workspace in the library's own device array): two
calls in a row, the second with a smaller batch, so the second call runs over scratch the
first one left behind."""
import ctypes

import numpy as np
import pytest

from ternary_weight_matmul_amd import synth
from parity import bf16_tensor, dev, make_pair

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, P, x, h, out):
    import torch
    from ternary_weight_matmul_amd.binding import _dtype_code, _ptr
    cw = P.c()
    st = lib.mmf_layer_decode_step_noalloc(ctypes.byref(cw), _ptr(x), _ptr(out), _dtype_code(x.dtype), x.shape[0],
                                           _ptr(h), None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.mmf_last_error()


@pytest.mark.parametrize("d,inner,batches,act", [(2048, 5632, (16, 3), "bf16"), (2048, 5632, (64, 1), "bf16"),
                                                  (1024, 2816, (12, 5), "f32")])
def test_noalloc_decode_matches_workspace_decode(gpu, d, inner, batches, act):
    import torch
    import ternary_weight_matmul_amd as mmf
    lib = mmf.load()
    _, P = make_pair(d, inner, 4100 + d + batches[0], gpu)
    for i, b in enumerate(batches):
        xs = synth.activations((b, d), 4200 + 10 * i + b, act)
        x = bf16_tensor(xs, gpu) if act == "bf16" else dev(xs, gpu)
        h0 = dev(synth.activations((b, d), 4300 + 10 * i + b), gpu)
        h_ref = h0.clone()
        out_ref = mmf.layer_decode_step(P, x, h_ref)
        path_ref = mmf.last_path()
        h = h0.clone()
        out = torch.empty_like(x)
        _call_noalloc(lib, P, x, h, out)
        torch.cuda.synchronize()
        assert mmf.last_path() == path_ref, (mmf.last_path(), path_ref)
        assert torch.equal(out, out_ref), (b, "out")
        assert torch.equal(h, h_ref), (b, "h")


def test_noalloc_decode_rejects_what_does_not_fit(gpu):
    import torch
    import ternary_weight_matmul_amd as mmf
    _, P = make_pair(2048, 5632, 4400, gpu)
    b = 512
    x = torch.zeros((b, 2048), dtype=torch.bfloat16, device=gpu)
    h = torch.zeros((b, 2048), dtype=torch.float32, device=gpu)
    with pytest.raises(mmf.MMFError) as ei:
        mmf.layer_decode_step_noalloc(P, x, h, torch.empty_like(x))
    assert ei.value.status == 3 and "scratch" in str(ei.value)
