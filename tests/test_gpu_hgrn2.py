"""GPU parity of the expanded-state recurrence (mmf_hgrn2_scan_fwd) against oracle.hgrn2_scan.

Both forms (step-wise; chunked, for heads of 64 and 128). Shapes cover every head width, sequence
lengths that leave a ragged last chunk of tokens, grids that are and are not whole rounds of the
eight XCDs, the decode step (one token, the state read and written in place), saturated gates and
the full prefill shape of the benchmark (16 x 2048 tokens, d = 2048, heads of 128), checked on
sampled heads.
"""
import numpy as np
import pytest

import oracle
from ternary_weight_matmul_amd import synth
from parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def _mmf():
    import ternary_weight_matmul_amd as mmf
    return mmf


def _state(b, d, e, seed):
    return synth.activations((b, d // e, e, e), seed)


CASES = [
    (1, 1, 16, 16, False),
    (2, 37, 256, 64, True),
    (3, 50, 96, 32, True),
    (1, 300, 256, 16, False),
    (2, 129, 512, 128, True),
    (5, 17, 384, 128, True),     # 60 workgroups: not a whole round of XCDs
    (8, 33, 1024, 128, True),    # 256 workgroups: dealt by XCD
    (2, 1, 128, 64, True),       # one token: a single, partial chunk
    (1, 16, 128, 128, False),    # exactly one chunk
]


@pytest.mark.parametrize("mode", ["recurrent", "chunk"])
@pytest.mark.parametrize("b,t,d,e,with_s0", CASES)
def test_hgrn2_parity(gpu, b, t, d, e, with_s0, mode):
    import torch
    mmf = _mmf()
    if mode == "chunk" and e < 64:
        pytest.skip("the chunked form takes heads of 64 or 128")
    f, i, o = synth.hgrn2_inputs(b, t, d, 900 + t + d + e)
    s0 = _state(b, d, e, 901 + e) if with_s0 else None
    s_last = torch.empty((b, d // e, e, e), device=gpu)
    y = mmf.hgrn2_scan_fwd(dev(f, gpu), dev(i, gpu), dev(o, gpu), e, dev(s0, gpu) if with_s0 else None,
                           s_last=s_last, mode=mode)
    assert mmf.last_path() == ("hgrn2_chunk<%d>" if mode == "chunk" else "hgrn2_scan<%d>") % e
    ry, rs = oracle.hgrn2_scan(f, i, o, e, s0)
    assert_close(host(y), ry, 1e-4, "y")
    assert_close(host(s_last), rs, 1e-4, "s_last")


def test_hgrn2_token_steps_match_one_call(gpu):
    """Step-wise form: t calls of one token, the state updated in place, give the bits of one call
    over t tokens."""
    import torch
    mmf = _mmf()
    b, t, d, e = 4, 21, 512, 128
    f, i, o = synth.hgrn2_inputs(b, t, d, 910)
    s0 = dev(_state(b, d, e, 911), gpu)
    fd, idv, od = dev(f, gpu), dev(i, gpu), dev(o, gpu)
    s_whole = torch.empty_like(s0)
    y = mmf.hgrn2_scan_fwd(fd, idv, od, e, s0, s_last=s_whole, mode="recurrent")
    st = s0.clone()
    for k in range(t):
        yk = mmf.hgrn2_scan_fwd(fd[:, k:k + 1].contiguous(), idv[:, k:k + 1].contiguous(),
                                od[:, k:k + 1].contiguous(), e, st, s_last=st, mode="recurrent")
        assert torch.equal(yk[:, 0], y[:, k]), k
    assert torch.equal(st, s_whole)


def test_hgrn2_empty_and_zero_state(gpu):
    import torch
    mmf = _mmf()
    b, d, e = 3, 256, 64
    s0 = dev(_state(b, d, e, 912), gpu)
    s_last = torch.full_like(s0, 7.0)
    empty = torch.empty((b, 0, d), device=gpu)
    mmf.hgrn2_scan_fwd(empty, empty, empty, e, s0, s_last=s_last)
    assert torch.equal(s_last, s0)
    mmf.hgrn2_scan_fwd(empty, empty, empty, e, None, s_last=s_last)
    assert not s_last.any()
    f, i, o = synth.hgrn2_inputs(b, 5, d, 913)
    y = mmf.hgrn2_scan_fwd(dev(f, gpu), dev(i, gpu), dev(o, gpu), e, None, s_last=s_last)
    ry, rs = oracle.hgrn2_scan(f, i, o, e)
    assert_close(host(y), ry, 1e-4, "y from zeros")
    assert_close(host(s_last), rs, 1e-4, "s_last from zeros")


def test_hgrn2_decode_step_full_width(gpu):
    """The decode shape: 16 sequences, d = 2048, heads of 128, one token, the state in place."""
    mmf = _mmf()
    b, d, e = 16, 2048, 128
    f, i, o = synth.hgrn2_inputs(b, 1, d, 914)
    s0 = _state(b, d, e, 915)
    st = dev(s0, gpu)
    y = mmf.hgrn2_scan_fwd(dev(f, gpu), dev(i, gpu), dev(o, gpu), e, st, s_last=st)
    ry, rs = oracle.hgrn2_scan(f, i, o, e, s0)
    assert_close(host(y), ry, 1e-4, "y")
    assert_close(host(st), rs, 1e-4, "state")


@pytest.mark.parametrize("e", [64, 128])
def test_hgrn2_chunk_saturated_gates_and_in_place(gpu, e):
    """The chunked form with gates of exactly 0 and 1 and with the state updated in place,
    against the oracle. Chunks 0 and 2 hold zero gates (their A and K^ come from running
    products, by the workgroup's vote), chunk 1 has gates of 1 on half the channels, the
    others are ordinary (A = Q~ K~^T): both paths alternate within one sequence."""
    mmf = _mmf()
    b, t, d = 2, 70, 256
    f, i, o = synth.hgrn2_inputs(b, t, d, 918)
    f = f.copy()
    f[:, 5:9] = 0.0
    f[:, 20:40, :64] = 1.0
    f[:, 41] = 0.0
    s0 = _state(b, d, e, 919)
    st = dev(s0, gpu)
    y = mmf.hgrn2_scan_fwd(dev(f, gpu), dev(i, gpu), dev(o, gpu), e, st, s_last=st, mode="chunk")
    assert mmf.last_path() == "hgrn2_chunk<%d>" % e
    ry, rs = oracle.hgrn2_scan(f, i, o, e, s0)
    assert_close(host(y), ry, 1e-4, "y")
    assert_close(host(st), rs, 1e-4, "state")


@pytest.mark.timeout(600)
def test_hgrn2_full_size_sampled(gpu):
    """16 x 2048 tokens, d = 2048, heads of 128 (the launch the benchmark times: the chunked form),
    and the step-wise form on the same inputs, checked on sampled (sequence, head) pairs against
    the oracle run on those heads alone."""
    import torch
    mmf = _mmf()
    b, t, d, e = 16, 2048, 2048, 128
    f, i, o = synth.hgrn2_inputs(b, t, d, 916)
    s0 = _state(b, d, e, 917)
    fd, idv, od, sd = dev(f, gpu), dev(i, gpu), dev(o, gpu), dev(s0, gpu)
    runs = {}
    for mode in ("auto", "recurrent"):
        s_last = torch.empty((b, d // e, e, e), device=gpu)
        y = mmf.hgrn2_scan_fwd(fd, idv, od, e, sd, s_last=s_last, mode=mode)
        runs[mode] = (mmf.last_path(), host(y), host(s_last))
    assert runs["auto"][0] == "hgrn2_chunk<128>" and runs["recurrent"][0] == "hgrn2_scan<128>"
    for bi, n in ((0, 0), (7, 9), (15, 15), (3, 4)):
        ch = slice(n * e, (n + 1) * e)
        ry, rs = oracle.hgrn2_scan(f[bi:bi + 1, :, ch], i[bi:bi + 1, :, ch], o[bi:bi + 1, :, ch], e,
                                   s0[bi:bi + 1, n:n + 1])
        for mode, (_, y, sl) in runs.items():
            assert_close(y[bi:bi + 1, :, ch], ry, 1e-4, "%s y (%d, %d)" % (mode, bi, n))
            assert_close(sl[bi:bi + 1, n:n + 1], rs, 1e-4, "%s s_last (%d, %d)" % (mode, bi, n))
