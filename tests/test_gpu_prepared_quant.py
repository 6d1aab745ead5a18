"""The prepared argmax calls over quantized heads (PreparedArgmaxFp8,
PreparedArgmaxMxfp4, PreparedArgmaxNvfp4): checked once, then one C call
per step.  Each step must equal the plain binding's call on the same buffers
bit for bit, follow hidden rows rewritten in place, and reject what the plain
call rejects at construction.  The plain calls meet the parity rule against
the oracle in the format tests; this checks the binding, through the C ABI."""
import numpy as np
import pytest

import synth
from devcopy import dev_bf16, dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def _heads(L, r, k):
    w = dev_bf16(synth.normal_bf16(71, r, k, 0.02))
    fp8 = L.lmhead_quantize_fp8(w)
    mx = L.lmhead_quantize_mxfp4(w)
    nv = L.lmhead_quantize_nvfp4(w)
    torch.cuda.synchronize()
    return fp8, mx, nv


@pytest.mark.parametrize("m,r", [(1, 3000), (3, 16000), (24, 5000)])
def test_prepared_quantized_equal_plain_calls(L, m, r):
    k = 2560
    (q8, s8), (q4, s4), (qn, sn, gn) = _heads(L, r, k)
    d2t = dev_i32((np.arange(r, dtype=np.int32) * 3 + 7))
    h = dev_bf16(synth.hidden(72, 0, m, k))
    preps = [
        (L.PreparedArgmaxFp8(h, q8, s8, d2t), lambda: L.draft_project_argmax_fp8(h, q8, s8, d2t)),
        (L.PreparedArgmaxMxfp4(h, q4, s4, d2t), lambda: L.draft_project_argmax_mxfp4(h, q4, s4, d2t)),
        (L.PreparedArgmaxNvfp4(h, qn, sn, gn, d2t), lambda: L.draft_project_argmax_nvfp4(h, qn, sn, gn, d2t)),
    ]
    for draw in range(3):
        h.copy_(dev_bf16(synth.hidden(72, draw, m, k)))      # rewritten in place
        for prep, plain in preps:
            i, lg = prep()
            pi, pl = plain()
            assert torch.equal(i, pi), draw
            assert torch.equal(lg.view(torch.int32), pl.view(torch.int32)), draw


def test_prepared_quantized_reject_at_construction(L):
    k, r = 512, 100
    (q8, s8), (q4, s4), (qn, sn, gn) = _heads(L, r, k)
    h = dev_bf16(synth.hidden(73, 0, 2, k))
    bad_h = h.float()
    with pytest.raises((ValueError, TypeError)):
        L.PreparedArgmaxFp8(bad_h, q8, s8)
    with pytest.raises((ValueError, TypeError)):
        L.PreparedArgmaxMxfp4(bad_h, q4, s4)
    with pytest.raises((ValueError, TypeError)):
        L.PreparedArgmaxNvfp4(bad_h, qn, sn, gn)
    with pytest.raises((ValueError, TypeError)):
        L.PreparedArgmaxFp8(h, q8, s8, dev_i32(np.arange(r + 1, dtype=np.int32)))
