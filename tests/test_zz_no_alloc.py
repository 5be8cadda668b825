"""mla_dsa_decode_noalloc (the decode step on the library's static scratch, for callers that cannot
allocate) against mla_dsa_decode with a caller workspace: two calls in a row on the same GPU, the
second with a smaller input, each equal to the workspace call bit for bit (scores, sel, nsel, out)."""
import math

import numpy as np
import pytest

from mla_latent_kv_dsa_amd import synth
from tests.helpers import dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_dsa_amd as mla  # noqa: E402


def _case(seed, B, T, seq_len):
    d = synth.decode(seed, T, B=B, dsa=True)
    kv = mla.KvCache(dev_bf16(d.lc), dev_bf16(d.rc), dev(d.ic), seq_len=dev(np.asarray(seq_len, np.int32)),
                     max_seq_len=T, seq_stride=T)
    args = (dev_bf16(d.q_nope), dev_bf16(d.q_rope), dev(d.q_idx), dev(d.w_idx), dev_bf16(d.kv_b), kv)
    return d, args


def _compare(args, T, k, sm):
    ref = [host(x) for x in mla.mla_dsa_decode(*args, T, k, sm)]
    got = [host(x) for x in mla.mla_dsa_decode(*args, T, k, sm, noalloc=True)]
    torch.cuda.synchronize()
    assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))   # scores
    assert np.array_equal(got[2], ref[2]) and np.array_equal(got[3], ref[3])  # sel, nsel
    assert np.array_equal(got[0].view(np.uint32), ref[0].view(np.uint32))   # out
    return got


def test_noalloc_decode_equals_workspace_call_twice():
    sm = 1.0 / math.sqrt(synth.QK_NOPE + synth.QK_ROPE)
    log("noalloc: B=3 T=20000 k=2048")
    d, args = _case(400, 3, 20000, [20000, 13001, 1500])
    got = _compare(args, 20000, 2048, sm)
    assert int(got[3][2]) == 1500
    log("noalloc: smaller input B=1 T=3000 k=512")
    d, args = _case(401, 1, 3000, [3000])
    got = _compare(args, 3000, 512, sm)
    assert int(got[3][0]) == 512
