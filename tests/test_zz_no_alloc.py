"""qs_moe_decode_static -- the decode call whose scratch lives in the
library's static device array -- against qs_moe_decode, through the C ABI:
two calls in a row (the second with a smaller batch, so a different kernel
and a smaller carve of the same array) must give bitwise the same outputs,
ids and weights as the allocating entry point, and a batch whose scratch does
not fit the array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import check_layer, make_handle, say, workload

pytestmark = pytest.mark.gpu


def _pair(lib, moe, wl, T, L, batch):
    x = torch.from_numpy(synth.tokens(wl, T, batch)).cuda()
    outs = []
    for fn in (lib.qs_moe_decode, lib.qs_moe_decode_static):
        y = torch.empty_like(x)
        ids = torch.empty((L, T, wl.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((L, T, wl.top_k), dtype=torch.float32, device="cuda")
        fn(moe.h, 0, L, x, y, T, lib.QS_DECODE_RESIDUAL | lib.QS_DECODE_RMSNORM, ids, w)
        outs.append((y, ids, w))
    moe.sync_status()
    (y0, i0, w0), (y1, i1, w1) = outs
    assert torch.equal(i0, i1), f"T={T}: expert ids differ"
    assert torch.equal(w0, w1), f"T={T}: router weights differ"
    assert torch.equal(y0, y1), f"T={T}: outputs differ"
    return x, y1, i1


@pytest.mark.parametrize("name,L,Ts", [("a3b_stack40_zipf", 3, (64, 4)), ("tiny_q2k", 1, (16, 1)),
                                       ("a3b_stack40_zipf", 2, (4, 1))])
def test_static_scratch_matches_decode(lib, name, L, Ts):
    wl = workload(name)
    moe, lws = make_handle(lib, wl, n_layers=L, max_tokens=max(Ts))
    with moe:
        for i, T in enumerate(Ts):
            say(f"static scratch {name} L={L} T={T} (call {i + 1} of {len(Ts)})")
            x, y, ids = _pair(lib, moe, wl, T, L, 20 + i)
            if L == 1:   # and to the oracle's bar
                check_layer(wl, lws[0], x.cpu().numpy(), y.cpu().numpy(), ids[0].cpu().numpy(),
                            residual=True, prenorm=True, label=f"static {name} T={T}")


def test_static_scratch_refuses_oversize(lib):
    """The large-layer shape at 64 tokens needs more scratch than the static
    array holds: QS_E_UNSUPPORTED, nothing enqueued; 8 tokens fit."""
    wl = workload("flash_stack8_zipf")
    moe, _ = make_handle(lib, wl, n_layers=1, max_tokens=64)
    with moe:
        say("static scratch flash T=64 (refused) and T=8")
        x = torch.from_numpy(synth.tokens(wl, 64, 1)).cuda()
        y = torch.empty_like(x)
        rc = lib.LIB.qs_moe_decode_static(moe.h, 0, 1, x.data_ptr(), y.data_ptr(), 64, 0, None, None,
                                          torch.cuda.current_stream().cuda_stream)
        assert rc == lib.QS_E_UNSUPPORTED
        _pair(lib, moe, wl, 8, 1, 3)
