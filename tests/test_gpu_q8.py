"""GPU parity of the 8-bit shared expert (d binary16 + 32 int8 per 32
weights) against the oracle, through the C ABI: the handle's shared matrices
dequantise bit-exactly, and decode calls of both kernels (small-batch and
batched, GEMV and MFMA items) match the oracle's layer."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import check_layer, make_handle, say, workload

pytestmark = pytest.mark.gpu

# the A3B layer with an 8-bit shared expert; a small shape whose shared width
# (192) is not a multiple of the 512-weight lane stride and whose padded
# shared rows (192 + 12 bytes -> 208) carry padding
Q8_SHAPES = {
    "a3b": dict(base="a3b_layer", shared_format="q8"),
    "tiny": dict(base="tiny_q2k", shared_ffn=192, shared_format="q8", name="tiny_q8"),
}


def _wl(key):
    kw = dict(Q8_SHAPES[key])
    return workload(kw.pop("base"), **kw)


@pytest.fixture(scope="module", params=sorted(Q8_SHAPES))
def q8(lib, request):
    wl = _wl(request.param)
    moe, lws = make_handle(lib, wl, max_tokens=64)
    yield request.param, wl, moe, lws
    moe.close()


@pytest.mark.parametrize("which", [3, 4, 5])
def test_shared_dequant_bit_exact(q8, which):
    key, wl, moe, lws = q8
    say(f"shared dequant {key} matrix {which}")
    got = moe.dequant(0, 0, which).cpu().numpy()
    raw = (lws[0].shared_gate, lws[0].shared_up, lws[0].shared_down)[which - 3]
    ref = om.dequant_matrix(raw, "q8")
    assert got.shape == ref.shape
    assert np.all(got == ref)


def test_shared_dequant_bf16(lib):
    """The bf16 shared matrices as the handle holds them widen exactly."""
    wl = workload("tiny_q2k", shared_ffn=192, name="tiny_bf16s")
    moe, lws = make_handle(lib, wl, max_tokens=4)
    with moe:
        for which in (3, 4, 5):
            say(f"shared dequant bf16 matrix {which}")
            got = moe.dequant(0, 0, which).cpu().numpy()
            raw = (lws[0].shared_gate, lws[0].shared_up, lws[0].shared_down)[which - 3]
            ref = (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
            assert np.all(got == ref)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 16, 64])
def test_decode_q8_shared(q8, T):
    key, wl, moe, lws = q8
    if key == "a3b" and T > 16:
        pytest.skip("the oracle's A3B layer at 64 tokens dequantises every expert (minutes of CPU)")
    say(f"decode {key} q8 shared T={T}")
    x = synth.tokens(wl, T, 2)
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
    y = moe.decode(torch.from_numpy(x).cuda(), ids_out=ids, w_out=w)
    moe.sync_status()
    check_layer(wl, lws[0], x, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(),
                label=f"{key} q8 T={T}")


@pytest.mark.parametrize("T", [1, 7, 32])
def test_decode_q8_shared_mfma(lib, T):
    """Every bucket on the matrix-core items (mfma_min_tokens = 1)."""
    wl = _wl("a3b")
    say(f"decode a3b q8 shared mfma1 T={T}")
    moe, lws = make_handle(lib, wl, max_tokens=32, mfma_min_tokens=1)
    with moe:
        x = synth.tokens(wl, T, 3)
        y = moe.decode(torch.from_numpy(x).cuda())
        moe.sync_status()
        check_layer(wl, lws[0], x, y.cpu().numpy(), label=f"a3b q8 mfma1 T={T}")


def test_q8_shared_chain_prenorm(lib):
    """Three layers, pre-norm residual stream: the full call equals chained
    single-layer calls bitwise, and each layer matches the oracle."""
    wl = workload("a3b_stack40_zipf_q8")
    L, T = 3, 4
    say(f"q8 shared chain {L} layers T={T}")
    moe, lws = make_handle(lib, wl, n_layers=L, max_tokens=8)
    with moe:
        x = torch.from_numpy(synth.tokens(wl, T, 1)).cuda()
        y_all = moe.decode(x, n_layers=L, residual=True, prenorm=True)
        cur = x
        for l in range(L):
            ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
            nxt = moe.decode(cur, layer0=l, n_layers=1, residual=True, prenorm=True, ids_out=ids)
            moe.sync_status()
            check_layer(wl, lws[l], cur.cpu().numpy(), nxt.cpu().numpy(), ids.cpu().numpy(),
                        residual=True, prenorm=True, label=f"q8 chain layer {l}")
            cur = nxt
        assert torch.equal(y_all, cur)


def test_q8_halves_shared_bytes(lib):
    """The handle's resident bytes drop by the shared expert's saving: per
    layer 3 * Fs * H * (2 - 34/32) bytes (up to the padding of the rows)."""
    wl = workload("a3b_layer")
    a, _ = make_handle(lib, wl, max_tokens=4, layers=[])
    b, _ = make_handle(lib, _wl("a3b"), max_tokens=4, layers=[])
    with a, b:
        saved = a.memory_bytes() - b.memory_bytes()
        want = 3 * wl.shared_ffn * wl.hidden * (2 - 34 / 32)
        say(f"bf16 - q8 shared bytes: {saved} (blocks alone {want:.0f})")
        assert abs(saved - want) <= 4096
