"""GPU parity of the steered combine (QuarkStar README, "Steering": each
layer's MoE output m becomes m - s * d * (d . m) before the residual add)
against the oracle, through the C ABI, for both persistent kernels."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import check_layer, make_handle, say, workload

pytestmark = pytest.mark.gpu


def _dirs(n_layers, hidden, seed):
    v = np.random.default_rng(seed).standard_normal((n_layers, hidden))
    return (v / np.linalg.norm(v, axis=1, keepdims=True)).astype(np.float32)


@pytest.fixture(scope="module")
def a3b(lib):
    wl = workload("a3b_layer")
    moe, lws = make_handle(lib, wl, max_tokens=16)
    yield wl, moe, lws
    moe.close()


@pytest.mark.parametrize("T", [1, 3, 4, 7, 16])      # small-batch kernel up to 4, batched above
@pytest.mark.parametrize("scale", [0.8, -0.5])
def test_steered_layer(a3b, T, scale):
    wl, moe, lws = a3b
    d = _dirs(1, wl.hidden, 10 + T)
    moe.set_steering(d, scale)
    say(f"steered a3b layer T={T} scale={scale}")
    x = synth.tokens(wl, T, 4)
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    y = moe.decode(torch.from_numpy(x).cuda(), ids_out=ids, steer=True)
    moe.sync_status()
    check_layer(wl, lws[0], x, y.cpu().numpy(), ids.cpu().numpy(), steering=(d[0], scale),
                label=f"steer T={T} s={scale}")


@pytest.mark.parametrize("T", [2, 16])
def test_scale_one_removes_the_direction(a3b, T):
    """With scale 1 the steered output has no component along d, up to the
    fp32 rounding of the sums."""
    wl, moe, _ = a3b
    d = _dirs(1, wl.hidden, 20)
    moe.set_steering(d, 1.0)
    x = torch.from_numpy(synth.tokens(wl, T, 5)).cuda()
    y = moe.decode(x, steer=True).double().cpu().numpy()
    m = moe.decode(x).double().cpu().numpy()
    moe.sync_status()
    along = np.abs(y @ d[0].astype(np.float64))
    before = np.abs(m @ d[0].astype(np.float64))
    say(f"  T={T}: |d.y| max {along.max():.3e}, |d.m| min {before.min():.3e}")
    assert np.all(along <= 1e-5 * np.linalg.norm(m, axis=1))
    assert np.all(before > 1e3 * along)                  # there was a component to remove


@pytest.mark.parametrize("T", [1, 16])
def test_zero_scale_is_the_plain_combine_bitwise(a3b, T):
    wl, moe, _ = a3b
    moe.set_steering(_dirs(1, wl.hidden, 30), 0.0)
    x = torch.from_numpy(synth.tokens(wl, T, 6)).cuda()
    y0 = moe.decode(x)
    ys = moe.decode(x, steer=True)
    moe.sync_status()
    assert torch.equal(y0, ys)


def test_steer_without_directions_is_a_state_error(lib):
    wl = workload("tiny_q2k")
    moe, _ = make_handle(lib, wl, max_tokens=4)
    with moe:
        x = torch.zeros((2, wl.hidden), device="cuda")
        with pytest.raises(lib.QsError) as e:
            moe.decode(x, steer=True)
        assert e.value.status == lib.QS_E_STATE
        with pytest.raises(lib.QsError) as e:
            moe.set_steering(_dirs(1, wl.hidden, 1), float("nan"))
        assert e.value.status == lib.QS_E_INVAL
        before = moe.memory_bytes()
        moe.set_steering(_dirs(1, wl.hidden, 1), 1.0)
        assert moe.memory_bytes() == before + wl.hidden * 4
        moe.decode(x, steer=True)
        moe.set_steering(None)
        assert moe.memory_bytes() == before
        with pytest.raises(lib.QsError):
            moe.decode(x, steer=True)
        moe.sync_status()


def _steered_chain(lib, wl, L, T, max_tokens, scale=0.9):
    """L steered layers in one call against chained single-layer calls
    (bitwise) and each layer against the oracle on the GPU's own x_l."""
    dirs = _dirs(L, wl.hidden, 40 + T)
    moe, lws = make_handle(lib, wl, n_layers=L, max_tokens=max_tokens)
    with moe:
        moe.set_steering(dirs, scale)
        x = torch.from_numpy(synth.tokens(wl, T, 1)).cuda()
        ids = torch.empty((L, T, wl.top_k), dtype=torch.int32, device="cuda")
        y_all = moe.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids, steer=True)
        cur = x
        for l in range(L):
            nxt = moe.decode(cur, layer0=l, n_layers=1, residual=True, prenorm=True, steer=True)
            moe.sync_status()
            check_layer(wl, lws[l], cur.cpu().numpy(), nxt.cpu().numpy(), ids[l].cpu().numpy(),
                        residual=True, prenorm=True, steering=(dirs[l], scale),
                        label=f"{wl.name} steered T={T} layer {l}")
            cur = nxt
        assert torch.equal(y_all, cur), "multi-layer steered call differs from chained single layers"
        ys = moe.decode_static(x, n_layers=L, residual=True, prenorm=True, steer=True)
        moe.sync_status()
        assert torch.equal(ys, y_all), "static-scratch steered call differs"


@pytest.mark.parametrize("T", [1, 4, 8])
def test_steered_stack(lib, T):
    say(f"steered 3-layer A3B stack T={T}")
    _steered_chain(lib, workload("a3b_stack40_zipf"), 3, T, 8)


@pytest.mark.parametrize("T", [1, 3])
def test_steered_small_hidden_stack(lib, T):
    """H = 512: 64 workgroups in the small-batch kernel, the partial words
    reused from layer to layer."""
    say(f"steered 4-layer tiny stack T={T}")
    _steered_chain(lib, workload("tiny_q2k", n_layers=4, shared_ffn=128, zipf_s=1.1), 4, T, 4)
