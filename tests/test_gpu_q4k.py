"""GPU parity of the Q4_K-style routed layers (the pages' models keep the
last layers' experts at a 4-bit K type) against the oracle, through the C
ABI: bit-exact dequantisation, single Q4_K layers at every batch class, and
stacks that mix 2-bit and Q4_K layers in one decode call (two launches)."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import check_layer, make_handle, say, workload

pytestmark = pytest.mark.gpu

SHAPES = {
    "a3b": dict(base="a3b_layer", tail_layers=1, name="a3b_q4k"),
    "tiny": dict(base="tiny_q2k", tail_layers=1, shared_ffn=128, name="tiny_q4k"),
}


def _wl(key):
    kw = dict(SHAPES[key])
    return workload(kw.pop("base"), **kw)


@pytest.fixture(scope="module", params=sorted(SHAPES))
def q4(lib, request):
    wl = _wl(request.param)
    moe, lws = make_handle(lib, wl, max_tokens=32)
    yield request.param, wl, moe, lws
    moe.close()


@pytest.mark.parametrize("which", [0, 1, 2])
def test_q4k_dequant_bit_exact(q4, which):
    key, wl, moe, lws = q4
    for e in (0, wl.n_experts // 2, wl.n_experts - 1):
        say(f"q4k dequant {key} expert {e} matrix {which}")
        got = moe.dequant(0, e, which).cpu().numpy()
        raw = (lws[0].gate, lws[0].up, lws[0].down)[which][e]
        assert np.all(got == om.dequant_matrix(raw, "q4k"))


@pytest.mark.parametrize("T", [1, 3, 4, 7, 16, 32])
def test_q4k_layer(q4, T):
    key, wl, moe, lws = q4
    if key == "a3b" and T > 16:
        pytest.skip("the oracle's A3B layer at 32 tokens dequantises most experts (minutes of CPU)")
    say(f"q4k layer {key} T={T}")
    x = synth.tokens(wl, T, 3)
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
    y = moe.decode(torch.from_numpy(x).cuda(), ids_out=ids, w_out=w)
    moe.sync_status()
    check_layer(wl, lws[0], x, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), label=f"{key} q4k T={T}")


def _mixed_chain(lib, wl, L, T, steer=False):
    """L layers whose last tail_layers are Q4_K: the one call (two launches)
    equals chained single-layer calls bitwise, each layer matches the oracle
    on the GPU's own x_l, and the ids of both kinds of layer come back."""
    moe, lws = make_handle(lib, wl, n_layers=L, max_tokens=16)
    dirs = None
    with moe:
        if steer:
            v = np.random.default_rng(5).standard_normal((L, wl.hidden))
            dirs = (v / np.linalg.norm(v, axis=1, keepdims=True)).astype(np.float32)
            moe.set_steering(dirs, 0.7)
        x = torch.from_numpy(synth.tokens(wl, T, 1)).cuda()
        ids = torch.full((L, T, wl.top_k), -1, dtype=torch.int32, device="cuda")
        w = torch.empty((L, T, wl.top_k), dtype=torch.float32, device="cuda")
        y_all = moe.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids, w_out=w, steer=steer)
        moe.sync_status()
        cur = x
        for l in range(L):
            nxt = moe.decode(cur, layer0=l, n_layers=1, residual=True, prenorm=True, steer=steer)
            moe.sync_status()
            check_layer(wl, lws[l], cur.cpu().numpy(), nxt.cpu().numpy(), ids[l].cpu().numpy(),
                        w[l].cpu().numpy(), residual=True, prenorm=True,
                        steering=None if dirs is None else (dirs[l], 0.7),
                        label=f"{wl.name} T={T} layer {l} ({lws[l].gate_up_format})")
            cur = nxt
        assert torch.equal(y_all, cur), "mixed-format call differs from chained single layers"


@pytest.mark.parametrize("T", [1, 4, 16])
def test_mixed_stack(lib, T):
    wl = workload("a3b_stack40_q4tail", n_layers=4, tail_layers=2)
    say(f"mixed 2-bit / Q4_K stack, 4 layers (2 tail) T={T}")
    _mixed_chain(lib, wl, 4, T)


def test_mixed_stack_steered(lib):
    wl = workload("a3b_stack40_q4tail", n_layers=3, tail_layers=1)
    say("mixed stack, steered, T=2")
    _mixed_chain(lib, wl, 3, 2, steer=True)


def test_tail_only_and_memory(lib):
    """A handle of only tail layers runs no 2-bit kernel; a Q4_K expert
    holds 148/144 of its raw bytes resident (its scales unpacked)."""
    wl = workload("tiny_q2k", tail_layers=2, n_layers=2, shared_ffn=0, name="tiny_tail2")
    say("tail-only stack T=5")
    _mixed_chain(lib, wl, 2, 5)
    a, _ = make_handle(lib, workload("tiny_q2k"), max_tokens=4, layers=[])
    b, _ = make_handle(lib, workload("tiny_q2k", tail_layers=1, name="t1"), max_tokens=4, layers=[])
    with a, b:
        H, F, E = 512, 256, 16
        q2 = 3 * E * F * H // 256 * 84
        q4 = 3 * E * F * H // 256 * 148
        diff = b.memory_bytes() - a.memory_bytes()
        say(f"  resident bytes Q4_K - Q2_K layer: {diff} (blocks {q4 - q2})")
        assert abs(diff - (q4 - q2)) <= 3 * 256
