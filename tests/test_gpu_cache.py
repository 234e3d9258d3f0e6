"""GPU parity of expert paging (QuarkStar README, "Running Models Larger
Than Available Memory"): routed experts of the later layers in pinned host
memory behind a bounded HBM cache, a resident prefix, a hotlist preload.

* Outputs and ids of a paged handle equal a fully resident handle's bitwise,
  at every batch class, cold, warm and after evictions (where an expert is
  read from never changes its value), and a paged layer matches the oracle.
* The cache's slot table and counters equal the policy model's
  (oracle/cache.py) fed with the ids the calls returned."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from oracle.cache import ExpertCacheModel, STATS
from tests.gpu_util import check_layer, say, workload

pytestmark = pytest.mark.gpu

L_ALL, R, SLOTS = 5, 2, 12


@pytest.fixture(scope="module")
def pair(lib):
    """A resident and a paged handle over the same 5 layers of the Zipf A3B stack."""
    wl = workload("a3b_stack40_zipf")
    cb = synth.codebook()
    lws = [synth.layer_weights(wl, l) for l in range(L_ALL)]
    res = lib.MoE.for_workload(wl, cb, n_layers=L_ALL, max_tokens=32)
    pag = lib.MoE.for_workload(wl, cb, n_layers=L_ALL, max_tokens=32, resident_layers=R, cache_slots=SLOTS)
    for l, lw in enumerate(lws):
        res.upload(l, lw)
        pag.upload(l, lw)
    yield wl, lws, res, pag
    res.close()
    pag.close()


def _call(moe, x, L, **kw):
    T = x.shape[0]
    k = moe.cfg.top_k
    ids = torch.full((L, T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    y = moe.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids, w_out=w, **kw)
    return y, ids, w


def _model_check(moe, model, label):
    st = moe.cache_stats()
    got = {n: st[n] for n in STATS}
    assert got == model.stats, f"{label}: counters {got} != model {model.stats}"
    assert np.array_equal(moe.cache_slots(), model.table()), f"{label}: slot table differs"
    assert st["slots_used"] == sum(o is not None for o in model.owner)


@pytest.mark.parametrize("T", [1, 4, 16, 32])
def test_paged_equals_resident(pair, T):
    """Three calls in a row (the cache changes between them), each bitwise
    equal to the resident handle; T = 16, 32 take the batched kernel."""
    wl, lws, res, pag = pair
    for b in range(3):
        say(f"paged vs resident T={T} call {b}")
        x = torch.from_numpy(synth.tokens(wl, T, 10 + b)).cuda()
        y0, i0, w0 = _call(res, x, L_ALL)
        y1, i1, w1 = _call(pag, x, L_ALL)
        pag.sync_status()
        assert torch.equal(i0, i1), "ids differ"
        assert torch.equal(w0, w1), "weights differ"
        assert torch.equal(y0, y1), "outputs differ"


@pytest.mark.parametrize("slots", [SLOTS, 96])
def test_policy_matches_model(lib, pair, slots):
    """Calls with a cache sync after each: slot table and counters equal the
    model's after every call, on a fresh paged handle (its history is this
    test's alone).  12 slots thrash (every call uses more experts than that);
    96 keep the popular experts."""
    wl, lws, _, _ = pair
    pag = lib.MoE.for_workload(wl, synth.codebook(), n_layers=L_ALL, max_tokens=32, resident_layers=R,
                               cache_slots=slots)
    with pag:
        for l, lw in enumerate(lws):
            pag.upload(l, lw)
        model = ExpertCacheModel(slots)
        _model_check(pag, model, "fresh")
        for i, T in enumerate([1, 1, 4, 2, 16, 1, 3]):
            x = torch.from_numpy(synth.tokens(wl, T, 30 + i)).cuda()
            layer0, nL = (0, L_ALL) if i % 3 else (3, 2)   # some calls start inside the paged layers
            ids = torch.full((nL, T, wl.top_k), -1, dtype=torch.int32, device="cuda")
            pag.decode(x, layer0=layer0, n_layers=nL, residual=True, prenorm=True, ids_out=ids)
            pag.cache_sync()
            hits = model.call(ids.cpu().numpy(), layer0, R)
            say(f"  call {i}: T={T} layers [{layer0},{layer0 + nL}) uses {len(hits)} hits {sum(hits)}")
            _model_check(pag, model, f"call {i}")
        assert model.stats["evictions"] > 0
        if slots > SLOTS:
            assert model.stats["hits"] > 0


def test_preload_then_calls(lib):
    """A hotlist warm start (each paged layer's most popular experts first)
    and then calls that hit it; a call with no ids_out still feeds the cache."""
    wl = workload("a3b_stack40_zipf")
    L, Rl, S = 4, 1, 20
    cb = synth.codebook()
    lws = [synth.layer_weights(wl, l) for l in range(L)]
    pag = lib.MoE.for_workload(wl, cb, n_layers=L, max_tokens=8, resident_layers=Rl, cache_slots=S)
    ref = lib.MoE.for_workload(wl, cb, n_layers=L, max_tokens=8)
    with pag, ref:
        for l, lw in enumerate(lws):
            pag.upload(l, lw)
            ref.upload(l, lw)
        hot = synth.hotlist(wl, range(Rl, L))
        pag.cache_preload(hot)
        model = ExpertCacheModel(S)
        model.preload(hot)
        _model_check(pag, model, "preload")
        for i, T in enumerate([1, 4, 1, 8]):
            x = torch.from_numpy(synth.tokens(wl, T, 50 + i)).cuda()
            ids = torch.full((L, T, wl.top_k), -1, dtype=torch.int32, device="cuda")
            if i == 2:   # no ids_out: the library keeps the ids itself (the resident handle's are the same)
                pag.decode(x, n_layers=L, residual=True, prenorm=True)
                ref.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids)
            else:
                pag.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids)
            pag.cache_sync()
            hits = model.call(ids.cpu().numpy(), 0, Rl)
            say(f"  call {i}: T={T} uses {len(hits)} hits {sum(hits)}")
            _model_check(pag, model, f"call {i}")
        assert model.stats["hits"] > 0


def test_paged_layer_matches_oracle(pair):
    """A single paged layer (cold: read from host memory) against the oracle."""
    wl, lws, _, pag = pair
    for T in (1, 4):
        x = synth.tokens(wl, T, 70 + T)
        ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
        y = pag.decode(torch.from_numpy(x).cuda(), layer0=L_ALL - 1, ids_out=ids, w_out=w)
        pag.sync_status()
        check_layer(wl, lws[L_ALL - 1], x, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(),
                    label=f"paged layer {L_ALL - 1} T={T}")


@pytest.mark.parametrize("which", [0, 1, 2])
def test_paged_dequant(pair, which):
    wl, lws, _, pag = pair
    for e in (0, 77, wl.n_experts - 1):
        got = pag.dequant(R, e, which).cpu().numpy()
        raw = (lws[R].gate, lws[R].up, lws[R].down)[which][e]
        fmt = lws[R].down_format if which == 2 else lws[R].gate_up_format
        assert np.array_equal(got, om.dequant_matrix(raw, fmt, synth.codebook()))


def test_static_decode_reads_through_map(pair):
    """qs_moe_decode_static on a paged handle: the same outputs, and the
    cache is not updated by it."""
    wl, lws, res, pag = pair
    pag.cache_sync()
    before = pag.cache_stats()
    x = torch.from_numpy(synth.tokens(wl, 2, 90)).cuda()
    y0 = res.decode(x, n_layers=L_ALL, residual=True, prenorm=True)
    y1 = pag.decode_static(x, n_layers=L_ALL, residual=True, prenorm=True)
    pag.sync_status()
    pag.cache_sync()
    assert torch.equal(y0, y1)
    assert pag.cache_stats() == before


def test_q4k_tail_paged_and_steered(lib):
    """Paged layers in both routed formats (2-bit, then Q4_K-style tail
    layers: two launches per call) with steering, against the resident
    handle; then a re-upload of a paged layer drops its cached experts."""
    wl = workload("a3b_stack40_q4tail", n_layers=5, tail_layers=2)
    cb = synth.codebook()
    lws = [synth.layer_weights(wl, l) for l in range(5)]
    res = lib.MoE.for_workload(wl, cb, n_layers=5, max_tokens=16)
    pag = lib.MoE.for_workload(wl, cb, n_layers=5, max_tokens=16, resident_layers=1, cache_slots=10)
    with res, pag:
        for l, lw in enumerate(lws):
            res.upload(l, lw)
            pag.upload(l, lw)
        v = np.random.default_rng(4).standard_normal((5, wl.hidden))
        dirs = (v / np.linalg.norm(v, axis=1, keepdims=True)).astype(np.float32)
        res.set_steering(dirs, 0.6)
        pag.set_steering(dirs, 0.6)
        for T in (1, 4, 16):
            for steer in (False, True):
                say(f"q4 tail paged T={T} steer={steer}")
                x = torch.from_numpy(synth.tokens(wl, T, T)).cuda()
                y0, i0, _ = _call(res, x, 5, steer=steer)
                y1, i1, _ = _call(pag, x, 5, steer=steer)
                pag.sync_status()
                assert torch.equal(i0, i1) and torch.equal(y0, y1)
        pag.cache_sync()
        held = pag.cache_slots()
        assert (held[:, 0] == 4).any(), "no expert of the last (Q4_K-style) layer got cached"
        pag.upload(4, lws[4])
        held2 = pag.cache_slots()
        assert not (held2[:, 0] == 4).any()
        assert np.array_equal(held2[held[:, 0] != 4], held[held[:, 0] != 4])
        x = torch.from_numpy(synth.tokens(wl, 4, 99)).cuda()
        y0, _, _ = _call(res, x, 5)
        y1, _, _ = _call(pag, x, 5)
        pag.sync_status()
        assert torch.equal(y0, y1)


def test_memory_split(lib):
    """Paged layers hold no routed expert in HBM: the device bytes drop by
    their experts and grow by the slots; the host bytes are the records."""
    wl = workload("tiny_q2k", n_layers=3)
    a = lib.MoE.for_workload(wl, synth.codebook(), n_layers=3, max_tokens=4)
    b = lib.MoE.for_workload(wl, synth.codebook(), n_layers=3, max_tokens=4, resident_layers=1, cache_slots=5)
    with a, b:
        H, F, E = wl.hidden, wl.expert_ffn, wl.n_experts
        rec = 3 * F * H // 256 * 84          # gate, up, down of one expert (256-byte aligned already)
        st = b.cache_stats()
        assert st["host_bytes"] == 2 * E * rec and st["slots"] == 5
        drop = a.memory_bytes() - b.memory_bytes()
        say(f"  device bytes resident - paged: {drop}")
        # the experts of 2 layers, less 5 slots, the map and the ids buffer
        assert drop == 2 * E * rec - 5 * rec - 2 * E * 8 - 3 * 4 * wl.top_k * 4
