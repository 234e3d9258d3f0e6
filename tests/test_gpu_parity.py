"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: bit-exact dequantised weights, expert ids and grouping; router weights
within 1e-6; layer outputs within a max relative L2 error of 1e-3."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import TOL_REL_L2, check_layer, make_handle, oracle_layer, say, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny(lib):
    wl = workload("tiny_q2k")
    moe, lws = make_handle(lib, wl, max_tokens=64)
    yield wl, moe, lws
    moe.close()


@pytest.fixture(scope="module")
def a3b(lib):
    wl = workload("a3b_layer")
    moe, lws = make_handle(lib, wl, max_tokens=16)
    yield wl, moe, lws
    moe.close()


@pytest.fixture(scope="module", params=["tiny_q2k", "a3b_layer"])
def gemv_only(lib, request):
    """A threshold no bucket reaches: every batch size on the GEMV items."""
    wl = workload(request.param)
    moe, lws = make_handle(lib, wl, max_tokens=16, mfma_min_tokens=1024)
    yield wl, moe, lws
    moe.close()


def _equal_fp32(a, b):
    return bool(np.all(a == b))          # +0 == -0


@pytest.mark.parametrize("which", [0, 1, 2])
def test_dequant_bit_exact_tiny(tiny, which):
    wl, moe, lws = tiny
    for e in (0, 7, wl.n_experts - 1):
        say(f"dequant tiny expert {e} matrix {which}")
        got = moe.dequant(0, e, which).cpu().numpy()
        raw = (lws[0].gate, lws[0].up, lws[0].down)[which][e]
        fmt = wl.gate_up_format if which < 2 else wl.down_format
        assert _equal_fp32(got, om.dequant_matrix(raw, fmt, synth.codebook()))


@pytest.mark.parametrize("which", [0, 1, 2])
def test_dequant_bit_exact_a3b(a3b, which):
    wl, moe, lws = a3b
    for e in (0, 128, 255):
        say(f"dequant a3b expert {e} matrix {which}")
        got = moe.dequant(0, e, which).cpu().numpy()
        raw = (lws[0].gate, lws[0].up, lws[0].down)[which][e]
        fmt = wl.gate_up_format if which < 2 else wl.down_format
        ref = om.dequant_matrix(raw, fmt, synth.codebook())
        assert _equal_fp32(got, ref)


def _route_check(wl, moe, lw, T, batch=0):
    x = synth.tokens(wl, T, batch)
    r = moe.route(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    lg_ref = om.router_logits(x, lw.router, lw.router_bias)
    ids_ref, w_ref, gap = om.top_k(lg_ref, wl.top_k)
    cnt, off, pairs, active = om.group_by_expert(ids_ref, wl.n_experts)
    lg = r["logits"].cpu().numpy()
    scale = np.abs(x).astype(np.float64) @ np.abs(lw.router.astype(np.float64)).T
    assert np.all(np.abs(lg - lg_ref) <= 1e-13 * (scale + 1.0)), "logits differ beyond fp64 rounding"
    assert np.all(gap > 1e-9)
    assert np.array_equal(r["ids"].cpu().numpy(), ids_ref)
    assert np.max(np.abs(r["w"].cpu().numpy() - w_ref)) < 1e-6
    assert np.array_equal(r["counts"].cpu().numpy(), cnt)
    assert np.array_equal(r["offsets"].cpu().numpy(), off)
    assert np.array_equal(r["pairs"].cpu().numpy(), pairs)
    na = int(r["n_active"].item())
    assert na == len(active)
    act = r["active"].cpu().numpy()
    assert np.array_equal(act[:na], active) and np.all(act[na:] == -1)


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_route_tiny(tiny, T):
    wl, moe, lws = tiny
    say(f"route tiny T={T}")
    _route_check(wl, moe, lws[0], T)


@pytest.mark.parametrize("T", [1, 5, 16])
def test_route_a3b(a3b, T):
    wl, moe, lws = a3b
    say(f"route a3b T={T}")
    _route_check(wl, moe, lws[0], T)


def _decode_check(wl, moe, lw, T, batch=0, label=""):
    x = synth.tokens(wl, T, batch)
    xd = torch.from_numpy(x).cuda()
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
    y = moe.decode(xd, ids_out=ids, w_out=w)
    moe.sync_status()
    return check_layer(wl, lw, x, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), label=label)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 16, 33, 64])
def test_decode_tiny(tiny, T):
    wl, moe, lws = tiny
    say(f"decode tiny T={T}")
    _decode_check(wl, moe, lws[0], T, label=f"tiny T={T}")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 16])
def test_decode_a3b(a3b, T):
    wl, moe, lws = a3b
    say(f"decode a3b T={T}")
    _decode_check(wl, moe, lws[0], T, label=f"a3b T={T}")


def test_batch_invariance_and_determinism(gemv_only):
    """On the GEMV items a token's output does not depend on its batch: T = 1
    (small-batch kernel) equals the same token inside T = 8 (batched kernel)."""
    wl, moe, _ = gemv_only
    T = 8
    say(f"batch invariance {wl.name} T={T}")
    x = torch.from_numpy(synth.tokens(wl, T, 3)).cuda()
    y = moe.decode(x)
    y2 = moe.decode(x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "two runs differ"
    for t in (0, 3, T - 1):
        yt = moe.decode(x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(yt[0], y[t]), f"token {t} differs between T=1 and T={T}"
    perm = torch.tensor([5, 2, 7, 0, 1, 6, 4, 3], device="cuda")
    yp = moe.decode(x[perm].contiguous())
    moe.sync_status()
    assert torch.equal(yp, y[perm]), "permuting tokens does not permute outputs"


# ---- MFMA path (buckets of at least mfma_min_tokens tokens) ------------------
# mfma_min_tokens=1 sends every bucket through the matrix-core items, =4 mixes
# GEMV and MFMA buckets inside one call.

@pytest.fixture(scope="module", params=[1, 4], ids=["mfma1", "mfma4"])
def tiny_mfma(lib, request):
    wl = workload("tiny_q2k")
    moe, lws = make_handle(lib, wl, max_tokens=64, mfma_min_tokens=request.param)
    yield wl, moe, lws, request.param
    moe.close()


@pytest.fixture(scope="module", params=[1, 4], ids=["mfma1", "mfma4"])
def a3b_mfma(lib, request):
    wl = workload("a3b_layer")
    moe, lws = make_handle(lib, wl, max_tokens=32, mfma_min_tokens=request.param)
    yield wl, moe, lws, request.param
    moe.close()


@pytest.mark.parametrize("T", [1, 5, 16, 64])
def test_decode_tiny_mfma(tiny_mfma, T):
    wl, moe, lws, thr = tiny_mfma
    say(f"decode tiny T={T} mfma_min={thr}")
    _decode_check(wl, moe, lws[0], T, label=f"tiny mfma{thr} T={T}")


@pytest.mark.parametrize("T", [1, 7, 32])
def test_decode_a3b_mfma(a3b_mfma, T):
    wl, moe, lws, thr = a3b_mfma
    say(f"decode a3b T={T} mfma_min={thr}")
    _decode_check(wl, moe, lws[0], T, label=f"a3b mfma{thr} T={T}")


def test_mfma_deterministic_and_permutation(a3b_mfma):
    wl, moe, _, thr = a3b_mfma
    T = 24
    say(f"mfma determinism a3b T={T} mfma_min={thr}")
    x = torch.from_numpy(synth.tokens(wl, T, 4)).cuda()
    y = moe.decode(x)
    y2 = moe.decode(x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "two runs differ"
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(3)).cuda()
    yp = moe.decode(x[perm].contiguous())
    torch.cuda.synchronize()
    # a bucket's tokens sit in other MFMA columns after the permutation; the
    # integer sums are exact, so only fp32 rounding of the block scales differs
    err = float(np.max(om.rel_l2(yp.cpu().numpy(), y[perm].cpu().numpy())))
    say(f"  permuted vs unpermuted: max rel-L2 {err:.3e}, bitwise {torch.equal(yp, y[perm])}")
    assert err <= 1e-6


def test_zero_input_gives_zero(a3b):
    wl, moe, _ = a3b
    say("zero input")
    x = torch.zeros((3, wl.hidden), device="cuda")
    y = moe.decode(x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_ties_break_to_lower_index(lib):
    wl = workload("tiny_q2k")
    cb = synth.codebook()
    lw = synth.layer_weights(wl, 0)
    lw.router[9] = lw.router[3]
    lw.router[12] = lw.router[3]
    say("ties")
    with lib.MoE.for_workload(wl, cb, max_tokens=16) as moe:
        moe.upload(0, lw)
        x = synth.tokens(wl, 16, 5)
        r = moe.route(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        ids_ref, _, _ = om.top_k(om.router_logits(x, lw.router), wl.top_k)
        assert np.array_equal(r["ids"].cpu().numpy(), ids_ref)
        lg = r["logits"].cpu().numpy()
        assert np.array_equal(lg[:, 3], lg[:, 9]) and np.array_equal(lg[:, 3], lg[:, 12])


@pytest.mark.parametrize("T", [1, 3, 16])
def test_decode_ties_break_to_lower_index(lib, T):
    """Three experts with exactly equal logits at the top of the routing set
    (router row and bias copied), through the decode kernels of each batch
    class: the tie goes to the lower expert index, as in the oracle's order."""
    wl = workload("a3b_layer")
    cb = synth.codebook()
    lw = synth.layer_weights(wl, 0)
    x1 = synth.tokens(wl, 1, 7)
    top = int(np.argmax(om.router_logits(x1, lw.router, lw.router_bias)[0]))
    lo, hi = (top + 97) % wl.n_experts, (top + 161) % wl.n_experts
    for e in (lo, hi):
        lw.router[e] = lw.router[top]
        if lw.router_bias is not None:
            lw.router_bias[e] = lw.router_bias[top]
    x = np.repeat(x1, T, axis=0)
    say(f"decode ties T={T}")
    with lib.MoE.for_workload(wl, cb, max_tokens=16) as moe:
        moe.upload(0, lw)
        ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
        y = moe.decode(torch.from_numpy(x).cuda(), ids_out=ids, w_out=w)
        torch.cuda.synchronize()
        ids_np = ids.cpu().numpy()
        assert np.array_equal(ids_np[:, :3], np.tile(sorted([top, lo, hi]), (T, 1)))
        check_layer(wl, lw, x, y.cpu().numpy(), ids_np, w.cpu().numpy(), label=f"ties T={T}")


@pytest.mark.parametrize("T", [1, 3])
def test_decode_many_experts(lib, T):
    """E = 512 (> 256): the small-batch kernel's general top-k (keys and group
    maxima by (token, group) threads, an LDS threshold) instead of the
    register one."""
    wl = synth.Workload("e512", 43, 512, 512, 6, 256, 64, "cb2", "q2k", 1, (1,))
    say(f"E = 512 T={T}")
    moe, lws = make_handle(lib, wl, max_tokens=4)
    with moe:
        _decode_check(wl, moe, lws[0], T, label=f"E=512 T={T}")


def test_all_experts_selected(lib):
    """k = E: every expert is used by every token."""
    wl = synth.Workload("all", 41, 512, 4, 4, 256, 64, "cb2", "q2k", 1, (1,))
    say("k = E")
    moe, lws = make_handle(lib, wl, max_tokens=8)
    with moe:
        _decode_check(wl, moe, lws[0], 8, label="k=E T=8")


def test_max_tokens_edge(lib):
    """T = max_tokens with T*k at the pair budget (256 tokens x 4 = 1024)."""
    wl = synth.Workload("maxT", 42, 256, 32, 4, 256, 0, "cb2", "q2k", 1, (1,))
    say("T = 256, k = 4")
    moe, lws = make_handle(lib, wl, max_tokens=256)
    with moe:
        _decode_check(wl, moe, lws[0], 256, label="T=256 k=4")


def _chain_check(lib, wl, L, T, prenorm, max_tokens=8):
    """An L-layer call against chained single-layer calls (bitwise) and each
    layer against the oracle, teacher-forced on the GPU's own x_l; then the
    same call in place."""
    moe, lws = make_handle(lib, wl, n_layers=L, max_tokens=max_tokens)
    with moe:
        x = torch.from_numpy(synth.tokens(wl, T, 1)).cuda()
        ids = torch.empty((L, T, wl.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((L, T, wl.top_k), dtype=torch.float32, device="cuda")
        y_all = moe.decode(x, n_layers=L, residual=True, prenorm=prenorm, ids_out=ids, w_out=w)
        cur = x
        for l in range(L):
            nxt = moe.decode(cur, layer0=l, n_layers=1, residual=True, prenorm=prenorm)
            moe.sync_status()
            check_layer(wl, lws[l], cur.cpu().numpy(), nxt.cpu().numpy(), ids[l].cpu().numpy(),
                        w[l].cpu().numpy(), residual=True, prenorm=prenorm,
                        label=f"{wl.name} T={T} layer {l} (teacher-forced)")
            cur = nxt
        moe.sync_status()
        assert torch.equal(y_all, cur), "multi-layer call differs from chained single layers"
        xin = x.clone()
        moe.decode(xin, y=xin, n_layers=L, residual=True, prenorm=prenorm)
        moe.sync_status()
        assert torch.equal(xin, y_all), "in-place decode differs"


@pytest.mark.parametrize("prenorm", [False, True])
def test_residual_chain_and_in_place(lib, prenorm):
    say(f"residual chain 3 layers prenorm={prenorm}")
    _chain_check(lib, workload("a3b_stack40_zipf"), 3, 4, prenorm)


@pytest.mark.parametrize("T", [1, 2, 4])
def test_multilayer_small_hidden(lib, T):
    """Several layers of a shape with H / 8 < 256 output-row tiles: the
    small-batch kernel runs on fewer workgroups (one down tile each), so the
    flagged words reused from layer to layer are rewritten only after every
    workgroup has read them."""
    say(f"5-layer tiny stack T={T}")
    _chain_check(lib, workload("tiny_q2k", n_layers=5, zipf_s=1.1), 5, T, True)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_exclusive_launch_same_bits(lib, T):
    """QS_DECODE_EXCLUSIVE dispatches the same persistent kernel as an
    ordinary launch: outputs, ids and weights equal the cooperative launch's
    bitwise (fixed-shape small-batch kernel at T = 1, 4, batched at 16, and
    the generic small-batch kernel of the tiny shape)."""
    for wl, L in ((workload("a3b_stack40_zipf"), 3), (workload("tiny_q2k", n_layers=3, zipf_s=1.1), 3)):
        say(f"exclusive launch {wl.name} T={T}")
        moe, _ = make_handle(lib, wl, n_layers=L, max_tokens=16)
        with moe:
            x = torch.from_numpy(synth.tokens(wl, T, 5)).cuda()
            out = []
            for excl in (False, True, False, True):
                ids = torch.full((L, T, wl.top_k), -1, dtype=torch.int32, device="cuda")
                w = torch.empty((L, T, wl.top_k), dtype=torch.float32, device="cuda")
                y = moe.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids, w_out=w, exclusive=excl)
                moe.sync_status()
                out.append((y, ids, w))
            for y, ids, w in out[1:]:
                assert torch.equal(y, out[0][0]) and torch.equal(ids, out[0][1]) and torch.equal(w, out[0][2])


def test_wait_limit_reports_give_up(lib):
    """A wait limit of one poll makes the kernels' bounded waits give up while
    data is still on its way; every workgroup leaves through its normal path,
    qs_moe_sync_status reports QS_E_HIP once, and after the limit is restored
    the next call is clean and matches the oracle."""
    wl = workload("a3b_stack40_zipf")
    L = 4
    moe, lws = make_handle(lib, wl, n_layers=L, max_tokens=16)
    with moe:
        for T in (1, 16):                        # small-batch and batched kernels
            say(f"wait limit 1, T={T}")
            x = torch.from_numpy(synth.tokens(wl, T, 2)).cuda()
            moe.set_wait_limit(1)
            seen = False
            for _ in range(5):                   # a give-up is (almost) certain on the first call
                moe.decode(x, n_layers=L, residual=True, prenorm=True)
                try:
                    moe.sync_status()
                except lib.QsError as e:
                    assert e.status == lib.QS_E_HIP
                    seen = True
                    break
            assert seen, "no wait gave up with a limit of one poll"
            moe.sync_status()                    # reported once, then clear
            moe.set_wait_limit(0)
            ids = torch.empty((L, T, wl.top_k), dtype=torch.int32, device="cuda")
            y = moe.decode(x, n_layers=1, residual=True, prenorm=True, ids_out=ids)
            moe.sync_status()
            check_layer(wl, lws[0], x.cpu().numpy(), y.cpu().numpy(), ids[0].cpu().numpy(),
                        residual=True, prenorm=True, label=f"after give-up T={T}")
            y4 = moe.decode(x, n_layers=L, residual=True, prenorm=True)
            moe.sync_status()
            assert torch.isfinite(y4).all()
        with pytest.raises(lib.QsError):
            moe.set_wait_limit(-1)


@pytest.mark.parametrize("T", [1, 5])
def test_prenorm_single_layer(a3b, T):
    wl, moe, lws = a3b
    say(f"prenorm a3b T={T}")
    x = synth.tokens(wl, T, 9) * 3.0
    xd = torch.from_numpy(x).cuda()
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    y = moe.decode(xd, prenorm=True, ids_out=ids)
    r = moe.route(xd, prenorm=True)
    torch.cuda.synchronize()
    check_layer(wl, lws[0], x, y.cpu().numpy(), ids.cpu().numpy(), prenorm=True,
                label=f"prenorm T={T}")
    lg_ref = om.moe_layer(oracle_layer(wl, lws[0]), x, prenorm=True)["logits"]
    assert np.allclose(r["logits"].cpu().numpy(), lg_ref, rtol=1e-12, atol=1e-12)


def test_error_statuses_with_gpu(lib):
    wl = workload("tiny_q2k")
    cb = synth.codebook()
    say("error statuses")
    with lib.MoE.for_workload(wl, cb, n_layers=2, max_tokens=4) as moe:
        moe.upload(0, synth.layer_weights(wl, 0))
        x = torch.zeros((4, wl.hidden), device="cuda")
        y = torch.empty_like(x)
        st = torch.cuda.current_stream().cuda_stream
        L = lib.LIB
        assert L.qs_moe_decode(moe.h, 1, 1, x.data_ptr(), y.data_ptr(), 4, 0, None, None, st) == lib.QS_E_STATE
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr(), y.data_ptr(), 5, 0, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr(), y.data_ptr(), 0, 0, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_decode(moe.h, 0, 2, x.data_ptr(), y.data_ptr(), 4, 0, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr(), x.data_ptr(), 4, 0, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr() + 4, y.data_ptr(), 2, 0, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr(), y.data_ptr(), 4, 16, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr(), y.data_ptr(), 4, 32, None, None, st) == lib.QS_E_INVAL
        # steering asked for before any directions were set
        assert L.qs_moe_decode(moe.h, 0, 1, x.data_ptr(), y.data_ptr(), 4, 4, None, None, st) == lib.QS_E_STATE
        assert L.qs_moe_decode(moe.h, 2, 1, x.data_ptr(), y.data_ptr(), 4, 0, None, None, st) == lib.QS_E_INVAL
        assert L.qs_moe_dequant(moe.h, 0, wl.n_experts, 0, y.data_ptr(), st) == lib.QS_E_INVAL
        assert L.qs_moe_dequant(moe.h, 0, 0, 3, y.data_ptr(), st) == lib.QS_E_INVAL
        assert moe.memory_bytes() > 0
