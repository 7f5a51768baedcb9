"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: expert ids bit-exact as ordered lists, |dw| <= 1e-5, and
max|dy| <= 2e-3 * max|y| over the compared tensor, on seeded inputs screened
for router near-ties (no two of a token's 11 largest logits within 1e-4).
"""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle.screen as scr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hz.qm().lib()
    yield
    hz.drop_stores()
    torch.cuda.empty_cache()


def _say(msg):
    print(msg, flush=True)


def test_device_fill_matches_host_generator():
    _say("case: device fill vs host generator, seed 0 layer 0 and seed 2 layer 47")
    s = hz.store(0, 0).view(512, -1)
    for e in (0, 1, 255, 511):
        assert np.array_equal(s[e].cpu().numpy(), inputs.gen_blob(0, e)), e
    import torch
    one = torch.empty(inputs.blob_bytes(), dtype=torch.uint8, device="cuda")
    inputs.fill_blobs_device(one, 2, 47 * 512 + 5, 1)
    assert np.array_equal(one.cpu().numpy(), inputs.gen_blob(2, 47 * 512 + 5))


@pytest.mark.parametrize("name", ["layer-T1", "layer-T4-window"])
def test_decode_workloads(name):
    c = inputs.WORKLOADS[name]
    _say(f"case: {name}, T={c['T']}, seed {c['seed']}")
    x, R, _ = hz.single_layer_case(c["seed"], c["T"])
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(c["seed"]))
    oids, ow, oy = hz.oracle_rows(x, R, c["seed"], np.arange(c["T"]))
    hz.check(name, ids, w, y, oids, ow, oy)


@pytest.mark.parametrize("T", [2, 3, 5, 8, 16])
def test_decode_sizes(T):
    seed = 1000 + T
    _say(f"case: decode T={T}, seed {seed}")
    x, R, _ = hz.single_layer_case(seed, T)
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed))
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T))
    hz.check(f"decode T={T}", ids, w, y, oids, ow, oy)


def test_decode_prefill_boundary_agree():
    """The same 16 tokens through the decode arithmetic (T = 16: 16-bit
    integer dot products) and the prefill arithmetic (T = 17, the 16 plus one
    more token: fp16 MFMA).  Ids are identical, w agree to the w bar, and both
    meet the oracle's bar, so their outputs agree within twice the y bar."""
    seed = 1616
    _say(f"case: decode T=16 vs prefill T=17 on the same tokens, seed {seed}")
    x, R, _ = hz.single_layer_case(seed, 17)
    blobs = hz.store(seed)
    ids16, w16, y16, _ = hz.gpu_layer(x[:16].copy(), R, blobs)
    ids17, w17, y17, _ = hz.gpu_layer(x, R, blobs)
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(17))
    hz.check("boundary T=16 (decode)", ids16, w16, y16, oids[:16], ow[:16], oy[:16])
    hz.check("boundary T=17 (prefill)", ids17, w17, y17, oids, ow, oy)
    assert np.array_equal(ids16, ids17[:16])
    assert np.max(np.abs(w16 - w17[:16])) <= hz.W_TOL
    d = np.max(np.abs(y16 - y17[:16])) / np.max(np.abs(oy[:16]))
    _say(f"  decode vs prefill max|dy|/max|y| = {d:.2e}")
    assert d <= 2 * hz.Y_TOL


@pytest.mark.parametrize("T", [17, 64, 100, 257])
def test_prefill_sizes(T):
    seed = 2000 + T
    _say(f"case: prefill T={T}, seed {seed}")
    x, R, _ = hz.single_layer_case(seed, T)
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed))
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T))
    hz.check(f"prefill T={T}", ids, w, y, oids, ow, oy)


def test_prefill_skewed_multi_chunk_experts():
    """A Zipf-biased router sends more than 64 tokens to the hottest experts,
    so their rows span several 64-token chunks with a ragged last chunk."""
    seed, T = 3001, 300
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    bias = inputs.draw_zipf_bias(st.bias)
    x, _ = scr.screened_x(st, T, R, bias=bias)
    _say(f"case: skewed prefill T={T}, seed {seed}")
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed), bias=bias)
    counts = np.bincount(ids.ravel(), minlength=512)
    assert counts.max() > 64, counts.max()
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T), bias=bias)
    hz.check("skewed prefill", ids, w, y, oids, ow, oy)


@pytest.mark.timeout(900)
def test_layer_t2048_prefill_full():
    """The T = 2048 prefill layer compared with the oracle on every row."""
    c = inputs.WORKLOADS["layer-T2048-prefill"]
    _say(f"case: layer-T2048-prefill T={c['T']} seed {c['seed']}, all rows")
    x, R, redrawn = hz.single_layer_case(c["seed"], c["T"])
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(c["seed"]))
    oids, ow, oy = hz.oracle_rows(x, R, c["seed"], np.arange(c["T"]))
    hz.check("layer-T2048-prefill all rows", ids, w, y, oids, ow, oy)
    load = np.bincount(ids.ravel(), minlength=512)
    _say(f"layer-T2048-prefill: {redrawn} rows redrawn; tokens per expert {load.min()}..{load.max()}")


@pytest.mark.timeout(1200)
def test_max_T_full():
    """The largest chunk, T = 8192, compared with the oracle on every row."""
    T, seed = 8192, 8192
    _say(f"case: T={T} (largest chunk) seed {seed}, all rows")
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    x, _ = scr.screened_x(st, T, R)
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed))
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T), chunk=1024)
    hz.check("T=8192 all rows", ids, w, y, oids, ow, oy)


@pytest.mark.parametrize("T,flags", [(1, 0), (2, 0), (4, 0), (8, 0), (16, 0), (1, 1), (4, 1),
                                     (16, 1)])
def test_decode_with_router_bias(T, flags):
    """Decode-sized calls with a Zipf router bias (and RMSNorm when flags = 1)
    against the oracle layer of the same input."""
    seed = 1100 + 10 * T + flags
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    bias = inputs.draw_zipf_bias(st.bias)
    x, _ = scr.screened_x(st, T, R, bias=bias, rmsnorm=bool(flags & 1))
    _say(f"case: decode T={T} flags={flags} with a Zipf router bias, seed {seed}")
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed), bias=bias, flags=flags)
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T), bias=bias, rmsnorm=bool(flags & 1))
    hz.check(f"decode T={T} flags={flags} biased", ids, w, y, oids, ow, oy)


@pytest.mark.parametrize("T,scale", [(64, 1e5), (64, 1e-5), (300, 3e4), (4, 1e5), (4, 1e-5)])
def test_input_magnitude(T, scale):
    """Activations far from unit size, with the router scaled by the inverse
    so that routing stays as for unit-size inputs: without RMSNorm the
    experts see |x| up to ~4e5 (prefill: beyond fp16's range unless scaled)
    or ~4e-5 (fp16's subnormal range), and the outputs scale as x^2."""
    seed = 1500 + T
    st = inputs.Streams(seed)
    R = inputs.f32_to_bf16_bits(scr.bf16_values(inputs.draw_router(st.router)) / np.float32(scale))
    x, _ = scr.screened_x(st, T, R, x_scale=scale)
    _say(f"case: T={T} with |x| scaled by {scale:g}, seed {seed}")
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed))
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T))
    assert np.all(np.isfinite(y))
    hz.check(f"T={T} |x| x {scale:g}", ids, w, y, oids, ow, oy)


def test_mixed_row_magnitudes_share_experts():
    """Prefill rows of different magnitudes in one call, so that the items of
    an expert hold rows with different exponents: token t is scaled by
    (0.2, 1, 3, 0.5)[t % 4] (max |x| ~0.8, ~4, ~12, ~2: rows inside [1, 8)
    stored unscaled, the others with their own power-of-two scales), no
    RMSNorm.  Rows are redrawn until the scaled logits clear the near-tie
    margin, and the test checks that the ten largest probabilities stay
    far from fp32's subnormal range."""
    T, seed = 256, 1777
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    scale = np.array([0.2, 1.0, 3.0, 0.5], np.float32)[np.arange(T) % 4][:, None]
    x = (inputs.draw_x(st.x, T) * scale).astype(np.float32)
    for _ in range(100):
        gap = scr.top11_gap(scr.logits_np(x.astype(np.float64), R, None))
        bad = np.nonzero(gap <= scr.TIE_MARGIN)[0]
        if bad.size == 0:
            break
        for t in bad:
            x[t] = (inputs.draw_x(st.x_redraw, 1)[0] * scale[t]).astype(np.float32)
    else:
        raise RuntimeError("near-tie screen did not converge")
    lg = scr.logits_np(x.astype(np.float64), R, None)
    top = np.sort(lg, axis=1)[:, -10:]
    assert np.all(top[:, -1] - top[:, 0] < 60.0), "softmax tail near fp32 underflow"
    mx = np.abs(x).max(axis=1)
    assert mx[0::4].max() < 1.0 and mx[2::4].min() >= 8.0 and 1.0 <= mx[1::4].min()
    _say(f"case: T={T} mixed row magnitudes, seed {seed}")
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed))
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T))
    assert np.all(np.isfinite(y))
    hz.check(f"T={T} mixed row magnitudes", ids, w, y, oids, ow, oy)


@pytest.mark.parametrize("T", [1, 2, 4, 100])
def test_layer_equals_composition_and_is_deterministic(T):
    seed = 4000 + T
    _say(f"case: layer vs composition T={T}")
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    ids, w, y, _ = hz.gpu_layer(x, R, st)
    ids2, w2, y2, _ = hz.gpu_layer(x, R, st)
    comp = hz.gpu_composed(x, R, st)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2) and np.array_equal(y, y2)
    assert np.array_equal(ids, comp["ids"]) and np.array_equal(w, comp["w"])
    assert np.array_equal(y, comp["y"])


def test_decode_batch_invariance():
    """Each token of a T=4 window gets bitwise the T=1 result."""
    seed = 4100
    x, R, _ = hz.single_layer_case(seed, 4)
    st = hz.store(seed)
    _say("case: batch invariance T=4 vs T=1")
    ids, w, y, _ = hz.gpu_layer(x, R, st)
    for t in range(4):
        i1, w1, y1, _ = hz.gpu_layer(x[t:t + 1], R, st)
        assert np.array_equal(i1[0], ids[t]) and np.array_equal(w1[0], w[t])
        assert np.array_equal(y1[0], y[t]), t


@pytest.mark.parametrize("T", [1, 4, 64])
def test_timing_hook_records_and_leaves_results_alone(T):
    """strata_moe_time_next_kernel: the armed call records both events around
    one kernel (positive elapsed time), gives bitwise the unarmed results, and
    the hook is used up by that call."""
    import torch
    m = hz.qm()
    seed = 4200 + T
    _say(f"case: timing hook T={T}")
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    ids, w, y, _ = hz.gpu_layer(x, R, st)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    stale = e0.elapsed_time(e1)
    m.strata_moe_time_next_kernel(e0, e1)
    ids2, w2, y2, _ = hz.gpu_layer(x, R, st)
    ms = e0.elapsed_time(e1)
    assert ms > 0.0 and ms != stale and ms < 100.0, ms
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2) and np.array_equal(y, y2)
    ids3, w3, y3, _ = hz.gpu_layer(x, R, st)   # disarmed: events stay where they were
    assert e0.elapsed_time(e1) == ms
    assert np.array_equal(y, y3)
    with pytest.raises(ValueError):
        m.strata_moe_time_next_kernel(torch.cuda.Event(enable_timing=True), e1)


def test_prefill_experts_row_boundaries():
    """Experts entry point on a hand-made routing that gives experts exactly
    1, 15, 16, 17, 48, 49, 64, 65 and 128 rows: every count of 16-row
    subtiles an item can have, items that fill their 64-token chunk exactly,
    and experts split over two and three chunks with ragged last chunks.  The
    per-slot outputs are compared with the oracle's expert FFN."""
    import torch
    import oracle
    m = hz.qm()
    seed, T = 11, 200
    rng = np.random.default_rng(seed)
    counts = {0: 1, 1: 15, 2: 16, 3: 17, 4: 48, 5: 49, 6: 64, 7: 65, 8: 128}
    rows = [[] for _ in range(T)]
    for e, c in counts.items():
        for t in rng.choice(T, c, replace=False):
            rows[t].append(e)
    for t in range(T):   # fill each token up to 10 distinct experts from 9..511
        rest = rng.choice(np.arange(9, 512), 10 - len(rows[t]), replace=False)
        rows[t] += list(rest)
        rng.shuffle(rows[t])
    ids = np.array(rows, dtype=np.int32)
    cnt = np.bincount(ids.ravel(), minlength=512)
    assert all(cnt[e] == c for e, c in counts.items())
    x = rng.standard_normal((T, inputs.H)).astype(np.float32)
    _say(f"case: prefill experts row boundaries T={T}, seed {seed}")
    xd = hz.cuda(x)
    ws = m.workspace(T)
    offsets = torch.empty(513, dtype=torch.int32, device="cuda")
    slots = torch.empty(T * 10, dtype=torch.int32, device="cuda")
    active = torch.empty(513, dtype=torch.int32, device="cuda")
    out = torch.empty((T * 10, inputs.H), dtype=torch.float32, device="cuda")
    m.strata_moe_group(hz.cuda(ids), offsets, slots, active, ws)
    m.strata_moe_experts(xd, hz.store(seed), offsets, slots, active, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    blobs = scr.BlobSource(seed).get_many(np.unique(ids))
    ref = oracle.experts(x.astype(np.float64), ids, blobs, inputs.E, inputs.H, inputs.FF)
    for e in counts:   # the boundary experts, slot by slot
        sl = np.nonzero(ids.ravel() == e)[0]
        rel = float(np.max(np.abs(got[sl] - ref[sl])) / np.max(np.abs(ref[sl])))
        _say(f"  expert {e} ({counts[e]} rows): max|do|/max|o| = {rel:.3e}")
        assert rel <= hz.Y_TOL, (e, rel)
    rel = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    _say(f"  all slots: max|do|/max|o| = {rel:.3e}")
    assert rel <= hz.Y_TOL


def test_group_matches_cpu_counting_sort():
    import torch
    m = hz.qm()
    rng = np.random.default_rng(9)
    for T in (1, 4, 37, 300, 2048, 8192):
        _say(f"case: group T={T}")
        ids = rng.integers(0, 512, (T, 10)).astype(np.int32)
        if T == 300:   # skewed: most slots on a few experts, across many blocks
            hot = rng.random((T, 10)) < 0.7
            ids[hot] = rng.choice([7, 8, 511], size=int(hot.sum()))
        if T == 37:
            ids[3, 4] = 600     # out-of-range ids are dropped
            ids[5, 0] = -1
        idd = hz.cuda(ids)
        offsets = torch.empty(513, dtype=torch.int32, device="cuda")
        slots = torch.full((T * 10,), -7, dtype=torch.int32, device="cuda")
        active = torch.empty(513, dtype=torch.int32, device="cuda")
        m.strata_moe_group(idd, offsets, slots, active, m.workspace(T))
        torch.cuda.synchronize()
        flat = ids.ravel()
        ok = (flat >= 0) & (flat < 512)
        cnt = np.bincount(flat[ok], minlength=512)
        ref_off = np.concatenate([[0], np.cumsum(cnt)])
        assert np.array_equal(offsets.cpu().numpy(), ref_off)
        order = np.nonzero(ok)[0]
        order = order[np.argsort(flat[order], kind="stable")]
        assert np.array_equal(slots.cpu().numpy()[: order.size], order)
        act = np.nonzero(cnt)[0]
        a = active.cpu().numpy()
        assert a[0] == act.size and np.array_equal(a[1:1 + act.size], act)


def test_error_codes():
    import torch
    m = hz.qm()
    x = torch.zeros((2, 2560), device="cuda")
    R = torch.zeros((512, 2560), dtype=torch.int16, device="cuda")
    ids = torch.empty((2, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((2, 10), device="cuda")
    ws = m.workspace(2)
    L = m.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.strata_moe_route(None, 2, R.data_ptr(), None, 0, ids.data_ptr(), w.data_ptr(),
                              ws.data_ptr(), ws.numel(), s) == m.E_ARG
    assert L.strata_moe_route(x.data_ptr(), 0, R.data_ptr(), None, 0, ids.data_ptr(),
                              w.data_ptr(), ws.data_ptr(), ws.numel(), s) == m.E_SHAPE
    assert L.strata_moe_route(x.data_ptr(), 8193, R.data_ptr(), None, 0, ids.data_ptr(),
                              w.data_ptr(), ws.data_ptr(), ws.numel(), s) == m.E_SHAPE
    assert L.strata_moe_route(x.data_ptr(), 2, R.data_ptr(), None, 0, ids.data_ptr(),
                              w.data_ptr(), ws.data_ptr(), 100, s) == m.E_WORKSPACE
    assert L.strata_moe_route(x.data_ptr() + 4, 2, R.data_ptr(), None, 0, ids.data_ptr(),
                              w.data_ptr(), ws.data_ptr(), ws.numel(), s) == m.E_ALIGN
    assert L.strata_moe_route(x.data_ptr(), 2, R.data_ptr(), None, 8, ids.data_ptr(),
                              w.data_ptr(), ws.data_ptr(), ws.numel(), s) == m.E_ARG
    misaligned = torch.zeros(512 * m.BLOB + 256, dtype=torch.uint8, device="cuda")[1:]
    with pytest.raises(m.StrataError) as err:
        m.strata_moe_layer(x, R, misaligned, ws, y=x)
    assert err.value.rc == m.E_ALIGN


def _tie_router(x, R, rmsnorm=False):
    """Duplicate the top expert's router row into two higher ids (a tie at
    ranks 1-3), and the 8th-ranked row -- rank 10 once the two copies sit
    above it -- into a higher id, so a tie straddles ranks 10 and 11."""
    xh = scr.rms_np(x) if rmsnorm else x.astype(np.float64)
    lg = scr.logits_np(xh[:1], R)[0]
    order = np.argsort(-lg, kind="stable")
    R = R.copy()
    top, tenth = order[0], order[7]
    higher = [e for e in order[20:] if e > max(top, tenth)][:3]
    R[higher[0]] = R[top]
    R[higher[1]] = R[top]
    R[higher[2]] = R[tenth]
    return R, top, tenth, higher


@pytest.mark.parametrize("T", [2, 20])
def test_stable_tie_order(T):
    seed = 5000 + T
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    x, _ = scr.screened_x(st, T, R)
    R2, top, tenth, higher = _tie_router(x, R)
    _say(f"case: tie order T={T}, tie {top}={higher[:2]}, {tenth}={higher[2]}")
    ids, w, y, _ = hz.gpu_layer(x, R2, hz.store(seed))
    oids, ow, oy = hz.oracle_rows(x[:1], R2, seed, np.arange(1))
    assert np.array_equal(ids[0], oids[0]), (ids[0], oids[0])
    assert list(ids[0][:3]) == [top] + sorted(higher[:2]) and ids[0][9] == tenth
    assert w[0][0] == w[0][1] == w[0][2]


def test_zero_input_and_zero_experts():
    import torch
    T = 3
    _say("case: zero activations; all-zero-weight experts")
    R = inputs.draw_router(np.random.default_rng(1))
    zero_store = torch.full((512 * inputs.blob_bytes(),), 0x55, dtype=torch.uint8, device="cuda")
    for Tz in (1, T):   # one token takes its own path (the routing in the gate/up launch)
        x = np.zeros((Tz, 2560), dtype=np.float32)
        for flags in (0, 1):
            ids, w, y, _ = hz.gpu_layer(x, R, hz.store(0), flags=flags)
            assert np.all(ids == np.arange(10)) and np.allclose(w, 0.1, atol=1e-7)
            assert np.all(y == 0.0)
    xr = np.random.default_rng(2).standard_normal((20, 2560)).astype(np.float32)
    for T2 in (2, 20):
        _, _, y, _ = hz.gpu_layer(xr[:T2], R, zero_store)
        assert np.all(y == 0.0)


@pytest.mark.parametrize("T", [1, 4, 64])
def test_layer_keeps_ids_and_weights_in_the_workspace(T):
    """ids and w may be NULL: the layer keeps them in its workspace and its
    output is bitwise that of a call that returns them."""
    import torch
    m = hz.qm()
    seed = 4300 + T
    _say(f"case: layer without ids / w outputs, T={T}")
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    ids, w, y, _ = hz.gpu_layer(x, R, st)
    xd = hz.cuda(x)
    y2 = torch.full_like(xd, float("nan"))
    m.strata_moe_layer(xd, hz.router_dev(R), st, m.workspace(T), y=y2)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy(), y)


def test_graph_capture_replays_match_eager():
    import torch
    m = hz.qm()
    seed, T = 6000, 4
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    _say("case: HIP graph capture of the layer, 3 replays")
    xd, Rd = hz.cuda(x), hz.router_dev(R)
    ws = m.workspace(T)
    y = torch.empty_like(xd)
    ids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 10), device="cuda")
    m.strata_moe_layer(xd, Rd, st, ws, y=y, ids=ids, w=w)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.strata_moe_layer(xd, Rd, st, ws, y=y, ids=ids, w=w, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), i
        _ = (xd * 2).sum().item()   # eager work between replays
