"""CPU checks of the C-ABI library: it loads, exports every entry point the
public header declares, and validates arguments on the host (each call below
fails validation, so nothing reaches the GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            names += re.findall(r"STRATA_API\s+[\w\s\*]+?\b(strata_\w+)\s*\(", txt)
    return sorted(set(names))


@pytest.fixture(scope="module")
def m():
    import quantized_routed_expert_router_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.lib()
    return m


def test_exports_every_declared_symbol(m):
    names = declared()
    assert len(names) == 17, names
    assert set(names) == set(m.EXPORTS)
    for n in names:
        assert hasattr(m.lib(), n), n


def test_sizes(m):
    assert m.strata_moe_blob_bytes() == 1382400
    assert m.strata_moe_workspace_bytes(0) == 0
    assert m.strata_moe_workspace_bytes(8193) == 0
    prev = 0
    for T in (1, 4, 16, 17, 2048, 8192):
        n = m.strata_moe_workspace_bytes(T)
        assert n > 0 and n % 256 == 0
        assert n >= T * 10 * 2560 * 4
        if T != 17:
            assert n >= prev
        prev = n


def test_host_validation_rejects_before_launch(m):
    L = m.lib()
    fake = 0x10000  # never dereferenced: every call below fails validation
    ws_need = m.strata_moe_workspace_bytes(4)
    assert L.strata_moe_route(None, 4, fake, None, 0, fake, fake, fake, ws_need, None) == m.E_ARG
    assert L.strata_moe_route(fake, 0, fake, None, 0, fake, fake, fake, ws_need, None) == m.E_SHAPE
    assert L.strata_moe_route(fake, 9000, fake, None, 0, fake, fake, fake, ws_need, None) == m.E_SHAPE
    assert L.strata_moe_route(fake, 4, fake, None, 0, fake, fake, fake, ws_need - 1, None) == m.E_WORKSPACE
    assert L.strata_moe_route(fake, 4, fake, None, 0, fake, fake, None, ws_need, None) == m.E_WORKSPACE
    assert L.strata_moe_route(fake + 4, 4, fake, None, 0, fake, fake, fake, ws_need, None) == m.E_ALIGN
    assert L.strata_moe_route(fake, 4, fake, None, 4, fake, fake, fake, ws_need, None) == m.E_ARG
    assert L.strata_moe_route(fake, 4, fake, None, 0, fake, fake, fake + 16, ws_need, None) == m.E_ALIGN
    assert L.strata_moe_group(fake, 4, None, fake, fake, fake, ws_need, None) == m.E_ARG
    assert L.strata_moe_experts(fake, 4, fake + 128, fake, fake, fake, 0, fake, fake, ws_need, None) == m.E_ALIGN
    assert L.strata_moe_combine(fake, fake, 4, 0, None, None) == m.E_ARG
    assert L.strata_moe_combine(fake, fake + 2, 4, 0, fake, None) == m.E_ALIGN
    # y may be NULL only with STRATA_RESIDUAL
    assert L.strata_moe_layer(fake, 4, fake, None, fake, 0, None, None, None, fake, ws_need, None) == m.E_ARG
    assert L.strata_moe_layer(fake, 4, fake, None, fake, 3, None, None, None, fake, 0, None) == m.E_WORKSPACE
    # lookahead: decode sizes only, and both next-layer pointers required
    LA = L.strata_moe_layer_lookahead
    assert LA(fake, 9, fake, None, fake, 2, None, None, None, fake, None, fake, None, None, fake,
              m.strata_moe_workspace_bytes(9), None) == m.E_SHAPE
    assert LA(fake, 0, fake, None, fake, 2, None, None, None, fake, None, fake, None, None, fake,
              ws_need, None) == m.E_SHAPE
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, None, None, fake, None, None, fake,
              ws_need, None) == m.E_ARG
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, fake, None, None, None, None, fake,
              ws_need, None) == m.E_ARG
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, fake, None, fake + 16, None, None,
              fake, ws_need, None) == m.E_ALIGN
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, fake, None, fake, None, None, fake,
              ws_need - 1, None) == m.E_WORKSPACE
    # a misaligned hint at T = 1 (the only size that reads one)
    assert LA(fake, 1, fake, None, fake, 2, None, None, None, fake, None, fake, None, fake + 2,
              fake, m.strata_moe_workspace_bytes(1), None) == m.E_ALIGN
    # the timing hook takes both events or neither (arming touches no device)
    assert L.strata_moe_time_next_kernel(fake, None) == m.E_ARG
    assert L.strata_moe_time_next_kernel(None, fake) == m.E_ARG
    assert L.strata_moe_time_next_kernel(None, None) == m.OK
    # the static-workspace layer: T beyond its limit is refused before any
    # device call
    assert L.strata_moe_layer_static(fake, 65, fake, None, fake, 2, None, None, None, None) == m.E_SHAPE
    assert L.strata_moe_layer_static(fake, 0, fake, None, fake, 2, None, None, None, None) == m.E_SHAPE
    # status entry points: argument checks need no device
    assert L.strata_moe_read_status(None, 256, None, None) == m.E_ARG
    assert L.strata_moe_clear_status(None, 256, None) == m.E_ARG
    assert L.strata_moe_clear_status(fake, 255, None) == m.E_WORKSPACE
    assert L.strata_moe_clear_status(fake + 4, 256, None) == m.E_ALIGN
    assert L.strata_moe_set_wait_limit(-1) == m.E_ARG
    assert L.strata_moe_set_wait_limit(0) == m.OK
    for rc in (0, -1, -2, -3, -4, -5):
        assert m.strata_moe_status_string(rc) != "unknown status"
    assert m.strata_moe_status_string(-99) == "unknown status"


def test_binding_refuses_host_tensors(m):
    import torch
    x = torch.zeros((1, 2560))
    with pytest.raises(ValueError):
        m.strata_moe_route(x, x, x, x, x)


def test_binding_checks_sizes_before_the_call(m):
    """Every wrapper checks shapes and sizes before it passes a pointer: an
    undersized tensor raises ValueError naming it, on the host."""
    import torch
    T = 4
    x = torch.zeros((T, 2560))
    R = torch.zeros((512, 2560), dtype=torch.int16)
    ids = torch.zeros((T, 10), dtype=torch.int32)
    w = torch.zeros((T, 10))
    ws = torch.zeros(m.strata_moe_workspace_bytes(T), dtype=torch.uint8)
    store = torch.zeros(512 * 1382400, dtype=torch.uint8)
    offsets = torch.zeros(513, dtype=torch.int32)
    slots = torch.zeros(T * 10, dtype=torch.int32)
    active = torch.zeros(513, dtype=torch.int32)
    out = torch.zeros((T * 10, 2560))

    def bad(fn, *a, what, **k):
        with pytest.raises(ValueError, match=what):
            fn(*a, **k)

    bad(m.strata_moe_route, x[:, :2559], R, ids, w, ws, what="x must")
    bad(m.strata_moe_route, torch.zeros((0, 2560)), R, ids, w, ws, what="T = 0")
    bad(m.strata_moe_route, x, R[:511], ids, w, ws, what="router")
    bad(m.strata_moe_route, x, R, ids[:3], w, ws, what="ids")
    bad(m.strata_moe_route, x, R, ids, w[:, :9], ws, what="w must")
    bad(m.strata_moe_route, x, R, ids, w, ws[:-1], what="workspace")
    bad(m.strata_moe_route, x, R, ids, w, ws, bias=torch.zeros(511), what="bias")
    bad(m.strata_moe_group, ids[:, :9], offsets, slots, active, ws, what="ids")
    bad(m.strata_moe_group, ids, offsets[:512], slots, active, ws, what="offsets")
    bad(m.strata_moe_group, ids, offsets, slots[:-1], active, ws, what="slots")
    bad(m.strata_moe_group, ids, offsets, slots, active[:1], ws, what="active")
    bad(m.strata_moe_experts, x, store[:-1], offsets, slots, active, out, ws, what="blobs")
    bad(m.strata_moe_experts, x, store, offsets, slots, active, out[:-1], ws, what="out")
    bad(m.strata_moe_combine, out[:-10], w, x, what="out")
    bad(m.strata_moe_combine, out, w[:2], x, what="w must")
    bad(m.strata_moe_layer, x, R, store[:100], ws, y=x, what="blobs")
    bad(m.strata_moe_layer, x, R, store, ws, y=x[:2], what="y must")
    bad(m.strata_moe_layer, x, R, store, ws, y=x, ids=ids[:1], what="ids")
    bad(m.strata_moe_layer, x, R, store, ws[:10], y=x, what="workspace")
    bad(m.strata_moe_layer_lookahead, x, R, store, ws, R[:1], store, y=x, what="router_next")
    bad(m.strata_moe_layer_lookahead, x, R, store, ws, R, store[:5], y=x, what="blobs_next")
    bad(m.strata_moe_layer_lookahead, x, R, store, ws, R, store, y=x, pred=ids[:2],
        what="pred")
    bad(m.strata_moe_layer_lookahead, x, R, store, ws, R, store, y=x, hint=ids[:2],
        what="hint")
    # right sizes, host memory: refused for not being on the GPU
    bad(m.strata_moe_route, x, R, ids, w, ws, what="GPU")
    bad(m.strata_moe_layer, x, R, store, ws, y=x, ids=ids, w=w, what="GPU")
