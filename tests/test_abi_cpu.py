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
    assert len(names) == 10, names
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
    assert LA(fake, 9, fake, None, fake, 2, None, None, None, fake, None, fake, None, fake,
              m.strata_moe_workspace_bytes(9), None) == m.E_SHAPE
    assert LA(fake, 0, fake, None, fake, 2, None, None, None, fake, None, fake, None, fake,
              ws_need, None) == m.E_SHAPE
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, None, None, fake, None, fake,
              ws_need, None) == m.E_ARG
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, fake, None, None, None, fake,
              ws_need, None) == m.E_ARG
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, fake, None, fake + 16, None, fake,
              ws_need, None) == m.E_ALIGN
    assert LA(fake, 4, fake, None, fake, 2, None, None, None, fake, None, fake, None, fake,
              ws_need - 1, None) == m.E_WORKSPACE
    # the timing hook takes both events or neither (arming touches no device)
    assert L.strata_moe_time_next_kernel(fake, None) == m.E_ARG
    assert L.strata_moe_time_next_kernel(None, fake) == m.E_ARG
    assert L.strata_moe_time_next_kernel(None, None) == m.OK
    for rc in (0, -1, -2, -3, -4, -5):
        assert m.strata_moe_status_string(rc) != "unknown status"
    assert m.strata_moe_status_string(-99) == "unknown status"


def test_binding_refuses_host_tensors(m):
    import torch
    x = torch.zeros((1, 2560))
    with pytest.raises(ValueError):
        m.strata_moe_route(x, x, x, x, x)
