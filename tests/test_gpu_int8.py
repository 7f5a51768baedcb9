"""The integer prefill variant (STRATA_INT8, T > 16): 2-bit codes times int8
activations on the int8 matrix cores with the code-offset correction of the
pages' CPU kernel ("Strata in the source...", section "The CPU kernels").

Bar: expert ids bit-exact and |dw| <= 1e-5 (the routing is the exact path's),
and max|dy| <= Y_TOL_INT8 * max|y| over the compared tensor.  The looser
output bound comes from the int8 rounding of x and h per 64-value block
(scale max|v| / 127), which the exact oracle does not have: about 0.5% RMS
per rounded operand, about 1.2% RMS in y, about 1.2e-2 of max|y| at the
largest error of a 2048 x 2560 output; Y_TOL_INT8 leaves a factor ~2.5."""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle.screen as scr

pytestmark = pytest.mark.gpu
Y_TOL_INT8 = 3e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hz.qm().lib()
    yield
    hz.drop_stores()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,zipf,flags", [(17, False, 0), (64, False, 0), (300, True, 0),
                                          (257, False, 1)])
def test_int8_layer_against_the_oracle(T, zipf, flags):
    m = hz.qm()
    seed = 8800 + T
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    bias = inputs.draw_zipf_bias(st.bias) if zipf else None
    x, _ = scr.screened_x(st, T, R, bias=bias, rmsnorm=bool(flags & 1))
    print(f"case: int8 layer T={T} zipf={zipf} flags={flags}", flush=True)
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(seed), bias=bias, flags=flags | m.INT8)
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T), bias=bias, rmsnorm=bool(flags & 1))
    hz.check(f"int8 T={T}", ids, w, y, oids, ow, oy, y_tol=Y_TOL_INT8)


@pytest.mark.timeout(900)
def test_int8_layer_t2048_all_rows():
    m = hz.qm()
    c = inputs.WORKLOADS["layer-T2048-prefill"]
    x, R, _ = hz.single_layer_case(c["seed"], c["T"])
    print("case: int8 layer T=2048, all rows", flush=True)
    ids, w, y, _ = hz.gpu_layer(x, R, hz.store(c["seed"]), flags=m.INT8)
    oids, ow, oy = hz.oracle_rows(x, R, c["seed"], np.arange(c["T"]))
    hz.check("int8 T=2048 all rows", ids, w, y, oids, ow, oy, y_tol=Y_TOL_INT8)


def test_int8_composition_and_decode_sizes():
    """experts(INT8) + combine equals layer(INT8) bitwise and is deterministic;
    at decode sizes the flag changes nothing."""
    import torch
    m = hz.qm()
    seed, T = 8900, 100
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    print("case: int8 composition T=100; flag at T=4", flush=True)
    ids, w, y, _ = hz.gpu_layer(x, R, st, flags=m.INT8)
    ids2, w2, y2, _ = hz.gpu_layer(x, R, st, flags=m.INT8)
    assert np.array_equal(y, y2)
    ref = hz.gpu_composed(x, R, st)
    xd = hz.cuda(x)
    ws = m.workspace(T)
    out = torch.empty((T * 10, 2560), dtype=torch.float32, device="cuda")
    yy = torch.empty_like(xd)
    m.strata_moe_experts(xd, st, hz.cuda(ref["offsets"]), hz.cuda(ref["slots"]),
                         hz.cuda(ref["active"]), out, ws, flags=m.INT8)
    m.strata_moe_combine(out, hz.cuda(w), yy)
    torch.cuda.synchronize()
    assert np.array_equal(yy.cpu().numpy(), y)
    xs, Rs, _ = hz.single_layer_case(seed + 1, 4)
    a = hz.gpu_layer(xs, Rs, st)
    b = hz.gpu_layer(xs, Rs, st, flags=m.INT8)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
