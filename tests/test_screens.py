"""The stored near-tie screen decisions (inputs/screens.json) are the ones the
oracle-side screen makes now, and inputs.workload_inputs() replays them into
exactly the screened inputs of the parity tests (so bench.py times those)."""
import json
import os

import numpy as np

import inputs
import oracle.screen as scr
from oracle import write_screens


def test_stored_screens_match_a_fresh_derivation():
    path = os.path.join(os.path.dirname(inputs.__file__), "screens.json")
    with open(path) as f:
        stored = json.load(f)
    assert stored == json.loads(json.dumps(write_screens.derive()))


def test_workload_inputs_replay_the_screen():
    for name in ("layer-T1", "layer-T4-window", "layer-T2048-prefill"):
        c = inputs.WORKLOADS[name]
        st = inputs.Streams(c["seed"])
        R = inputs.draw_router(st.router)
        x, _ = scr.screened_x(st, c["T"], R)
        x2, routers, biases = inputs.workload_inputs(name)
        assert np.array_equal(x, x2) and np.array_equal(routers[0], R) and biases is None
    c = inputs.WORKLOADS["layer-T4-correlated-window"]
    st = inputs.Streams(c["seed"])
    R = inputs.draw_router(st.router)
    wins, _ = scr.screened_windows(st, c["T"], 1, R)
    x2, routers, _ = inputs.workload_inputs("layer-T4-correlated-window")
    assert np.array_equal(wins[0], x2) and np.array_equal(routers[0], R)


def test_stack_routers_replay_the_screen():
    c = inputs.WORKLOADS["stack48-T1"]
    x, routers, _ = inputs.workload_inputs("stack48-T1")
    st = inputs.Streams(c["seed"])
    x0 = inputs.draw_x(st.x, 1)
    ref, _ = scr.screened_stack_routers(st, x0, scr.BlobSource(c["seed"]), c["layers"],
                                        write_screens.STACK_MARGIN_T1)
    assert np.array_equal(x, x0)
    assert all(np.array_equal(a, b) for a, b in zip(routers, ref)) and len(routers) == 48
