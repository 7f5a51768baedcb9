"""Write inputs/screens.json: the near-tie screen's decisions for the workload
configurations -- TEST INFRASTRUCTURE (calls only oracle/ and inputs/).

The screen (oracle.screen) needs router logits, which the input generator
does not compute.  Its decisions -- which rows of x were redrawn, in which
order, and how often each stacked layer's router was redrawn -- are stored so
that inputs.workload_inputs() replays them with the generator's own streams,
and bench.py times exactly the screened inputs the parity tests check.
tests/test_screens.py re-derives the file and requires equality.

Run: python -m oracle.write_screens
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import inputs  # noqa: E402
import oracle.screen as scr  # noqa: E402

STACK_MARGIN_T1 = 1e-3   # the T=1 stack's router margin (see tests/test_gpu_stacks.py)


def derive():
    out = {}
    for name in ("layer-T1", "layer-T4-window", "layer-T2048-prefill"):
        c = inputs.WORKLOADS[name]
        st = inputs.Streams(c["seed"])
        R = inputs.draw_router(st.router)
        _, rows = scr.screened_x_rows(st, c["T"], R)
        out[name] = {"x_redraw_rows": rows}
    c = inputs.WORKLOADS["layer-T4-correlated-window"]
    st = inputs.Streams(c["seed"])
    R = inputs.draw_router(st.router)
    _, n = scr.screened_windows(st, c["T"], 1, R)
    out["layer-T4-correlated-window"] = {"window_redraws": n}
    c = inputs.WORKLOADS["stack48-T1"]
    st = inputs.Streams(c["seed"])
    x0 = inputs.draw_x(st.x, 1)
    per = []
    scr.screened_stack_routers(st, x0, scr.BlobSource(c["seed"]), c["layers"], STACK_MARGIN_T1,
                               per_layer=per)
    out["stack48-T1"] = {"router_redraws": per, "margin": STACK_MARGIN_T1}
    return out


def main():
    path = os.path.join(ROOT, "inputs", "screens.json")
    with open(path, "w") as f:
        json.dump(derive(), f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
