"""Benchmark of the routed-expert MoE layer on one MI355X.

Headline workload: one MoE layer, T = 4 verify-window tokens (1 committed +
3 drafts), 512 Q2_0 experts, top-10 -- the decode-window configuration the
headline metric (routed-expert GB/s and tok/s per MoE layer) is quoted on.
A step is one whole layer call: router GEMV, softmax/top-10, grouping, the
experts (each distinct expert's 1,382,400-byte blob read once) and the
combine.  One layer's working set (~54 MB) would sit in the 256 MB memory-side
cache on repeats, so consecutive steps use 48 copies of the layer's store
(and router) at distinct HBM addresses in turn; every step reads cold memory
and computes the same result.

The same run also measures the metric's other configurations, each in its
own object under "workloads" (same --steps / --warmup): the T = 1 layer, the
T = 2048 prefill layer, and the two 48-layer stacks (a step is one token
through 48 layers, or one 2048-token chunk through 48 Zipf-biased layers).
Inputs are the workloads' screened inputs (inputs.workload_inputs).

Timing: --warmup steps, then exactly --steps steps, each as a HIP graph
replayed on one stream (single layers: one graph of exactly that many steps;
stacks: one graph per step, replayed step by step), bracketed by device
synchronisation; ms_per_step = the steps' event-timed total / steps.  Every
graph is uploaded to the device (hipGraphUpload) after capture, so no timed
replay includes that one-time transfer.  Before the warmup steps the
workload runs untimed for --settle-ms of wall time (default 300; 0 turns it
off; the value is in the JSON line): on a fresh GPU the first tens of
milliseconds of this work run slower -- a T = 2048 prefill step 526 us
against 447 us once settled, with the same kernels -- and the timed steps
are meant to see the settled GPU a serving loop runs on.  A stack's residual
input is restored after the settling.  The
dominant kernel of a workload is timed live with HIP events attached to its
own dispatch (strata_moe_time_next_kernel) over eager calls of the same
steps: its mean duration prices the roofline object.  Each such call is
preceded by a spin kernel of ~80 us on the stream, so that the call's launches
are queued before the GPU reaches them, as in a graph replay; otherwise the
host's own launch gaps would fall inside a two-launch span.

Prints one JSON line.  With --gpus > 1 it exits: the measurement is of one GPU.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16/bf16 MFMA, TFLOP/s
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, TOP/s
GATEUP_FLOP_PER_SLOT = 2 * 2 * 2560 * 640

WORKLOADS = {
    "window": dict(wl="layer-T4-window", T=4, layers=1, copies=48),
    "window-corr": dict(wl="layer-T4-correlated-window", T=4, layers=1, copies=48),
    "token": dict(wl="layer-T1", T=1, layers=1, copies=48),
    "stack-decode": dict(wl="stack48-T1", T=1, layers=48, copies=1),
    "stack-decode-lookahead": dict(wl="stack48-T1", T=1, layers=48, copies=1, lookahead=True),
    "prefill": dict(wl="layer-T2048-prefill", T=2048, layers=1, copies=4),
    # the integer variant (STRATA_INT8: int8 activations on the int8 matrix cores)
    "prefill-i8": dict(wl="layer-T2048-prefill", T=2048, layers=1, copies=4, int8=True),
    "stack-prefill": dict(wl="stack48-T32768-zipf", T=2048, layers=48, copies=1),
}
# cycles of the spin kernel ahead of each event-timed call (~80 us)
SPIN_CYCLES = 200_000
# measured beside the headline in a default run
ALSO = ("token", "prefill", "prefill-i8", "stack-decode", "stack-prefill")


# HBM traffic of the dominant kernel from committed rocprofv3 counter
# summaries (profiles/<kernel>_traffic_<workload>.txt): used only while the
# kernel sources still hash to the value recorded there.
TRAFFIC = {
    ("dec_experts", "window"): ("T4_window", ["experts_decode.hip", "quant.hpp", "common.hpp"]),
    ("pf_gateup", "prefill"): ("T2048_prefill", ["experts_prefill.hip", "common.hpp"]),
    ("pq_gateup", "prefill-i8"): ("T2048_prefill_int8", ["experts_prefill_i8.hip", "common.hpp"]),
}


def traffic_from_profile(kernel, workload):
    import hashlib
    key = TRAFFIC.get((kernel, workload))
    if key is None:
        return None
    tag, files = key
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic_{tag}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quantized_routed_expert_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest() or "hbm_bytes_per_launch" not in fields:
        return None
    return float(fields["hbm_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--workload", default="window", choices=sorted(WORKLOADS))
    ap.add_argument("--only", action="store_true",
                    help="measure the chosen workload alone (no 'workloads' objects)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time of the headline workload's cpu_baseline")
    ap.add_argument("--cpu-seconds-also", type=float, default=6.0,
                    help="oracle time of each other workload's cpu_baseline")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of graphs")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed wall-clock milliseconds of the workload before the warmup steps")
    ap.add_argument("--copies", type=int, default=0,
                    help="store copies cycled by single-layer workloads (default: the workload's; "
                         "1 keeps the layer's experts in cache between steps, a diagnostic)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only run a device copy of this many MB (counter calibration)")
    return ap.parse_args()


_hip = None


def upload_graph(g, stream):
    """hipGraphUpload of a captured graph on `stream`: the one-time transfer
    of the graph to the device, which a graph's first replay would otherwise
    include (setup, not per-step work)."""
    global _hip
    import ctypes
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipGraphUpload.restype = ctypes.c_int
    rc = _hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                             ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"hipGraphUpload failed: {rc}")


def measure(name, a, cpu_seconds):
    """One workload: returns its result object."""
    import torch
    import inputs
    import quantized_routed_expert_router_amd as m
    wl = WORKLOADS[name]
    cfg = inputs.WORKLOADS[wl["wl"]]
    T, L, seed = wl["T"], wl["layers"], cfg["seed"]
    stack = L > 1
    prefill = T > 16
    flags = (m.RMSNORM | m.RESIDUAL) if stack else 0
    int8 = bool(wl.get("int8"))
    if int8:
        flags |= m.INT8
    x, routers, biases = inputs.workload_inputs(wl["wl"], T=T)
    x = np.ascontiguousarray(x[:T])
    blob = inputs.blob_bytes()
    per_layer = 512 * blob

    # Device state: stores (copies of the same layer for single-layer runs,
    # the 48 distinct layers for stacks), routers, workspace, outputs.
    copies = (a.copies or wl["copies"]) if not stack else 1
    n_store = L if stack else copies
    store = torch.empty(n_store * per_layer, dtype=torch.uint8, device="cuda")
    for i in range(n_store):
        inputs.fill_blobs_device(store[i * per_layer:(i + 1) * per_layer], seed,
                                 (i if stack else 0) * 512, 512)
    Rd = [torch.from_numpy(R.view(np.int16)).cuda() for R in routers]
    if not stack:
        Rd = [Rd[0].clone() for _ in range(copies)]
    bd = None if biases is None else [torch.from_numpy(b).cuda() for b in biases]
    x0 = torch.from_numpy(x).cuda()
    xd = x0.clone()
    ws = m.workspace(T)
    y = torch.empty_like(xd)
    ids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 10), device="cuda")
    torch.cuda.synchronize()

    lookahead = bool(wl.get("lookahead"))
    pred_t = [torch.empty((T, 10), dtype=torch.int32, device="cuda") for _ in range(L)]

    def layer_call(l, i, ids_o, stream):
        """Layer l (store copy i for single layers); with the lookahead, layers
        0 .. L-2 also predict layer l+1's experts and warm its blobs, and take
        the previous layer's prediction as their hint."""
        sto = store[i * per_layer:(i + 1) * per_layer]
        if lookahead and l + 1 < L:
            m.strata_moe_layer_lookahead(
                xd, Rd[i], sto, ws, Rd[i + 1], store[(i + 1) * per_layer:(i + 2) * per_layer],
                bias=None if bd is None else bd[l], bias_next=None if bd is None else bd[l + 1],
                flags=flags, y=y, ids=ids_o, w=w, pred=pred_t[l],
                hint=pred_t[l - 1] if l > 0 else None, stream=stream)
        else:
            m.strata_moe_layer(xd, Rd[i], sto, ws, bias=None if bd is None else bd[l],
                               flags=flags, y=y, ids=ids_o, w=w, stream=stream)

    def one_step(i, stream=None, ids_o=None):
        ids_o = ids if ids_o is None else ids_o
        if stack:
            for l in range(L):
                layer_call(l, l, ids_o[l] if isinstance(ids_o, list) else ids_o, stream)
        else:
            layer_call(0, i % copies, ids_o, stream)

    # Routing facts of the workload (from the GPU's own ids).
    one_step(0)
    torch.cuda.synchronize()
    distinct = int(np.unique(ids.cpu().numpy()).size)
    if stack:
        xd.copy_(x0)

    # Timed region: exactly a.warmup, then exactly a.steps steps.  Single
    # layers: one graph per count holding that many consecutive steps; stacks:
    # one graph of one step (48 layers), replayed step by step.  A stack's
    # residual stream keeps moving from step to step (its inputs are the
    # previous step's outputs); the work per step is the same.
    stream = torch.cuda.Stream()

    def capture(n, first):
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    one_step(first + i, stream=stream)
        torch.cuda.current_stream().wait_stream(stream)
        upload_graph(g, stream)
        torch.cuda.synchronize()
        return g

    # The timed steps continue the warmup's walk over the store copies, so
    # none of them finds its copy still in the memory-side cache.
    graphs = {}
    if not a.eager:
        if stack:
            graphs["step"] = capture(1, 0)
        else:
            if a.warmup:
                graphs["warmup"] = capture(a.warmup, 0)
            graphs["steps"] = capture(a.steps, a.warmup)

    def run(n, key, first):
        if n == 0:
            return
        with torch.cuda.stream(stream):
            if a.eager:
                for i in range(n):
                    one_step(first + i, stream=stream)
            elif stack:
                for _ in range(n):
                    graphs["step"].replay()
            else:
                graphs[key].replay()

    if a.settle_ms > 0:   # untimed, before the warmup steps (see the module docstring)
        key = "step" if stack else ("warmup" if a.warmup else "steps")
        t_s = time.perf_counter()
        while (time.perf_counter() - t_s) * 1e3 < a.settle_ms:
            with torch.cuda.stream(stream):
                if a.eager:
                    one_step(0, stream=stream)
                else:
                    graphs[key].replay()
            torch.cuda.synchronize()
        if stack:
            xd.copy_(x0)
            torch.cuda.synchronize()
    run(a.warmup, "warmup", 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    run(a.steps, "steps", a.warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps
    del graphs

    # The dominant kernel, timed live with HIP events that the library records
    # on its stream just around it (strata_moe_time_next_kernel): the fused
    # decode experts kernel, or the prefill gate/up GEMM.  Eager layer calls
    # on the same stores; a stack re-runs its 48 layers from x0.
    n_pass = 2 if stack else max(2, (max(copies * 4, 48) + copies - 1) // copies)
    ids_t = [torch.empty((T, 10), dtype=torch.int32, device="cuda") for _ in range(L)]
    evs = []
    with torch.cuda.stream(stream):
        for p in range(n_pass):
            if stack:
                xd.copy_(x0)
            for i in range(L if stack else copies):
                ev0 = torch.cuda.Event(enable_timing=True)
                ev1 = torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(SPIN_CYCLES)   # the call's launches queue behind it
                ev0.record(stream)
                ev1.record(stream)
                m.strata_moe_time_next_kernel(ev0, ev1)
                l = i if stack else 0                  # layer (store copy i otherwise)
                layer_call(l, i, ids_t[l], stream)
                if p > 0:
                    evs.append((ev0, ev1, l))
    torch.cuda.synchronize()
    per_l = [int(np.unique(t.cpu().numpy()).size) for t in ids_t]
    k_ms = float(np.mean([ev0.elapsed_time(ev1) for ev0, ev1, _ in evs]))
    if prefill:
        units = [T * 10 for _ in evs]              # (token, expert) slots per launch
        per_unit = GATEUP_FLOP_PER_SLOT            # gate and up flops per slot
    else:
        units = [per_l[l] for _, _, l in evs]      # distinct experts per launch
        per_unit = blob                            # weight bytes per distinct expert
    k_work = float(np.mean(units)) * per_unit

    tok_s = T / (ms / 1e3)
    if prefill and int8:
        roof = {"bound": "mfma", "achieved": k_work / (k_ms / 1e3) / 1e12,
                "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s"}
    elif prefill:
        roof = {"bound": "mfma", "achieved": k_work / (k_ms / 1e3) / 1e12,
                "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": k_work / (k_ms / 1e3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # A layer of up to 3 tokens runs its experts as two launches, gate/up then
    # dec_down; the events span both dispatches (the experts stage, all of its
    # weight bytes).  The gate/up launch, dec_route_gateup, also routes the
    # tokens, so the span includes that.
    roof["kernel"] = (("pq_gateup" if int8 else "pf_gateup") if prefill
                      else "dec_route_gateup+dec_down" if T <= 3 else "dec_experts")
    # HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or null
    roof["traffic"] = traffic_from_profile(roof["kernel"], name)
    if roof["traffic"] is not None and not prefill:
        roof["traffic_per_algorithmic_byte"] = roof["traffic"] / k_work
    roof["traffic_unit"] = "bytes per launch"
    roof["ms_per_launch"] = k_ms
    roof["launches"] = len(evs)
    roof["work_per_launch"] = (f"{float(np.mean(units)):.1f} slots x {per_unit} flops" if prefill
                               else f"{float(np.mean(units)):.2f} distinct experts x {per_unit} B")

    if stack:
        value, unit = tok_s, "tok/s"
        metric = "routed-expert tok/s, 48-layer stack"
        step_bytes = sum(per_l) * blob if not prefill else None
    elif prefill:
        value, unit = tok_s, "tok/s"
        metric = "routed-expert tok/s per MoE layer (prefill)"
        step_bytes = distinct * blob
    else:
        step_bytes = distinct * blob
        value = step_bytes / (ms / 1e3) / 1e9
        unit, metric = "GB/s", "routed-expert GB/s per MoE layer (decode)"

    res = {
        "metric": metric, "value": value, "unit": unit, "ms_per_step": ms,
        "steps": a.steps, "warmup": a.warmup,
        "dtype": ("i8-mfma/f32-acc" if int8 else "f16-mfma/f32-acc") if prefill
                 else "i4dot-16bit/f32-acc",
        "config": {"workload": f"{name}: {cfg['name']}, T={T}, layers={L}, "
                               f"512 Q2_0 experts, top-10",
                   "global_batch": T, "seq_len": T if prefill else 1,
                   "timing": "eager" if a.eager else "hipGraph replay",
                   "settle_ms": a.settle_ms, "store_copies": copies},
        "tok_per_s": tok_s, "layer_ms": ms / L, "distinct_experts": distinct,
        "expert_bytes_per_step": step_bytes, "wall_s": wall,
        "roofline": roof,
    }
    if stack and not prefill:
        res["expert_gbs"] = step_bytes / (ms / 1e3) / 1e9
    if lookahead:
        # How often a routed expert of layer l+1 was among those predicted
        # (and warmed) while layer l ran, over the eager pass's tokens.
        hits = []
        pbytes = 0
        for l in range(L - 1):
            nxt, prd = ids_t[l + 1].cpu().numpy(), pred_t[l].cpu().numpy()
            hits += [len(set(nxt[t]) & set(prd[t])) / 10.0 for t in range(T)]
            pbytes += int(np.unique(prd).size) * blob
        res["lookahead"] = {"hit_rate": float(np.mean(hits)),
                            "prefetched_bytes_per_step": pbytes,
                            "note": "prefetched bytes are read in addition to the routed "
                                    "experts' own; tok/s counts the whole 48-layer step"}
    del store, Rd, ws, xd, x0, y, ids, w, pred_t, ids_t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cpu_seconds, x, routers, biases, seed, stack, prefill,
                                           T, blob)
    return res


def cpu_baseline(seconds, x, routers, biases, seed, stack, prefill, T, blob):
    """The oracle timed on the host cores on a bounded sample of the same
    workload: whole layers (route, experts, combine) for the workload's first
    layer, repeated until `seconds` have passed (at most 64 tokens)."""
    import oracle
    import oracle.screen as scr
    n = min(T, 64)
    xs = x[:n]
    R = routers[0]
    b = None if biases is None else biases[0]
    src = scr.BlobSource(seed)
    ids, _, _ = oracle.route(xs, R, 10, bias=b, rmsnorm_flag=stack)
    src.get_many(np.unique(ids))          # input generation, not timed
    reps, t0 = 0, time.perf_counter()
    while True:
        ids, w, y = scr.oracle_layer(xs, R, src, 0, bias=b, rmsnorm=stack)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    distinct = int(np.unique(ids).size)
    per_rep = el / reps
    if not prefill and not stack:
        value, unit = distinct * blob / per_rep / 1e9, "GB/s"
    else:
        value, unit = n / per_rep, "token-layers/s"
    return {"value": value, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} x one layer on {n} token(s) of the workload ({distinct} distinct "
                      f"experts), {el:.1f} s", "seconds_per_layer": per_rep}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the layer would shard by tokens: each GPU holds the whole store and runs its own "
              "tokens, with no collective)", file=sys.stderr)
        sys.exit(2)
    if a.steps < 1 or a.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.calibrate_copy_mb:
        n = a.calibrate_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))
        return
    import quantized_routed_expert_router_amd as m
    m.lib()
    head = measure(a.workload, a, a.cpu_seconds)
    res = {
        "metric": head["metric"], "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic (seeded generator; no trained weights)",
        "config": dict(head["config"], parallelism="single GPU"),
    }
    for k in ("tok_per_s", "layer_ms", "distinct_experts", "expert_bytes_per_step", "wall_s",
              "roofline", "lookahead", "cpu_baseline"):
        if k in head:
            res[k] = head[k]
    if not a.only:
        res["workloads"] = {}
        for name in ALSO:
            if name == a.workload:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            res["workloads"][name] = measure(name, a, a.cpu_seconds_also)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
