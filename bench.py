"""Benchmark of the FP8_DYNAMIC W8A8 Linear on one MI355X.

One step = one pass of the whole hot path (per-token activation quantization,
FP8 GEMM, scale epilogue) through the 7 quantized Linears of one
self-attention layer (q, k, v, o, gate, up, down) on a 4096-token prefill
chunk of seeded synthetic data.  ``value`` is that step's throughput in
TFLOP/s (2*M*N*K summed over the 7 Linears; quantization flops not counted).

Also measured and printed on the same JSON line:
* ``roofline``: the dominant kernel (the FP8 GEMM) timed alone with HIP events
  on its own stream, against the FP8 dense MFMA peak (5.0 PFLOP/s);
  (the step itself is replayed from a HIP graph of its 7 fused calls;)
* ``decode``: the decode step of one layer at M = 1 (7 fused calls replayed
  from a HIP graph, rotating over 4 copies of the layer's weights so that the
  weight bytes come from HBM, not from the 256 MB last-level cache), in GB/s
  of algorithmic bytes against 8 TB/s;
* ``packed``: the same two measurements with the layer's Linears packed the
  way the checkpoint's packed modules are (q|k|v as one 6144 x 4096 Linear,
  gate|up as one 24576 x 4096 Linear), so that each distinct input is
  quantized once and a layer is 4 calls instead of 7;
* ``rmsnorm_quant``: the fused BF16 RMSNorm -> per-token quantization
  kernel (the norm ahead of q/k/v and gate/up) at M = 4096 and M = 1, in GB/s
  of algorithmic bytes against 8 TB/s, beside the unfused sequence;
* ``swiglu_quant``: the fused SiLU-gated activation -> per-token quantization
  kernel (down_proj's input) at M = 4096 and M = 1, likewise;
* ``kv_cache_fp8``: the FP8 E4M3 KV-cache codec (quantizing a 4096-token
  chunk into the cache, reading a 32768-token window back), GB/s;
* ``kv_cache_int8``: the INT8 group-64 KV cache with its 128-token BF16
  residual window (quantizing into the store; reading history + tail);
* ``layer_with_fusions``: one layer's whole Linear path with the fused norms
  and activation (norm -> q|k|v, o, norm -> gate|up, SwiGLU -> down) at
  M = 4096 and M = 1 through the single-call entries (at M = 1 the norm and
  the activation run inside the GEMV), beside the same chain as separate
  calls and beside the unfused chain;
* ``cpu_baseline``: the CPU oracle timed on a bounded sample of the same
  workload on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
PREFILL_M = 4096
DECODE_M = 1
DECODE_COPIES = 4             # 4 x 193 MB of weights > 2 x the 256 MB MALL

# HBM bytes per launch (or per prefill step, for the GEMM: its 7 dispatches)
# from rocprofv3 FETCH_SIZE (x2, calibrated) and WRITE_SIZE passes over this
# script (profiles/hbm_traffic_counters_prefill_layer.txt), each valid for the
# source whose SHA-1 (comments and blank lines stripped) is given; reported
# as null once that code differs.
KERNEL_TRAFFIC = {
    "gemm": {"files": ("gemm.hip", "device_common.h"),
             "sha1": "444f460f7dc9991ea3d98b3f7609807aaac9e82b",
             "bytes": 1493419 * 1024},
    "gemv_group": {"files": ("gemv.hip", "row_ops.h", "device_common.h"),
                   "sha1": "3a03b37f980147340cfe1bf8c5ab1fecf7d3aabd",
                   "bytes": (94860 * 2 + 101) * 1024},
    "rmsnorm_quant": {"files": ("norm.hip", "row_ops.h", "device_common.h"),
                      "sha1": "c296ce5eeaa5bc30817865676bfb4f34f7514481",
                      "bytes": (16492 * 2 + 16416) * 1024},
    "swiglu_quant": {"files": ("swiglu.hip", "row_ops.h", "device_common.h"),
                     "sha1": "ec70ba76bffcc6b866b9ec5dbc6dd93875e57d26",
                     "bytes": (98412 * 2 + 49280) * 1024},
    "kv_dequant": {"files": ("kvcache.hip", "device_common.h"),
                   "sha1": "83d24ec97a97cb29dc032c3d41475d8a58bd8239",
                   "bytes": (16908 * 2 + 65629) * 1024},
    "kv_int8_read": {"files": ("kvcache.hip", "device_common.h"),
                     "sha1": "83d24ec97a97cb29dc032c3d41475d8a58bd8239",
                     "bytes": (18501 * 2 + 65619) * 1024},
}


def code_sha1(files):
    """SHA-1 of the given csrc files, comments and blank lines stripped."""
    import hashlib
    import re
    code = []
    for name in files:
        with open(os.path.join(ROOT, "fp8_w8a8_dynamic_amd", "csrc", name)) as f:
            code += [re.sub(r"//.*", "", line).rstrip() for line in f]
    return hashlib.sha1("\n".join(c for c in code if c).encode()).hexdigest()


def kernel_traffic(name):
    """The counted HBM bytes of `name` if its code is still the code the
    counters were taken on, else None."""
    t = KERNEL_TRAFFIC[name]
    return t["bytes"] if code_sha1(t["files"]) == t["sha1"] else None


def gemm_code_sha1():
    return code_sha1(KERNEL_TRAFFIC["gemm"]["files"])


def gemm_traffic():
    return kernel_traffic("gemm")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to("cuda")


# Every timed leg is first run for at least this long (besides any count of
# warm-up calls): after an idle moment the GPU's clocks ramp up over several
# milliseconds, and a fixed number of warm-up calls of a short leg would
# leave its timed calls on the ramp.
WARM_S = 0.25


def warm_for(torch, fn, seconds=WARM_S):
    """Call fn() (and synchronize) until at least `seconds` of wall time have
    passed; returns the number of calls."""
    t0 = time.perf_counter()
    calls, batch = 0, 1
    while True:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        calls += batch
        if time.perf_counter() - t0 >= seconds:
            return calls
        batch = min(2 * batch, 64)


def time_events(torch, fn, reps):
    """Average duration of fn() over reps calls, HIP events on the current
    stream (the stream the library launches on)."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def time_chunks(torch, fn, reps, chunks=5):
    """time_events over reps calls, with an event between `chunks` equal
    slices of them (no synchronization in between): returns the average per
    call over all reps and the average per call of each slice."""
    s = torch.cuda.current_stream()
    cuts = [round(i * reps / chunks) for i in range(chunks + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in cuts]
    ev[0].record(s)
    for i in range(chunks):
        for _ in range(cuts[i + 1] - cuts[i]):
            fn()
        ev[i + 1].record(s)
    ev[-1].synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / max(1, cuts[i + 1] - cuts[i])
           for i in range(chunks)]
    return ev[0].elapsed_time(ev[-1]) * 1e-3 / reps, per


def spread(rates):
    """Median, p10 and p90 of the rates of the timed slices."""
    return {"median": round(float(np.median(rates)), 2),
            "p10": round(float(np.percentile(rates, 10)), 2),
            "p90": round(float(np.percentile(rates, 90)), 2), "slices": len(rates)}


def setup_layer(torch, fq, m, cfg, packed=False):
    """The 7 Linears of one layer (seeded weights quantized on the GPU, one
    seeded input per Linear); packed: q|k|v and gate|up concatenated along
    the output channels (rows of W and of the channel scales), taking the
    input of q and of gate respectively."""
    from workloads import LAYER_SHAPES
    from workloads.generators import c3_x, outlier_act_bf16, rng_for, weight_bf16
    layer = []
    for j, (name, n, k) in enumerate(LAYER_SHAPES):
        w = weight_bf16(cfg, 0, j, n, k)
        qw, sw = fq.quantize_weight_channelwise(to_dev(w, torch))
        if cfg == 3:
            x = c3_x(m, k, j)
        else:
            x = outlier_act_bf16(rng_for(2, m, j, 0), (m, k))
        xd = to_dev(x, torch)
        layer.append(dict(name=name, n=n, k=k, x=xd, qw=qw, sw=sw))
    if packed:
        def pack(idx, name):
            parts = [layer[i] for i in idx]
            return dict(name=name, n=sum(L["n"] for L in parts), k=parts[0]["k"],
                        x=parts[0]["x"],
                        qw=torch.cat([L["qw"].view(torch.uint8) for L in parts]),
                        sw=torch.cat([L["sw"] for L in parts]))
        layer = [pack([0, 1, 2], "qkv_proj"), layer[3],
                 pack([4, 5], "gate_up_proj"), layer[6]]
    for L in layer:
        L["y"] = torch.empty((m, L["n"]), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    return layer


def bench_prefill(torch, fq, steps, warmup, packed=False):
    layer = setup_layer(torch, fq, PREFILL_M, 3, packed)
    flops = sum(2 * PREFILL_M * L["n"] * L["k"] for L in layer)
    wsb = max(fq.workspace_bytes(PREFILL_M, L["n"], L["k"], True) for L in layer)
    ws = fq.init_workspace(torch.empty(max(wsb, 1 << 20), dtype=torch.uint8, device="cuda"))

    def calls():
        for L in layer:
            fq.quant_linear(L["x"], L["qw"], L["sw"], out=L["y"], workspace=ws)

    # The step's calls are captured once in a HIP graph and replayed (as a
    # serving loop would), so host-side launch cost stays out of the timing.
    for _ in range(max(1, warmup)):
        calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        calls()                            # first use of this stream, uncaptured
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            calls()
    torch.cuda.synchronize()
    step = g.replay
    for _ in range(warmup):
        step()
    warm_for(torch, step)
    t0 = time.perf_counter()
    step_time, slices = time_chunks(torch, step, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    slice_tflops = [flops / t / 1e12 for t in slices]
    if packed:
        del layer
        torch.cuda.empty_cache()
        return dict(step_time=step_time, wall=wall, flops=flops, slices=slice_tflops)

    # Dominant kernel: the GEMM on pre-quantized activations, timed with HIP
    # events on the launching stream while the 7 GEMMs of the layer run in
    # sequence (as in the step: operands rotate through 7 Linears, 300+ MB,
    # more than the last-level cache holds).
    for L in layer:
        L["qx"], L["sx"] = fq.quantize_act_per_token(L["x"])
    s = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layer] for _ in range(steps)]
    def gemms():
        for L in layer:
            fq.fp8_linear(L["qx"], L["sx"], L["qw"], L["sw"], out=L["y"])
    warm_for(torch, gemms)
    for it in range(steps):
        for j, L in enumerate(layer):
            ev[it][j][0].record(s)
            fq.fp8_linear(L["qx"], L["sx"], L["qw"], L["sw"], out=L["y"])
            ev[it][j][1].record(s)
    torch.cuda.synchronize()
    gemm_t = [sum(ev[it][j][0].elapsed_time(ev[it][j][1]) for it in range(steps))
              * 1e-3 / steps for j in range(len(layer))]
    # The roofline figure: the same 7 launches back to back, two events
    # around the whole timed region (per-launch events add small gaps and
    # scatter; they give the per-Linear split only).
    warm_for(torch, gemms)
    gemm_region = time_events(torch, gemms, steps)
    lib_tflops = library_gemm_tflops(torch, layer, flops, steps)
    quant_t = []
    for L in layer:
        q = lambda L=L: fq.quantize_act_per_token(L["x"])
        warm_for(torch, q, 0.05)
        quant_t.append(time_events(torch, q, max(10, steps)))
    per = {L["name"]: {"gemm_us": round(t * 1e6, 2),
                       "gemm_tflops": round(2 * PREFILL_M * L["n"] * L["k"] / t / 1e12, 1),
                       "quant_us": round(tq * 1e6, 2),
                       "quant_gbs": round((3 * PREFILL_M * L["k"] + 4 * PREFILL_M) / tq / 1e9, 0)}
           for L, t, tq in zip(layer, gemm_t, quant_t)}
    gemm_tflops = flops / gemm_region / 1e12
    del layer
    torch.cuda.empty_cache()
    return dict(step_time=step_time, wall=wall, flops=flops, slices=slice_tflops,
                gemm_tflops=gemm_tflops, gemm_time=gemm_region, per_linear=per,
                lib_tflops=lib_tflops)


def library_gemm_tflops(torch, layer, flops, steps):
    """For comparison only: the vendor library's FP8 GEMM (hipBLASLt behind
    torch._scaled_mm) on the same quantized operands, with the same
    per-token x per-channel float32 scales and bf16 output, timed the same
    way (the 7 GEMMs back to back).  None where torch does not offer it."""
    try:
        ops = [(L["qx"].view(torch.float8_e4m3fn), L["qw"].view(torch.float8_e4m3fn).t(),
                L["sx"].view(-1, 1), L["sw"].view(1, -1)) for L in layer]

        def seq():
            for a, b, sa, sb in ops:
                torch._scaled_mm(a, b, scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        warm_for(torch, seq)
        return round(flops / time_events(torch, seq, steps) / 1e12, 2)
    except Exception as e:                 # not offered by this torch build
        log(f"library comparison skipped: {type(e).__name__}: {e}")
        return None


def bench_decode(torch, fq, reps, packed=False, m=DECODE_M):
    """One layer's 7 fused calls (4 when packed) at m tokens, captured in a
    HIP graph over DECODE_COPIES copies of the weights; GB/s of algorithmic
    bytes."""
    base = setup_layer(torch, fq, m, 2, packed)
    copies = [base]
    for _ in range(DECODE_COPIES - 1):
        copies.append([dict(L, qw=L["qw"].clone(), sw=L["sw"].clone(),
                            y=torch.empty_like(L["y"])) for L in base])
    nbytes = sum(L["n"] * L["k"] + 4 * L["n"] + 2 * m * L["k"]
                 + 2 * m * L["n"] for L in base)
    wsb = max(fq.workspace_bytes(m, L["n"], L["k"], True) for L in base)
    ws = fq.init_workspace(torch.empty(max(wsb, 1 << 20), dtype=torch.uint8, device="cuda"))

    def layer_pass(layer):
        for L in layer:
            fq.quant_linear(L["x"], L["qw"], L["sw"], out=L["y"], workspace=ws)

    for c in copies:                       # warm-up outside capture
        layer_pass(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        layer_pass(copies[0])              # first use of this stream, uncaptured
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for c in copies:
                layer_pass(c)
    torch.cuda.synchronize()
    for _ in range(max(3, reps // 2)):
        g.replay()
    warm_for(torch, g.replay)
    t, slices = time_chunks(torch, g.replay, reps)
    t /= DECODE_COPIES
    del g
    single = None
    if m == 1 and not packed:
        # The same 7 Linears of each copy as one grouped call (one launch per
        # layer copy: fp8w8a8_quant_linear_group_m1, outputs bit-identical
        # to the 7 calls): the ceiling of one long weight stream.
        def grouped(layer):
            fq.quant_linear_group_m1([L["x"] for L in layer], [L["qw"] for L in layer],
                                     [L["sw"] for L in layer], [L["y"] for L in layer])
        gg = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            grouped(copies[0])
            torch.cuda.synchronize()
            with torch.cuda.graph(gg, stream=cap):
                for c in copies:
                    grouped(c)
        torch.cuda.synchronize()
        warm_for(torch, gg.replay)
        tg, gslices = time_chunks(torch, gg.replay, reps)
        tg /= DECODE_COPIES
        single = {"us_per_layer": round(tg * 1e6, 3), "value": round(nbytes / tg / 1e9, 1),
                  "unit": "GB/s", "frac_of_hbm": round(nbytes / tg / 1e9 / HBM_PEAK_GBS, 4),
                  "slice_gbs": spread([nbytes * DECODE_COPIES / ts / 1e9 for ts in gslices])}
        del gg
    grouped = None
    if 1 < m <= 64 and not packed:
        # The same 7 Linears of each copy as two launches: their 7 inputs
        # quantized in one (fp8w8a8_quantize_act_group), then one grouped
        # call on the codes (fp8w8a8_fp8_linear_group; weights tiled
        # beforehand, as an offline step next to their quantization).
        for c in copies:
            for L in c:
                L["qt"] = fq.tile_weights(L["qw"])

        # Down (K = 12288, three times the stages of the others) has its K
        # summed in ranges that are units of their own in the launch, then
        # added in order by one more kernel (fp8w8a8_fp8_linear_group_requant
        # without re-quantization); also timed: the one launch unsplit.
        wsd = torch.empty(8 * m * 4096 * 4, dtype=torch.uint8, device="cuda")

        def grouped_pass(layer):
            qs = fq.quantize_act_group([L["x"] for L in layer])
            fq.fp8_linear_group_requant(
                [q for q, _ in qs], [sc for _, sc in qs], [L["qt"] for L in layer],
                [L["sw"] for L in layer], [L["n"] for L in layer], 6,
                outs=[L["y"] for L in layer], workspace=wsd, requant=False)

        def unsplit_pass(layer):
            qs = fq.quantize_act_group([L["x"] for L in layer])
            fq.fp8_linear_group([q for q, _ in qs], [sc for _, sc in qs],
                                [L["qt"] for L in layer], [L["sw"] for L in layer],
                                [L["n"] for L in layer], outs=[L["y"] for L in layer])
        timed = {}
        for name, fn in (("split", grouped_pass), ("unsplit", unsplit_pass)):
            gt = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                fn(copies[0])
                torch.cuda.synchronize()
                with torch.cuda.graph(gt, stream=cap):
                    for c in copies:
                        fn(c)
            torch.cuda.synchronize()
            warm_for(torch, gt.replay)
            tt, tslices = time_chunks(torch, gt.replay, reps)
            timed[name] = (tt / DECODE_COPIES, tslices)
            del gt
        tt, tslices = timed["split"]
        tu = timed["unsplit"][0]
        grouped = {"us_per_layer": round(tt * 1e6, 3), "value": round(nbytes / tt / 1e9, 1),
                   "unit": "GB/s", "frac_of_hbm": round(nbytes / tt / 1e9 / HBM_PEAK_GBS, 4),
                   "slice_gbs": spread([nbytes * DECODE_COPIES / ts / 1e9 for ts in tslices]),
                   "what": "the 7 inputs quantized in one launch, then the 7 Linears in "
                           "one grouped launch on MFMA-tiled weights, down's K summed in "
                           "ranges spread over the launch and added by one more kernel",
                   "unsplit": {"us_per_layer": round(tu * 1e6, 3),
                               "value": round(nbytes / tu / 1e9, 1),
                               "what": "the same with down's units unsplit (one launch "
                                       "after the quantization)"}}
        for c in copies:
            for L in c:
                L.pop("qt", None)
    del copies
    # Each Linear on its own: a graph of that Linear's call on copies of its
    # weights in turn (at least ROTATE_BYTES of distinct weights per replay,
    # so they come from HBM), replayed; GB/s of its own algorithmic bytes.
    per = {}
    for L in base:
        lb = L["n"] * L["k"] + 4 * L["n"] + 2 * m * L["k"] + 2 * m * L["n"]
        nc = max(2, -(-ROTATE_BYTES // lb))
        ws_copies = [(L["qw"], L["sw"])] + [(L["qw"].clone(), L["sw"].clone())
                                             for _ in range(nc - 1)]
        gj = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(gj, stream=cap):
                for qw, sw in ws_copies:
                    fq.quant_linear(L["x"], qw, sw, out=L["y"], workspace=ws)
        torch.cuda.synchronize()
        warm_for(torch, gj.replay, 0.05)
        tj = time_events(torch, gj.replay, max(10, reps // 4)) / nc
        per[L["name"]] = {"us": round(tj * 1e6, 3), "gbs": round(lb / tj / 1e9, 1),
                          "frac_of_hbm": round(lb / tj / 1e9 / HBM_PEAK_GBS, 4),
                          "weight_copies": nc}
        del gj, ws_copies
    del base
    torch.cuda.empty_cache()
    return dict(layer_us=t * 1e6, gbs=nbytes / t / 1e9, bytes=nbytes, per_linear=per,
                single_launch=single, grouped=grouped,
                slices=[nbytes * DECODE_COPIES / ts / 1e9 for ts in slices])


def launch_floor(torch, sizes, reps=40):
    """The bound that separate launches cannot pass: a HIP graph of one
    plain streaming read (the measured-peak read kernel) per size in
    `sizes`, back to back, over buffer copies past the last-level cache:
    us per sequence and GB/s of the bytes read.  Compared with one read of
    the summed size, it gives the fixed cost of each extra launch."""
    import ctypes
    from fp8_w8a8_dynamic_amd import build as fbuild
    lib = ctypes.CDLL(fbuild.PEAKS_LIB_PATH)
    lib.fp8w8a8_peaks_read_stream.restype = ctypes.c_int
    lib.fp8w8a8_peaks_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_void_p]
    total = sum(sizes)
    copies = max(2, -(-ROTATE_BYTES // total))
    bufs = [[torch.empty(sz, dtype=torch.uint8, device="cuda") for sz in sizes]
            for _ in range(copies)]
    one = [torch.empty(total, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    out = torch.empty(1024 * 256, dtype=torch.int32, device="cuda")

    def seq(c, parts):
        st = torch.cuda.current_stream().cuda_stream
        for b in parts:
            if lib.fp8w8a8_peaks_read_stream(b.data_ptr(), b.numel(), out.data_ptr(), st):
                raise RuntimeError("read_stream failed")
    res = {}
    for name, sets in (("separate", bufs), ("one_read", [[o] for o in one])):
        gr = graph_of(torch, rotating([lambda c=c: seq(0, c) for c in sets]), len(sets))
        warm_for(torch, gr.replay, 0.1)
        t = time_events(torch, gr.replay, reps) / len(sets)
        res[name] = {"us": round(t * 1e6, 3), "gbs": round(total / t / 1e9, 1)}
        del gr
    res["launches"] = len(sizes)
    res["fixed_cost_us_per_extra_launch"] = round(
        (res["separate"]["us"] - res["one_read"]["us"]) / max(1, len(sizes) - 1), 3)
    del bufs, one, out
    torch.cuda.empty_cache()
    return res


def bench_stack(torch, fq, m, passes):
    """The 36-layer stack at m tokens: 252 fused calls per pass over
    6.946 GB of FP8 weights resident in HBM, with the stack's data flow
    (q, k, v, o, gate, up read the layer input, down reads up's output, and
    down's output is the next layer's input).  Weight codes are seeded
    random bytes (NaN codes excluded) with random channel scales: the timing
    does not depend on the values, and quantizing 6.9 GB of bf16 weights
    first would dominate the run."""
    from workloads import LAYER_SHAPES
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    layers = []
    for _ in range(36):
        lw = []
        for _, n, k in LAYER_SHAPES:
            c = torch.randint(0, 256, (n, k), dtype=torch.uint8, device="cuda", generator=gen)
            c[(c & 0x7F) == 0x7F] -= 1
            lw.append((c, torch.rand(n, device="cuda", generator=gen) * 1e-3 + 1e-4))
        layers.append(lw)
    x0 = torch.randn(m, 4096, device="cuda", generator=gen).to(torch.bfloat16)
    ys = [torch.empty(m, n, dtype=torch.bfloat16, device="cuda") for _, n, _ in LAYER_SHAPES]
    xs = [x0] + [torch.empty(m, 4096, dtype=torch.bfloat16, device="cuda") for _ in range(36)]
    wsb = max(fq.workspace_bytes(m, n, k, True) for _, n, k in LAYER_SHAPES)
    ws = fq.init_workspace(torch.empty(max(wsb, 1 << 20), dtype=torch.uint8, device="cuda"))

    def one_pass():
        for li, lw in enumerate(layers):
            x = xs[li]
            for j in range(6):
                fq.quant_linear(x, lw[j][0], lw[j][1], out=ys[j], workspace=ws)
            fq.quant_linear(ys[5], lw[6][0], lw[6][1], out=xs[li + 1], workspace=ws)

    # The same stack as the checkpoint's packed modules run it: q|k|v and
    # gate|up concatenated along the output channels, and each distinct
    # input quantized once (X_l for qkv, o, gate_up; up's output for down):
    # 4 matmuls per layer instead of 7 fused calls, with up's output
    # quantized on its own and down's output re-quantized for the next
    # layer by down's own call (fp8_linear_requant; the last layer's output
    # is not).
    packed = [(torch.cat([lw[0][0], lw[1][0], lw[2][0]]), torch.cat([lw[0][1], lw[1][1], lw[2][1]]),
               lw[3], torch.cat([lw[4][0], lw[5][0]]), torch.cat([lw[4][1], lw[5][1]]), lw[6])
              for lw in layers]
    y_qkv = torch.empty(m, 6144, dtype=torch.bfloat16, device="cuda")
    y_gu = torch.empty(m, 24576, dtype=torch.bfloat16, device="cuda")
    wsp = max(fq.workspace_bytes(m, n, k, False) for n, k in
              ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)))
    ws2 = fq.init_workspace(torch.empty(max(wsp, 1 << 20), dtype=torch.uint8, device="cuda"))

    def down_of(li, qu, su, wd, sd, ws):
        """Down; its output re-quantized for the next layer unless last."""
        if li + 1 < 36:
            _, qn, sn = fq.fp8_linear_requant(qu, su, wd, sd, out=xs[li + 1], workspace=ws)
            return qn, sn
        fq.fp8_linear(qu, su, wd, sd, out=xs[li + 1], workspace=ws)
        return None, None

    def packed_pass():
        qx, sx = fq.quantize_act_per_token(xs[0])
        for li, (wqkv, sqkv, (wo, so), wgu, sgu, (wd, sd)) in enumerate(packed):
            fq.fp8_linear(qx, sx, wqkv, sqkv, out=y_qkv, workspace=ws2)
            fq.fp8_linear(qx, sx, wo, so, out=ys[3], workspace=ws2)
            fq.fp8_linear(qx, sx, wgu, sgu, out=y_gu, workspace=ws2)
            qu, su = fq.quantize_act_per_token(y_gu[:, 12288:])
            qx, sx = down_of(li, qu, su, wd, sd, ws2)

    for _ in range(3):
        one_pass()
    warm_for(torch, one_pass)
    # Eagerly launched from Python (each call's host-side cost included) ...
    t_eager = time_events(torch, one_pass, passes)
    # ... and the pass captured once in a HIP graph and replayed (as a
    # serving loop would): the GPU-side figure.
    gr = graph_of(torch, one_pass, 1)
    warm_for(torch, gr.replay)
    t = time_events(torch, gr.replay, passes)
    del gr
    gp = graph_of(torch, packed_pass, 1)
    warm_for(torch, gp.replay)
    t_packed = time_events(torch, gp.replay, passes)
    del gp, packed
    # At up to 64 tokens, on weights tiled offline: per layer q, o, gate and
    # up in one grouped launch (one round of 64-row units), up's output
    # quantized, then down -- its K summed in ranges that are units of
    # their own -- beside k and v in a second grouped launch, whose ranges
    # one kernel adds, writes and re-quantizes as the next layer's input.
    # Also timed: the six Linears that read the layer input in one launch,
    # then down through fp8_linear_requant (the previous arrangement).
    grouped = None
    # (The grouped call takes up to 256 tokens, but at 256 the stack passed
    # in 5.0 ms this way against 3.9 ms packed: not timed there.)
    if m <= 64:
        tiled = [[fq.tile_weights(lw[j][0]) for j in range(7)] for lw in layers]
        ns = [n for _, n, _ in LAYER_SHAPES]
        first, second = (0, 3, 4, 5), (6, 1, 2)
        ws3 = torch.empty(8 * m * 4096 * 4, dtype=torch.uint8, device="cuda")

        def grouped_pass():
            qx, sx = fq.quantize_act_per_token(xs[0])
            for li, lw in enumerate(layers):
                fq.fp8_linear_group([qx] * 4, [sx] * 4, [tiled[li][j] for j in first],
                                    [lw[j][1] for j in first], [ns[j] for j in first],
                                    outs=[ys[j] for j in first])
                qu, su = fq.quantize_act_per_token(ys[5])
                # (The last layer's output is re-quantized too: a few KB.)
                _, qx, sx = fq.fp8_linear_group_requant(
                    [qu, qx, qx], [su, sx, sx], [tiled[li][j] for j in second],
                    [lw[j][1] for j in second], [ns[j] for j in second], 0,
                    outs=[xs[li + 1], ys[1], ys[2]], workspace=ws3)

        def grouped_six_pass():
            qx, sx = fq.quantize_act_per_token(xs[0])
            for li, lw in enumerate(layers):
                fq.fp8_linear_group([qx] * 6, [sx] * 6, tiled[li][:6],
                                    [lw[j][1] for j in range(6)], ns[:6], outs=ys[:6])
                qu, su = fq.quantize_act_per_token(ys[5])
                qx, sx = down_of(li, qu, su, lw[6][0], lw[6][1], ws2)

        timed = {}
        for name, fn in (("grouped", grouped_pass), ("six", grouped_six_pass)):
            for _ in range(2):
                fn()
            gg = graph_of(torch, fn, 1)
            warm_for(torch, gg.replay)
            timed[name] = time_events(torch, gg.replay, passes)
            del gg
        del tiled
        t_grouped = timed["grouped"]
        grouped = {"ms_per_pass": round(t_grouped * 1e3, 4),
                   "gbs": None, "frac_of_hbm": None,
                   "us_per_layer": round(t_grouped * 1e6 / 36, 2),
                   "what": "per layer q, o, gate, up in one grouped launch on MFMA-tiled "
                           "weights, up's output quantized, then down (K summed in ranges "
                           "spread over the launch) beside k and v in a second grouped "
                           "launch, down's output re-quantized as the next layer's input",
                   "six_in_one_launch": {
                       "ms_per_pass": round(timed["six"] * 1e3, 4),
                       "what": "q, k, v, o, gate, up in one grouped launch, up's output "
                               "quantized, then down through fp8_linear_requant"}}
    nbytes = 36 * sum(n * k + 4 * n + 2 * m * k + 2 * m * n for _, n, k in LAYER_SHAPES)
    flops = 36 * sum(2 * m * n * k for _, n, k in LAYER_SHAPES)
    if grouped is not None:
        grouped["gbs"] = round(nbytes / t_grouped / 1e9, 1)
        grouped["frac_of_hbm"] = round(nbytes / t_grouped / 1e9 / HBM_PEAK_GBS, 4)
    del layers, xs, ys
    torch.cuda.empty_cache()
    return {"m": m, "ms_per_pass": round(t * 1e3, 4), "gbs": round(nbytes / t / 1e9, 1),
            "frac_of_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(flops / t / 1e12, 2),
            "frac_of_fp8_peak": round(flops / t / 1e12 / FP8_PEAK_TFLOPS, 4),
            "us_per_layer": round(t * 1e6 / 36, 2),
            "eager_ms_per_pass": round(t_eager * 1e3, 4),
            "packed": {"ms_per_pass": round(t_packed * 1e3, 4),
                       "gbs": round(nbytes / t_packed / 1e9, 1),
                       "frac_of_hbm": round(nbytes / t_packed / 1e9 / HBM_PEAK_GBS, 4),
                       "us_per_layer": round(t_packed * 1e6 / 36, 2),
                       "what": "q|k|v and gate|up packed, each distinct input quantized "
                               "once (down re-quantizes its output as the next layer's "
                               "input): 4 matmuls + 1 quantization per layer"},
            "grouped": grouped}


def graph_of(torch, fn, calls):
    """A HIP graph of `calls` back-to-back fn() calls (outputs allocated at
    capture and reused by every replay), so that replays time the kernels
    without the host's per-call overhead."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fn()                               # first use of this stream, uncaptured
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for _ in range(calls):
                fn()
    torch.cuda.synchronize()
    return g


NORM_CALLS_PER_GRAPH = 20
ROTATE_BYTES = 600 << 20      # distinct bytes per replay: > 2x the 256 MB MALL


MAX_COPIES = 64


def copies_for(nbytes):
    """Copies of a call's buffers such that one replay of the graph touches
    ROTATE_BYTES of distinct memory: the last-level cache (256 MB) then holds
    none of a call's data when that call comes round again, so every figure
    of a call of 10 MB or more is an HBM figure.  At most MAX_COPIES (calls
    smaller than that, e.g. one decode token's row, are cache-resident in
    use anyway)."""
    return max(1, min(MAX_COPIES, -(-ROTATE_BYTES // nbytes)))


def rotating(fns):
    """One callable that runs fns[0], fns[1], ... in turn, one per call (so
    the calls captured into a graph cycle through the buffer copies)."""
    state = [0]

    def f():
        fns[state[0] % len(fns)]()
        state[0] += 1
    return f


def time_graph(torch, fns, reps, nbytes):
    """HIP-graph replays of max(NORM_CALLS_PER_GRAPH, len(fns)) calls cycling
    over fns (one per set of buffer copies), events on the replay stream:
    us and GB/s of `nbytes` algorithmic bytes per call."""
    calls = max(NORM_CALLS_PER_GRAPH, len(fns))
    gr = graph_of(torch, rotating(fns), calls)
    for _ in range(max(10, reps // 10)):
        gr.replay()
    warm_for(torch, gr.replay, 0.1)
    t, slices = time_chunks(torch, gr.replay, max(10, reps // 4))
    del gr
    t /= calls
    return {"us": round(t * 1e6, 3), "gbs": round(nbytes / t / 1e9, 1),
            "frac_of_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "buffer_copies": len(fns),
            "slice_gbs": spread([nbytes * calls / ts / 1e9 for ts in slices])}


def bench_norm(torch, fq, reps, m=PREFILL_M, k=4096, eps=1e-6):
    """The fused BF16 RMSNorm -> per-token quantization (the input norm of
    q/k/v and of gate/up) on m tokens of hidden size k: GB/s of algorithmic
    bytes (x and gamma in; codes, scales and, when stored, the bf16 norm
    output out), with and without the bf16 output, and the unfused sequence
    (torch's bf16 rms_norm, then this library's quantizer) for comparison.
    Each figure is a HIP-graph replay whose calls cycle over copies of the
    buffers (time_graph)."""
    from workloads import norm_inputs
    xb, gb = norm_inputs(m, k, seed=0)
    x0, g = to_dev(xb, torch), to_dev(gb, torch)
    base = 2 * m * k + 2 * k + m * k + 4 * m
    nc = copies_for(base)
    xs = [x0] + [x0.clone() for _ in range(nc - 1)]
    ys = [torch.empty_like(x0) for _ in range(nc)]

    def unfused(i):
        n = torch.nn.functional.rms_norm(xs[i], (k,), weight=g, eps=eps)
        fq.quantize_act_per_token(n)

    res = {}
    for name, mk, nbytes in (
            ("fused", lambda i: lambda: fq.rmsnorm_quantize(xs[i], g, eps), base),
            ("fused_with_normed_output",
             lambda i: lambda: fq.rmsnorm_quantize(xs[i], g, eps, out=ys[i]),
             base + 2 * m * k),
            ("unfused_torch_rms_norm_then_quantize", lambda i: lambda: unfused(i), base)):
        res[name] = time_graph(torch, [mk(i) for i in range(nc)], reps, nbytes)
    del xs, ys, g
    torch.cuda.empty_cache()
    return res


def bench_swiglu(torch, fq, reps, m=PREFILL_M, n=12288):
    """The fused SiLU-gated activation -> per-token quantization (down_proj's
    input) on m tokens of width n, reading the two halves of a packed
    gate_up output [m, 2n]: GB/s of algorithmic bytes (gate and up in; codes
    and scales out; plus h when stored), beside the unfused sequence (torch's
    bf16 silu and multiply, then this library's quantizer).  HIP-graph
    replays over buffer copies, as for the norm."""
    from workloads import swiglu_inputs
    gb, ub = swiglu_inputs(m, n, seed=0)
    gu0 = to_dev(np.concatenate([gb, ub], axis=1), torch)
    base = 4 * m * n + m * n + 4 * m
    nc = copies_for(base)
    gus = [gu0] + [gu0.clone() for _ in range(nc - 1)]
    hs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in range(nc)]

    def unfused(i):
        a = torch.nn.functional.silu(gus[i][:, :n]) * gus[i][:, n:]
        fq.quantize_act_per_token(a)

    res = {}
    for name, mk, nbytes in (
            ("fused", lambda i: lambda: fq.swiglu_quantize(gus[i][:, :n], gus[i][:, n:]),
             base),
            ("fused_with_h_output",
             lambda i: lambda: fq.swiglu_quantize(gus[i][:, :n], gus[i][:, n:], out=hs[i]),
             base + 2 * m * n),
            ("unfused_torch_silu_mul_then_quantize", lambda i: lambda: unfused(i), base)):
        res[name] = time_graph(torch, [mk(i) for i in range(nc)], reps, nbytes)
    del gus, hs
    torch.cuda.empty_cache()
    return res


def bench_fused_layer(torch, fq, m, steps, copies=1, eps=1e-6):
    """One layer's Linear path with the adjacent fusions, HIP-graph replays:
        rmsnorm_quant_linear(x1, q|k|v)         [6144 x 4096]
        quant_linear(attention out)             (o_proj)
        rmsnorm_quant_linear(x2, gate|up)       [24576 x 4096]
        swiglu_quant_linear(gate, up, down)     [4096 x 12288]
    (at decode sizes each of these is one kernel; otherwise the pre-step
    kernel and then the Linear), beside the same chain as separate
    rmsnorm_quantize / swiglu_quantize + fp8_linear calls and beside torch's
    bf16 rms_norm and silu * up feeding quant_linear.  Attention and the
    residual adds are not part of it (their inputs are seeded data).
    `copies` layers with distinct weights run per replay so that
    decode-sized steps read their weights from HBM."""
    from workloads import norm_inputs
    base = setup_layer(torch, fq, m, 3 if m == PREFILL_M else 2, packed=True)
    layers = [base]
    for _ in range(copies - 1):
        layers.append([dict(L, qw=L["qw"].clone(), sw=L["sw"].clone(),
                            y=torch.empty_like(L["y"])) for L in base])
    _, g1 = norm_inputs(1, 4096, seed=11)
    _, g2 = norm_inputs(1, 4096, seed=12)
    g1, g2 = to_dev(g1, torch), to_dev(g2, torch)
    qkv, o, gu, down = base
    inter = gu["n"] // 2
    wsb = max(fq.workspace_bytes(m, L["n"], L["k"], mode) for L in base for mode in (1, 2, 3))
    ws = fq.init_workspace(torch.empty(max(wsb, 1 << 20), dtype=torch.uint8, device="cuda"))
    flops = sum(2 * m * L["n"] * L["k"] for L in base)
    nbytes = (sum(L["n"] * L["k"] + 4 * L["n"] + 2 * m * L["k"] + 2 * m * L["n"] for L in base)
              + 2 * (2 * 4096) + 2 * 2 * m * inter)      # gammas, gate/up re-read

    def fused(layer):
        qkv, o, gu, down = layer
        fq.rmsnorm_quant_linear(qkv["x"], g1, eps, qkv["qw"], qkv["sw"], out=qkv["y"],
                                workspace=ws)
        fq.quant_linear(o["x"], o["qw"], o["sw"], out=o["y"], workspace=ws)
        fq.rmsnorm_quant_linear(gu["x"], g2, eps, gu["qw"], gu["sw"], out=gu["y"],
                                workspace=ws)
        fq.swiglu_quant_linear(gu["y"][:, :inter], gu["y"][:, inter:], down["qw"],
                               down["sw"], out=down["y"], workspace=ws)

    def two_step(layer):
        qkv, o, gu, down = layer
        qx, sx = fq.rmsnorm_quantize(qkv["x"], g1, eps)
        fq.fp8_linear(qx, sx, qkv["qw"], qkv["sw"], out=qkv["y"], workspace=ws)
        fq.quant_linear(o["x"], o["qw"], o["sw"], out=o["y"], workspace=ws)
        qx, sx = fq.rmsnorm_quantize(gu["x"], g2, eps)
        fq.fp8_linear(qx, sx, gu["qw"], gu["sw"], out=gu["y"], workspace=ws)
        qh, sh = fq.swiglu_quantize(gu["y"][:, :inter], gu["y"][:, inter:])
        fq.fp8_linear(qh, sh, down["qw"], down["sw"], out=down["y"], workspace=ws)

    def unfused(layer):
        qkv, o, gu, down = layer
        n1 = torch.nn.functional.rms_norm(qkv["x"], (4096,), weight=g1, eps=eps)
        fq.quant_linear(n1, qkv["qw"], qkv["sw"], out=qkv["y"], workspace=ws)
        fq.quant_linear(o["x"], o["qw"], o["sw"], out=o["y"], workspace=ws)
        n2 = torch.nn.functional.rms_norm(gu["x"], (4096,), weight=g2, eps=eps)
        fq.quant_linear(n2, gu["qw"], gu["sw"], out=gu["y"], workspace=ws)
        a = torch.nn.functional.silu(gu["y"][:, :inter]) * gu["y"][:, inter:]
        fq.quant_linear(a, down["qw"], down["sw"], out=down["y"], workspace=ws)

    res = {}
    for name, fn in (("fused", fused), ("two_step", two_step),
                     ("unfused_torch_norm_and_silu", unfused)):
        gr = graph_of(torch, lambda: [fn(L) for L in layers], 1)
        for _ in range(max(5, steps // 4)):
            gr.replay()
        warm_for(torch, gr.replay)
        t, slices = time_chunks(torch, gr.replay, steps)
        t /= copies
        res[name] = {"us_per_layer": round(t * 1e6, 2),
                     "tflops": round(flops / t / 1e12, 2),
                     "gbs": round(nbytes / t / 1e9, 1),
                     "slice_us": spread([ts * 1e6 / copies for ts in slices])}
        del gr
    del layers, base
    torch.cuda.empty_cache()
    res["flops_per_layer"] = flops
    res["bytes_per_layer"] = nbytes
    return res


def bench_kv(torch, fq, reps, t_write=PREFILL_M, t_read=32768, width=1024, group=128):
    """The FP8 E4M3 KV-cache codec: quantizing one prefill chunk's K (or V)
    rows into the cache (t_write tokens x 8 KV heads x 128) and reading a
    t_read-token window back to bf16, one scale per head; GB/s of
    algorithmic bytes (bf16 in/out, codes, scales), HIP-graph replays over
    buffer copies (time_graph)."""
    from workloads import kv_inputs
    x0 = to_dev(kv_inputs(t_write, width, seed=0), torch)
    win = to_dev(kv_inputs(t_read, width, seed=1), torch)
    cache0, cscale0 = fq.kv_quantize_fp8(win, group)
    del win
    qbytes = 3 * t_write * width + 4 * t_write * width // group
    rbytes = 3 * t_read * width + 4 * t_read * width // group
    res = {}
    nq = copies_for(qbytes)
    xs = [x0] + [x0.clone() for _ in range(nq - 1)]
    cq = [torch.empty((t_write, width), dtype=torch.uint8, device="cuda") for _ in range(nq)]
    sq = [torch.empty((t_write, width // group), dtype=torch.float32, device="cuda")
          for _ in range(nq)]
    res["quantize"] = time_graph(
        torch, [(lambda i: lambda: fq.kv_quantize_fp8(xs[i], group, cq[i], sq[i]))(i)
                for i in range(nq)], reps, qbytes)
    del xs, cq, sq
    nr = copies_for(rbytes)
    cs = [cache0] + [cache0.clone() for _ in range(nr - 1)]
    ss = [cscale0] + [cscale0.clone() for _ in range(nr - 1)]
    outs = [torch.empty((t_read, width), dtype=torch.bfloat16, device="cuda")
            for _ in range(nr)]
    res["dequantize"] = time_graph(
        torch, [(lambda i: lambda: fq.kv_dequantize_fp8(cs[i], ss[i], group, out=outs[i]))(i)
                for i in range(nr)], reps, rbytes)
    del cs, ss, outs, x0, cache0, cscale0
    torch.cuda.empty_cache()
    return res


def bench_kv_int8(torch, fq, reps, t_write=PREFILL_M, t_read=32768, width=1024,
                  group=64, residual=128):
    """The INT8 group-wise KV cache with its BF16 residual window (groups of
    64, newest 128 positions in bf16): quantizing t_write tokens into the
    INT8 store, and the cache read of a t_read-token window (t_read - 128
    dequantized history rows followed by the 128-row bf16 tail); GB/s of
    algorithmic bytes, HIP-graph replays over buffer copies."""
    from workloads import kv_inputs
    x0 = to_dev(kv_inputs(t_write, width, seed=0), torch)
    hist = t_read - residual
    win = to_dev(kv_inputs(t_read, width, seed=1), torch)
    codes0, sc0, mn0 = fq.kv_quantize_int8(win[:hist], group)
    tail0 = win[hist:].clone()
    del win
    g = width // group
    qbytes = 3 * t_write * width + 8 * t_write * g
    rbytes = hist * width + 8 * hist * g + 2 * residual * width + 2 * t_read * width
    res = {}
    nq = copies_for(qbytes)
    xs = [x0] + [x0.clone() for _ in range(nq - 1)]
    cq = [torch.empty((t_write, width), dtype=torch.uint8, device="cuda") for _ in range(nq)]
    sq = [torch.empty((t_write, g), dtype=torch.float32, device="cuda") for _ in range(nq)]
    mq = [torch.empty((t_write, g), dtype=torch.float32, device="cuda") for _ in range(nq)]
    res["quantize"] = time_graph(
        torch, [(lambda i: lambda: fq.kv_quantize_int8(xs[i], group, cq[i], sq[i], mq[i]))(i)
                for i in range(nq)], reps, qbytes)
    del xs, cq, sq, mq
    nr = copies_for(rbytes)
    rc = [(codes0, sc0, mn0, tail0)] + [
        (codes0.clone(), sc0.clone(), mn0.clone(), tail0.clone()) for _ in range(nr - 1)]
    outs = [torch.empty((t_read, width), dtype=torch.bfloat16, device="cuda")
            for _ in range(nr)]
    res["read_history_and_tail"] = time_graph(
        torch, [(lambda i: lambda: fq.kv_read_int8(*rc[i][:3], tail=rc[i][3], group=group,
                                                   out=outs[i]))(i)
                for i in range(nr)], reps, rbytes)
    del rc, outs, x0, codes0, sc0, mn0, tail0
    torch.cuda.empty_cache()
    return res


def host_info(threads):
    """The host the CPU leg ran on: logical CPUs, lscpu's model name, the
    BLAS thread count."""
    import subprocess
    model = None
    try:
        res = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=30)
        for line in res.stdout.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:                            # noqa: BLE001 - report only
        pass
    return {"os_cpu_count": os.cpu_count(), "lscpu_model_name": model,
            "blas_threads": int(threads)}


def cpu_baseline(target_s=8.0, decode_frac=4, long_m=1024, long_frac=8):
    """The oracle as it stands, timed on samples of the same workloads, with
    the quantization and the matmul + epilogue timed separately:
    * prefill: all 7 Linears of the M=4096 layer, a subset of tokens and of
      output channels (weights quantized by the oracle beforehand, untimed,
      as the offline step), grown until the timed part reaches ~target_s;
    * decode: the M=1 layer's 7 Linears on 1/decode_frac of their output
      channels, GB/s of the same algorithmic bytes as the GPU figure;
    * long prefill: the 7 Linears once on the long-prefill distribution
      (Student-t, nu = 3, with its all-zero, x1e4 and saturating rows) at
      long_m tokens and 1/long_frac of the output channels."""
    import oracle
    from workloads import LAYER_SHAPES
    from workloads.generators import c3_x, c5_x, outlier_act_bf16, rng_for, weight_bf16
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1

    def run(m_s, n_frac, decode=False, long=False):
        r = dict(flops=0, quant_s=0.0, mm_s=0.0, quant_bytes=0, mm_bytes=0)
        for j, (_, n, k) in enumerate(LAYER_SHAPES):
            n_s = max(16, n // n_frac)
            if long:
                x = c5_x(m_s, k, j)
            elif decode:
                x = outlier_act_bf16(rng_for(2, m_s, j, 0), (m_s, k))
            else:
                x = c3_x(PREFILL_M, k, j, rows=m_s)
            w = weight_bf16(5 if long else 2 if decode else 3, 0, j, n, k, rows=n_s)
            qw, sw = oracle.quant_weight_ref(w)
            t0 = time.perf_counter()
            qx, sx = oracle.quant_act_ref(x)
            t1 = time.perf_counter()
            oracle.linear_ref(qx, sx, qw, sw)
            t2 = time.perf_counter()
            r["quant_s"] += t1 - t0
            r["mm_s"] += t2 - t1
            r["flops"] += 2 * m_s * n_s * k
            r["quant_bytes"] += 3 * m_s * k + 4 * m_s
            r["mm_bytes"] += n_s * k + 4 * n_s + m_s * k + 4 * m_s + 2 * m_s * n_s
        return r

    # Grow the prefill sample until the timed oracle work reaches target_s.
    sizes = [(64, 16), (256, 8), (512, 4), (1024, 4), (2048, 4), (4096, 4), (4096, 2),
             (4096, 1)]
    for m_s, n_frac in sizes:
        r = run(m_s, n_frac)
        if r["quant_s"] + r["mm_s"] >= target_s:
            break
    secs = r["quant_s"] + r["mm_s"]
    d = run(1, decode_frac, decode=True)
    dsecs = d["quant_s"] + d["mm_s"]
    lp = run(long_m, long_frac, long=True)
    lsecs = lp["quant_s"] + lp["mm_s"]
    # Algorithmic bytes of the fused decode call, as on the GPU.
    dbytes = sum(max(16, n // decode_frac) * k + 4 * max(16, n // decode_frac) + 2 * k
                 + 2 * max(16, n // decode_frac) for _, n, k in LAYER_SHAPES)
    return {"value": round(r["flops"] / secs / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"prefill M=4096 layer, {m_s} tokens x 1/{n_frac} of the "
                      f"output channels of each of the 7 Linears; quantize + "
                      f"fp64 matmul + epilogue; {secs:.1f} s",
            "quant_gbs": round(r["quant_bytes"] / r["quant_s"] / 1e9, 3),
            "matmul_gflops": round(r["flops"] / r["mm_s"] / 1e9, 2),
            "matmul_gbs": round(r["mm_bytes"] / r["mm_s"] / 1e9, 3),
            "quant_s": round(r["quant_s"], 3), "matmul_s": round(r["mm_s"], 3),
            "decode": {"value": round(dbytes / dsecs / 1e9, 3), "unit": "GB/s",
                       "sample": f"decode M=1 layer, 1/{decode_frac} of the output "
                                 f"channels of each of the 7 Linears; quantize + fp64 "
                                 f"matmul + epilogue; {dsecs:.2f} s",
                       "quant_s": round(d["quant_s"], 4), "matmul_s": round(d["mm_s"], 3)},
            "long_prefill": {"value": round(lp["flops"] / lsecs / 1e12, 6), "unit": "TFLOP/s",
                             "sample": f"long-prefill distribution (Student-t nu=3 with "
                                       f"all-zero, x1e4 and saturating rows) at {long_m} "
                                       f"tokens x 1/{long_frac} of the output channels of "
                                       f"each of the 7 Linears, once; quantize + fp64 matmul "
                                       f"+ epilogue; {lsecs:.2f} s",
                             "quant_gbs": round(lp["quant_bytes"] / lp["quant_s"] / 1e9, 3),
                             "matmul_gflops": round(lp["flops"] / lp["mm_s"] / 1e9, 2),
                             "quant_s": round(lp["quant_s"], 3),
                             "matmul_s": round(lp["mm_s"], 3)},
            "host": host_info(threads)}


def rocm_smi_clocks():
    """rocm-smi's clock report (sclk, mclk, ...) for GPU 0, taken as a child
    process before this process touches the GPU; None if unavailable."""
    import subprocess
    try:
        res = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                             text=True, timeout=60)
        card = json.loads(res.stdout or "{}").get("card0", {})
        return {k: v for k, v in card.items() if "clock" in k.lower()} or None
    except Exception as e:                       # noqa: BLE001 - report only
        return {"error": f"{type(e).__name__}: {e}"[:200]}


def measured_peaks(torch, reps=10, wg=2048, iters=2048, read_bytes=2 << 30):
    """The two roofs as this GPU sustains them (libfp8w8a8_peaks.so): an
    MFMA-only loop of v_mfma_f32_32x32x64_f8f6f4 (TFLOP/s, and the shader
    clock it ran at from the in-kernel cycle and 100 MHz counters), and a
    streaming read of 2 GiB, 8x the last-level cache (GB/s).  HIP events on
    the stream the kernels are launched on."""
    import ctypes
    from fp8_w8a8_dynamic_amd import build as fbuild
    path = fbuild.PEAKS_LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the library first")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fp8w8a8_peaks_mfma_out_floats.restype = i64
    lib.fp8w8a8_peaks_mfma_out_floats.argtypes = [i64]
    lib.fp8w8a8_peaks_mfma_flops.restype = i64
    lib.fp8w8a8_peaks_mfma_flops.argtypes = [i64, ctypes.c_int]
    lib.fp8w8a8_peaks_read_workgroups.restype = i64
    lib.fp8w8a8_peaks_read_workgroups.argtypes = [i64]
    lib.fp8w8a8_peaks_mfma_loop.restype = ctypes.c_int
    lib.fp8w8a8_peaks_mfma_loop.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.fp8w8a8_peaks_read_stream.restype = ctypes.c_int
    lib.fp8w8a8_peaks_read_stream.argtypes = [vp, i64, vp, vp]
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty(lib.fp8w8a8_peaks_mfma_out_floats(wg), dtype=torch.float32,
                      device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")

    def mfma():
        st = lib.fp8w8a8_peaks_mfma_loop(out.data_ptr(), clk.data_ptr(), wg, iters, stream)
        if st != 0:
            raise RuntimeError(f"fp8w8a8_peaks_mfma_loop: status {st}")

    for _ in range(3):
        mfma()
    torch.cuda.synchronize()
    t = time_events(torch, mfma, reps)
    cycles, ticks = (int(v) for v in clk.cpu())
    mfma_tflops = lib.fp8w8a8_peaks_mfma_flops(wg, iters) / t / 1e12
    del out, clk
    buf = torch.empty(read_bytes, dtype=torch.uint8, device="cuda")
    rout = torch.empty(lib.fp8w8a8_peaks_read_workgroups(read_bytes) * 256,
                       dtype=torch.int32, device="cuda")

    def read():
        st = lib.fp8w8a8_peaks_read_stream(buf.data_ptr(), read_bytes, rout.data_ptr(),
                                           stream)
        if st != 0:
            raise RuntimeError(f"fp8w8a8_peaks_read_stream: status {st}")

    for _ in range(3):
        read()
    torch.cuda.synchronize()
    tr = time_events(torch, read, 2 * reps)
    del buf, rout
    torch.cuda.empty_cache()
    return {"mfma_fp8_tflops": round(mfma_tflops, 1),
            "mfma_loop_sclk_ghz": round(cycles / (ticks / 100e6) / 1e9, 3) if ticks else None,
            "mfma_loop_us": round(t * 1e6, 1),
            "hbm_read_gbs": round(read_bytes / tr / 1e9, 1),
            "hbm_read_us": round(tr * 1e6, 1),
            "what": "MFMA-only loop (2048 workgroups x 4 waves x 8 accumulators x 2048 "
                    "v_mfma_f32_32x32x64_f8f6f4); a persistent read of 2 GiB (1024 workgroups, "
                    "16-byte nontemporal loads, 8 in flight per thread)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks ramp for several milliseconds after an idle period:
    # the warm-up is long enough (tens of ms of work) that the timed steps
    # see the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 36-layer stack leg")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA / HBM-read peaks")
    ap.add_argument("--only-stack", action="store_true",
                    help="run only the 36-layer stack leg (M = 64 and 256) and print "
                         "its figures (for profiling that leg on its own)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; "
                          "run with --gpus 1"}))
        return 2
    smi = None if args.no_peaks else rocm_smi_clocks()
    import torch
    import fp8_w8a8_dynamic_amd as fq
    fq.load_library()
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        # A plain elementwise kernel of known traffic: reads 256 MiB, writes
        # 256 MiB (torch's vectorized add on uint8).
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 3 x (268435456 B read + 268435456 B written)")
        del src, dst
    if args.only_stack:
        passes = [bench_stack(torch, fq, m, max(3, args.steps // 20)) for m in (64, 256)]
        print(json.dumps({"stack_36_layers": {"passes": passes}}), flush=True)
        return 0
    log("prefill ...")
    pre = bench_prefill(torch, fq, args.steps, args.warmup)
    tflops = pre["flops"] / pre["step_time"] / 1e12
    log(f"prefill step {pre['step_time']*1e6:.1f} us  {tflops:.1f} TFLOP/s; "
        f"GEMM alone {pre['gemm_tflops']:.1f} TFLOP/s")
    dec = None
    if not args.no_decode:
        log("decode ...")
        dec = bench_decode(torch, fq, max(20, args.steps))
        log(f"decode layer {dec['layer_us']:.2f} us  {dec['gbs']:.0f} GB/s; one launch "
            f"{dec['single_launch']}")
        from workloads import LAYER_SHAPES
        dec_floor = launch_floor(torch, [n * k for _, n, k in LAYER_SHAPES])
        dec_floor["what"] = ("plain streaming reads of the 7 weight matrices' bytes as 7 "
                             "launches in a graph, against one read of their sum")
        log(f"launch floor {dec_floor}")
        dec_more = {mm: bench_decode(torch, fq, max(20, args.steps // 2), m=mm)
                    for mm in (4, 8)}
        log("decode M=4, 8: " + ", ".join(f"{v['layer_us']:.1f} us {v['gbs']:.0f} GB/s "
                                          f"(grouped {v['grouped']['us_per_layer']} us)"
                                          for v in dec_more.values()))
    log("packed layer ...")
    pre_p = bench_prefill(torch, fq, args.steps, args.warmup, packed=True)
    packed = {"linears": "qkv_proj (6144x4096), o_proj, gate_up_proj (24576x4096), "
                         "down_proj: 4 calls, one quantization per distinct input",
              "prefill": {"value": round(pre_p["flops"] / pre_p["step_time"] / 1e12, 2),
                          "unit": "TFLOP/s",
                          "ms_per_step": round(pre_p["step_time"] * 1e3, 4),
                          "slice_tflops": spread(pre_p["slices"])}}
    log(f"packed prefill {packed['prefill']}")
    if not args.no_decode:
        dec_p = bench_decode(torch, fq, max(20, args.steps), packed=True)
        packed["decode"] = {"slice_gbs": spread(dec_p["slices"]),
                            "value": round(dec_p["gbs"], 1), "unit": "GB/s",
                            "us_per_layer": round(dec_p["layer_us"], 3),
                            "frac_of_hbm": round(dec_p["gbs"] / HBM_PEAK_GBS, 4),
                            "per_linear": dec_p["per_linear"]}
        log(f"packed decode {packed['decode']}")
    stack = None
    if not args.no_stack:
        log("36-layer stack ...")
        stack = [bench_stack(torch, fq, m, max(5, args.steps // 20)) for m in (64, 256)]
        log(f"stack {stack}")
    log("rmsnorm -> quant ...")
    norm = bench_norm(torch, fq, args.steps)
    norm_dec = bench_norm(torch, fq, args.steps, m=DECODE_M)
    log(f"rmsnorm quant {norm}; M=1 {norm_dec['fused']['us']} us")
    log("swiglu -> quant ...")
    swi = bench_swiglu(torch, fq, args.steps)
    swi_dec = bench_swiglu(torch, fq, args.steps, m=DECODE_M)
    log(f"swiglu quant {swi}; M=1 {swi_dec['fused']['us']} us")
    log("kv cache codec ...")
    kv = bench_kv(torch, fq, args.steps)
    log(f"kv fp8 {kv}")
    kv8 = bench_kv_int8(torch, fq, args.steps)
    log(f"kv int8 {kv8}")
    log("layer with fused norms and activation ...")
    fl = bench_fused_layer(torch, fq, PREFILL_M, max(20, args.steps // 4))
    fl_dec = None
    if not args.no_decode:
        fl_dec = bench_fused_layer(torch, fq, DECODE_M, max(20, args.steps), DECODE_COPIES)
    log(f"fused layer M=4096 {fl}; M=1 {fl_dec}")
    peaks = None
    if not args.no_peaks:
        log("measured peaks ...")
        peaks = measured_peaks(torch)
        peaks["rocm_smi_before_run"] = smi
        log(f"measured peaks {peaks}")
    cpu = None
    if not args.no_cpu:
        log("cpu oracle ...")
        cpu = cpu_baseline()
        log(f"cpu oracle {cpu}")

    out = {
        "metric": "FP8_DYNAMIC linear TFLOP/s @M=4096 (%MFMA peak); GB/s @M=1 (%HBM)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["step_time"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> f32 acc -> bf16",
        "data": "synthetic (seeded; no datasets or trained weights)",
        "config": {"workload": "prefill chunk of one self-attention layer: "
                               "M=4096 tokens through q,k,v,o (4096|1024 x 4096), "
                               "gate,up (12288 x 4096), down (4096 x 12288); "
                               "fused per-token quant + FP8 GEMM + epilogue",
                   "m": PREFILL_M, "linears": 7,
                   "frac_of_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
                   "slice_tflops": spread(pre["slices"])},
        "roofline": {"bound": "mfma", "achieved": round(pre["gemm_tflops"], 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre["gemm_tflops"] / FP8_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic(),
                     "traffic_scope": "HBM bytes of one step's 7 GEMM dispatches "
                                      "(rocprofv3 FETCH_SIZE x2 + WRITE_SIZE); "
                                      "algorithmic 663 MB",
                     "kernel": "gemm_fp8_kernel",
                     "mfma_busy": {
                         "counted_equals_algorithmic":
                             True if code_sha1(KERNEL_TRAFFIC["gemm"]["files"])
                             == KERNEL_TRAFFIC["gemm"]["sha1"] else None,
                         "frac_of_gemm_time_at_2p4ghz": round(
                             pre["gemm_tflops"] * 1e12 * 64 / (131072 * 1024) / 2.4e9, 4),
                         "source": "profiles/gemm_fp8_kernel_mfma_busy_lds_conflicts_"
                                   "prefill_layer.txt (SQ_VALU_MFMA_BUSY_CYCLES / 1024 "
                                   "SIMDs = the algorithmic 64 cycles per MFMA)"},
                     "library_same_operands_tflops": pre.get("lib_tflops"),
                     "library": "hipBLASLt via torch._scaled_mm, row-wise scales (comparison only)",
                     "per_linear": pre["per_linear"]},
    }
    if dec is not None:
        out["decode"] = {"m": DECODE_M, "metric": "GB/s of algorithmic bytes, "
                         "7 fused calls of one layer, HIP graph replay",
                         "value": round(dec["gbs"], 1), "unit": "GB/s",
                         "us_per_layer": round(dec["layer_us"], 3),
                         "frac_of_hbm": round(dec["gbs"] / HBM_PEAK_GBS, 4),
                         "bytes_per_layer": dec["bytes"],
                         "slice_gbs": spread(dec["slices"]),
                         "per_linear": dec["per_linear"],
                         "single_launch": dict(
                             dec["single_launch"] or {},
                             what="the same 7 Linears of the layer (independent inputs) "
                                  "as ONE grouped call, fp8w8a8_quant_linear_group_m1 "
                                  "(outputs bit-identical to the 7 calls)",
                             kernel="gemv_group_kernel",
                             traffic=kernel_traffic("gemv_group"),
                             traffic_scope="HBM bytes of one launch (one layer; rocprofv3 "
                                           "FETCH_SIZE x2 + WRITE_SIZE); algorithmic "
                                           "193,245,184"),
                         "launch_floor": dec_floor,
                         "other_token_counts": {
                             f"m{mm}": {"value": round(v["gbs"], 1), "unit": "GB/s",
                                        "us_per_layer": round(v["layer_us"], 3),
                                        "frac_of_hbm": round(v["gbs"] / HBM_PEAK_GBS, 4),
                                        "grouped": v["grouped"]}
                             for mm, v in dec_more.items()}}
    out["packed"] = packed
    if stack is not None:
        out["stack_36_layers"] = {
            "metric": "one pass of the 36-layer stack (252 fused calls, 6.946 GB of "
                      "FP8 weights in HBM, layer outputs chained), captured in a HIP "
                      "graph and replayed: GB/s of algorithmic bytes and TFLOP/s "
                      "(eager_ms_per_pass: the same calls launched from Python)",
            "passes": stack}
    f = norm["fused"]
    out["rmsnorm_quant"] = {
        "workload": f"BF16 RMSNorm fused with per-token FP8 quantization of its output, "
                    f"M={PREFILL_M}, hidden 4096 (the input norm of q/k/v and gate/up)",
        "roofline": {"bound": "hbm", "achieved": f["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": f["frac_of_hbm"],
                     "traffic": kernel_traffic("rmsnorm_quant"),
                     "traffic_scope": "HBM bytes of one launch without the norm output "
                                      "(rocprofv3 FETCH_SIZE x2 + WRITE_SIZE); "
                                      "algorithmic 50,356,224",
                     "kernel": "rmsnorm_quant_kernel"},
        "m4096": norm, "m1_us": norm_dec["fused"]["us"]}
    f = swi["fused"]
    out["swiglu_quant"] = {
        "workload": f"SiLU-gated activation fused with per-token FP8 quantization of its "
                    f"output, M={PREFILL_M}, width 12288 (gate/up halves of the packed "
                    f"gate_up output -> down_proj's input)",
        "roofline": {"bound": "hbm", "achieved": f["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": f["frac_of_hbm"],
                     "traffic": kernel_traffic("swiglu_quant"),
                     "traffic_scope": "HBM bytes of one launch without the activation "
                                      "output (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE); "
                                      "algorithmic 251,674,624",
                     "kernel": "swiglu_quant_kernel"},
        "m4096": swi, "m1_us": swi_dec["fused"]["us"]}
    d = kv["dequantize"]
    out["kv_cache_fp8"] = {
        "workload": "FP8 E4M3 KV-cache codec, 8 KV heads x 128, one scale per "
                    "(token, head): quantize a 4096-token chunk into the cache, read a "
                    "32768-token window back to bf16",
        "roofline": {"bound": "hbm", "achieved": d["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": d["frac_of_hbm"],
                     "traffic": kernel_traffic("kv_dequant"),
                     "traffic_scope": "HBM bytes of one 32768-token read (rocprofv3 "
                                      "FETCH_SIZE x2 + WRITE_SIZE); algorithmic 101,711,872",
                     "kernel": "kv_dequant_kernel"},
        "quantize": kv["quantize"], "dequantize": d}
    d = kv8["read_history_and_tail"]
    out["kv_cache_int8"] = {
        "workload": "INT8 group-wise KV cache (groups of 64, min-max) with the newest 128 "
                    "positions in bf16: quantize a 4096-token chunk into the INT8 store, "
                    "read a 32768-token window (32640 history + 128 tail) back to bf16",
        "roofline": {"bound": "hbm", "achieved": d["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": d["frac_of_hbm"],
                     "traffic": kernel_traffic("kv_int8_read"),
                     "traffic_scope": "HBM bytes of one 32768-token read (rocprofv3 "
                                      "FETCH_SIZE x2 + WRITE_SIZE); algorithmic 104,972,288",
                     "kernel": "kv_int8_read_kernel"},
        "quantize": kv8["quantize"], "read": d}
    out["layer_with_fusions"] = {
        "workload": "one layer's Linear path with the adjacent fusions: "
                    "rmsnorm_quant_linear(q|k|v), quant_linear(o), "
                    "rmsnorm_quant_linear(gate|up), swiglu_quant_linear(down) "
                    "(attention and residual adds excluded), beside the same chain as "
                    "separate pre-step + fp8_linear calls (two_step) and with torch bf16 "
                    "rms_norm / silu*up feeding quant_linear",
        "m4096": fl, "m1": fl_dec}
    if peaks is not None:
        out["measured_peaks"] = peaks
        # Every roofline also against what this GPU sustained in the same run.
        for key in ("roofline", "rmsnorm_quant", "swiglu_quant", "kv_cache_fp8",
                    "kv_cache_int8"):
            rf = out[key] if key == "roofline" else out[key]["roofline"]
            meas = peaks["mfma_fp8_tflops"] if rf["bound"] == "mfma" else peaks["hbm_read_gbs"]
            rf["measured_peak"] = meas
            rf["frac_of_measured_peak"] = round(rf["achieved"] / meas, 4)
        for d in (out.get("decode"), out["packed"].get("decode")):
            if d:
                d["frac_of_measured_hbm"] = round(d["value"] / peaks["hbm_read_gbs"], 4)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
