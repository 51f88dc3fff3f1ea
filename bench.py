"""Benchmark of the theta-bundle reconstructed linear on one MI355X.

Default workload (one JSON line on stdout): the Gemma-3-1B-shaped decoder,
26 layers, bf16, rank 16, decode batches M = 1, 4 and 16 tokens.  One step is a
full pass of all 26 layers at each of the three batch sizes; a layer is four
dispatches (fused Q/K/V, o, fused gate/up, down).  The weights of all 26 layers
(1.4 GB of W0) stay resident in HBM, far beyond the 256 MB Infinity Cache, and
are visited in model order, so every dispatch streams its weights from HBM.

Other workloads (``--workload``): gemma_prefill (M = 512, 2048; rank 64),
large_decoder (8 layers in 4 shared-W0 bands, rank 32, M = 1, 32, 512),
materialize_fp4 (7 families x 26 layers, 13 bands, rank 64: W_eff then FP4).

The step is timed as a captured HIP graph (launch cost excluded, as in serving)
and, for comparison, eagerly.  The dominant kernel is also timed per launch with
HIP events on the launch stream, queued behind a GPU sleep so that no CPU launch
gap falls inside an event pair.  The CPU baseline is the fp64 oracle on a bounded
sample of the same workload, on this host's cores.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6    # dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- workload

class Call:
    """One pre-marshalled C-ABI call (pointers, strides and stream fixed)."""

    def __init__(self, fn, args, nbytes, flops, name, grid_key):
        self.fn, self.args = fn, args
        self.nbytes, self.flops, self.name, self.grid_key = nbytes, flops, name, grid_key

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            from rank_shared_block_amd import binding as B
            raise RuntimeError(f"{self.name}: {B.status_string(st)}: {B.last_error()}")


def _dispatch_bytes(M, K, bundles):
    """Algorithmic bytes of one recon dispatch (bf16): every operand once."""
    b = M * K * 2
    for (N, r) in bundles:
        b += (N * K + N + N * r + r * K) * 2 + M * N * 2
    return b


def _dispatch_flops(M, K, bundles):
    f = 0
    for (N, r) in bundles:
        f += 2 * M * K * (N + r) + 2 * M * r * N
    return f


def make_recon_calls(torch, B, I, shapes, layer_dev, layer_np, M, x_tag, dtype="bf16"):
    """Per layer, the four dispatches as pre-marshalled calls."""
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream().cuda_stream
    calls = []
    keep = []
    lib = B.lib()
    for l, fam_dev in enumerate(layer_dev):
        for name, fams in I.LAYER_DISPATCHES:
            K = shapes[fams[0]][0]
            x = torch.from_numpy(I.activations("gemma_decode", x_tag + len(name), M, K, dtype)).to(dev).to(torch.bfloat16)
            projs = [B.make_proj(*fam_dev[f]) for f in fams]
            arr = (B.aq_proj * len(fams))(*projs)
            ntot = sum(p.N for p in projs)
            y = torch.empty((M, ntot), dtype=torch.bfloat16, device=dev)
            need = lib.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, K, arr, len(fams))
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            fn = {"qkv": lib.aq_recon_qkv_fused, "gateup": lib.aq_recon_gateup_fused}.get(name, lib.aq_recon_linear)
            args = (B.AQ_BF16, M, K, x.data_ptr(), K, arr, y.data_ptr(), ntot, ws.data_ptr(), ws.numel(), stream)
            nr = [(shapes[f][1], layer_np[l][f]["U"].shape[1]) for f in fams]
            calls.append(Call(fn, args, _dispatch_bytes(M, K, nr), _dispatch_flops(M, K, nr), f"L{l}.{name}.M{M}", name))
            keep += [x, y, ws, arr]
    return calls, keep


def upload_layers(torch, I, layer_np):
    dev = torch.device("cuda", 0)
    shared = {}
    out = []
    for l in sorted(layer_np):
        d = {}
        for f, bd in layer_np[l].items():
            key = id(bd["W0"])
            if key not in shared:
                shared[key] = torch.from_numpy(bd["W0"]).to(dev).to(torch.bfloat16)
            d[f] = (shared[key],) + tuple(torch.from_numpy(bd[k]).to(dev).to(torch.bfloat16) for k in ("s", "U", "Vt"))
        out.append(d)
    return out


# --------------------------------------------------------------------------- timing

def time_graph(torch, calls, steps, warmup):
    """Capture `calls` in one HIP graph; replay warmup + steps; return ms per replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:             # eager warm-up on the capture stream
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        # the calls were marshalled with the ambient stream; re-marshal for the capture stream
        cap = torch.cuda.current_stream().cuda_stream
        for c in calls:
            a = list(c.args)
            a[-1] = cap
            st = c.fn(*a)
            assert st == 0, c.name
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, g


def time_graph_streams(torch, calls, nstreams, steps, warmup):
    """Like time_graph, but the calls (independent of each other) are issued
    round-robin on `nstreams` streams forked from and joined back to the capture
    stream, as a loader issues independent projections."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    side = [torch.cuda.Stream() for _ in range(nstreams)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for st in side:
            st.wait_stream(cap)
        for i, c in enumerate(calls):
            st = side[i % nstreams]
            a = list(c.args)
            a[-1] = st.cuda_stream
            assert c.fn(*a) == 0, c.name
        for st in side:
            cap.wait_stream(st)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_eager(torch, calls, steps, warmup):
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        for c in calls:
            c()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_per_launch(torch, calls, reps):
    """Average duration of one launch of `calls`' kernel: HIP events around
    replays of a graph that holds only these launches back to back, on the
    stream the graph runs on.  Consecutive kernels of a graph abut on the GPU,
    so this equals the average kernel duration that rocprofv3 reports for the
    same replays (start to start)."""
    ms, _ = time_graph(torch, calls, reps, 2)
    return ms / len(calls)


# --------------------------------------------------------------------------- CPU baseline

def cpu_baseline(I, layer_np, shapes, Ms, x_tag, budget_s, layers_sample):
    """The oracle on a bounded sample: `layers_sample` layers, every M, repeated
    until `budget_s` of oracle time; returns GB/s of algorithmic bytes."""
    import oracle
    from threadpoolctl import threadpool_info
    ls = sorted(layer_np)[:layers_sample]
    conv = {}
    for l in ls:
        for f, bd in layer_np[l].items():
            conv[(l, f)] = tuple(bd[k].astype(np.float64) for k in ("W0", "s", "U", "Vt"))
    xs = {}
    for M in Ms:
        for name, fams in I.LAYER_DISPATCHES:
            K = shapes[fams[0]][0]
            xs[(M, name)] = I.activations("gemma_decode", x_tag(M) + len(name), M, K, "bf16").astype(np.float64)
    nbytes, t_used, passes = 0, 0.0, 0
    while t_used < budget_s:
        for M in Ms:
            for l in ls:
                for name, fams in I.LAYER_DISPATCHES:
                    K = shapes[fams[0]][0]
                    t0 = time.perf_counter()
                    oracle.recon_fused(xs[(M, name)], [conv[(l, f)] for f in fams])
                    t_used += time.perf_counter() - t0
                    nbytes += _dispatch_bytes(M, K, [(shapes[f][1], conv[(l, f)][2].shape[1]) for f in fams])
        passes += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(nbytes / t_used / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(ls)} of 26 layers x M in {list(Ms)} x 4 dispatches, {passes} passes, "
                      f"{t_used:.1f} s of numpy float64 oracle time (bf16->fp64 conversion excluded)"}


# --------------------------------------------------------------------------- counters

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SOURCES = {"decode_gateup": "rank_shared_block_amd/csrc/recon_decode.hip",
           "fp4_gemv_gateup": "rank_shared_block_amd/csrc/fp4_gemv.hip"}
PMC_KERNELS = {"decode_gateup": (("k_decode_bf16",), "k_decode_bf16 (fused gate/up)"),
               "fp4_gemv_gateup": (("k_fp4_gemv", "<2, false>"), "k_fp4_gemv / k_fp4_gemv_m4 (FP4 stacked gate/up)")}


def source_digest(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(key):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256_16") != source_digest(SOURCES[key]):
        return None
    return t.get("bytes_per_launch")


def run_pmc_probe(args, torch, B, I):
    """Workload for the counter runs: a plain copy of known size (calibration),
    then the 78 fused gate/up launches of a bench step, eagerly."""
    dev = torch.device("cuda", 0)
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    layer_np = I.layer_bundles("gemma_decode", I.GEMMA_1B, layers=26, r=16, dtype="bf16",
                               families=("gate", "up"))
    layer_dev = upload_layers(torch, I, layer_np)
    for M in (1, 4, 16):
        lib = B.lib()
        stream = torch.cuda.current_stream().cuda_stream
        for l in range(26):
            x = torch.from_numpy(I.activations("gemma_decode", 10 * M + 6, M, 1152, "bf16")).to(dev).to(torch.bfloat16)
            arr = (B.aq_proj * 2)(*[B.make_proj(*layer_dev[l][f]) for f in ("gate", "up")])
            y = torch.empty((M, 13824), dtype=torch.bfloat16, device=dev)
            need = lib.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, 1152, arr, 2)
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            st = lib.aq_recon_gateup_fused(B.AQ_BF16, M, 1152, x.data_ptr(), 1152, arr, y.data_ptr(), 13824,
                                           ws.data_ptr(), ws.numel(), stream)
            assert st == 0
    torch.cuda.synchronize()
    return {"probe": "copy of %d bytes, then 78 fused gate/up decode launches" % CALIB_BYTES}


def run_pmc_probe_fp4(args, torch, B, I):
    """Counter-run workload for the FP4 GEMV: the copy calibration, then 78
    stacked gate/up launches (13824 x 1152 packed; 26 layers, each its own
    weight, x M in {1, 4, 16}), eagerly."""
    dev = torch.device("cuda", 0)
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    N, K = 13824, 1152
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    packs = [B.quant_fp4_block16((torch.randn(N, K, device=dev, generator=g) * K ** -0.5).to(torch.bfloat16))
             for _ in range(26)]
    for M in (1, 4, 16):
        x = (torch.randn(M, K, device=dev, generator=g)).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for l in range(26):
            B.fp4_linear(x, *packs[l], y=y)
    torch.cuda.synchronize()
    return {"probe": "copy of %d bytes, then 78 FP4 stacked gate/up GEMV launches" % CALIB_BYTES}


CALIB_BYTES = 256 * 2 ** 20


def summarize_profiles(args):
    """Turn rocprofv3 CSV output (kernel trace, and optionally the two counter
    runs) into the markdown summary committed under profiles/."""
    import csv
    import collections

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    out = []
    if args.trace:
        tr = rows(args.trace)
        agg = collections.defaultdict(list)
        for r in tr:
            wg = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) // int(r["Workgroup_Size_X"])
            agg[(r["Kernel_Name"], wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out.append("| kernel | workgroups | launches | avg us | median us | total us |")
        out.append("|---|---|---|---|---|---|")
        for (name, wg), d in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:14]:
            d.sort()
            out.append(f"| `{name[:80]}` | {wg} | {len(d)} | {sum(d)/len(d):.3f} | {d[len(d)//2]:.3f} | {sum(d):.1f} |")
        if args.calls:
            # A prefill call is its kernels in launch order up to the main GEMM
            # (MODE 0, which may also run the rank-r pass in its first
            # workgroups), or up to the fold that follows a K-split main GEMM
            # (MODE 1).
            seq = []
            for r in sorted(tr, key=lambda r: int(r["Start_Timestamp"])):
                if "aq::" not in r["Kernel_Name"]:
                    continue
                name = r["Kernel_Name"].split("(")[0].replace("void aq::", "").replace("aq::", "")
                wg = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) // int(r["Workgroup_Size_X"])
                seq.append((name, wg, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
            def mode(n):             # k_gemm_bf16<BM, BN, BK, NST, MODE, NW>
                return int(n[n.index("<") + 1:-1].split(", ")[4]) if n.startswith("k_gemm_bf16<") else -1
            calls, cur = collections.defaultdict(list), []
            for k in seq:
                cur.append(k)
                # a call ends with its main pass (MODE 0, or 3: tiles with their
                # own t), or with the fold after a K-split main pass (MODE 1)
                if mode(k[0]) in (0, 3) or (k[0] == "k_prefill_reduce" and any(mode(c[0]) == 1 for c in cur)):
                    calls[tuple((c[0], c[1]) for c in cur)].append([c[2] for c in cur])
                    cur = []
            out.append("")
            out.append("| calls | kernels (grid) in order: mean us | total us |")
            out.append("|---|---|---|")
            for key, runs in sorted(calls.items(), key=lambda kv: -sum(map(sum, kv[1])) / len(kv[1]) * len(kv[1])):
                means = [sum(r[i] for r in runs) / len(runs) for i in range(len(key))]
                parts = " + ".join(f"`{key[i][0]}` [{key[i][1]}] {means[i]:.2f}" for i in range(len(key)))
                out.append(f"| {len(runs)} | {parts} | {sum(means):.2f} |")
    if args.fetch and args.write:
        res = {}
        for key, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
            rs = rows(path)
            val = lambda r: float(r.get("Counter_Value", r.get("value", 0)))
            copy = [val(r) for r in rs if "copyBuffer" in r["Kernel_Name"]]
            dec = [val(r) for r in rs if all(k in r["Kernel_Name"] for k in PMC_KERNELS[args.traffic_key][0])]
            res[key] = (max(copy) if copy else None, float(np.mean(dec)) if dec else None, len(dec))
        # scale: a copy of CALIB_BYTES reads and writes CALIB_BYTES each
        fscale = CALIB_BYTES / (res["FETCH_SIZE"][0] * 1024)
        wscale = CALIB_BYTES / (res["WRITE_SIZE"][0] * 1024)
        fetch_b = res["FETCH_SIZE"][1] * 1024 * fscale
        write_b = res["WRITE_SIZE"][1] * 1024 * wscale
        out.append("")
        out.append(f"FETCH_SIZE copy calibration: {res['FETCH_SIZE'][0]:.0f} KiB for {CALIB_BYTES} B read "
                   f"(scale {fscale:.4f}); WRITE_SIZE: {res['WRITE_SIZE'][0]:.0f} KiB for {CALIB_BYTES} B written "
                   f"(scale {wscale:.4f}).")
        out.append(f"{PMC_KERNELS[args.traffic_key][1]}, mean over {res['FETCH_SIZE'][2]} launches: "
                   f"fetch {fetch_b/1e6:.3f} MB, write {write_b/1e6:.3f} MB per launch "
                   f"(scaled), total {(fetch_b + write_b)/1e6:.3f} MB.")
        t = {}
        try:
            with open(TRAFFIC_FILE) as f:
                t = json.load(f)
        except (OSError, ValueError):
            pass
        t[args.traffic_key] = {"bytes_per_launch": int(fetch_b + write_b), "fetch_bytes": int(fetch_b),
                               "write_bytes": int(write_b), "fetch_scale": fscale, "write_scale": wscale,
                               "source_sha256_16": source_digest(SOURCES[args.traffic_key])}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
    print("\n".join(out))


# --------------------------------------------------------------------------- workloads

def run_gemma_decode(args, torch, B, I):
    Ms = (1, 4, 16)
    L = 26
    t0 = time.time()
    layer_np = I.layer_bundles("gemma_decode", I.GEMMA_1B, layers=L, r=16, dtype="bf16")
    log(f"generated inputs in {time.time() - t0:.1f} s")
    layer_dev = upload_layers(torch, I, layer_np)
    torch.cuda.synchronize()
    log(f"uploaded {L} layers")
    xtag = lambda M: 10 * M
    per_M = {}
    all_calls = []
    keep = []
    for M in Ms:
        calls, k = make_recon_calls(torch, B, I, I.GEMMA_1B, layer_dev, layer_np, M, xtag(M))
        keep += k
        per_M[M] = calls
        all_calls += calls
    step_bytes = sum(c.nbytes for c in all_calls)

    # Headline: one graph for the whole step.
    ms_step, g = time_graph(torch, all_calls, args.steps, args.warmup)
    log(f"graph step: {ms_step:.4f} ms")
    us_layer = {}
    for M in Ms:
        ms, _ = time_graph(torch, per_M[M], max(5, args.steps // 2), 2)
        us_layer[f"M{M}"] = round(ms * 1e3 / L, 3)
    ms_eager = time_eager(torch, all_calls, max(3, args.steps // 4), 1)

    # Dominant kernel: the fused gate/up dispatch (59% of the bytes of a layer).
    gu = [c for c in all_calls if c.grid_key == "gateup"]
    avg_ms = time_per_launch(torch, gu, max(5, args.roofline_reps))
    gu_bytes = float(np.mean([c.nbytes for c in gu]))
    achieved = gu_bytes / (avg_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic("decode_gateup"),
            "kernel": "k_decode_bf16 (fused gate/up, K=1152, N=2x6912, r=16, M in {1,4,16}, 26 layers)",
            "bytes_per_launch": int(gu_bytes), "avg_launch_us": round(avg_ms * 1e3, 3),
            "launches_per_replay": len(gu)}

    line = {
        "metric": "reconstructed-linear µs/layer + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1/in) W0, U(0.9,1.1) s, N(0,0.02) U/V, N(0,1) x)",
        "config": {"workload": "gemma-3-1b-shaped decode: 26 layers x (fused QKV, o, fused gate/up, down), "
                               "hidden 1152, rank 16, bf16, M in {1,4,16} tokens per step",
                   "layers": L, "rank": 16, "tokens": list(Ms), "launch": "hip graph per step"},
        "us_per_layer": us_layer,
        "frac_of_hbm_peak_step": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "bytes_per_step": int(step_bytes),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(I, layer_np, I.GEMMA_1B, Ms, xtag, args.cpu_budget, 4)
    return line


def run_gemma_prefill(args, torch, B, I):
    Ms = (512, 2048)
    L = args.layers or 26
    layer_np = I.layer_bundles("gemma_prefill", I.GEMMA_1B, layers=L, r=64, dtype="bf16")
    layer_dev = upload_layers(torch, I, layer_np)
    res = {}
    for M in Ms:
        calls, keep = make_recon_calls(torch, B, I, I.GEMMA_1B, layer_dev, layer_np, M, 5 * M)
        ms, _ = time_graph(torch, calls, args.steps, args.warmup)
        fl = sum(c.flops for c in calls)
        # dense baseline: torch.matmul (hipBLASLt) on W_eff of the identical stacked shapes
        dense = []
        dev = torch.device("cuda", 0)
        for l in range(L):
            for name, fams in I.LAYER_DISPATCHES:
                K = I.GEMMA_1B[fams[0]][0]
                N = sum(I.GEMMA_1B[f][1] for f in fams)
                dense.append((torch.randn(M, K, device=dev, dtype=torch.bfloat16),
                              torch.randn(N, K, device=dev, dtype=torch.bfloat16) * 0.03))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        outs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for x, w in dense:
                torch.matmul(x, w.t())
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(g):
            for x, w in dense:
                outs.append(torch.matmul(x, w.t()))
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_dense = e0.elapsed_time(e1) / args.steps
        dfl = sum(2 * x.shape[0] * x.shape[1] * w.shape[0] for x, w in dense)
        res[f"M{M}"] = {"us_per_layer": round(ms * 1e3 / L, 2), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                        "frac_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                        "dense_us_per_layer": round(ms_dense * 1e3 / L, 2),
                        "dense_tflops": round(dfl / (ms_dense * 1e-3) / 1e12, 1),
                        "recon_over_dense": round(ms / ms_dense, 3)}
        del dense, outs, g
    return {"workload": f"gemma-3-1b-shaped prefill, {L} layers, rank 64, bf16", "results": res}


def run_large_decoder(args, torch, B, I):
    Ms = (1, 32, 512)
    L = 8
    layer_np = I.layer_bundles("large_decoder", I.LARGE_DECODER, layers=L, r=32, dtype="bf16", num_bands=4)
    layer_dev = upload_layers(torch, I, layer_np)
    res = {}
    for M in Ms:
        calls, keep = make_recon_calls(torch, B, I, I.LARGE_DECODER, layer_dev, layer_np, M, 9 * M)
        ms, _ = time_graph(torch, calls, args.steps, args.warmup)
        nb = sum(c.nbytes for c in calls)
        fl = sum(c.flops for c in calls)
        res[f"M{M}"] = {"us_per_layer": round(ms * 1e3 / L, 2),
                        "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                        "note": "bands of 2 layers share W0: the second layer may hit the Infinity Cache"}
    return {"workload": "large-decoder-shaped, 8 layers in 4 W0 bands, rank 32, bf16", "results": res}


def run_materialize_fp4(args, torch, B, I):
    L, G = 26, 13
    layer_np = I.layer_bundles("materialize_fp4", I.GEMMA_1B, layers=L, r=64, dtype="bf16", num_bands=G)
    layer_dev = upload_layers(torch, I, layer_np)
    dev = torch.device("cuda", 0)
    lib = B.lib()
    stream = torch.cuda.current_stream().cuda_stream
    mats, packs, keep = [], [], []
    mbytes = pbytes = 0
    for l in range(L):
        for f in I.FAMILIES:
            K, N = I.GEMMA_1B[f]
            bd = layer_dev[l][f]
            w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
            p = B.make_proj(*bd)
            pa = (B.aq_proj * 1)(p)
            mats.append(Call(lib.aq_materialize_weff, (B.AQ_BF16, K, pa, w.data_ptr(), K, stream),
                             (2 * N * K + N + N * 64 + 64 * K) * 2, 2 * N * K * 64, f"mat.L{l}.{f}", "mat"))
            packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
            gs = torch.empty((1,), dtype=torch.float32, device=dev)
            wsb = 65536 + 4096
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            packs.append(Call(lib.aq_quant_fp4_block16, (N, K, w.data_ptr(), K, packed.data_ptr(), sc.data_ptr(),
                                                         gs.data_ptr(), ws.data_ptr(), wsb, stream),
                              2 * N * K * 2 + N * K // 2 + N * K // 16, 0, f"fp4.L{l}.{f}", "fp4"))
            keep += [w, packed, sc, gs, ws, pa]
            mbytes += mats[-1].nbytes
            pbytes += packs[-1].nbytes
    ms_m, _ = time_graph(torch, mats, args.steps, args.warmup)
    ms_p, _ = time_graph(torch, packs, args.steps, args.warmup)
    ms_m4 = time_graph_streams(torch, mats, 4, args.steps, args.warmup)
    ms_p4 = time_graph_streams(torch, packs, 4, args.steps, args.warmup)
    mat_avg = time_per_launch(torch, mats, 2)
    # the largest projections alone (gate, up, down: 6912 x 1152 elements)
    big = [c for c in mats if c.name.split(".")[-1] in ("gate", "up", "down")]
    big_avg = time_per_launch(torch, big, 2)
    big_bytes = big[0].nbytes

    def leg(ms, nb):
        return {"ms": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return {"workload": "materialise + FP4 pack, 7 families x 26 layers (Gemma-3-1B shapes), 13 W0 bands, rank 64",
            "note": "serial: the 182 calls of each kind back to back in one graph; 4 streams: the same "
                    "independent calls round-robin on 4 streams inside one graph",
            "materialize": dict(leg(ms_m, mbytes), bytes=mbytes, avg_launch_us=round(mat_avg * 1e3, 2),
                                streams4=leg(ms_m4, mbytes),
                                largest_projection={"bytes": big_bytes, "avg_launch_us": round(big_avg * 1e3, 2),
                                                    "GBps": round(big_bytes / (big_avg * 1e-3) / 1e9, 1)}),
            "fp4_pack": dict(leg(ms_p, pbytes), bytes=pbytes, streams4=leg(ms_p4, pbytes))}


def run_fp4_decode(args, torch, B, I):
    """Gemma-3-1B-shaped decode layer on FP4-packed W_eff: the four dispatches
    (stacked QKV 1536 x 1152, o 1152 x 1024, stacked gate/up 13824 x 1152, down
    1152 x 6912) per layer, 26 layers, M in {1, 4, 16}; each layer's weights are
    its own W_eff (materialised from the materialise workload's rank-64
    bundles in 13 W0 bands) packed on the GPU."""
    L = 26
    layer_np = I.layer_bundles("materialize_fp4", I.GEMMA_1B, layers=L, r=64, dtype="bf16", num_bands=13)
    dev = torch.device("cuda", 0)
    lib = B.lib()
    stream = torch.cuda.current_stream().cuda_stream
    groups = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",))]
    packed = []                        # per layer: [(name, N, K, packed, scales, g)]
    layer_dev = upload_layers(torch, I, layer_np)
    for l in range(L):
        row = []
        for name, fams in groups:
            w = torch.cat([B.materialize(layer_dev[l][f]) for f in fams], 0)
            p, s, g = B.quant_fp4_block16(w)
            row.append((name, w.shape[0], w.shape[1], p, s, g))
            del w
        packed.append(row)
    del layer_dev
    torch.cuda.synchronize()
    Ms = (1, 4, 16)
    wsz = max(lib.aq_workspace_bytes(B.AQ_OP_FP4_LINEAR, B.AQ_BF16, M, K,
                                     (B.aq_proj * 1)(B.aq_proj(N, 0, None, None, None, None)), 1)
              for M in Ms for (_, N, K, _, _, _) in packed[0])
    ws = torch.zeros(max(wsz, 256), dtype=torch.uint8, device=dev)
    keep, per_m, gu = [], {}, []
    for M in Ms:
        calls = []
        for l in range(L):
            for (name, N, K, p, s, g) in packed[l]:
                x = (torch.randn(M, K, device=dev) * 0.5).to(torch.bfloat16)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                keep += [x, y]
                nb = N * K // 2 + N * K // 16 + 4 + M * K * 2 + M * N * 2
                c = Call(lib.aq_fp4_linear, (M, N, K, x.data_ptr(), K, p.data_ptr(), s.data_ptr(), g.data_ptr(),
                                             y.data_ptr(), N, ws.data_ptr(), ws.numel(), stream),
                         nb, 2 * M * N * K, f"fp4lin.L{l}.{name}.M{M}", name)
                calls.append(c)
                if name == "gateup":
                    gu.append(c)
        per_m[M] = calls
    res = {}
    for M in Ms:
        ms, _ = time_graph(torch, per_m[M], args.steps, args.warmup)
        nb = sum(c.nbytes for c in per_m[M])
        res[f"M{M}"] = {"us_per_layer": round(ms * 1e3 / L, 2), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    avg = time_per_launch(torch, gu, args.roofline_reps)
    gb = gu[0].nbytes
    return {"workload": "gemma-3-1b-shaped decode on FP4-packed W_eff, 26 layers, M in {1, 4, 16}",
            "results": res,
            "dominant": {"kernel": "k_fp4_gemv (stacked gate/up, 13824 x 1152)", "bytes_per_launch_M1": gb,
                         "avg_launch_us": round(avg * 1e3, 3),
                         "GBps_M1_bytes": round(gb / (avg * 1e-3) / 1e9, 1),
                         "frac_hbm_peak": round(gb / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": "average over the M = 1, 4 and 16 launches; bytes are the M = 1 launch's "
                                 "(codes, scales, x, y)"}}


def run_fold(args, torch, B, I):
    """The in-graph fold against the factored form, per call: W_eff
    materialised into scratch every call, then a plain GEMM on it through the
    same library (s = 1, r = 0), against one factored dispatch; Gemma-3-1B
    shapes (QKV, o, gate/up, down), rank 64, 26 layers in 13 W0 bands, over M.
    The crossover M is where the fold starts to win."""
    L = 26
    layer_np = I.layer_bundles("materialize_fp4", I.GEMMA_1B, layers=L, r=64, dtype="bf16", num_bands=13)
    layer_dev = upload_layers(torch, I, layer_np)
    dev = torch.device("cuda", 0)
    lib = B.lib()
    stream = torch.cuda.current_stream().cuda_stream
    groups = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",))]
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    keep, res = [], {}
    for M in (16, 64, 128, 256, 512, 1024, 2048):
        fact, fold = [], []
        for l in range(L):
            for name, fams in groups:
                K = I.GEMMA_1B[fams[0]][0]
                Ns = [I.GEMMA_1B[f][1] for f in fams]
                Nt = sum(Ns)
                x = (torch.randn(M, K, device=dev) * 0.5).to(torch.bfloat16)
                y = torch.empty((M, Nt), dtype=torch.bfloat16, device=dev)
                ps = [B.make_proj(*layer_dev[l][f]) for f in fams]
                pa = (B.aq_proj * len(ps))(*ps)
                fn = {1: lib.aq_recon_linear, 2: lib.aq_recon_gateup_fused, 3: lib.aq_recon_qkv_fused}[len(ps)]
                fact.append(Call(fn, (B.AQ_BF16, M, K, x.data_ptr(), K, pa, y.data_ptr(), Nt, ws.data_ptr(),
                                      ws.numel(), stream), 0, 0, f"fact.{name}", name))
                # fold: every block's W_eff into one stacked scratch weight, then s = 1, r = 0
                weff = torch.empty((Nt, K), dtype=torch.bfloat16, device=dev)
                ones = torch.ones(Nt, dtype=torch.bfloat16, device=dev)
                r0 = 0
                for p1, n in zip(ps, Ns):
                    one = (B.aq_proj * 1)(p1)
                    fold.append(Call(lib.aq_materialize_weff, (B.AQ_BF16, K, one, weff[r0:].data_ptr(), K, stream),
                                     0, 0, f"fold.mat.{name}", name))
                    keep.append(one)
                    r0 += n
                dp = (B.aq_proj * 1)(B.aq_proj(Nt, 0, weff.data_ptr(), ones.data_ptr(), None, None))
                fold.append(Call(lib.aq_recon_linear, (B.AQ_BF16, M, K, x.data_ptr(), K, dp, y.data_ptr(), Nt,
                                                       ws.data_ptr(), ws.numel(), stream), 0, 0, f"fold.gemm.{name}",
                                 name))
                keep += [x, y, weff, ones, pa, dp]
        ms_f, _ = time_graph(torch, fact, args.steps, args.warmup)
        ms_d, _ = time_graph(torch, fold, args.steps, args.warmup)
        res[f"M{M}"] = {"factored_us_per_layer": round(ms_f * 1e3 / L, 2), "fold_us_per_layer": round(ms_d * 1e3 / L, 2),
                        "fold_over_factored": round(ms_d / ms_f, 3)}
        keep = keep[-8:]
    cross = next((m for m in (16, 64, 128, 256, 512, 1024, 2048) if res[f"M{m}"]["fold_over_factored"] < 1.0), None)
    return {"workload": "in-graph fold (materialise every call + GEMM) vs factored, Gemma-3-1B shapes, 26 layers, rank 64",
            "results": res, "fold_wins_from_M": cross}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gemma_decode",
                    choices=["gemma_decode", "gemma_prefill", "large_decoder", "materialize_fp4", "fp4_decode",
                             "fold", "pmc_probe", "pmc_probe_fp4"])
    ap.add_argument("--summarize", action="store_true",
                    help="summarise rocprofv3 CSVs (--trace, --fetch, --write) instead of running")
    ap.add_argument("--trace")
    ap.add_argument("--calls", action="store_true",
                    help="with --trace: also group the library's prefill kernels into calls")
    ap.add_argument("--fetch")
    ap.add_argument("--traffic-key", default="decode_gateup", choices=["decode_gateup", "fp4_gemv_gateup"],
                    help="with --fetch/--write: which kernel's counters to summarise")
    ap.add_argument("--write")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--roofline-reps", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_shared_block_amd import binding as B
    from rank_shared_block_amd import inputs as I
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    torch.cuda.set_device(0)
    fn = {"gemma_decode": run_gemma_decode, "gemma_prefill": run_gemma_prefill,
          "large_decoder": run_large_decoder, "materialize_fp4": run_materialize_fp4,
          "fp4_decode": run_fp4_decode, "fold": run_fold, "pmc_probe": run_pmc_probe,
          "pmc_probe_fp4": run_pmc_probe_fp4}[args.workload]
    out = fn(args, torch, B, I)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
