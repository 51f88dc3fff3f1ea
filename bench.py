"""Benchmark of the theta-bundle reconstructed linear on one MI355X.

Default run (one JSON line on stdout): the large-decoder-shaped model -- hidden
5376; q 5376->4096, k/v 5376->2048, o 4096->5376, gate/up 5376->21504, down
21504->5376 -- with 8 layers sharing W0 in 4 bands of 2 (per-layer s, U, Vt),
rank 32, bf16.  One step is a full pass of the 8 layers at each of M = 1 and 32
tokens (decode) and M = 512 tokens (prefill); a layer is four dispatches (fused
Q/K/V, o, fused gate/up, down), every one captured in one HIP graph (launch cost
excluded, as in serving).  All weights (3.3 GB of W0) stay resident in HBM.

The line reports:
* ``value``: microseconds per layer over the step (the sum of the three batch
  sizes), from exactly ``--steps`` timed graph replays after ``--warmup``;
* ``decode`` / ``prefill``: per batch size the median (p10, p90) of >= 50
  replays, achieved HBM GB/s (decode) or MFMA TFLOP/s (prefill) as a fraction of
  the MI355X peak, and the same stacked shapes as a dense ``torch.matmul``
  (hipBLASLt) on a materialised-size weight in the same graph mode
  (``recon_over_dense``);
* ``roofline``: the kernel that takes the most time in the step (the prefill
  gate/up dispatch), its algorithmic flops per launch over its average launch
  duration (HIP events around graph replays that hold only those launches, on
  the stream the graph runs on), against the bf16 dense MFMA peak;
  ``roofline_decode``: the same for the decode gate/up dispatch at M = 1 against
  the HBM peak; ``traffic`` from rocprofv3 FETCH_SIZE / WRITE_SIZE counters
  (profiles/traffic.json), null when the kernel source has changed since;
* ``cpu_baseline``: the fp64 oracle on a bounded sample of the same workload,
  on this host's cores, in the same unit;
* ``extra``: the Gemma-3-1B-shaped decode (26 layers, rank 16, M = 1, 4, 16),
  prefill (rank 64, M = 512, 2048, against dense) and the load-time materialise
  + FP4 pack of all 182 projections (13 bands, rank 64).

Other workloads (``--workload``) print their own JSON: gemma_decode,
gemma_prefill, large_decoder, materialize_fp4, fp4_decode, fold, rebuild, and
the counter-run probes.
"""

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6    # dense bf16 MFMA
METRIC = "reconstructed-linear µs/layer + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)"
DATA = "synthetic (seeded N(0,1/in) W0, U(0.9,1.1) s, N(0,0.02) U/V, N(0,1) x)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- workload

class Call:
    """One pre-marshalled C-ABI call (pointers, strides and stream fixed)."""

    def __init__(self, fn, args, nbytes, flops, name, grid_key):
        self.fn, self.args = fn, args
        self.nbytes, self.flops, self.name, self.grid_key = nbytes, flops, name, grid_key

    def __call__(self, stream=None):
        a = self.args if stream is None else self.args[:-1] + (stream,)
        st = self.fn(*a)
        if st != 0:
            from rank_shared_block_amd import binding as B
            raise RuntimeError(f"{self.name}: {B.status_string(st)}: {B.last_error()}")


class TorchCall:
    """A dense baseline launch (torch.matmul into a preallocated output)."""

    def __init__(self, torch, x, w, y, name, grid_key, flops):
        self.torch, self.x, self.w, self.y = torch, x, w, y
        self.name, self.grid_key, self.flops, self.nbytes = name, grid_key, flops, 0

    def __call__(self, stream=None):
        self.torch.matmul(self.x, self.w.t(), out=self.y)


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


def make_recon_calls(torch, B, I, workload, shapes, layer_dev, layer_np, M, x_tag):
    """Per layer, the four dispatches as pre-marshalled calls."""
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream().cuda_stream
    calls, keep = [], []
    lib = B.lib()
    for l, fam_dev in enumerate(layer_dev):
        for name, fams in I.LAYER_DISPATCHES:
            K = shapes[fams[0]][0]
            x = torch.from_numpy(I.activations(workload, x_tag + len(name), M, K, "bf16")).to(dev).to(torch.bfloat16)
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


def make_dense_calls(torch, I, shapes, L, M):
    """The same stacked shapes as plain dense GEMMs y = x W^T (torch.matmul,
    hipBLASLt) on random bf16 weights of the materialised size, one per layer."""
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(1234 + M)
    calls = []
    for l in range(L):
        for name, fams in I.LAYER_DISPATCHES:
            K = shapes[fams[0]][0]
            N = sum(shapes[f][1] for f in fams)
            x = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
            w = torch.randn(N, K, device=dev, dtype=torch.bfloat16, generator=g) * 0.03
            y = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
            calls.append(TorchCall(torch, x, w, y, f"dense.L{l}.{name}.M{M}", name, 2 * M * K * N))
    return calls


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

def capture(torch, calls):
    """One HIP graph holding `calls` in order (eager warm-up first, on the
    capture stream); the library calls are re-marshalled for that stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for c in calls:
            c(cap)
    torch.cuda.synchronize()
    return g


def time_steps(torch, g, steps, warmup):
    """`warmup` untimed replays, then exactly `steps` replays between two
    synchronisations; ms per replay."""
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


def replay_stats(torch, g, reps, warmup=3):
    """Median, p10 and p90 (ms) of `reps` replays, each between its own events."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90)), "n": int(reps)}


def time_graph(torch, calls, steps, warmup):
    g = capture(torch, calls)
    return time_steps(torch, g, steps, warmup), g


def time_per_launch(torch, calls, reps):
    """Average duration of one launch of `calls`: HIP events around replays of
    a graph that holds only these launches back to back, on the stream the
    graph runs on.  Consecutive kernels of a graph abut on the GPU, so this is
    the average kernel duration (start to start) that rocprofv3 reports for the
    same launches."""
    g = capture(torch, calls)
    st = replay_stats(torch, g, reps, 2)
    del g
    return st["median"] / len(calls)


def time_graph_streams(torch, calls, nstreams, steps, warmup):
    """Like time_graph, but the calls (independent of each other) are issued
    round-robin on `nstreams` streams forked from and joined back to the capture
    stream, as a loader issues independent projections."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    side = [torch.cuda.Stream() for _ in range(nstreams)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for st in side:
            st.wait_stream(cap)
        for i, c in enumerate(calls):
            c(side[i % nstreams].cuda_stream)
        for st in side:
            cap.wait_stream(st)
    return time_steps(torch, g, steps, warmup)


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


def _r(x, n=3):
    return None if x is None else round(float(x), n)


# --------------------------------------------------------------------------- host facts

def blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception as e:          # noqa: BLE001 -- informational only
        return {"error": str(e)}
    if not info:
        return {"vendor": None}
    p = info[0]
    return {"vendor": p.get("internal_api"), "version": p.get("version"), "threads": p.get("num_threads"),
            "architecture": p.get("architecture")}


def gpu_clocks():
    """Current GPU clocks as amd-smi reports them (child process; best effort)."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception as e:          # noqa: BLE001 -- informational only
        return {"error": str(e)[:200]}
    out = {}
    try:
        gpus = data.get("gpu_data", data) if isinstance(data, dict) else data
        clk = gpus[0]["clock"]
        gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
        out["gfx_mhz_min_max"] = [min(gfx), max(gfx)] if gfx else None
        for k in ("mem_0", "fclk_0", "socclk_0"):
            try:
                out[k.replace("_0", "_mhz")] = clk[k]["clk"]["value"]
            except (KeyError, TypeError):
                pass
    except Exception as e:          # noqa: BLE001 -- informational only
        out["error"] = str(e)[:200]
    return out


# --------------------------------------------------------------------------- CPU baseline

def cpu_baseline_layers(I, workload, shapes, layer_np, Ms, x_tag, layers, reps, per_m_layers=None):
    """The oracle (numpy float64, this host's BLAS threads) on a bounded sample:
    the four dispatches of `layers` at every M, each timed `reps` times (median),
    operands converted to float64 per projection outside the timed region.
    Returns microseconds per layer per M and their sum."""
    import oracle
    per_m = {}
    conv_s = 0.0
    for M in Ms:
        ls = layers if per_m_layers is None else per_m_layers.get(M, layers)
        tot = 0.0
        for l in ls:
            for name, fams in I.LAYER_DISPATCHES:
                K = shapes[fams[0]][0]
                t0 = time.perf_counter()
                bds = [tuple(layer_np[l][f][k].astype(np.float64) for k in ("W0", "s", "U", "Vt")) for f in fams]
                x = I.activations(workload, x_tag(M) + len(name), M, K, "bf16").astype(np.float64)
                conv_s += time.perf_counter() - t0
                ts = []
                for _ in range(reps):
                    t0 = time.perf_counter()
                    oracle.recon_fused(x, bds)
                    ts.append(time.perf_counter() - t0)
                tot += float(np.median(ts))
                del bds
        per_m[f"M{M}"] = round(tot / len(ls) * 1e6, 1)
    return per_m, conv_s


# --------------------------------------------------------------------------- counters

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SOURCES = {"decode_gateup": "rank_shared_block_amd/csrc/recon_decode.hip",
           "decode_gateup_large": "rank_shared_block_amd/csrc/recon_decode.hip",
           "prefill_gateup_large": ("rank_shared_block_amd/csrc/recon_prefill.hip",
                                    "rank_shared_block_amd/csrc/handoff.h"),
           "fp4_gemv_gateup": "rank_shared_block_amd/csrc/fp4_gemv.hip",
           "fp4_gemv_dot_large": "rank_shared_block_amd/csrc/fp4_gemv.hip",
           "materialize_batch": ("rank_shared_block_amd/csrc/materialize.hip",
                                 "rank_shared_block_amd/csrc/fp4_block.h"),
           "fp4_pack_batch": ("rank_shared_block_amd/csrc/fp4_pack.hip", "rank_shared_block_amd/csrc/fp4_block.h")}
PMC_KERNELS = {"decode_gateup": (("k_decode_bf16",), "k_decode_bf16 (fused gate/up, Gemma-3-1B-shaped)"),
               "decode_gateup_large": (("k_decode_bf16",), "k_decode_bf16 (gate/up, large-decoder-shaped, M = 1)"),
               "prefill_gateup_large": (("k_gemm_bf16",), "k_gemm_bf16 (gate/up, large-decoder-shaped, M = 512)"),
               "fp4_gemv_gateup": (("k_fp4_gemv", "<2, false>"), "k_fp4_gemv / k_fp4_gemv_m4 (FP4 stacked gate/up)"),
               "fp4_gemv_dot_large": (("k_fp4_gemv_dot",), "k_fp4_gemv_dot (FP4 large stacked gate/up, M = 1)"),
               "materialize_batch": (("k_materialize_batch",), "k_materialize_batch (182 Gemma-3-1B-shaped W_eff, "
                                                               "13 bands)"),
               "fp4_pack_batch": (("k_fp4_pack_batch",), "k_fp4_pack_batch (the same 182 W_eff)")}


def source_digest(rel):
    """Digest of a kernel's source file (or files, in order)."""
    import hashlib
    h = hashlib.sha256()
    for r in ((rel,) if isinstance(rel, str) else rel):
        with open(os.path.join(ROOT, r), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


CALIB_BYTES = 256 * 2 ** 20


def _calibration_copy(torch):
    dev = torch.device("cuda", 0)
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def run_pmc_probe(args, torch, B, I):
    """Workload for the counter runs: a plain copy of known size (calibration),
    then the dispatches named by --probe, eagerly:
    decode_gateup (Gemma-3-1B fused gate/up, 26 layers x M in {1, 4, 16}),
    decode_gateup_large (large-decoder gate/up at M = 1, 8 layers),
    decode_gateup_large32 (the same at M = 32),
    prefill_gateup_large (large-decoder gate/up at M = 512, 8 layers)."""
    _calibration_copy(torch)
    probe = args.probe
    if probe == "load_batch":
        # one aq_materialize_batch call over the 182 Gemma-3-1B-shaped
        # projections (13 bands of 2 layers, rank 64), then one
        # aq_quant_fp4_batch call with its maxima
        L = 26
        layer_np = I.layer_bundles("materialize_fp4", I.GEMMA_1B, layers=L, r=64, dtype="bf16", num_bands=13)
        layer_dev = upload_layers(torch, I, layer_np)
        bundles = [layer_dev[l][f] for f in I.FAMILIES for l in range(L)]
        ws, amax = B.materialize_batch(bundles, want_amax=True)
        B.quant_fp4_batch(ws, amax)
        torch.cuda.synchronize()
        return {"probe": f"copy of {CALIB_BYTES} bytes, then one batched materialisation and one batched pack "
                         f"of {len(bundles)} projections"}
    if probe == "decode_gateup":
        wl, shapes, L, G, r, Ms = "gemma_decode", I.GEMMA_1B, 26, None, 16, (1, 4, 16)
    else:
        wl, shapes, L, G, r = "large_decoder", I.LARGE_DECODER, 8, 4, 32
        Ms = {"decode_gateup_large": (1,), "decode_gateup_large32": (32,)}.get(probe, (512,))
    layer_np = I.layer_bundles(wl, shapes, layers=L, r=r, dtype="bf16", num_bands=G, families=("gate", "up"))
    layer_dev = upload_layers(torch, I, layer_np)
    dev = torch.device("cuda", 0)
    lib = B.lib()
    K = shapes["gate"][0]
    N = 2 * shapes["gate"][1]
    for M in Ms:
        x = torch.from_numpy(I.activations(wl, 10 * M + 6, M, K, "bf16")).to(dev).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for l in range(L):
            arr = (B.aq_proj * 2)(*[B.make_proj(*layer_dev[l][f]) for f in ("gate", "up")])
            need = lib.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, K, arr, 2)
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            B.check(lib.aq_recon_gateup_fused(B.AQ_BF16, M, K, x.data_ptr(), K, arr, y.data_ptr(), N,
                                              ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return {"probe": f"copy of {CALIB_BYTES} bytes, then {probe}: {L} layers x M in {list(Ms)}"}


def run_pmc_probe_fp4(args, torch, B, I):
    """Counter-run workload for the FP4 GEMV: the copy calibration, then 78
    stacked gate/up launches (13824 x 1152 packed; 26 layers, each its own
    weight, x M in {1, 4, 16}), eagerly."""
    _calibration_copy(torch)
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    if args.probe == "fp4_large":
        # the large decoder's stacked gate/up (43008 x 5376 packed), 8 weights,
        # one token: the packed-dot kernel
        N, K = 43008, 5376
        packs = [B.quant_fp4_block16((torch.randn(N, K, device=dev, generator=g) * K ** -0.5).to(torch.bfloat16))
                 for _ in range(8)]
        x = (torch.randn(1, K, device=dev, generator=g)).to(torch.bfloat16)
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        for l in range(8):
            B.fp4_linear(x, *packs[l], y=y)
        torch.cuda.synchronize()
        return {"probe": "copy of %d bytes, then 8 FP4 large stacked gate/up GEMV launches at M = 1" % CALIB_BYTES}
    N, K = 13824, 1152
    packs = [B.quant_fp4_block16((torch.randn(N, K, device=dev, generator=g) * K ** -0.5).to(torch.bfloat16))
             for _ in range(26)]
    for M in (1, 4, 16):
        x = (torch.randn(M, K, device=dev, generator=g)).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for l in range(26):
            B.fp4_linear(x, *packs[l], y=y)
    torch.cuda.synchronize()
    return {"probe": "copy of %d bytes, then 78 FP4 stacked gate/up GEMV launches" % CALIB_BYTES}


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
        for (name, wg), d in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:args.top]:
            d.sort()
            out.append(f"| `{name[:90]}` | {wg} | {len(d)} | {sum(d)/len(d):.3f} | {d[len(d)//2]:.3f} | {sum(d):.1f} |")
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
        match = tuple(args.kernel_match.split("|")) if args.kernel_match else PMC_KERNELS[args.traffic_key][0]
        for key, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
            rs = rows(path)
            val = lambda r: float(r.get("Counter_Value", r.get("value", 0)))
            copy = [val(r) for r in rs if "copyBuffer" in r["Kernel_Name"]]
            dec = [val(r) for r in rs if all(k in r["Kernel_Name"] for k in match)]
            res[key] = (max(copy) if copy else None, float(np.mean(dec)) if dec else None, len(dec),
                        float(np.sum(dec)) if dec else None)
        # scale: a copy of CALIB_BYTES reads and writes CALIB_BYTES each
        fscale = CALIB_BYTES / (res["FETCH_SIZE"][0] * 1024)
        wscale = CALIB_BYTES / (res["WRITE_SIZE"][0] * 1024)
        fetch_b = res["FETCH_SIZE"][1] * 1024 * fscale
        write_b = res["WRITE_SIZE"][1] * 1024 * wscale
        out.append("")
        out.append(f"FETCH_SIZE copy calibration: {res['FETCH_SIZE'][0]:.0f} KiB for {CALIB_BYTES} B read "
                   f"(scale {fscale:.4f}); WRITE_SIZE: {res['WRITE_SIZE'][0]:.0f} KiB for {CALIB_BYTES} B written "
                   f"(scale {wscale:.4f}).")
        out.append(f"{PMC_KERNELS[args.traffic_key][1]} (kernel name containing {list(match)}), mean over "
                   f"{res['FETCH_SIZE'][2]} launches: fetch {fetch_b/1e6:.3f} MB, write {write_b/1e6:.3f} MB per "
                   f"launch (scaled), total {(fetch_b + write_b)/1e6:.3f} MB; summed over those launches: fetch "
                   f"{res['FETCH_SIZE'][3] * 1024 * fscale / 1e6:.3f} MB, write "
                   f"{res['WRITE_SIZE'][3] * 1024 * wscale / 1e6:.3f} MB.")
        t = {}
        try:
            with open(TRAFFIC_FILE) as f:
                t = json.load(f)
        except (OSError, ValueError):
            pass
        t[args.traffic_key] = {"bytes_per_launch": int(fetch_b + write_b), "fetch_bytes": int(fetch_b),
                               "write_bytes": int(write_b), "fetch_scale": fscale, "write_scale": wscale,
                               "launches": res["FETCH_SIZE"][2],
                               "source_sha256_16": source_digest(SOURCES[args.traffic_key])}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
    if args.pmc:
        # any other counter run (e.g. MFMA busy): mean per kernel-name match
        rs = rows(args.pmc)
        match = tuple(args.kernel_match.split("|")) if args.kernel_match else ("aq::",)
        agg = collections.defaultdict(list)
        for r in rs:
            if all(k in r["Kernel_Name"] for k in match):
                agg[r.get("Counter_Name", "?")].append(float(r.get("Counter_Value", r.get("value", 0))))
        out.append("")
        out.append(f"Counters for kernels whose name contains {list(match)}:")
        out.append("")
        out.append("| counter | launches | mean per launch |")
        out.append("|---|---|---|")
        for name, v in sorted(agg.items()):
            out.append(f"| {name} | {len(v)} | {np.mean(v):.1f} |")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in agg:
            # one MOPS unit is 512 flops (the derived MfmaFlopsBF16 counter)
            out.append("")
            out.append(f"bf16 MFMA flops per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512): "
                       f"{np.mean(agg['SQ_INSTS_VALU_MFMA_MOPS_BF16']) * 512 / 1e9:.2f} GFLOP")
    print("\n".join(out))


# --------------------------------------------------------------------------- model workloads

class Model:
    """A decoder's bundles resident on the GPU, its recon calls and its dense
    baseline calls per batch size."""

    def __init__(self, torch, B, I, workload, shapes, L, G, r, Ms, x_tag, dense=True):
        t0 = time.time()
        self.I, self.workload, self.shapes, self.L, self.r, self.Ms = I, workload, shapes, L, r, Ms
        self.layer_np = I.layer_bundles(workload, shapes, layers=L, r=r, dtype="bf16", num_bands=G)
        log(f"{workload}: generated inputs in {time.time() - t0:.1f} s")
        self.layer_dev = upload_layers(torch, I, self.layer_np)
        torch.cuda.synchronize()
        self.x_tag = x_tag
        self.calls, self.keep, self.dense = {}, [], {}
        for M in Ms:
            c, k = make_recon_calls(torch, B, I, workload, shapes, self.layer_dev, self.layer_np, M, x_tag(M))
            self.calls[M] = c
            self.keep += k
            if dense:
                self.dense[M] = make_dense_calls(torch, I, shapes, L, M)
        log(f"{workload}: uploaded {L} layers")


def measure_model(torch, mdl, reps, prefill_Ms):
    """Per batch size: recon graph median/p10/p90, bytes and flops, and the dense
    baseline in the same graph mode."""
    out = {}
    for M in mdl.Ms:
        calls = mdl.calls[M]
        g = capture(torch, calls)
        st = replay_stats(torch, g, reps)
        del g
        ms = st["median"]
        nb = sum(c.nbytes for c in calls)
        fl = sum(c.flops for c in calls)
        res = {"us_per_layer": _r(ms * 1e3 / mdl.L, 2),
               "us_per_layer_p10": _r(st["p10"] * 1e3 / mdl.L, 2), "us_per_layer_p90": _r(st["p90"] * 1e3 / mdl.L, 2)}
        if M in prefill_Ms:
            res.update({"tflops": _r(fl / (ms * 1e-3) / 1e12, 1),
                        "frac_mfma_peak": _r(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)})
        else:
            res.update({"GBps": _r(nb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm_peak": _r(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        if M in mdl.dense:
            gd = capture(torch, mdl.dense[M])
            sd = replay_stats(torch, gd, reps)
            del gd
            dfl = sum(c.flops for c in mdl.dense[M])
            res.update({"dense_us_per_layer": _r(sd["median"] * 1e3 / mdl.L, 2),
                        "dense_tflops": _r(dfl / (sd["median"] * 1e-3) / 1e12, 1),
                        "recon_over_dense": _r(ms / sd["median"], 3)})
        res["replays"] = st["n"]
        out[f"M{M}"] = res
    return out


def dominant(torch, mdl, reps):
    """Per-launch time of every dispatch kind at every M: {(M, kind): ms}."""
    d = {}
    for M in mdl.Ms:
        for kind, _ in mdl.I.LAYER_DISPATCHES:
            cs = [c for c in mdl.calls[M] if c.grid_key == kind]
            d[(M, kind)] = (time_per_launch(torch, cs, reps), cs)
    return d


def roofline_of(M, kind, ms, cs, prefill_Ms, traffic_key, what):
    fl = float(np.mean([c.flops for c in cs]))
    nb = float(np.mean([c.nbytes for c in cs]))
    if M in prefill_Ms:
        ach = fl / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": _r(ach, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": _r(ach / MFMA_BF16_PEAK_TFS, 4), "flops_per_launch": int(fl)}
    else:
        ach = nb / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": _r(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": _r(ach / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": read_traffic(traffic_key) if traffic_key else None,
                 "bytes_per_launch": int(nb), "avg_launch_us": _r(ms * 1e3, 3), "launches_per_replay": len(cs),
                 "kernel": what})
    return roof


def run_headline(args, torch, B, I):
    Ms, PF = (1, 32, 512), (512,)
    L = 8
    clocks0 = gpu_clocks()
    mdl = Model(torch, B, I, "large_decoder", I.LARGE_DECODER, L, 4, 32, Ms, lambda M: 9 * M)
    step_calls = [c for M in Ms for c in mdl.calls[M]]
    g = capture(torch, step_calls)
    ms_step = time_steps(torch, g, args.steps, args.warmup)
    del g
    log(f"large decoder step: {ms_step:.4f} ms")
    reps = max(50, args.steps)
    per_m = measure_model(torch, mdl, reps, PF)
    dom = dominant(torch, mdl, max(10, args.roofline_reps))
    tot = {k: v[0] * len(v[1]) for k, v in dom.items()}
    (Mk, kind) = max(tot, key=tot.get)
    roof = roofline_of(Mk, kind, dom[(Mk, kind)][0], dom[(Mk, kind)][1], PF,
                       "prefill_gateup_large" if (Mk, kind) == (512, "gateup") else None,
                       f"{kind} dispatch at M = {Mk} (large-decoder-shaped, rank 32, {L} layers): "
                       + ("k_gemm_bf16 main pass with the rank-r tiles in the same launch" if Mk in PF else
                          "k_decode_bf16"))
    roof_dec = roofline_of(1, "gateup", dom[(1, "gateup")][0], dom[(1, "gateup")][1], PF, "decode_gateup_large",
                           f"gate/up dispatch at M = 1 (K = 5376, N = 2 x 21504, rank 32, {L} layers): k_decode_bf16")
    share = {f"M{M}.{k}": _r(v / sum(tot.values()), 3) for (M, k), v in sorted(tot.items(), key=lambda kv: -kv[1])}
    step_bytes = sum(c.nbytes for M in Ms if M not in PF for c in mdl.calls[M])
    step_flops = sum(c.flops for M in PF for c in mdl.calls[M])
    line = {
        "metric": METRIC,
        "value": _r(ms_step * 1e3 / L, 2),
        "unit": "us/layer (M=1 + M=32 + M=512)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": _r(ms_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": DATA,
        "config": {"workload": "large-decoder-shaped: 8 layers, W0 shared in 4 bands of 2, x (fused QKV, o, "
                               "fused gate/up, down), hidden 5376, rank 32, bf16, M in {1, 32, 512} tokens per step",
                   "layers": L, "bands": 4, "rank": 32, "tokens": list(Ms), "launch": "hip graph per step",
                   "note": "the second layer of a band reads the same W0 (826 MB per layer, > the 256 MB "
                           "Infinity Cache): effective, MALL-assisted at most marginally"},
        "decode": {k: v for k, v in per_m.items() if int(k[1:]) not in PF},
        "prefill": {k: v for k, v in per_m.items() if int(k[1:]) in PF},
        "decode_GBps_step": _r(step_bytes / (sum(per_m[f"M{M}"]["us_per_layer"] for M in Ms if M not in PF)
                                              * L * 1e-6) / 1e9, 1),
        "prefill_tflops_step": _r(step_flops / (sum(per_m[f"M{M}"]["us_per_layer"] for M in PF) * L * 1e-6) / 1e12, 1),
        "roofline": roof,
        "roofline_decode": roof_dec,
        "time_share_by_dispatch": share,
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        per, conv = cpu_baseline_layers(I, "large_decoder", I.LARGE_DECODER, mdl.layer_np, Ms, mdl.x_tag,
                                        layers=[0, 1], reps=3, per_m_layers={512: [0]})
        bl = blas_info()
        line["cpu_baseline"] = {
            "value": _r(sum(per.values()), 1), "unit": "us/layer (M=1 + M=32 + M=512)",
            "cores": int(bl.get("threads") or os.cpu_count() or 1), "kind": "oracle",
            "sample": f"layers 0 and 1 (one W0 band) at M = 1 and 32, layer 0 at M = 512; all four dispatches; "
                      f"median of 3 runs each; numpy float64 ({bl.get('vendor')} {bl.get('version')}, "
                      f"{bl.get('threads')} threads); bf16->fp64 conversion ({conv:.1f} s) excluded",
            "per_M_us_per_layer": per, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "blas": bl, "wall_s": _r(time.time() - t0, 1)}
    del mdl
    torch.cuda.empty_cache()
    if not args.no_extras:
        line["extra"] = {}
        for name, fn in (("gemma_decode", run_gemma_decode), ("gemma_prefill", run_gemma_prefill),
                         ("materialize_fp4", run_materialize_fp4)):
            t0 = time.time()
            line["extra"][name] = fn(args, torch, B, I, nested=True)
            torch.cuda.empty_cache()
            log(f"extra {name}: {time.time() - t0:.1f} s")
    line["clocks"] = {"before": clocks0, "after": gpu_clocks()}
    return line


def run_gemma_decode(args, torch, B, I, nested=False):
    Ms = (1, 4, 16)
    L = 26
    mdl = Model(torch, B, I, "gemma_decode", I.GEMMA_1B, L, None, 16, Ms, lambda M: 10 * M, dense=True)
    step = [c for M in Ms for c in mdl.calls[M]]
    g = capture(torch, step)
    ms_step = time_steps(torch, g, args.steps, args.warmup)
    del g
    step_bytes = sum(c.nbytes for c in step)
    per_m = measure_model(torch, mdl, max(50, args.steps), ())
    gu = [c for c in step if c.grid_key == "gateup"]
    ms = time_per_launch(torch, gu, max(10, args.roofline_reps))
    roof = roofline_of(1, "gateup", ms, gu, (), "decode_gateup",
                       "k_decode_bf16 (fused gate/up, K=1152, N=2x6912, r=16, M in {1,4,16}, 26 layers)")
    res = {"workload": "gemma-3-1b-shaped decode: 26 layers x (fused QKV, o, fused gate/up, down), hidden 1152, "
                       "rank 16, bf16, M in {1, 4, 16}",
           "ms_per_step": _r(ms_step, 4), "GBps_step": _r(step_bytes / (ms_step * 1e-3) / 1e9, 1),
           "frac_hbm_peak_step": _r(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "results": per_m, "roofline": roof}
    if not nested:
        res = {"metric": METRIC, "value": res["GBps_step"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": DATA,
               "config": {"workload": res["workload"]}, **res}
        if not args.no_cpu_baseline:
            per, conv = cpu_baseline_layers(I, "gemma_decode", I.GEMMA_1B, mdl.layer_np, Ms, mdl.x_tag,
                                            layers=[0, 1, 2, 3], reps=5)
            res["cpu_baseline"] = {"per_M_us_per_layer": per, "kind": "oracle", "blas": blas_info()}
    return res


def run_gemma_prefill(args, torch, B, I, nested=False):
    Ms = (512, 2048)
    L = args.layers or 26
    mdl = Model(torch, B, I, "gemma_prefill", I.GEMMA_1B, L, None, 64, Ms, lambda M: 5 * M)
    per_m = measure_model(torch, mdl, max(50, args.steps) if not nested else 50, Ms)
    return {"workload": f"gemma-3-1b-shaped prefill, {L} layers, rank 64, bf16", "results": per_m}


def run_large_decoder(args, torch, B, I, nested=False):
    Ms = (1, 32, 512)
    mdl = Model(torch, B, I, "large_decoder", I.LARGE_DECODER, 8, 4, 32, Ms, lambda M: 9 * M)
    per_m = measure_model(torch, mdl, max(50, args.steps), (512,))
    return {"workload": "large-decoder-shaped, 8 layers in 4 W0 bands, rank 32, bf16", "results": per_m}


def run_materialize_fp4(args, torch, B, I, nested=False):
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
    steps, warm = (10, 2) if nested else (args.steps, args.warmup)
    ms_m, _ = time_graph(torch, mats, steps, warm)
    ms_p, _ = time_graph(torch, packs, steps, warm)
    ms_m4 = time_graph_streams(torch, mats, 4, steps, warm)
    ms_p4 = time_graph_streams(torch, packs, 4, steps, warm)
    mat_avg = time_per_launch(torch, mats, 3)
    big = [c for c in mats if c.name.split(".")[-1] in ("gate", "up", "down")]
    big_avg = time_per_launch(torch, big, 3)
    big_bytes = big[0].nbytes

    def leg(ms, nb):
        return {"ms": _r(ms, 4), "GBps": _r(nb / (ms * 1e-3) / 1e9, 1),
                "frac_hbm_peak": _r(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # The batched load-time calls: the whole model in one aq_materialize_batch
    # call (family by family, the two layers of each band next to each other,
    # so each W0 tile is read once per band) that also reports each W_eff's
    # largest magnitude, then one aq_quant_fp4_batch call that takes them and
    # reads each W_eff once.
    order = [(f, l) for f in I.FAMILIES for l in range(L)]
    n = len(order)
    mitems, fitems = (B.aq_mat_item * n)(), (B.aq_fp4_item * n)()
    xitems = (B.aq_mat_fp4_item * n)()
    amax = torch.zeros(n, dtype=torch.int32, device=dev)
    bmat = bpack = bfused = 0
    seen = set()
    for i, (f, l) in enumerate(order):
        K, N = I.GEMMA_1B[f]
        bd = layer_dev[l][f]
        w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
        gs = torch.empty((1,), dtype=torch.float32, device=dev)
        mitems[i] = B.aq_mat_item(K, B.make_proj(*bd), w.data_ptr(), K)
        fitems[i] = B.aq_fp4_item(N, K, K, w.data_ptr(), packed.data_ptr(), sc.data_ptr(), gs.data_ptr())
        packed2 = torch.empty_like(packed)
        sc2 = torch.empty_like(sc)
        gs2 = torch.empty_like(gs)
        xitems[i] = B.aq_mat_fp4_item(K, B.make_proj(*bd), packed2.data_ptr(), sc2.data_ptr(), gs2.data_ptr())
        keep += [w, packed, sc, gs, packed2, sc2, gs2]
        if bd[0].data_ptr() not in seen:              # W0 read once per band
            seen.add(bd[0].data_ptr())
            bmat += N * K * 2
            bfused += 2 * N * K * 2                   # ... in each of the two passes
        bmat += (N * K + N + N * 64 + 64 * K) * 2     # W_eff written; s, U, Vt read
        bpack += N * K * 2 + N * K // 2 + N * K // 16
        bfused += 2 * (N + N * 64 + 64 * K) * 2 + N * K // 2 + N * K // 16
    keep += [mitems, fitems]
    matb = Call(lib.aq_materialize_batch, (B.AQ_BF16, n, mitems, amax.data_ptr(), stream), bmat,
                2 * sum(I.GEMMA_1B[f][0] * I.GEMMA_1B[f][1] for f, _ in order) * 64, "mat.batch", "matb")
    packb = Call(lib.aq_quant_fp4_batch, (n, fitems, amax.data_ptr(), None, 0, stream), bpack, 0, "fp4.batch",
                 "fp4b")
    fws_bytes = lib.aq_materialize_fp4_batch_workspace_bytes(n)
    fws = torch.zeros(fws_bytes, dtype=torch.uint8, device=dev)
    keep += [xitems, fws]
    fusedb = Call(lib.aq_materialize_fp4_batch, (n, xitems, fws.data_ptr(), fws_bytes, stream), bfused, 0,
                  "matfp4.batch", "mfb")
    ms_mb, _ = time_graph(torch, [matb], steps, warm)
    ms_pb, _ = time_graph(torch, [packb], steps, warm)
    ms_both, _ = time_graph(torch, [matb, packb], steps, warm)
    ms_fused, _ = time_graph(torch, [fusedb], steps, warm)
    # Ceilings for this traffic mix, in the same graph setting: a device copy
    # (read + write) and a fill (write only) of 1 GiB.
    class _Op:
        def __init__(self, fn):
            self.fn = fn

        def __call__(self, stream=None):
            self.fn()
    big_a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    big_b = torch.empty_like(big_a)
    ms_copy, _ = time_graph(torch, [_Op(lambda: big_b.copy_(big_a))], steps, warm)
    ms_fill, _ = time_graph(torch, [_Op(lambda: big_b.fill_(1.0))], steps, warm)
    calib = {"copy_1GiB": leg(ms_copy, 2 << 30), "fill_1GiB": leg(ms_fill, 1 << 30)}
    del big_a, big_b
    batched = {"materialize": dict(leg(ms_mb, bmat), bytes=bmat,
                                   bytes_note="W0 once per band (13 x 7), W_eff written, s, U, V read"),
               "fp4_pack": dict(leg(ms_pb, bpack), bytes=bpack, bytes_note="W_eff read once, codes and scales written"),
               "both": dict(leg(ms_both, bmat + bpack), bytes=bmat + bpack),
               "fp4_without_w_eff": dict(leg(ms_fused, bfused), bytes=bfused,
                                         bytes_note="aq_materialize_fp4_batch: W0 once per band, s, U, V read "
                                                    "in each of its two passes; codes and scales written",
                                         vs_both=_r(ms_fused / ms_both, 3))}
    return {"workload": "materialise + FP4 pack, 7 families x 26 layers (Gemma-3-1B shapes), 13 W0 bands, rank 64",
            "batched": batched, "calibration": calib,
            "note": "batched: one aq_materialize_batch call for all 182 projections, then one "
                    "aq_quant_fp4_batch call with its maxima; serial: the 182 one-projection calls of each "
                    "kind back to back in one graph; 4 streams: the same independent calls round-robin on 4 "
                    "streams inside one graph",
            "materialize": dict(leg(ms_m, mbytes), bytes=mbytes, avg_launch_us=_r(mat_avg * 1e3, 2),
                                streams4=leg(ms_m4, mbytes),
                                largest_projection={"bytes": big_bytes, "avg_launch_us": _r(big_avg * 1e3, 2),
                                                    "GBps": _r(big_bytes / (big_avg * 1e-3) / 1e9, 1)}),
            "fp4_pack": dict(leg(ms_p, pbytes), bytes=pbytes, streams4=leg(ms_p4, pbytes))}


def _fp4_decode_model(args, torch, B, I, wl, shapes, L, G, r, Ms, label):
    """One decoder on FP4-packed W_eff: per layer the four dispatches (stacked
    QKV, o, stacked gate/up, down), each layer's weights its own W_eff
    (materialised from its bundles) packed on the GPU; per M the layer time and
    the stacked gate/up launch's average duration."""
    layer_np = I.layer_bundles(wl, shapes, layers=L, r=r, dtype="bf16", num_bands=G)
    dev = torch.device("cuda", 0)
    lib = B.lib()
    stream = torch.cuda.current_stream().cuda_stream
    groups = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",))]
    packed = []
    layer_dev = upload_layers(torch, I, layer_np)
    del layer_np
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
    wsz = max(lib.aq_workspace_bytes(B.AQ_OP_FP4_LINEAR, B.AQ_BF16, M, K,
                                     (B.aq_proj * 1)(B.aq_proj(N, 0, None, None, None, None)), 1)
              for M in Ms for (_, N, K, _, _, _) in packed[0])
    ws = torch.zeros(max(wsz, 256), dtype=torch.uint8, device=dev)
    keep, per_m, gu = [], {}, {}
    for M in Ms:
        calls = []
        gu[M] = []
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
                    gu[M].append(c)
        per_m[M] = calls
    res = {}
    for M in Ms:
        ms, _ = time_graph(torch, per_m[M], args.steps, args.warmup)
        nb = sum(c.nbytes for c in per_m[M])
        avg = time_per_launch(torch, gu[M], max(10, args.roofline_reps))
        gb = gu[M][0].nbytes
        res[f"M{M}"] = {"us_per_layer": _r(ms * 1e3 / L, 2), "GBps": _r(nb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm_peak": _r(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "gateup_avg_launch_us": _r(avg * 1e3, 3),
                        "gateup_GBps": _r(gb / (avg * 1e-3) / 1e9, 1),
                        "gateup_frac_hbm_peak": _r(gb / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    N, K = packed[0][2][1], packed[0][2][2]
    return {"workload": label, "results": res,
            "gateup": f"k_fp4_gemv, stacked gate/up {N} x {K}: {N * K // 2 + N * K // 16} bytes of codes and "
                      f"scales per launch"}


def run_fp4_decode(args, torch, B, I, nested=False):
    """Decode on FP4-packed W_eff: the Gemma-3-1B-shaped decoder (stacked QKV
    1536 x 1152, o 1152 x 1024, stacked gate/up 13824 x 1152, down 1152 x 6912;
    26 layers, rank-64 bundles in 13 W0 bands, M in {1, 4, 16}) and the
    large-decoder-shaped one (8 layers, rank 32, 4 bands, M in {1, 16}; its
    stacked gate/up streams 130 MB of codes and scales per launch)."""
    gem = _fp4_decode_model(args, torch, B, I, "materialize_fp4", I.GEMMA_1B, 26, 13, 64, (1, 4, 16),
                            "gemma-3-1b-shaped decode on FP4-packed W_eff, 26 layers, M in {1, 4, 16}")
    torch.cuda.empty_cache()
    large = _fp4_decode_model(args, torch, B, I, "large_decoder", I.LARGE_DECODER, 8, 4, 32, (1, 16),
                              "large-decoder-shaped decode on FP4-packed W_eff, 8 layers, M in {1, 16}")
    g1, l1 = gem["results"]["M1"], large["results"]["M1"]
    return {"workload": "decode on FP4-packed W_eff", "gemma": gem, "large_decoder": large,
            "dominant": {"kernel": "k_fp4_gemv_m4 (Gemma-3-1B stacked gate/up, 13824 x 1152, M = 1)",
                         "avg_launch_us": g1["gateup_avg_launch_us"], "GBps": g1["gateup_GBps"],
                         "frac_hbm_peak": g1["gateup_frac_hbm_peak"],
                         "traffic": read_traffic("fp4_gemv_gateup")},
            "dominant_large": {"kernel": "k_fp4_gemv_dot (large-decoder stacked gate/up, 43008 x 5376, M = 1)",
                               "avg_launch_us": l1["gateup_avg_launch_us"], "GBps": l1["gateup_GBps"],
                               "frac_hbm_peak": l1["gateup_frac_hbm_peak"],
                               "traffic": read_traffic("fp4_gemv_dot_large")}}


def run_fold(args, torch, B, I, nested=False):
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
        res[f"M{M}"] = {"factored_us_per_layer": _r(ms_f * 1e3 / L, 2), "fold_us_per_layer": _r(ms_d * 1e3 / L, 2),
                        "fold_over_factored": _r(ms_d / ms_f, 3)}
        keep = keep[-8:]
    cross = next((m for m in (16, 64, 128, 256, 512, 1024, 2048) if res[f"M{m}"]["fold_over_factored"] < 1.0), None)
    return {"workload": "in-graph fold (materialise every call + GEMM) vs factored, Gemma-3-1B shapes, 26 layers, "
                        "rank 64", "results": res, "fold_wins_from_M": cross}


def make_rebuild_calls(torch, B, I, workload, shapes, layer_dev, layer_np, M, x_tag):
    """Per layer, the four dispatches through the per-element rebuild entry point."""
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream().cuda_stream
    calls, keep = [], []
    lib = B.lib()
    for l, fam_dev in enumerate(layer_dev):
        for name, fams in I.LAYER_DISPATCHES:
            K = shapes[fams[0]][0]
            x = torch.from_numpy(I.activations(workload, x_tag + len(name), M, K, "bf16")).to(dev).to(torch.bfloat16)
            projs = [B.make_proj(*fam_dev[f]) for f in fams]
            arr = (B.aq_proj * len(fams))(*projs)
            ntot = sum(p.N for p in projs)
            y = torch.empty((M, ntot), dtype=torch.bfloat16, device=dev)
            need = lib.aq_workspace_bytes(B.AQ_OP_REBUILD, B.AQ_BF16, M, K, arr, len(fams))
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            args = (B.AQ_BF16, M, K, x.data_ptr(), K, arr, len(fams), y.data_ptr(), ntot, ws.data_ptr(), ws.numel(),
                    stream)
            nr = [(shapes[f][1], layer_np[l][f]["U"].shape[1]) for f in fams]
            calls.append(Call(lib.aq_rebuild_linear, args, _dispatch_bytes(M, K, nr), _dispatch_flops(M, K, nr),
                              f"rb.L{l}.{name}.M{M}", name))
            keep += [x, y, ws, arr]
    return calls, keep


def run_rebuild(args, torch, B, I, nested=False):
    """The per-element rebuild (every weight rebuilt inside the kernel, no t)
    against the factored form, per rank and batch size: Gemma-3-1B-shaped
    layers (26, ranks 4, 16, 64) and large-decoder-shaped layers (8 in 4 W0
    bands, rank 32); us per layer, both as HIP graphs."""
    res = {}
    cases = [("gemma_decode", I.GEMMA_1B, 26, None, r, (1, 4, 16)) for r in (4, 16, 64)]
    cases.append(("large_decoder", I.LARGE_DECODER, 8, 4, 32, (1, 16)))
    for wl, shapes, L, G, r, Ms in cases:
        layer_np = I.layer_bundles(wl, shapes, layers=L, r=r, dtype="bf16", num_bands=G)
        layer_dev = upload_layers(torch, I, layer_np)
        for M in Ms:
            fc, k1 = make_recon_calls(torch, B, I, wl, shapes, layer_dev, layer_np, M, 11 * M)
            rc, k2 = make_rebuild_calls(torch, B, I, wl, shapes, layer_dev, layer_np, M, 11 * M)
            gf, gr = capture(torch, fc), capture(torch, rc)
            sf, sr = replay_stats(torch, gf, 30), replay_stats(torch, gr, 30)
            del gf, gr, k1, k2
            nb = sum(c.nbytes for c in fc)
            res[f"{wl}.r{r}.M{M}"] = {"factored_us_per_layer": _r(sf["median"] * 1e3 / L, 2),
                                      "rebuild_us_per_layer": _r(sr["median"] * 1e3 / L, 2),
                                      "rebuild_over_factored": _r(sr["median"] / sf["median"], 3),
                                      "rebuild_GBps": _r(nb / (sr["median"] * 1e-3) / 1e9, 1)}
            log(f"rebuild {wl} r={r} M={M}: {res[f'{wl}.r{r}.M{M}']}")
        del layer_dev
        torch.cuda.empty_cache()
    return {"workload": "per-element rebuild vs factored form, decode batch sizes", "results": res}


def run_decompose(args, torch, B, I, nested=False):
    """The decomposition on the GPU (least-squares scale, randomized SVD of the
    residual at rank 64 with 10 probes of oversampling and 2 subspace steps,
    float64) for the seven Gemma-3-1B-shaped projections of one layer, against
    the oracle's on this host's cores (one projection, q)."""
    dev = torch.device("cuda", 0)
    r, q = 64, 2
    res, keep = {}, []
    total_ms = 0.0
    for fam in I.FAMILIES:
        K, N = I.GEMMA_1B[fam]
        W = torch.from_numpy(I.trained_weight("decompose", 0, fam, K, N, "bf16", waves=32)).to(dev).to(torch.bfloat16)
        W0 = torch.from_numpy(I.bundle("decompose", 0, fam, K, N, 0, "bf16")["W0"]).to(dev).to(torch.bfloat16)
        l = B.probe_width(N, K, r)
        om = torch.from_numpy(I.gaussian_probe("decompose", 7, l, K)).to(dev)
        ws = B.Workspace()
        for _ in range(2):
            B.decompose(W, W0, r, om, q=q, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            B.decompose(W, W0, r, om, q=q, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        total_ms += ms
        # contractions with R, each 2 N K l flops (the l x l work is second
        # order): R Omega^T, then per subspace step R^T Q and R Q', then
        # B = Q^T R; where l = N, B = R (one pass); where l = K, no steps
        passes = 1 if l == N else (2 if l == K else 2 * q + 2)
        flop = passes * 2.0 * N * K * l
        res[fam] = {"N": N, "K": K, "l": l, "ms": _r(ms, 3), "fp64_GFLOP": _r(flop / 1e9, 2),
                    "fp64_TFLOPs": _r(flop / (ms * 1e-3) / 1e12, 2)}
        keep += [W, W0, om]
    out = {"workload": "decomposition of the 7 Gemma-3-1B-shaped projections of one layer (rank 64, p = 10, "
                       "q = 2, fp64)", "per_projection": res, "ms_per_layer": _r(total_ms, 3)}
    if not args.no_cpu_baseline:
        import oracle
        for fam in ("q", "k"):         # the randomized branch, and the full SVD (min(N, K) = 256)
            K, N = I.GEMMA_1B[fam]
            Wn = I.trained_weight("decompose", 0, fam, K, N, "bf16", waves=32).astype(np.float64)
            W0n = I.bundle("decompose", 0, fam, K, N, 0, "bf16")["W0"].astype(np.float64)
            omn = I.gaussian_probe("decompose", 7, B.probe_width(N, K, r), K)
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.decompose_randomized(Wn, W0n, r, omn, q)
                ts.append((time.perf_counter() - t0) * 1e3)
            out[f"cpu_baseline_{fam}_proj_ms"] = _r(float(np.median(ts)), 1)
        out["cpu_baseline_blas"] = blas_info()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "gemma_decode", "gemma_prefill", "large_decoder", "materialize_fp4",
                             "fp4_decode", "fold", "rebuild", "decompose", "pmc_probe", "pmc_probe_fp4"])
    ap.add_argument("--probe", default="decode_gateup",
                    choices=["decode_gateup", "decode_gateup_large", "decode_gateup_large32", "prefill_gateup_large",
                             "load_batch", "fp4_large"],
                    help="with --workload pmc_probe: which dispatches the counter run covers")
    ap.add_argument("--summarize", action="store_true",
                    help="summarise rocprofv3 CSVs (--trace, --fetch/--write, --pmc) instead of running")
    ap.add_argument("--trace")
    ap.add_argument("--top", type=int, default=16)
    ap.add_argument("--calls", action="store_true",
                    help="with --trace: also group the library's prefill kernels into calls")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--pmc", help="with --summarize: a counter CSV to average per counter")
    ap.add_argument("--kernel-match", default="", help="with --summarize: '|'-separated substrings of the kernel name")
    ap.add_argument("--traffic-key", default="decode_gateup", choices=sorted(PMC_KERNELS),
                    help="with --fetch/--write: which kernel's counters to summarise")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--roofline-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline only (no Gemma-3-1B / materialise keys)")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the reconstructed linear here runs on a single GPU and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_shared_block_amd import binding as B
    from rank_shared_block_amd import inputs as I
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    torch.cuda.set_device(0)
    fn = {"headline": run_headline, "gemma_decode": run_gemma_decode, "gemma_prefill": run_gemma_prefill,
          "large_decoder": run_large_decoder, "materialize_fp4": run_materialize_fp4,
          "fp4_decode": run_fp4_decode, "fold": run_fold, "rebuild": run_rebuild, "decompose": run_decompose,
          "pmc_probe": run_pmc_probe,
          "pmc_probe_fp4": run_pmc_probe_fp4}[args.workload]
    t0 = time.time()
    out = fn(args, torch, B, I)
    out["bench_wall_s"] = _r(time.time() - t0, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
