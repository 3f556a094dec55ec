#!/usr/bin/env python3
"""Benchmark: NVFP4 W4A16 MoE grouped GEMM at 16-64 tokens per expert on one
MI355X.

One step = the three grouped GEMMs that span the decode range where the pages
report utilization collapsing ("The FP4 Frontier", section "The Context":
15-55 TFLOPS at 16-64 tokens per expert on their hardware):
  1. up projection, 64 experts, N=4096, K=6144, 128 tokens top-8 uniform
     over 60 experts (~16 rows per expert, 4 experts empty);
  2. up projection, 64 experts, N=4096, K=6144, 512 tokens top-8 with
     Zipf(1.2) expert skew (~64 rows per expert on average);
  3. down projection of the same routing, N=6144, K=2048.
Weights are NVFP4 (encoded once by nvfp4_quantize before timing, as a model
load would); activations and outputs BF16; all inputs are resident in HBM
when the timed region starts.  Each launch streams more weight bytes (0.45 to
0.91 GB) than the 256 MB Infinity Cache holds, so weights come from HBM.

Output: one JSON line.  value = useful TFLOPS of the step (2 * rows * N * K
summed over the three launches, divided by wall time of the timed steps);
roofline = algorithmic HBM bytes per launch of the dominant kernel over its
average launch time (HIP events on the launch stream), against 8 TB/s;
cpu_baseline = the CPU oracle timed on a bounded sample of launch 1 (plus its
quantize, and single-thread figures for the small dense and decode shapes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOPS + HBM GB/s (% roofline), NVFP4 grouped GEMM at 16-64 tok/expert"
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0
KERNEL_SOURCE = os.path.join(ROOT, "block_scaled_fp4_nibble_amd", "csrc", "gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense decode / 8192^3 / quantize side measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent on the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run five 1 GiB device-to-device copies (run under rocprofv3 "
                         "--pmc to calibrate FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--dense", nargs=3, type=int, metavar=("M", "N", "K"),
                    help="only time one dense GEMM of this shape (e.g. to profile its kernel) "
                         "and print one JSON line")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                           "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs of a bench "
                         "run and of --copy-calibration (no GPU needed)")
    return ap.parse_args()


def grouped_bytes(counts, n, k):
    """Algorithmic HBM bytes of one grouped launch: each non-empty expert's
    packed weight + scales + global scale once, activations read once, output
    written once, offsets read once."""
    nonempty = sum(1 for c in counts if c > 0)
    rows = int(sum(counts))
    return nonempty * (n * k * 9 // 16 + 4) + 2 * rows * k + 2 * rows * n + 4 * (len(counts) + 1)


def dense_bytes(m, n, k):
    return n * k * 9 // 16 + 4 + 2 * m * k + 2 * m * n


def randn_bf16(shape, std, seed, device="cuda"):
    """Seeded N(0, std^2) BF16 tensor drawn on the GPU (torch's generator)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def build_workload():
    import numpy as np
    import torch
    import block_scaled_fp4_nibble_amd as nv
    import workloads as W

    launches = []
    specs = [
        ("up_uniform_16tpe", W.moe_uniform_routing(), 4096, 6144, 101),
        ("up_zipf_64tpe", W.moe_zipf_routing(), 4096, 6144, 102),
        ("down_zipf_64tpe", W.moe_zipf_routing(), 6144, 2048, 103),
    ]
    for name, r, n, k, seed in specs:
        E = r.num_experts
        w = randn_bf16((E, n, k), 0.02, seed)
        qw = nv.quantize(w)
        del w
        x = randn_bf16((r.rows, k), 1.0, seed + 1000)
        off = torch.from_numpy(r.offsets.astype(np.int32)).cuda()
        y = torch.empty((r.rows, n), dtype=torch.bfloat16, device="cuda")
        launches.append(dict(name=name, qw=qw, x=x, off=off, y=y, n=n, k=k, rows=r.rows,
                             counts=r.counts.tolist(), experts=E, tokens=r.tokens,
                             row_token=torch.from_numpy(r.row_token.astype(np.int32)).cuda(),
                             kernel=nv.nvfp4_kernel_name(r.rows, E, n, k, 1),
                             flops=2 * r.rows * n * k, bytes=grouped_bytes(r.counts, n, k)))
    torch.cuda.synchronize()
    return launches


def run_launch(L):
    import block_scaled_fp4_nibble_amd as nv
    nv.grouped_gemm(L["x"], L["off"], L["qw"], out=L["y"])


def traffic_record(kernel_name):
    """HBM traffic measured with rocprofv3 counters, if the record matches the
    current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    ent = rec.get(kernel_name)
    if not ent or ent.get("source_sha256") != sha:
        return None
    return ent.get("bytes_per_launch")


_SINGLE_THREAD_SCRIPT = r"""
import json, sys, time
sys.path.insert(0, "@ROOT@")
import oracle, workloads as W
out = {}
def timed(fn, min_s=0.3):
    n, t0 = 0, time.perf_counter()
    while True:
        fn(); n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / n
x, w = W.small_dense()
t = timed(lambda: oracle.quantize(w))
p, s, g = oracle.quantize(w)
out["small_dense_16x256x512"] = {
    "quantize_GBps": w.nbytes / t / 1e9,
    "gemm_GFLOPS": 2 * 16 * 256 * 512 / timed(lambda: oracle.gemm(x, p, s, g[0])) / 1e9}
w = W.decode_weight()
t0 = time.perf_counter(); p, s, g = oracle.quantize(w); tq = time.perf_counter() - t0
d = {"quantize_GBps": w.nbytes / tq / 1e9,
     "gemm_sample": "the first 128 of the 4096 weight rows (output columns)"}
for m in (1, 16, 64):
    x = W.decode_act(m)
    d["gemm_m%d_GFLOPS" % m] = 2 * m * 128 * 7168 / timed(
        lambda: oracle.gemm(x, p[:128], s[:128], g[0]), 0.2) / 1e9
out["decode_4096x7168"] = d
print(json.dumps(out))
"""


def cpu_baseline(min_seconds):
    """The CPU oracle (plain C, OpenMP over rows) on whole expert segments of
    launch 1 until at least `min_seconds` of wall time have been spent, its
    quantize on the same experts' weights, and -- in a child process with one
    OpenMP thread -- the small dense product and the decode sweep (quantize
    and M = 1 / 16 / 64 at N = 4096, K = 7168)."""
    import subprocess
    import numpy as np
    import oracle
    import workloads as W

    r = W.moe_uniform_routing()
    n, k = 4096, 6144
    flops = 0
    elapsed = 0.0
    q_elapsed = 0.0
    q_bytes = 0
    experts = 0
    rows = 0
    for e in range(r.num_experts):
        c = int(r.counts[e])
        if c == 0:
            continue
        w = W.normal_bf16((1, n, k), 0.02, (W.SEED, W.W_MOE_UNIFORM, W.S_WEIGHT, 500 + e))
        x = W.normal_bf16((c, k), 1.0, (W.SEED, W.W_MOE_UNIFORM, W.S_ACT, 500 + e))
        t0 = time.perf_counter()
        p, s, g = oracle.quantize(w)
        q_elapsed += time.perf_counter() - t0
        q_bytes += w.nbytes
        off = np.array([0, c], np.int32)
        t0 = time.perf_counter()
        oracle.grouped_gemm(x, off, p, s, g)
        elapsed += time.perf_counter() - t0
        flops += 2 * c * n * k
        experts += 1
        rows += c
        if elapsed >= min_seconds:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    res = {"value": flops / elapsed / 1e12, "unit": "TFLOPS", "cores": threads,
           "kind": "oracle",
           "sample": "%d experts (%d rows) of the ~16 tok/expert up projection "
                     "(N=4096, K=6144), FP64-accumulate oracle GEMM, %.1f s" %
                     (experts, rows, elapsed),
           "quantize": {"GBps": q_bytes / q_elapsed / 1e9, "cores": threads,
                        "sample": "the same %d experts' 4096 x 6144 BF16 weights, %.1f s" %
                                  (experts, q_elapsed)}}
    env = dict(os.environ, OMP_NUM_THREADS="1")
    t0 = time.perf_counter()
    out = subprocess.run([sys.executable, "-c", _SINGLE_THREAD_SCRIPT.replace("@ROOT@", ROOT)], env=env,
                         capture_output=True, text=True, timeout=600)
    if out.returncode == 0:
        st = json.loads(out.stdout.strip().splitlines()[-1])
        st["cores"] = 1
        st["seconds"] = time.perf_counter() - t0
        res["single_thread"] = st
    else:
        res["single_thread"] = {"error": out.stderr[-500:]}
    return res


def time_fn(fn, iters, warm):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters  # ms


def extras():
    """Side measurements on the other workloads (not the headline value)."""
    import torch
    import block_scaled_fp4_nibble_amd as nv

    out = {}
    # dense decode: N=4096, K=7168.  Warm: 4 weight copies rotated, so each
    # launch reads a copy not touched for 3 launches (3 x 16.5 MB, inside the
    # 256 MB Infinity Cache).  Cold: 72 copies (1.19 GB), so each launch reads a
    # copy not touched for more than 1 GB of traffic and comes from HBM.
    n, k = 4096, 7168
    ws = [nv.quantize(randn_bf16((n, k), 0.02, 200 + i)) for i in range(4)]
    cold = [nv.QuantizedWeight(ws[i % 4].packed.clone(), ws[i % 4].scales.clone(),
                               ws[i % 4].global_scale.clone()) for i in range(72)]
    for m in (1, 16, 64):
        x = randn_bf16((m, k), 1.0, 300 + m)
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        for tag, pool, iters in (("", ws, 50), ("_cold", cold, 144)):
            it = [0]

            def f():
                nv.gemm(x, pool[it[0] % len(pool)], out=y)
                it[0] += 1
            ms = time_fn(f, iters, len(pool))
            out["dense_decode_m%d%s" % (m, tag)] = {
                "us": ms * 1e3, "GBps": dense_bytes(m, n, k) / (ms * 1e-3) / 1e9,
                "TFLOPS": 2 * m * n * k / (ms * 1e-3) / 1e12}
        # 16 chained launches (the 4 warm copies in turn) captured once as a
        # HIP graph and replayed: per-launch time without the host launch path
        chain = 16
        nv.gemm(x, ws[0], out=y)  # workspace allocated before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(chain):
                nv.gemm(x, ws[i % 4], out=y)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            for i in range(chain):
                nv.gemm(x, ws[i % 4], out=y)
        ms = time_fn(graph.replay, 10, 2) / chain
        out["dense_decode_m%d_graph" % m] = {
            "us": ms * 1e3, "GBps": dense_bytes(m, n, k) / (ms * 1e-3) / 1e9}
        del graph
    del ws, cold
    # 8192^3 dense GEMM and the bulk quantize of its weight
    m = n = k = 8192
    w = randn_bf16((n, k), 0.02, 400)
    qw = nv.quantize(w)
    x = randn_bf16((m, k), 1.0, 401)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    # 10 warm-up launches: the first few run at a lower clock (1.05-1.2 ms
    # against ~0.95 ms from the fifth launch on)
    ms = time_fn(lambda: nv.gemm(x, qw, out=y), 20, 10)
    tf = 2 * m * n * k / (ms * 1e-3) / 1e12
    out["dense_8192_cubed"] = {"ms": ms, "TFLOPS": tf,
                               "frac_of_bf16_peak": tf / BF16_DENSE_PEAK_TFLOPS}
    ms = time_fn(lambda: nv.quantize(w), 10, 2)
    qbytes = 2 * (n * k * 2) + n * k * 9 // 16 + 4  # two reads of W, one write
    out["quantize_8192x8192"] = {"us": ms * 1e3, "GBps": qbytes / (ms * 1e-3) / 1e9}
    # measured ceilings on this machine, as context for the spec peaks: the BF16
    # GEMM of the same shape through torch (hipBLASLt; contiguous operands)
    # and a device-to-device copy of 1 GiB (bytes read + bytes written)
    wt = w.t().contiguous()
    ms = time_fn(lambda: torch.matmul(x, wt, out=y), 20, 10)
    out["measured_bf16_gemm_8192_cubed"] = {"ms": ms, "TFLOPS": 2 * m * n * k / (ms * 1e-3) / 1e12}
    del wt, w, qw, x, y
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = time_fn(lambda: dst.copy_(src), 10, 3)
    out["measured_copy_1GiB"] = {"us": ms * 1e3, "GBps": 2 * src.numel() / (ms * 1e-3) / 1e9}
    del src, dst
    return out


def swiglu_extras(launches):
    """The gate_up launches with the SiLU(gate) * up epilogue (h [rows, n/2]
    leaves the kernel), against the plain launch followed by SiLU and the
    product as separate torch kernels on its output."""
    import torch
    import block_scaled_fp4_nibble_amd as nv

    out = {}
    for L in launches:
        if not L["name"].startswith("up_"):
            continue
        rows, n = L["rows"], L["n"]
        h = torch.empty((rows, n // 2), dtype=torch.bfloat16, device="cuda")

        def fused():
            nv.grouped_gemm_swiglu(L["x"], L["off"], L["qw"], out=h)

        def unfused():
            nv.grouped_gemm(L["x"], L["off"], L["qw"], out=L["y"])
            torch.mul(torch.nn.functional.silu(L["y"][:, :n // 2]), L["y"][:, n // 2:], out=h)
        # alternated, best of two rounds each (the clock drifts between runs)
        ms, ms_u = float("inf"), float("inf")
        for _ in range(2):
            ms = min(ms, time_fn(fused, 20, 3))
            ms_u = min(ms_u, time_fn(unfused, 20, 3))
        nbytes = L["bytes"] - 2 * rows * n + 2 * rows * (n // 2)
        out["swiglu_" + L["name"]] = {
            "us": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "TFLOPS": L["flops"] / (ms * 1e-3) / 1e12,
            "unfused_us": ms_u * 1e3}
    return out


def gather_extras(launches):
    """The up launches reading their routed rows from the token matrix through
    the routing index, against the plain launch on pre-permuted rows (the
    step's own form) and against torch's index_select followed by it."""
    import torch
    import block_scaled_fp4_nibble_amd as nv

    out = {}
    for L in launches:
        if not L["name"].startswith("up_"):
            continue
        x_tok = randn_bf16((L["tokens"], L["k"]), 1.0, 500)
        xp = torch.empty_like(L["x"])

        def gathered():
            nv.grouped_gemm_gather(x_tok, L["row_token"], L["off"], L["qw"], out=L["y"])

        def permuted():
            torch.index_select(x_tok, 0, L["row_token"], out=xp)
            nv.grouped_gemm(xp, L["off"], L["qw"], out=L["y"])
        # alternated, best of two rounds each
        ms_g = ms_p = ms_s = float("inf")
        for _ in range(2):
            ms_g = min(ms_g, time_fn(gathered, 20, 3))
            ms_p = min(ms_p, time_fn(lambda: run_launch(L), 20, 3))
            ms_s = min(ms_s, time_fn(permuted, 20, 3))
        out["gather_" + L["name"]] = {"us": ms_g * 1e3, "prepermuted_us": ms_p * 1e3,
                                      "index_select_then_gemm_us": ms_s * 1e3}
    return out


def combine_extras(launches):
    """The MoE combine after the down launch: each token's router-weighted sum
    of its routed rows, against torch's gather-multiply-sum of the same."""
    import numpy as np
    import torch
    import block_scaled_fp4_nibble_amd as nv
    import workloads as W

    out = {}
    for L in launches:
        if not L["name"].startswith("down_"):
            continue
        r = W.moe_zipf_routing()
        assert r.rows == L["rows"]
        tr = torch.from_numpy(r.token_rows()).cuda()
        wts = torch.rand((r.tokens, r.topk), generator=torch.Generator("cuda").manual_seed(600),
                         device="cuda")
        o = torch.empty((r.tokens, L["n"]), dtype=torch.bfloat16, device="cuda")
        y = L["y"]

        def ours():
            nv.moe_combine(y, tr, wts, out=o)

        def torch_ref():
            (y[tr].float() * wts[..., None]).sum(1).to(torch.bfloat16)
        ms_c = ms_t = float("inf")
        for _ in range(2):
            ms_c = min(ms_c, time_fn(ours, 50, 5))
            ms_t = min(ms_t, time_fn(torch_ref, 20, 3))
        nbytes = (r.rows * L["n"] + r.tokens * L["n"]) * 2 + r.rows * 8
        out["combine_" + L["name"]] = {"us": ms_c * 1e3, "GBps": nbytes / (ms_c * 1e-3) / 1e9,
                                       "frac_of_hbm": nbytes / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                       "bytes": nbytes, "torch_gather_mul_sum_us": ms_t * 1e3}
    return out


def moe_layer_extras(launches):
    """A whole routed MoE layer at ~64 tok/expert (Zipf): gather + gate_up with
    the SiLU(gate) * up epilogue (N = 4096 fused, K = 6144) -> down projection
    (N = 6144, K = 2048) -> router-weighted combine of each token's 8 rows,
    timed as eager launches and as one captured HIP graph replayed."""
    import torch
    import block_scaled_fp4_nibble_amd as nv
    import workloads as W

    up = next(L for L in launches if L["name"] == "up_zipf_64tpe")
    down = next(L for L in launches if L["name"] == "down_zipf_64tpe")
    r = W.moe_zipf_routing()
    x_tok = randn_bf16((r.tokens, up["k"]), 1.0, 700)
    tr = torch.from_numpy(r.token_rows()).cuda()
    wts = torch.rand((r.tokens, r.topk), generator=torch.Generator("cuda").manual_seed(701),
                     device="cuda")
    h = torch.empty((r.rows, up["n"] // 2), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((r.rows, down["n"]), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((r.tokens, down["n"]), dtype=torch.bfloat16, device="cuda")

    def layer():
        nv.grouped_gemm_gather(x_tok, up["row_token"], up["off"], up["qw"], act="swiglu", out=h)
        nv.grouped_gemm(h, down["off"], down["qw"], out=y)
        nv.moe_combine(y, tr, wts, out=out)
    layer()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer()
    ms_e = ms_g = float("inf")
    for _ in range(2):
        ms_e = min(ms_e, time_fn(layer, 20, 3))
        ms_g = min(ms_g, time_fn(g.replay, 20, 3))
    flops = 2 * r.rows * up["n"] * up["k"] + 2 * r.rows * down["n"] * down["k"]
    return {"moe_layer_zipf_64tpe": {"eager_us": ms_e * 1e3, "graph_us": ms_g * 1e3,
                                     "TFLOPS_graph": flops / (ms_g * 1e-3) / 1e12,
                                     "tokens": r.tokens, "topk": r.topk}}


def mlp_extras(launches):
    """The MoE MLP (gate_up with the SiLU(gate) * up epilogue, then the down
    projection N = 6144, K = 2048) as one persistent launch, against the two
    launches in a row (each planned on its own, K split where the planner
    splits it).  ~64 tok/expert uses the Zipf down weight; ~16 tok/expert a
    down weight drawn for it."""
    import torch
    import block_scaled_fp4_nibble_amd as nv

    out = {}
    down = next(L for L in launches if L["name"] == "down_zipf_64tpe")
    for L in launches:
        if not L["name"].startswith("up_"):
            continue
        if L["name"] == "up_zipf_64tpe":
            qd = down["qw"]
        else:
            w = randn_bf16((L["experts"], down["n"], down["k"]), 0.02, 800)
            qd = nv.quantize(w)
            del w
        rows = L["rows"]
        h = torch.empty((rows, L["n"] // 2), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((rows, down["n"]), dtype=torch.bfloat16, device="cuda")

        def fused():
            nv.grouped_mlp(L["x"], L["off"], L["qw"], qd, out=y, h=h)

        def two():
            nv.grouped_gemm_swiglu(L["x"], L["off"], L["qw"], out=h)
            nv.grouped_gemm(h, L["off"], qd, out=y)
        ms_f = ms_t = float("inf")
        for _ in range(2):
            ms_f = min(ms_f, time_fn(fused, 20, 3))
            ms_t = min(ms_t, time_fn(two, 20, 3))
        flops = L["flops"] + 2 * rows * down["n"] * down["k"]
        name = L["name"].replace("up_", "mlp_")
        out[name] = {"us": ms_f * 1e3, "two_launches_us": ms_t * 1e3,
                     "TFLOPS": flops / (ms_f * 1e-3) / 1e12,
                     "kernel": nv.nvfp4_grouped_mlp_kernel_name(rows, L["experts"], down["n"],
                                                                 down["k"])}
    return out


def w4a4_extras(launches):
    """The ~16 tok/expert up launch with NVFP4 activations: quantizing the
    activations, then the W4A4 launch (decode of the activations included),
    against the W4A16 launch on the same shape."""
    import torch
    import block_scaled_fp4_nibble_amd as nv

    out = {}
    for L in launches:
        if L["name"] != "up_uniform_16tpe":
            continue
        xq = nv.quantize(L["x"])
        ms_q = ms_4 = ms_16 = float("inf")
        for _ in range(2):
            ms_q = min(ms_q, time_fn(lambda: nv.quantize(L["x"]), 20, 3))
            ms_4 = min(ms_4, time_fn(lambda: nv.grouped_gemm_w4a4(xq, L["off"], L["qw"],
                                                                   out=L["y"]), 20, 3))
            ms_16 = min(ms_16, time_fn(lambda: run_launch(L), 20, 3))
        out["w4a4_" + L["name"]] = {"us": ms_4 * 1e3, "w4a16_us": ms_16 * 1e3,
                                     "quantize_activations_us": ms_q * 1e3}
    return out


def dense_only(m, n, k):
    """One dense GEMM shape: 10 warm-up and 20 timed launches."""
    import torch
    import block_scaled_fp4_nibble_amd as nv
    qw = nv.quantize(randn_bf16((n, k), 0.02, 400))
    x = randn_bf16((m, k), 1.0, 401)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ms = time_fn(lambda: nv.gemm(x, qw, out=y), 20, 10)
    tf = 2 * m * n * k / (ms * 1e-3) / 1e12
    print(json.dumps({"dense": [m, n, k], "ms": ms, "TFLOPS": tf,
                      "frac_of_bf16_peak": tf / BF16_DENSE_PEAK_TFLOPS,
                      "GBps": dense_bytes(m, n, k) / (ms * 1e-3) / 1e9}), flush=True)


COPY_BYTES = 1 << 30


def copy_calibration():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": COPY_BYTES, "copies": 5}), flush=True)


def _counter_rows(path, counter):
    import csv
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter]


def traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per launch of each gemm kernel instantiation from rocprofv3
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the ratio of
    the known bytes of a 1 GiB copy to what the same counter reads for it."""
    def copy_kib(path, counter):
        vals = [v for n, v in _counter_rows(path, counter) if "copy" in n.lower() and v > 0]
        return max(vals)
    fetch_factor = COPY_BYTES / 1024.0 / copy_kib(copy_fetch_csv, "FETCH_SIZE")
    write_factor = COPY_BYTES / 1024.0 / copy_kib(copy_write_csv, "WRITE_SIZE")
    sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    out = {"_calibration": {"fetch_factor": fetch_factor, "write_factor": write_factor,
                            "copy_bytes": COPY_BYTES}}
    per = {}
    for counter, path, factor in (("FETCH_SIZE", fetch_csv, fetch_factor),
                                  ("WRITE_SIZE", write_csv, write_factor)):
        for name, v in _counter_rows(path, counter):
            if "gemm_kp_kernel" not in name and "gemm_reg_kernel" not in name:
                continue
            key = "nvfp4::" + name.split("nvfp4::", 1)[1].split("(")[0]
            per.setdefault(key, {}).setdefault(counter, []).append(v * 1024.0 * factor)
    for key, d in per.items():
        fetch = sum(d.get("FETCH_SIZE", [0])) / max(1, len(d.get("FETCH_SIZE", [])))
        write = sum(d.get("WRITE_SIZE", [0])) / max(1, len(d.get("WRITE_SIZE", [])))
        out[key] = {"source_sha256": sha, "bytes_per_launch": fetch + write,
                    "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
                    "dispatches": len(d.get("FETCH_SIZE", []))}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: every box here has a single MI355X, so "
              "--gpus %d is not supported (the sharding design is described in the docs)" %
              args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.dense:
        dense_only(*args.dense)
        return
    launches = build_workload()
    step_flops = sum(L["flops"] for L in launches)
    step_bytes = sum(L["bytes"] for L in launches)

    for _ in range(args.warmup):
        for L in launches:
            run_launch(L)
    torch.cuda.synchronize()

    # timed region: per-launch HIP events on the launch stream, wall clock
    # around the whole region with synchronization on both sides
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        for j, L in enumerate(launches):
            run_launch(L)
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    samples = [[evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]
               for j in range(len(launches))]
    launch_ms = [sum(v) / len(v) for v in samples]

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]

    # dominant kernel instantiation by total time (the library names the
    # kernel each launch runs)
    by_kernel = {}
    for L, ms in zip(launches, launch_ms):
        d = by_kernel.setdefault(L["kernel"], {"ms": 0.0, "bytes": 0, "launches": 0, "names": []})
        d["ms"] += ms
        d["bytes"] += L["bytes"]
        d["launches"] += 1
        d["names"].append(L["name"])
    kernel, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    avg_ms = dom["ms"] / dom["launches"]
    bytes_per_launch = dom["bytes"] / dom["launches"]
    achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    tr = traffic_record(kernel)

    result = {
        "metric": METRIC,
        "value": step_flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "moe_grouped_gemm_16_to_64_tok_per_expert",
            "experts": 64,
            "launches": [{"name": L["name"], "rows": L["rows"], "n": L["n"], "k": L["k"],
                          "nonempty_experts": sum(1 for c in L["counts"] if c),
                          "max_rows_per_expert": max(L["counts"]),
                          "us": ms * 1e3,
                          "us_p10_median_p90": [pct(v, q) * 1e3 for q in (0.1, 0.5, 0.9)],
                          "TFLOPS": L["flops"] / (ms * 1e-3) / 1e12,
                          "GBps": L["bytes"] / (ms * 1e-3) / 1e9}
                         for L, ms, v in zip(launches, launch_ms, samples)],
        },
        "hbm_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "launches": dom["names"],
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "avg_launch_us": avg_ms * 1e3,
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "traffic": tr,
        },
    }
    if not args.no_extras:
        # the epilogue and gather comparisons first: after the 8192^3 GEMMs in
        # extras() the clock runs lower for a while
        ex = swiglu_extras(launches)
        ex.update(gather_extras(launches))
        ex.update(combine_extras(launches))
        ex.update(w4a4_extras(launches))
        ex.update(moe_layer_extras(launches))
        ex.update(mlp_extras(launches))
        ex.update(extras())
        # the same rates against what this box measured (context for the
        # spec peaks): the dominant kernel's algorithmic GB/s over a device
        # copy's, the 8192^3 NVFP4 GEMM over hipBLASLt's BF16 GEMM
        ex["vs_measured_ceilings"] = {
            "roofline_kernel_frac_of_copy_GBps":
                achieved / ex["measured_copy_1GiB"]["GBps"],
            "dense_8192_cubed_frac_of_hipblaslt_bf16":
                ex["dense_8192_cubed"]["TFLOPS"] / ex["measured_bf16_gemm_8192_cubed"]["TFLOPS"],
        }
        result["extras"] = ex
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
