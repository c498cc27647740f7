"""Engram forward throughput on one MI355X.

One step = one engram_forward call over one batch of the workload (hash +
gather, K/V projection, gate, short conv + residual), inputs resident in HBM.
Prints one JSON line: tokens/s, per-kernel times from HIP events recorded
inside the timed region on the launch stream, the roofline of the dominant
kernel, and the oracle's single-thread CPU rate on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config b1_t32768]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram forward tokens/sec at 1 MI355X; gather/gate HBM GB/s as % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FP32_PEAK_TFLOPS = 157.3        # MI355X dense fp32 on the matrix cores (v_mfma_f32_32x32x2_f32)


def kernel_model(w, N, split=False, with_state=False):
    """Algorithmic work per launch of each kernel, as {"flops": F, "bytes": B}.
    Bytes count what the method must move through HBM (ids, table rows,
    activations, weights once, outputs, state), not re-reads; the GEMMs count
    their multiply-adds as 2 flops.  `split`: the fused GEMM covers the key
    channels and project_value_gemm the value channels."""
    s = 2 if w.dtype == "bf16" else 4
    E, d, hc, K = w.emb_dim, w.hidden, w.hc_mult, w.conv_kernel
    P = d // 128                                   # gate partial sums per (token, branch), 16 B each
    R = (K - 1) * w.conv_dilation + 1              # ring positions of the decode state
    B = w.batch
    hist = N * (w.max_order - 1) * 4 + B * 8 if with_state else 0
    ring = B * (R * (d * s + 4 * hc) + (w.max_order - 1) * 4 + 8) if with_state else 0
    w_all, w_keys, w_val = (hc + 1) * d * E * s, hc * d * E * s, d * E * s
    return {
        "hash_gather": {"flops": 0, "bytes": N * (4 + 2 * E * s) + hist},
        "project_gemm": {"flops": 2.0 * N * E * (hc + 1) * d, "bytes": N * E * s + w_all + N * (hc + 1) * d * s},
        "project_gate_gemm": {
            "flops": 2.0 * N * E * (hc if split else hc + 1) * d,
            "bytes": N * E * s + (w_keys if split else w_all) + N * hc * d * s + N * hc * P * 16
                     + (0 if split else N * d * s)},
        "project_value_gemm": {"flops": 2.0 * N * E * d,
                               "bytes": N * E * s + w_val + N * d * s + N * hc * (P * 16 + 4)},
        "gate": {"flops": 0, "bytes": N * (2 * hc * d * s + 4 * hc)},
        "gate_finalize": {"flops": 0, "bytes": N * hc * (16 * P + 4)},
        "short_conv": {"flops": 0, "bytes": N * (d * s + 4 * hc + hc * d * s) + ring},
        "advance_state": {"flops": 0, "bytes": ring},
        # one decode step: the partial sums, the value row, the K-1 history taps of
        # the rings and the new slot written, the output, the taps' weights, and
        # n_past / the token ring
        "decode_tail": {"flops": 0, "bytes": N * hc * (16 * P) + N * d * s + N * hc * d * s + hc * d * K * s
                        + K * N * (d * s + 4 * hc) + N * 28},
    }


def step_floor(w, N):
    """Whole-step floors: the bytes no schedule can avoid (ids, the gathered
    rows, the queries read and the outputs written -- every intermediate fused
    away -- and the weights once) and the projection's flops."""
    s = 2 if w.dtype == "bf16" else 4
    E, d, hc = w.emb_dim, w.hidden, w.hc_mult
    return {"bytes": N * (4 + E * s + 2 * hc * d * s) + (hc + 1) * d * E * s,
            "flops": 2.0 * N * E * (hc + 1) * d}


def roofline_of(work, us, dtype):
    """The kernel's binding roofline -- the larger of its HBM and matrix-core
    floors -- and its achieved rate against that peak."""
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if dtype == "bf16" else FP32_PEAK_TFLOPS
    t_mfma = work["flops"] / (mfma_peak * 1e12)
    t_hbm = work["bytes"] / (HBM_PEAK_GBS * 1e9)
    if work["flops"] and t_mfma >= t_hbm:
        ach = work["flops"] / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(ach / mfma_peak, 4), "work_per_launch": work["flops"]}
    ach = work["bytes"] / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "work_per_launch": work["bytes"]}


def step_roofline(w, N, step_us):
    f = step_floor(w, N)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    hbm_us = f["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6
    mfma_us = f["flops"] / (mfma_peak * 1e12) * 1e6
    return {"floor_bytes": f["bytes"], "floor_flops": f["flops"], "hbm_floor_us": round(hbm_us, 2),
            "mfma_floor_us": round(mfma_us, 2), "bound": "mfma" if mfma_us >= hbm_us else "hbm",
            "step_us": round(step_us, 2), "frac": round(max(hbm_us, mfma_us) / step_us, 4),
            "frac_of_serial_floor": round((hbm_us + mfma_us) / step_us, 4),
            "note": "frac = max(HBM floor, MFMA floor) / step time; the serial floor adds the two (the HBM-bound "
                    "and MFMA-bound kernels run one after the other)"}


def kernel_table(w, N, names, per_kernel_us, with_state=False):
    model = kernel_model(w, N, split="project_value_gemm" in names, with_state=with_state)
    out = []
    for name, us in zip(names, per_kernel_us):
        r = roofline_of(model[name], us, w.dtype)
        out.append({"name": name, "avg_us": round(us, 2), **r, "flops": model[name]["flops"],
                    "bytes": model[name]["bytes"]})
    return out


def measured_traffic(args, w, name):
    """HBM bytes per launch of `name` from the rocprofv3 counters in
    profiles/traffic.json, or None once a forward source changed since."""
    import hashed_gram_conditional_amd as eg

    if not os.path.exists(args.traffic):
        return None
    with open(args.traffic) as f:
        tr = json.load(f)
    if tr.get("source_hash") != eg.source_hash():
        return None
    return tr.get("workloads", {}).get(w.name, {}).get(name)


class Hip:
    """The few HIP runtime calls the timing needs (the runtime torch loaded)."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence: timing-only events, no cache flush

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def cpu_baseline(w, inp, budget_s=15.0):
    """The oracle (single-threaded C, double precision) over the first positions
    of the batch in order (sequence 0 first), sized to about budget_s seconds."""
    import numpy as np

    import oracle as orc

    B, T = w.batch, inp.seq_total
    o = orc.Oracle.from_workload(w, inp, batch=B, seqlen=T)
    idx = o.hash(inp.ids, remap=inp.remap).reshape(B * T, -1)
    off = np.concatenate([[0], np.cumsum(inp.primes)[:-1]])
    wkv, gk, gq, cw = inp.wkv(), inp.gamma_k(), inp.gamma_q(), inp.conv_w()

    def run(n):
        pos = np.arange(n, dtype=np.int64)
        rows = np.unique((idx[:n] + off).ravel())
        tab = inp.table_rows(rows)
        hid = inp.hidden_at(pos // T, pos % T).reshape(n, -1)
        t0 = time.perf_counter()
        o.forward_at(inp.ids, inp.remap, tab, wkv, gk, gq, cw, hid, pos, table_keys=rows, hidden_keys=pos)
        return time.perf_counter() - t0

    n0 = min(8, B * T)
    t_small = run(n0)
    n = int(min(B * T, max(n0, budget_s / max(t_small / n0, 1e-9))))
    dt = run(n) if n > n0 else t_small
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"full forward over the first {n} of {B * T} positions of {w.name} (sequence by "
                      f"sequence, {dt:.1f} s single-threaded, no BLAS)"}


def bench_decode(args, w):
    """Decode-shaped workload: the prompt is prefilled with state (untimed), then
    every sequence takes single-token steps.  The step loop is captured once in a
    HIP graph (torch.cuda.graph around the library's launches on the capture
    stream) and replayed; a separate eager pass with HIP events gives the
    per-kernel times.  tokens/s = batch * steps / time of the captured steps."""
    import torch

    import engram_synth as S
    import hashed_gram_conditional_amd as eg
    from engram_synth.device import device_inputs

    inp = S.Inputs(w)
    torch.cuda.set_device(0)
    d = device_inputs(inp)
    B, P = w.batch, w.decode_prompt
    steps = min(args.steps, w.decode_steps) if args.steps else w.decode_steps
    cfg1 = eg.EngramConfig.make(**w.config_kwargs(inp, batch=B, seqlen=1))
    cfgp = eg.EngramConfig.make(**w.config_kwargs(inp, batch=B, seqlen=P))
    p = eg.Params(remap=d["remap"], tables=d["tables"], w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                  conv_w=d["conv_w"])
    ids_steps = d["ids"][:, P:P + steps].t().contiguous()                 # [steps][B]
    hid_steps = d["hidden"][:, P:P + steps].transpose(0, 1).contiguous()  # [steps][B][hc][d]
    prompt_ids = d["ids"][:, :P].contiguous()
    prompt_hid = d["hidden"][:, :P].contiguous()
    del d["hidden"]
    st = eg.State(cfg1, B)
    ws = eg.alloc_workspace(cfgp)
    out1 = torch.empty((B, 1, w.hc_mult, w.hidden), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                       device="cuda")
    outp = torch.empty((B, P, w.hc_mult, w.hidden), dtype=out1.dtype, device="cuda")
    eg.forward(cfgp, p, prompt_ids, prompt_hid, state=st, out=outp, workspace=ws)
    torch.cuda.synchronize()

    # per-kernel times: eager single-token steps with events (they advance the state too)
    hip = Hip()
    names = eg.kernel_names(cfg1, with_state=True)
    nk = len(names)
    n_ev = min(32, steps)
    evs = [hip.events(2 * nk) for _ in range(n_ev)]
    for k in range(n_ev):
        eg.forward(cfg1, p, ids_steps[k], hid_steps[k], state=st, out=out1, workspace=ws, events=evs[k])
    torch.cuda.synchronize()
    per_kernel_us = [sum(hip.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evs) / n_ev * 1e3 for i in range(nk)]
    for e in evs:
        hip.destroy(e)

    graph = torch.cuda.graph_pool_handle()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, pool=graph, stream=s):
            for k in range(steps):
                eg.forward(cfg1, p, ids_steps[k], hid_steps[k], state=st, out=out1, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for _ in range(max(args.warmup, 1)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / steps
    res = {
        "metric": METRIC, "value": round(B * steps / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": max(args.warmup, 1), "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seqlen": 1, "decode_prompt": P, "decode_steps": steps,
                   "hidden": w.hidden, "hc_mult": w.hc_mult, "table_rows": w.table_rows,
                   "tokens_per_step": B, "parallelism": "single-gpu", "launch": "hip-graph of all steps"},
        "kernels_note": "eager single-token steps timed with HIP events (outside the graph)",
    }
    kernels = kernel_table(w, B, names, per_kernel_us, with_state=True)
    dom = max(kernels, key=lambda k: k["avg_us"])
    res["roofline"] = {"kernel": dom["name"], "bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                       "unit": dom["unit"], "frac": dom["frac"], "traffic": measured_traffic(args, w, dom["name"])}
    res["step_roofline"] = step_roofline(w, B, ms_per_step * 1e3)
    res["kernels"] = kernels
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(res))


def bench_offload(args, w):
    """Tables in pinned host memory mapped into the device (walk-through 4.4:
    the hash needs only the ids, so the rows are fetched while the layers before
    the Engram layer run).  Per step, with L layers of a dense FFN (d -> 4d -> d,
    bf16 matmuls) standing in for those layers:
      resident:  FFN x L, then engram_forward with the tables in HBM;
      offloaded: at the step start a side stream hashes the ids and gathers the
                 rows from host memory; the main stream runs FFN x L, waits for
                 the side stream, then engram_forward_gathered.
    Two ways to bring the rows in:
      zero-copy: a GPU gather reading the host table over the link (32
                 workgroups); it holds those CUs while it waits on the link;
      host+DMA:  the indices are copied to host memory, host threads copy the
                 rows into pinned staging (engram_gather_host), the DMA
                 engines copy them to HBM: no compute units taken.
    Reports the step times and the loss of each offloaded flow, for several L."""
    import torch

    import engram_synth as S
    import hashed_gram_conditional_amd as eg
    from engram_synth.device import device_inputs

    inp = S.Inputs(w)
    torch.cuda.set_device(0)
    d = device_inputs(inp)
    cfg = eg.EngramConfig.make(**w.config_kwargs(inp))
    p = eg.Params(remap=d["remap"], tables=d["tables"], w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                  conv_w=d["conv_w"])
    t = d["tables"]
    # pinned host memory mapped into the device serves both flows; where the
    # host cannot pin the whole table (the 77 GB one), ordinary pageable memory
    # serves the host+DMA flow alone (its reads are host threads' memcpy)
    nbytes = t.numel() * t.element_size()
    try:
        if nbytes > 32 << 30:
            raise MemoryError("table larger than the pinned host memory the box grants")
        host = eg.alloc_mapped_host(nbytes)
        host.copy_from(t)
        host_tab = host
    except MemoryError:
        host = None
        host_tab = torch.empty(t.shape, dtype=t.dtype)
        rows = 1 << 22
        for i in range(0, t.shape[0], rows):
            host_tab[i:i + rows].copy_(t[i:i + rows])
    ph = None if host is None else eg.Params(remap=d["remap"], tables=host, w_kv=d["w_kv"], gamma_k=d["gamma_k"],
                                             gamma_q=d["gamma_q"], conv_w=d["conv_w"])
    no_tables = eg.Params(remap=d["remap"], tables=None, w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                          conv_w=d["conv_w"])
    N = w.batch * w.seqlen
    free, total = torch.cuda.mem_get_info()
    print(f"device memory free {free / 2**30:.1f} of {total / 2**30:.1f} GiB after the tables", file=sys.stderr,
          flush=True)
    ws = eg.alloc_workspace(cfg)
    out = torch.empty((w.batch, w.seqlen, w.hc_mult, w.hidden), dtype=d["hidden"].dtype, device="cuda")
    idx = torch.empty((w.batch, w.seqlen, cfg.n_heads), dtype=torch.int32, device="cuda")
    e = torch.empty((w.batch, w.seqlen, cfg.emb_dim), dtype=d["hidden"].dtype, device="cuda")
    x = torch.randn(N, w.hidden, dtype=torch.bfloat16, device="cuda")
    w1 = torch.randn(w.hidden, 4 * w.hidden, dtype=torch.bfloat16, device="cuda") * 0.02
    w2 = torch.randn(4 * w.hidden, w.hidden, dtype=torch.bfloat16, device="cuda") * 0.02
    h1 = torch.empty(N, 4 * w.hidden, dtype=torch.bfloat16, device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    hip = Hip()

    def ffn(layers):
        for _ in range(layers):
            torch.matmul(x, w1, out=h1)
            torch.matmul(h1, w2, out=x)

    def resident(layers):
        ffn(layers)
        eg.forward(cfg, p, d["ids"], d["hidden"], out=out, workspace=ws, stream=main)

    def offloaded(layers):
        side.wait_stream(main)                     # the ids are known at the step start
        with torch.cuda.stream(side):
            eg.engram_hash(cfg, ph, d["ids"], out=idx, stream=side)
            eg.engram_gather(cfg, ph, idx, out=e, stream=side)
        ffn(layers)
        main.wait_stream(side)
        eg.forward_gathered(cfg, ph, e, d["hidden"], out=out, workspace=ws, stream=main)

    idx_h = torch.empty(idx.shape, dtype=torch.int32, pin_memory=True)
    e_h = torch.empty(e.shape, dtype=e.dtype, pin_memory=True)
    ev_idx = torch.cuda.Event()

    def offloaded_dma(layers):
        side.wait_stream(main)
        with torch.cuda.stream(side):
            eg.engram_hash(cfg, p, d["ids"], out=idx, stream=side)
            idx_h.copy_(idx, non_blocking=True)
            ev_idx.record(side)
        ffn(layers)
        ev_idx.synchronize()                       # the host waits for the indices only
        eg.engram_gather_host(cfg, host_tab, idx_h, e_h)
        with torch.cuda.stream(side):
            e.copy_(e_h, non_blocking=True)
        main.wait_stream(side)
        eg.forward_gathered(cfg, no_tables, e, d["hidden"], out=out, workspace=ws, stream=main)

    def timed(fn, steps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    steps = max(args.steps // 4, 10)
    # the two halves of the offloaded step alone: hash + gather from host vs from HBM
    gather_host = None if ph is None else timed(
        lambda: eg.engram_gather(cfg, ph, eg.engram_hash(cfg, ph, d["ids"], out=idx), out=e), steps)
    gather_dev = timed(lambda: eg.engram_gather(cfg, p, eg.engram_hash(cfg, p, d["ids"], out=idx), out=e), steps)
    idx_h.copy_(idx)
    eg.engram_gather_host(cfg, host_tab, idx_h, e_h)   # first touch of the pinned buffers
    t0 = time.perf_counter()
    for _ in range(steps):
        eg.engram_gather_host(cfg, host_tab, idx_h, e_h)
    gather_cpu = (time.perf_counter() - t0) / steps * 1e6
    h2d = timed(lambda: e.copy_(e_h, non_blocking=True), steps)
    rows_bytes = N * cfg.emb_dim * t.element_size()
    rows = []
    for layers in (0, 1, 2, 4, 8):
        # the GEMM-heavy steps run at a power-limited clock that drifts between
        # runs: the variants are measured in turns, three times, and the median kept
        runs = {"ffn": [], "r": [], "o": [], "od": []}
        for _ in range(3):
            runs["ffn"].append(timed(lambda: ffn(layers), steps) if layers else 0.0)
            runs["r"].append(timed(lambda: resident(layers), steps))
            runs["o"].append(timed(lambda: offloaded(layers), steps) if ph is not None else None)
            runs["od"].append(timed(lambda: offloaded_dma(layers), steps))
        ffn_us, r, od = (sorted(runs[k])[1] for k in ("ffn", "r", "od"))
        o = sorted(runs["o"])[1] if ph is not None else None
        rows.append({"ffn_layers": layers, "ffn_us": round(ffn_us, 1), "resident_us": round(r, 1),
                     "zero_copy_us": None if o is None else round(o, 1),
                     "zero_copy_loss": None if o is None else round(o / r - 1.0, 4),
                     "host_dma_us": round(od, 1), "host_dma_loss": round(od / r - 1.0, 4)})
    torch.cuda.synchronize()
    if host is not None:
        host.free()
    res = {
        "mode": "offload", "workload": w.name, "tokens_per_step": N, "table_bytes": t.numel() * t.element_size(),
        "host_tables": "pinned host memory, mapped, non-coherent (device may cache)" if host is not None else
                       "pageable host memory (pinning the whole table failed): host+DMA flow only",
        "hash_gather_from_host_us": None if gather_host is None else round(gather_host, 1),
        "hash_gather_from_hbm_us": round(gather_dev, 1),
        "host_rows_GBps": None if gather_host is None else round(rows_bytes / (gather_host * 1e-6) / 1e9, 1),
        "host_threads_gather_us": round(gather_cpu, 1), "rows_h2d_copy_us": round(h2d, 1),
        "steps": steps, "per_ffn_layers": rows,
    }
    print(json.dumps(res))


def bench_train(args, w):
    """One training step of the module (walk-through 4.4 trains the tables and
    weights with the model): engram_forward_train, which keeps the forward
    quantities in the backward workspace, then engram_backward_saved for a
    fixed upstream gradient.  The float32 gradients accumulate across steps, as
    over micro-batches; the optimiser's update is not part of the module.
    Also times engram_forward (inference) and engram_backward (recomputing the
    forward quantities), and gives the rate of the saved backward's GEMM flops
    (dE = dKV.W and dW = dKV^T.E) against the bf16 MFMA peak."""
    import torch

    import engram_synth as S
    import hashed_gram_conditional_amd as eg
    from engram_synth.device import device_inputs, fill

    inp = S.Inputs(w)
    torch.cuda.set_device(0)
    d = device_inputs(inp)
    cfg = eg.EngramConfig.make(**w.config_kwargs(inp))
    p = eg.Params(remap=d["remap"], tables=d["tables"], w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                  conv_w=d["conv_w"])
    N = w.batch * w.seqlen
    ws = eg.alloc_workspace(cfg)
    bws = eg.alloc_backward_workspace(cfg)
    out = torch.empty_like(d["hidden"])
    dy = torch.empty_like(d["hidden"])
    fill(dy, w.seed, *inp.recipe("dy"))
    # the table gradient: dense float32 where it fits beside the tables, else
    # row-sparse (the rows the step's hashes select, with their sums)
    dense_bytes = w.table_rows * w.head_dim * 4
    sparse = args.sparse or dense_bytes > 16 << 30
    stream = torch.cuda.current_stream()
    if sparse:
        d_hidden, grads, rows = eg.backward_sparse(cfg, p, d["ids"], d["hidden"], dy, workspace=bws)
    else:
        d_hidden, grads = eg.backward(cfg, p, d["ids"], d["hidden"], dy, workspace=bws)
        rows = None

    def fwd():
        eg.forward(cfg, p, d["ids"], d["hidden"], out=out, workspace=ws, stream=stream)

    def fwd_train():
        eg.forward_train(cfg, p, d["ids"], d["hidden"], bws, out=out, stream=stream)

    def bwd_saved():
        if sparse:
            eg.backward_saved_sparse(cfg, p, d["hidden"], dy, bws, grads=grads, rows=rows, d_hidden=d_hidden,
                                     stream=stream)
        else:
            eg.backward_saved(cfg, p, d["hidden"], dy, bws, grads=grads, d_hidden=d_hidden, stream=stream)

    def bwd():
        if sparse:
            eg.backward_sparse(cfg, p, d["ids"], d["hidden"], dy, grads=grads, rows=rows, d_hidden=d_hidden,
                               workspace=bws, stream=stream)
        else:
            eg.backward(cfg, p, d["ids"], d["hidden"], dy, grads=grads, d_hidden=d_hidden, workspace=bws,
                        stream=stream)

    def train():
        fwd_train()
        bwd_saved()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    train_ms = timed(train)
    fwd_train_ms = timed(fwd_train)
    bwd_saved_ms = train_ms - fwd_train_ms
    fwd_ms = timed(fwd)
    bwd_ms = timed(bwd)
    flops = 2 * 2.0 * N * cfg.emb_dim * (w.hc_mult + 1) * w.hidden
    tflops = flops / (bwd_saved_ms * 1e-3) / 1e12
    res = {
        "mode": "train", "metric": "Engram forward + backward tokens/sec at 1 MI355X",
        "value": round(N / (train_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(train_ms, 4),
        "forward_train_ms": round(fwd_train_ms, 4), "backward_saved_ms": round(bwd_saved_ms, 4),
        "inference_forward_ms": round(fwd_ms, 4), "backward_recompute_ms": round(bwd_ms, 4),
        "steps": args.steps, "warmup": args.warmup,
        "dtype": w.dtype, "data": "synthetic", "config": {"workload": w.name, "tokens_per_step": N},
        "table_gradient": "row-sparse (rows used: %d of %d)" % (int(rows["n_rows"].item()), w.table_rows)
                          if sparse else "dense float32",
        "backward_gemm_flops": flops, "backward_gemm_TFLOPs_over_backward_time": round(tflops, 1),
        "frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4) if w.dtype == "bf16" else None,
        "workspace_bytes": {"forward": ws.numel(), "backward": bws.numel()},
    }
    print(json.dumps(res))


def bench_vocab(args, w):
    """Compressed token ids (walk-through 2.2-1, 4.1): the host builder of the
    remap table on a synthetic vocabulary of the workload's size, best of 5;
    the oracle's builder timed once beside it as the CPU baseline."""
    from engram_synth.vocab import synthetic_vocab
    from hashed_gram_conditional_amd.compressed_vocab import build_remap

    texts = synthetic_vocab(w.seed, w.vocab)
    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        remap, n = build_remap(texts)
        times.append(time.perf_counter() - t0)
    best = min(times)
    res = {"mode": "vocab", "metric": "compressed-id table build, tokens/s (host)", "value": round(len(texts) / best, 1),
           "unit": "tokens/s", "seconds": round(best, 4), "vocab": len(texts), "compressed": int(n),
           "reduction": round(1 - n / len(texts), 4), "data": "synthetic vocabulary", "config": {"workload": w.name}}
    if not args.no_cpu_baseline:
        from oracle.compressed_vocab import compressed_ids

        t0 = time.perf_counter()
        compressed_ids(texts)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(len(texts) / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole {len(texts)}-token vocabulary"}
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="b1_t32768",
                    help="workload: b1_t32768 (default: the largest, 77 GB of tables), b8_t4096, b4_t1024, "
                         "tiny_fp32, decode_b256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    ap.add_argument("--zipf", type=float, default=None,
                    help="override the workload's Zipf exponent of the token stream (0 = uniform tokens: the "
                         "control without the cache reuse of frequent n-grams)")
    ap.add_argument("--offload", action="store_true",
                    help="tables in host memory: measure the prefetch flow against HBM-resident tables")
    ap.add_argument("--vocab", action="store_true",
                    help="host build of the compressed-id table from a synthetic vocabulary of the workload's size")
    ap.add_argument("--train", action="store_true",
                    help="forward + backward (gradients of the tables and weights) per step")
    ap.add_argument("--sparse", action="store_true",
                    help="with --train: the table gradient row-sparse (automatic when a dense one exceeds 16 GiB)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run a plain float32 copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Engram tables of every workload fit in one MI355X's HBM, and the "
              "library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import engram_synth as S
    import hashed_gram_conditional_amd as eg
    from engram_synth.device import device_inputs

    w = S.WORKLOADS[args.config]
    if args.zipf is not None:
        w = w.replace(zipf_a=args.zipf)
    if args.offload:
        return bench_offload(args, w)
    if args.train:
        return bench_train(args, w)
    if args.vocab:
        return bench_vocab(args, w)
    if w.decode_prompt:
        return bench_decode(args, w)
    inp = S.Inputs(w)
    torch.cuda.set_device(0)
    d = device_inputs(inp)
    cfg = eg.EngramConfig.make(**w.config_kwargs(inp))
    p = eg.Params(remap=d["remap"], tables=d["tables"], w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                  conv_w=d["conv_w"])
    ws = eg.alloc_workspace(cfg)
    out = torch.empty((w.batch, w.seqlen, w.hc_mult, w.hidden), dtype=d["hidden"].dtype, device="cuda")
    names = eg.kernel_names(cfg)
    nk = len(names)
    N = w.batch * w.seqlen

    if args.calibrate_copy_mb:
        src = torch.ones(args.calibrate_copy_mb * 2**18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        eg.forward(cfg, p, d["ids"], d["hidden"], out=out, workspace=ws)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # timed region: exactly K steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        eg.forward(cfg, p, d["ids"], d["hidden"], out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    # second timed region of K steps with every kernel bracketed by HIP events on
    # the launch stream (timing-only events: no system-scope fence), for the
    # per-kernel durations the roofline uses
    hip = Hip()
    evs = [hip.events(2 * nk) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        eg.forward(cfg, p, d["ids"], d["hidden"], out=out, workspace=ws, stream=stream, events=evs[k])
    torch.cuda.synchronize()
    per_kernel_ms = [sum(hip.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evs) / args.steps for i in range(nk)]
    step_gpu_ms = sum(hip.elapsed_ms(e[0], e[-1]) for e in evs) / args.steps
    for e in evs:
        hip.destroy(e)

    ms_per_step = dt * 1e3 / args.steps
    kernels = kernel_table(w, N, names, [ms * 1e3 for ms in per_kernel_ms])
    dom = max(kernels, key=lambda k: k["avg_us"])
    roofline = {"kernel": dom["name"], "bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                "unit": dom["unit"], "frac": dom["frac"], "traffic": measured_traffic(args, w, dom["name"])}
    hbm = [k for k in kernels if k["bound"] == "hbm" and k["work_per_launch"] > 0]
    hbm_bytes = sum(k["work_per_launch"] for k in hbm)
    hbm_us = sum(k["avg_us"] for k in hbm)
    s = 2 if w.dtype == "bf16" else 4
    hbm_path = {"kernels": [k["name"] for k in hbm], "achieved": round(hbm_bytes / (hbm_us * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(hbm_bytes / (hbm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "note": "the HBM-bound kernels only; on the fused plans the gate's sums run in the projection GEMM's "
                        "epilogue, so its largest read, the queries (%d bytes), is timed inside that MFMA-bound "
                        "kernel -- the whole step is measured by step_roofline" % (N * w.hc_mult * w.hidden * s)}

    res = {
        "metric": METRIC, "value": round(N / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "vocab": w.vocab, "zipf_a": w.zipf_a,
                   "orders": w.orders, "heads_per_order": w.heads_per_order, "head_dim": w.head_dim,
                   "hidden": w.hidden, "hc_mult": w.hc_mult, "table_rows": w.table_rows,
                   "tokens_per_step": N, "parallelism": "single-gpu"},
        "gpu_ms_per_step_events": round(step_gpu_ms, 4),
        "roofline": roofline, "step_roofline": step_roofline(w, N, ms_per_step * 1e3),
        "gather_gate_conv_hbm": hbm_path, "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
