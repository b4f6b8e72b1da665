"""Benchmark one routed-expert MoE layer forward on one MI355X.

A step is one moe_layer_forward over one seeded batch: gate scores, top-k +
counts + offsets, permutation, grouped SwiGLU expert GEMMs, combine (and the
latent projections for the latent layer).  Inputs and weights are resident in
HBM before timing starts.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

The default workload is the largest layer, DeepSeek-R1-shaped (T=8192,
H=7168, E=256, k=8, I=2048, bf16, Zipf-skewed routing).  Other configs:
qwen3_30b_a3b_shaped, k3_shaped_decode, k3_shaped_decode_t8, latent_moe,
tiny_f32, deepseek_r1_shaped_shared (the R1-shaped layer with a shared
expert of width 2048).

Per-stage times come from HIP events that moe_layer_forward records on the
stream the kernels run on.  The roofline object describes the dominant kernel
(the expert gate/up GEMM): algorithmic bytes per launch (the compulsory bytes:
touched experts' W1 and W3, one input row per routed assignment, the
intermediate written) over its average event-timed duration, against
MI355X's 8 TB/s HBM peak.  Which kernels run is the library's own decision,
read from moe_layer_plan.  cpu_baseline is the
CPU oracle (tests' reference implementation) timed on a bounded token sample of
the same layer on this host's cores.

Besides the contract's back-to-back steps, the line carries:
  cold            layers run after a 1 GiB write that evicts every XCD's L2 and
                  the 256 MB last-level cache (median / p95 of event times);
  combine_alone   moe_combine on its own, fused and as the unpermute +
                  weighted-reduce pair;
  permute_alone   moe_dispatch_permute on its own, writing the T*k*D*b
                  permuted copy (the fused layer writes only row metadata);
  ep_rank_share   (--ep-rank-share R) the grouped expert FFN at the share one
                  rank of R-way expert parallelism would run: R source batches
                  routed on this GPU, the rows of experts [0, E/R) gathered.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
F32_PEAK_TFLOPS = 157.3
GEMM_SRC = os.path.join(ROOT, "routing_dispatch_expert_logits_amd", "csrc", "gemm.hip")
# the headers gemm.hip includes: a change in either changes the compiled GEMM too
GEMM_HEADERS = [os.path.join(ROOT, "routing_dispatch_expert_logits_amd", "csrc", h)
                for h in ("moe_kernels.h", "moe_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{config}.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded.

    The events are timing-only: created with hipEventDisableSystemFence, so recording
    one does not write back and invalidate the caches (which slows the kernel that
    follows); every read of them comes after a device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
            assert rc == 0, f"hipEventCreateWithFlags failed: {rc}"
            evs.append(h.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert rc == 0, f"hipEventElapsedTime failed: {rc}"
        return ms.value

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        assert rc == 0, f"hipEventRecord failed: {rc}"

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def layer_plan(B, cfg):
    """The kernels moe_layer_forward runs for this layer (called without aux x_perm, as
    here): the library's own decision, from moe_layer_plan."""
    s = B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.dtype, cfg.shared_I, cfg.capacity,
                cfg.dispatch)
    return B.layer_plan(s, cfg.gate == "computed")


def stage_bytes_flops(cfg, counts, gath):
    """Algorithmic HBM bytes and FLOPs per stage for one layer forward.

    b = element bytes of activations/weights; touched = experts with >= 1 row; the
    row count R is the rows kept (all T*k unless an expert capacity drops some).
    gath: whether the gate/up GEMM reads the token rows through row_token (the plan's
    rows_gathered); then the permutation writes only the metadata.  The gate/up GEMM's
    bytes count one input row per routed assignment (R*D*b, the permuted operand it
    multiplies), whichever way it fetches it; "gemm_gate_up_gathered" counts the T
    token rows instead, the least a gathering kernel must fetch.
    """
    T, H, E, k, I, L, D = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.D
    R = int(sum(counts))
    b = cfg.elem_bytes
    touched = int(sum(1 for c in counts if c > 0))
    out_b = 2 if cfg.dtype == "bf16" else 4
    st = {}
    st["latent_down"] = (T * H * b + L * H * b + T * L * b, 2 * T * H * L) if L else (0, 0)
    st["gate"] = ((T * H * b + E * H * 4 + T * E * 4, 2 * T * H * E) if cfg.gate == "computed"
                  else (0, 0))
    st["route"] = (T * E * 4 + 8 * R + (2 * E + 1) * 4, 0)
    if cfg.dispatch == "mxfp8":
        # rows and W1 / W3 as one code byte per element plus one scale byte per 32
        q = D * 33 // 32
        st["permute"] = (T * D * b + (T if gath else R) * q + 12 * R, 0)
        st["gemm_gate_up"] = (touched * 2 * q * I + R * q + R * I * b, 4 * R * D * I)
        st["gemm_gate_up_gathered"] = (touched * 2 * q * I + T * q + R * I * b, 4 * R * D * I)
    else:
        st["permute"] = ((12 * R, 0) if gath else (T * D * b + R * D * b + 12 * R, 0))
        st["gemm_gate_up"] = (touched * 2 * D * I * b + R * D * b + R * I * b, 4 * R * D * I)
        st["gemm_gate_up_gathered"] = (touched * 2 * D * I * b + T * D * b + R * I * b, 4 * R * D * I)
    st["gemm_down"] = (touched * D * I * b + R * I * b + R * D * b, 2 * R * D * I)
    Is = cfg.shared_I
    st["shared_expert"] = ((T * H * b + 3 * Is * H * b + 2 * T * Is * b + T * H * b, 6 * T * H * Is)
                           if Is else (0, 0))
    st["combine"] = (R * D * b + 8 * R + T * D * (b if L else out_b) + (T * D * b if Is else 0), 0)
    st["latent_up"] = (T * L * b + H * L * b + T * H * out_b, 2 * T * L * H) if L else (0, 0)
    return st, touched


def sampled_steps(steps, samples=4):
    """The timed steps that record the two events around the gate/up GEMM: a fixed
    number (`samples`), spread evenly over the timed region whatever its length, so the
    idle time each event record adds between kernels stays a few microseconds per
    sampled step."""
    n = min(samples, steps)
    return sorted({(i * steps) // n + (steps // n) // 2 for i in range(n)})


def pct(vals, q):
    """Nearest-rank q-th percentile."""
    srt = sorted(vals)
    return float(srt[max(0, -(-q * len(srt) // 100) - 1)])


def time_combine_alone(B, torch, cfg, w, x, logits, od, s, ws, counts, stream, hip, reps=20):
    """moe_combine on its own over one layer's y_perm: fused, and the unpermute +
    weighted-reduce pair (UNFUSED); mean ms per call over `reps` calls each."""
    dev = x.device
    act = torch.int16 if cfg.dtype == "bf16" else torch.float32
    yp = torch.empty((cfg.R, cfg.D), dtype=act, device=dev)
    trow = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16 if od == B.MOE_BF16 else torch.float32, device=dev)
    B.layer_forward(w, x, logits, out, od, s, ws, aux={"counts": counts, "y_perm": yp, "token_row": trow,
                                                       "topk_w": tw}, stream=stream)
    cod = B.MOE_BF16 if cfg.dtype == "bf16" and (cfg.L or od == B.MOE_BF16) else B.MOE_F32
    oc = torch.empty((cfg.T, cfg.D), dtype=torch.int16 if cod == B.MOE_BF16 else torch.float32, device=dev)
    wsc = torch.empty(max(B.workspace_bytes(s, B.MOE_CALL_COMBINE), 256), dtype=torch.uint8, device=dev)
    res = {}
    for name, flag in (("fused_ms", B.MOE_COMBINE_FUSED), ("unpermute_plus_reduce_ms", B.MOE_COMBINE_UNFUSED)):
        B.combine(yp, trow, tw, oc, cod, flag, s, wsc, stream=stream)
        e = hip.create(2)
        hip.record(e[0], stream)
        for _ in range(reps):
            B.combine(yp, trow, tw, oc, cod, flag, s, wsc, stream=stream)
        hip.record(e[1], stream)
        torch.cuda.synchronize()
        res[name] = round(hip.elapsed_ms(e[0], e[1]) / reps, 5)
        hip.destroy(e)
    return res


def time_permute_alone(B, torch, cfg, w, x, logits, s, ws, stream, hip, reps=20):
    """moe_dispatch_permute on its own, writing the T*k*D*b permuted copy of the rows the
    layer dispatches (X, or Z for latent layers) on the layer's own routing: the call's
    three launches (per-block counts, expert scan, permutation) and its algorithmic
    bytes T*D*b + R*D*b + 12*R over the call time (mean ms per call over `reps`)."""
    dev = x.device
    act = torch.int16 if cfg.dtype == "bf16" else torch.float32
    T, k, D, R = cfg.T, cfg.k, cfg.D, cfg.R
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device=dev)
    aux = {"topk_ids": ids, "offsets": offs}
    z = None
    if cfg.L:
        z = torch.empty((T, cfg.L), dtype=act, device=dev)
        aux["z"] = z
    out = torch.empty((T, cfg.H), dtype=torch.float32, device=dev)
    B.layer_forward(w, x, logits, out, B.MOE_F32, s, ws, aux=aux, stream=stream)
    src = z if cfg.L else x
    xp = torch.empty((R, D), dtype=act, device=dev)
    rt = torch.empty((R,), dtype=torch.int32, device=dev)
    tr = torch.empty((T, k), dtype=torch.int32, device=dev)
    sd = B.shape(T, cfg.H, cfg.E, k, cfg.I, cfg.L, cfg.dtype, cfg.shared_I, cfg.capacity)
    wsd = torch.empty(max(B.workspace_bytes(sd, B.MOE_CALL_DISPATCH), 256), dtype=torch.uint8, device=dev)
    B.dispatch_permute(src, ids, offs, xp, rt, tr, sd, wsd, stream=stream)
    e = hip.create(2)
    hip.record(e[0], stream)
    for _ in range(reps):
        B.dispatch_permute(src, ids, offs, xp, rt, tr, sd, wsd, stream=stream)
    hip.record(e[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e[0], e[1]) / reps
    hip.destroy(e)
    kept = int(offs[-1].item())
    byt = T * D * cfg.elem_bytes + kept * D * cfg.elem_bytes + 12 * R
    return {"ms": round(ms, 5), "bytes": byt, "GB/s": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def ep_rank_share(B, torch, np, gen, cfg, ranks, up, stream, hip, reps=10):
    """The grouped expert FFN at one rank's share of `ranks`-way expert parallelism.

    Every rank holds E / ranks experts and receives, from each of the `ranks`
    source batches of T tokens (reseeded steps 0 .. ranks-1 of the same layer),
    the rows routed to its experts.  The batches are routed on this GPU; the rows
    of experts [0, E / ranks) form the rank-0 expert input (seeded random
    activations: the values do not change the time), and moe_grouped_ffn runs
    over them with those experts' weights."""
    dev = torch.device("cuda:0")
    assert cfg.E % ranks == 0, "experts must split evenly over the ranks"
    el = cfg.E // ranks
    s = B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.dtype)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    cnt = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device=dev)
    lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    wsr = torch.empty(max(B.workspace_bytes(s, B.MOE_CALL_ROUTE), 256), dtype=torch.uint8, device=dev)
    gw = up(gen.gate_weight(cfg)) if cfg.gate == "computed" else None
    bias = gen.zipf_bias(cfg)
    bias = up(bias) if bias is not None else None
    local = np.zeros(el, dtype=np.int64)
    for r in range(ranks):
        if cfg.gate == "computed":
            B.route_topk(up(gen.activations(cfg, r)), gw, bias, lg, ids, tw, cnt, offs, s, wsr, stream=stream)
        else:
            B.route_topk(None, None, bias, up(gen.drawn_logits(cfg, r)), ids, tw, cnt, offs, s, wsr,
                         stream=stream)
        local += cnt.cpu().numpy()[:el]
    rows = int(local.sum())
    offsets = np.concatenate([[0], np.cumsum(local)]).astype(np.int32)
    ls = B.shape(rows, cfg.H, el, 1, cfg.I, cfg.L, cfg.dtype)  # one row per assignment
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    xp = torch.randn((rows, cfg.D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    ew = gen.expert_weights(cfg, experts=range(el))
    w1, w3, w2 = up(ew["w1"]), up(ew["w3"]), up(ew["w2"])
    yp = torch.empty((rows, cfg.D), dtype=torch.int16, device=dev)
    wsf = torch.empty(max(B.workspace_bytes(ls, B.MOE_CALL_FFN), 256), dtype=torch.uint8, device=dev)
    doffs = torch.from_numpy(offsets).to(dev)
    B.grouped_ffn(xp, doffs, w1, w3, w2, yp, ls, wsf, stream=stream)
    e = hip.create(2)
    hip.record(e[0], stream)
    for _ in range(reps):
        B.grouped_ffn(xp, doffs, w1, w3, w2, yp, ls, wsf, stream=stream)
    hip.record(e[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e[0], e[1]) / reps
    hip.destroy(e)
    flops = 6.0 * rows * cfg.D * cfg.I
    wbytes = 3 * el * cfg.D * cfg.I * cfg.elem_bytes
    log(f"ep rank share: {rows} rows over {el} experts, {ms:.3f} ms, {flops / ms / 1e9:.0f} TFLOP/s")
    return {"ranks": ranks, "local_experts": el, "rows": rows,
            "rows_per_expert_mean": round(rows / el, 1), "rows_per_expert_max": int(local.max()),
            "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "weight_bytes": wbytes, "weight_gbps": round(wbytes / (ms * 1e-3) / 1e9, 1)}


def src_hash(path):
    """First 16 hex digits of the SHA-256 of the GEMM source (`path`) followed by the
    headers it includes: traffic counters are reported only for the code they
    were taken on."""
    h = hashlib.sha256(open(path, "rb").read())
    for inc in GEMM_HEADERS:
        h.update(open(inc, "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(cfg, inp, target_s):
    """Time the CPU oracle on the first n tokens of the same layer, growing n until
    about target_s / 3 seconds of work (or the whole layer); when the whole layer
    takes less than target_s, repeat it until about target_s seconds have run and
    report the mean; report assignments/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    n = min(8, cfg.T)
    while True:
        sub = dict(inp)
        sub["x"] = inp["x"][:n]
        if "logits" in inp:
            sub["logits"] = inp["logits"][:n]
        timers = {}
        t0 = time.perf_counter()
        oracle.layer_forward(sub, k=cfg.k, E=cfg.E, bf16=cfg.dtype == "bf16", timers=timers,
                             dispatch=cfg.dispatch)
        dt = time.perf_counter() - t0
        log(f"cpu oracle: {n} tokens in {dt:.2f} s")
        if dt >= target_s / 3 or n >= cfg.T:
            break
        n = min(cfg.T, n * 4)
    runs, total = 1, dt
    if n >= cfg.T:
        while total < target_s:
            t0 = time.perf_counter()
            oracle.layer_forward(sub, k=cfg.k, E=cfg.E, bf16=cfg.dtype == "bf16", timers=timers,
                                 dispatch=cfg.dispatch)
            total += time.perf_counter() - t0
            runs += 1
        log(f"cpu oracle: whole layer {runs} times in {total:.2f} s")
    dt = total / runs
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    try:
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                       if i.get("user_api") == "blas"})
    except Exception:  # pragma: no cover
        blas = []
    return {"value": n * cfg.k / dt, "unit": "assignments/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of the same layer (all {cfg.E} experts' "
                      f"weights), float64 numpy oracle, {runs} run(s), {dt:.2f} s each",
            "stages_s": {k_: round(v / runs, 4) for k_, v in timers.items()},
            "cpu_model": cpu, "blas": blas}


def traffic_from_pmc(fetch_csv, write_csv, config, copy_mib, fetch_cmd, write_cmd):
    """HBM bytes per launch of the expert gate/up GEMM from two rocprofv3 --pmc runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the same
    counter reads for the 1 GiB calibration copy (a plain device copy of known
    size in the same run), then averaged over the dispatches of the kernel the
    library's plan names for the layer's gate/up GEMM.
    """
    import csv

    def rows(path, counter):
        out = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return out

    copy_bytes = copy_mib << 20
    mx = config.endswith("_mxfp8")   # the MXFP8 kernels carry a trailing "true" template argument
    from routing_dispatch_expert_logits_amd import binding as B
    from workloads import FULL_CONFIGS
    cfg = FULL_CONFIGS[config[:-len("_mxfp8")] if mx else config]
    kern = layer_plan(B, cfg.with_(dispatch="mxfp8") if mx else cfg)["gate_up_kernel"]

    def dominant(name):
        return kern in name and (("true>" in name) == mx)

    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rs = rows(path, counter)
        copies = [v for n, v in rs if "copyBuffer" in n]
        big = max(copies)
        cal = [v for v in copies if v > 0.9 * big]
        scale = copy_bytes / (1024.0 * sum(cal) / len(cal))
        gemm = [v for n, v in rs if dominant(n)]
        kname = next(n for n, v in rs if dominant(n))
        res[counter] = {"kib_per_launch": sum(gemm) / len(gemm), "launches": len(gemm),
                        "copy_kib": sum(cal) / len(cal), "scale": scale, "kernel": kname.split("(")[0]}
    hbm = (res["FETCH_SIZE"]["kib_per_launch"] * 1024 * res["FETCH_SIZE"]["scale"] +
           res["WRITE_SIZE"]["kib_per_launch"] * 1024 * res["WRITE_SIZE"]["scale"])
    out = {"config": config, "kernel": res["FETCH_SIZE"]["kernel"],
           "gemm_src_sha256_16": src_hash(GEMM_SRC),
           "hbm_bytes_per_launch": int(hbm),
           "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
           "copy_calibration_bytes": copy_bytes,
           "commands": [fetch_cmd, write_cmd]}
    path = TRAFFIC_FILE.format(config=config)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main(argv=None):
    if argv is None:
        argv = sys.argv[1:]
    if argv and argv[0] == "--traffic-from":
        # python bench.py --traffic-from FETCH.csv WRITE.csv CONFIG COPY_MIB "fetch cmd" "write cmd"
        traffic_from_pmc(argv[1], argv[2], argv[3], int(argv[4]), argv[5], argv[6])
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deepseek_r1_shaped")
    ap.add_argument("--skew-steps", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra layers timed after a 1 GiB cache-evicting write each (0: none)")
    ap.add_argument("--dispatch", default="dtype", choices=["dtype", "mxfp8"],
                    help="mxfp8: dispatched rows and W1 / W3 as MXFP8 (value-changing; the accuracy "
                         "change against the bf16 layer is reported)")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="expert capacity C = ceil(f * T * k / E) rows (drops the rest; value-changing)")
    ap.add_argument("--ep-rank-share", type=int, default=0,
                    help="time the grouped expert FFN at one rank's share of R-way expert parallelism")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB 3 times "
                         "(reference kernel of known size for HBM counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs one GPU's share of the layer only; --gpus {args.gpus} is not "
              "supported (the library runs one GPU's share and has no collectives between GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from routing_dispatch_expert_logits_amd import binding as B
    from workloads import FULL_CONFIGS, generator as gen

    cfg = FULL_CONFIGS[args.config]
    if args.capacity_factor > 0:
        cfg = cfg.with_(capacity=int(np.ceil(args.capacity_factor * cfg.R / cfg.E)))
    if args.dispatch != "dtype":
        cfg = cfg.with_(dispatch=args.dispatch)
    plan = layer_plan(B, cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} L={cfg.L} {cfg.dtype}")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)

    t0 = time.perf_counter()
    inp = gen.layer_inputs(cfg)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    w = {n: up(inp[n]) for n in ("gate_w", "w1", "w3", "w2", "wd", "wu", "ws1", "ws3", "ws2") if n in inp}
    if "bias" in inp:
        w["gate_bias"] = up(inp["bias"])
    x = up(inp["x"])
    logits = up(inp["logits"]) if "logits" in inp else torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    s = B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.dtype, cfg.shared_I, cfg.capacity,
                cfg.dispatch)
    ws = torch.empty(B.workspace_bytes(s, B.MOE_CALL_LAYER), dtype=torch.uint8, device=dev)
    od = B.MOE_BF16 if args.out_dtype == "bf16" and cfg.dtype == "bf16" else B.MOE_F32
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16 if od == B.MOE_BF16 else torch.float32, device=dev)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    aux = {"counts": counts}
    mx_info = None
    if cfg.dispatch == "mxfp8":
        # the bf16 layer once on the same inputs (for the accuracy change), then W1 / W3
        # converted once on the GPU (offline weight preparation, timed on its own)
        s16 = B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.dtype, cfg.shared_I, cfg.capacity)
        ws16 = torch.empty(B.workspace_bytes(s16, B.MOE_CALL_LAYER), dtype=torch.uint8, device=dev)
        out16 = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
        B.layer_forward(w, x, logits, out16, B.MOE_F32, s16, ws16)
        del ws16
        hq = HipEvents()
        qe = hq.create(2)
        stream0 = torch.cuda.current_stream().cuda_stream
        hq.record(qe[0], stream0)
        for n in ("w1", "w3"):
            q = torch.empty((cfg.E, cfg.I, cfg.D), dtype=torch.uint8, device=dev)
            sc = torch.empty((cfg.E, cfg.I, cfg.D // 32), dtype=torch.uint8, device=dev)
            B.quantize_mxfp8(w[n], q, sc, stream=stream0)
            w[n], w[n + "_scale"] = q, sc
        hq.record(qe[1], stream0)
        torch.cuda.synchronize()
        mx_info = {"format": "MXFP8 E4M3, one E8M0 scale per 32 along K",
                   "weight_conversion_ms": round(hq.elapsed_ms(qe[0], qe[1]), 4),
                   "out_bf16_dispatch": out16}
        hq.destroy(qe)
    torch.cuda.synchronize()
    resident = sum(t.numel() * t.element_size() for t in w.values())
    log(f"uploaded; resident weights {resident / 1e9:.2f} GB, workspace {ws.numel() / 1e9:.2f} GB")

    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()
    nev = B.MOE_NUM_STAGE_EVENTS
    names = B.STAGE_NAMES
    # The timed steps record only the two events around the expert gate/up GEMM (the
    # dominant kernel the roofline object describes), on a fixed handful of sampled
    # steps whatever --steps is: every event record puts a few microseconds between
    # the kernels either side of it.  The per-stage breakdown comes from a separate
    # pass with every stage event, after the timed region.
    g = names.index("gemm_gate_up")
    sampled = sampled_steps(args.steps)
    gev = [hip.create(2) for _ in sampled]
    tev = [None] * args.steps
    for i, pair in zip(sampled, gev):
        arr = [None] * nev
        arr[g], arr[g + 1] = pair
        tev[i] = arr

    for _ in range(args.warmup):
        B.layer_forward(w, x, logits, out, od, s, ws, aux=aux, stream=stream)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    # timed region: exactly K steps, synchronised on both sides (one GPU: no barrier needed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        B.layer_forward(w, x, logits, out, od, s, ws, aux=aux, stage_events=tev[i], stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")
    gate_up_timed_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in gev]))
    for pair in gev:
        hip.destroy(pair)

    # stage pass: the same number of steps with every stage event
    evs = [hip.create(nev) for _ in range(args.steps)]
    for i in range(args.steps):
        B.layer_forward(w, x, logits, out, od, s, ws, aux=aux, stage_events=evs[i], stream=stream)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([hip.elapsed_ms(e[j], e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    layer_list = [hip.elapsed_ms(e[0], e[nev - 1]) for e in evs]
    layer_ev_ms = float(np.mean(layer_list))
    for e in evs:
        hip.destroy(e)
    stage_ms["gemm_gate_up"] = gate_up_timed_ms  # the timed steps' figure

    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cev = [hip.create(nev) for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(i & 0xFF)  # same stream: the write ends before the layer starts
            B.layer_forward(w, x, logits, out, od, s, ws, aux=aux, stage_events=cev[i], stream=stream)
        torch.cuda.synchronize()
        cl = [hip.elapsed_ms(e[0], e[nev - 1]) for e in cev]
        cst = {n: float(np.median([hip.elapsed_ms(e[j], e[j + 1]) for e in cev]))
               for j, n in enumerate(names)}
        for e in cev:
            hip.destroy(e)
        del flush
        cold = {"steps": args.cold_steps, "flush_bytes": 1 << 30,
                "ms_per_layer_median": round(float(np.median(cl)), 5),
                "ms_per_layer_p95": round(pct(cl, 95), 5),
                "value_median": round(cfg.R / (float(np.median(cl)) * 1e-3), 1),
                "stages_median_ms": cst}
        log(f"cold: {cold['ms_per_layer_median']:.4f} ms per layer (median of {args.cold_steps})")

    combine_alone = time_combine_alone(B, torch, cfg, w, x, logits, od, s, ws, counts, stream, hip)
    permute_alone = (time_permute_alone(B, torch, cfg, w, x, logits, s, ws, stream, hip)
                     if cfg.dispatch == "dtype" else None)
    ep_share = (ep_rank_share(B, torch, np, gen, cfg, args.ep_rank_share, up, stream, hip)
                if args.ep_rank_share > 1 and cfg.dispatch == "dtype" else None)
    if mx_info is not None:
        # the value change against the bf16 layer (same inputs, same routing)
        o32 = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
        B.layer_forward(w, x, logits, o32, B.MOE_F32, s, ws, stream=stream)
        torch.cuda.synchronize()
        ref16 = mx_info.pop("out_bf16_dispatch").double()
        d = o32.double() - ref16
        rms = float(torch.sqrt(torch.mean(ref16 * ref16)))
        mx_info["accuracy_vs_bf16_dispatch"] = {
            "max_abs_over_rms": round(float(d.abs().max()) / rms, 5),
            "rms_over_rms": round(float(torch.sqrt(torch.mean(d * d))) / rms, 5)}
        log(f"MXFP8 vs bf16 dispatch: {mx_info['accuracy_vs_bf16_dispatch']}")

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src_c = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
        log(f"copy calibration: 3 x {args.copy_calibration_mib} MiB device copies")

    cnt = counts.cpu().numpy()
    sb, touched = stage_bytes_flops(cfg, cnt, bool(plan["rows_gathered"]))
    stages = {}
    for n in names:
        byt, flp = sb[n]
        if byt == 0 and flp == 0:
            if cold:
                cold["stages_median_ms"].pop(n, None)
            continue
        if cold:
            cold["stages_median_ms"][n] = round(cold["stages_median_ms"][n], 5)
        t_s = stage_ms[n] * 1e-3
        stages[n] = {"ms": round(stage_ms[n], 5), "GB/s": round(byt / t_s / 1e9, 1) if t_s > 0 else None}
        if flp:
            stages[n]["TFLOP/s"] = round(flp / t_s / 1e12, 2)

    # p95 of the max/mean expert-load ratio over reseeded steps (route only)
    skews = []
    if args.skew_steps > 0:
        ids_b = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
        w_b = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
        offs_b = torch.empty((cfg.E + 1,), dtype=torch.int32, device=dev)
        lg_b = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
        ws_r = torch.empty(max(B.workspace_bytes(s, B.MOE_CALL_ROUTE), 256), dtype=torch.uint8, device=dev)
        for step in range(args.skew_steps):
            if cfg.gate == "computed":
                B.route_topk(up(gen.activations(cfg, step)), w["gate_w"], w.get("gate_bias"), lg_b,
                             ids_b, w_b, counts, offs_b, s, ws_r, stream=stream)
            else:
                B.route_topk(None, None, w.get("gate_bias"), up(gen.drawn_logits(cfg, step)), ids_b,
                             w_b, counts, offs_b, s, ws_r, stream=stream)
            c = counts.cpu().numpy()
            skews.append(float(c.max()) / (cfg.T * cfg.k / cfg.E))
        srt = sorted(skews)
        p95 = srt[int(np.ceil(0.95 * len(srt))) - 1]
        log(f"p95 skew over {len(skews)} steps: {p95:.3f}")
    else:
        p95 = None

    # roofline of the dominant kernel: the expert gate/up GEMM
    g_bytes, g_flops = sb["gemm_gate_up"]
    g_s = stage_ms["gemm_gate_up"] * 1e-3
    achieved = g_bytes / g_s / 1e9
    gg_bytes = sb["gemm_gate_up_gathered"][0]
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": plan["gate_up_kernel"] + " (expert gate/up GEMM" +
                      (", persistent" if plan["gate_up_persistent"] else "") +
                      (", token rows gathered through row_token" if plan["rows_gathered"] else "") + ")",
            "algorithmic_bytes": int(g_bytes),
            "algorithmic_bytes_note": "touched experts' W1+W3, one input row per routed assignment (R*D*b), "
                                      "the R*I intermediate written",
            "gathered_bytes": int(gg_bytes), "gathered_frac": round(gg_bytes / g_s / 1e9 / HBM_PEAK_GBS, 4),
            "avg_ms": round(stage_ms["gemm_gate_up"], 5), "sampled_launches": len(gev),
            "mfma_tflops": round(g_flops / g_s / 1e12, 1),
            "mfma_frac": round(g_flops / g_s / 1e12 / (
                F32_PEAK_TFLOPS if cfg.dtype != "bf16" else FP8_PEAK_TFLOPS if cfg.dispatch == "mxfp8"
                else BF16_PEAK_TFLOPS), 4)}
    tf = TRAFFIC_FILE.format(config=cfg.name + ("_mxfp8" if cfg.dispatch == "mxfp8" else ""))
    if os.path.exists(tf):
        tr = json.load(open(tf))
        if tr.get("gemm_src_sha256_16") == src_hash(GEMM_SRC):
            roof["traffic"] = tr.get("hbm_bytes_per_launch")

    gemm_ms = stage_ms["gemm_gate_up"] + stage_ms["gemm_down"]
    line = {
        "metric": "routed assignments/s per MoE layer",
        "value": round(cfg.R / (ms_per_step * 1e-3), 1),
        "unit": "assignments/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("mxfp8-e4m3/bf16" if cfg.dispatch == "mxfp8" else "bf16") if cfg.dtype == "bf16" else "f32",
        "data": "synthetic: seeded numpy PCG64 inputs, random-init weights",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "I": cfg.I, "L": cfg.L, "out_dtype": "bf16" if od == B.MOE_BF16 else "f32",
                   "dispatch": cfg.dispatch},
        "grouped_gemm_tflops": round((sb["gemm_gate_up"][1] + sb["gemm_down"][1]) / (gemm_ms * 1e-3) / 1e12, 1),
        "permute_gbps": stages["permute"]["GB/s"],
        "combine_gbps": stages["combine"]["GB/s"],
        "stage_timing": (f"timed steps record the two events around the expert gate/up GEMM on "
                         f"{len(gev)} sampled steps of {args.steps}; stages and layer_event_ms come "
                         "from a second pass of as many steps with every stage event"),
        "plan": plan,
        "layer_event_ms": round(layer_ev_ms, 5),
        "layer_event_ms_median": round(float(np.median(layer_list)), 5),
        "layer_event_ms_p95": round(pct(layer_list, 95), 5),
        "cold": cold,
        "combine_alone": combine_alone,
        "permute_alone": permute_alone,
        "ep_rank_share": ep_share,
        "stages": stages,
        "p95_skew": round(p95, 3) if p95 is not None else None,
        "touched_experts": touched,
        "expert_capacity": cfg.capacity,
        "dropped_assignments": int(cfg.R - int(cnt.sum())),
        "dispatch_bytes": (cfg.T * cfg.k * cfg.D * 33 // 32 if cfg.dispatch == "mxfp8"
                           else cfg.T * cfg.k * cfg.D * cfg.elem_bytes),
        "mxfp8": mx_info,
        "dispatch_bytes_full_width": cfg.T * cfg.k * cfg.H * cfg.elem_bytes,
        "resident_expert_bytes": resident,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
