#!/usr/bin/env python3
"""Throughput benchmark of the LoRA layer backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole backward of the workload through the C-ABI library:
lorabwd_layer_backward runs every step of the path (FFN backward,
O-projection backward, attention backward, inverse RoPE, and, where the
workload has adapters, LoRA gradients with AdamW) - for `stack36`, all 36
layers in reverse order.  The top layer reads the upstream gradient (never
written) and leaves dH1 in a separate buffer, which the layers below update
in place, so replaying a step needs no reset copy.  Inputs are resident in HBM before timing starts.
Steps rotate over enough input copies that HBM-bound work cannot be served
from the 256 MB Infinity Cache; one HIP graph holds the steps of all copies
in rotation order (as a model's backward holds its layers), so a graph
launch is paid once per round of copies, and a graph per copy covers a
step count that is not a whole number of rounds.

Workloads (default: stack36):
  decode       one token, 512-slot K/V cache, hidden 2560, ffn 6912, 20/5 heads
               of 128, ReLU^2 x up with sub-norms, ternary fp32 weights
  seq512       512 tokens, hidden 2560, ffn 9728, 32/8 heads, SwiGLU, LoRA r16, fp32
  seq2048bf16  the seq512 layer at 2048 tokens with bf16 activations/weights
  stack36      36 seq512-shaped layers at 1024 tokens, fp32
  seq512qk     the seq512 layer with QK-norm before RoPE
  decode_packed  the decode layer on packed ternary weights (2 bits per value)
  seq512ig, seq2048bf16ig
               those layers with the exact input gradient through attention
  tiny         hidden 64, 16 tokens (launch-bound; parity-size case)
  lmhead       the step upstream of the stack: lm_head backward of the stack36
               model (1024 tokens, hidden 2560, vocabulary 151936, fp32) -
               softmax cross-entropy, grad_hidden, dW with AdamW on the weight
               (lorabwd_lm_head_backward; metric lm_head-backward tokens/s)

Prints ONE JSON line.  `roofline` describes the kernel with the largest
share of the step, timed with HIP events recorded on the library's stream
right after each kernel (lorabwd_*_timed; the raw interval between
consecutive events, so it includes one event record) over steps run back
to back after the timed region; its algorithmic bytes / flops come from
the library.  `attn` sums the attention
launches of a layer (dA, softmax backward, dQ, dV and their helper launches)
against the three contractions on unmasked pairs.  `cpu_baseline` times the
float64 oracle on the host on a bounded sample of the same workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {  # MI355X published peaks (dense)
    "hbm_GBps": 8000.0,
    "f32_TFLOPs": 157.3,
    "bf16_TFLOPs": 2516.6,
}
COPIES = {"decode": 6, "tiny": 1, "seq512": 4, "seq2048bf16": 4, "stack36": 1, "seq512qk": 4,
          "seq512ig": 4, "seq2048bf16ig": 4, "decode_packed": 24, "lmhead": 1}
DEFAULT_STEPS = {"decode": 2000, "tiny": 2000, "seq512": 200, "seq2048bf16": 100, "stack36": 10,
                 "seq512qk": 200, "seq512ig": 200, "seq2048bf16ig": 100, "decode_packed": 4800,
                 "lmhead": 30}


def is_lm(cfg):
    return type(cfg).__name__ == "LmHeadConfig"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="stack36", choices=sorted(COPIES))
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline sample budget")
    ap.add_argument("--pmc-pass", metavar="RECORDS_JSON",
                    help="short eager run for a rocprofv3 --pmc pass: writes the step's kernel "
                         "records to RECORDS_JSON, runs 3 eager steps and a 256 MiB plain copy "
                         "(the counter calibration), prints nothing else")
    ap.add_argument("--sq-summary", nargs=2, metavar=("RECORDS_JSON", "SQ_CSV"),
                    help="per-kernel MFMA and LDS utilisation from one rocprofv3 --pmc pass of "
                         "SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT "
                         "GRBM_GUI_ACTIVE over --pmc-pass")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("RECORDS_JSON", "FETCH_CSV", "WRITE_CSV"),
                    help="turn the two counter passes (FETCH_SIZE, WRITE_SIZE) into "
                         "profiles/traffic.json and print the table; no GPU needed")
    return ap.parse_args()


# ------------------------------------------------------------------ HIP events via ctypes
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = e.value
        return arr

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        self.lib.hipEventSynchronize(b)
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value


# ------------------------------------------------------------------ workload
def layer_call(lbp, cfg, d, d_hidden, **kw):
    desc = lbp.make_desc(cfg.seq, cfg.kv_len, cfg.hidden, cfg.ffn, cfg.n_heads, cfg.n_kv_heads,
                         cfg.head_dim,
                         act=lbp.ACT_SWIGLU if cfg.act == "swiglu" else lbp.ACT_RELU2,
                         sub_norms=cfg.sub_norms, causal=cfg.causal,
                         dtype=lbp.BF16 if cfg.dtype == "bf16" else lbp.F32, pos0=cfg.pos0,
                         eps=cfg.eps, rope_base=cfg.rope_base, attn_scale=cfg.scale,
                         lora_alpha=cfg.alpha, qk_norm=cfg.qk_norm, input_grad=cfg.input_grad,
                         weight_format=1 if cfg.packed else 0)
    lora = d["lora"]
    hp = lbp.AdamW(cfg.lr, cfg.lr_b, cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay,
                   cfg.step) if lora else None
    return lbp.lorabwd_layer_backward(desc, d["weights"], d["saved"], d_hidden,
                                      q_state=lora["q"] if lora else None,
                                      v_state=lora["v"] if lora else None, adamw=hp,
                                      gnorm_sq=kw.pop("gnorm", None), **kw)


def pack_weights(lbp, d, torch):
    """Packed ternary storage of a drawn decode layer's four weight matrices
    (values 0.02 * {-1, 0, +1} in float32), with their scale."""
    import numpy as np
    for k in ("w_o", "w_gate", "w_up", "w_down"):
        d["weights"][k] = lbp.lorabwd_pack_ternary(d["weights"][k])
        d["weights"]["scale_" + k[2:]] = float(np.float32(0.02))
    torch.cuda.synchronize()
    return d


def lm_call(lbp, cfg, cp, **kw):
    return lbp.lorabwd_lm_head_backward(cp["h"], cp["logits"], cp["labels"], cp["W"], cp["m"],
                                        cp["v"], cp["grad_hidden"], cp["loss"], lr=cfg.lr,
                                        beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.adam_eps,
                                        weight_decay=cfg.weight_decay, step=cfg.step, **kw)


def build_copies(cfg, n_copies, torch, lbp=None):
    if is_lm(cfg):
        from synth.device import draw_lm_head_device
        copies = []
        for c in range(n_copies):
            cp = draw_lm_head_device(cfg, c)
            cp["grad_hidden"] = torch.empty((cfg.rows, cfg.hidden), device="cuda:0")
            cp["loss"] = torch.empty(1, device="cuda:0")
            copies.append(cp)
        return copies
    from synth.device import draw_timing_layer_device
    copies = []
    for c in range(n_copies):
        layers = [draw_timing_layer_device(cfg, c * cfg.n_layers + l) for l in range(cfg.n_layers)]
        if cfg.packed:
            layers = [pack_weights(lbp, d, torch) for d in layers]
        copies.append({"layers": layers, "d_out": layers[-1]["d_out"],
                       "d_hidden": torch.empty_like(layers[-1]["d_out"]),
                       "gnorm": torch.zeros(1, device="cuda:0")})
    return copies


def step_calls(lbp, cfg, cp):
    """The library calls of one step, each taking the call's keyword options
    (timing).  Layer workloads: the layers in reverse order (a single layer
    for one-layer workloads); the top layer reads the upstream gradient
    d_out, which is never written, and leaves dH1 in d_hidden; the layers
    below update d_hidden in place.  lmhead: one lm_head backward (AdamW
    updates the weight in place, as a training step does)."""
    if is_lm(cfg):
        return [lambda **kw: lm_call(lbp, cfg, cp, **kw)]
    return [lambda li=li, d=d, **kw: layer_call(lbp, cfg, d, cp["d_hidden"], gnorm=cp["gnorm"],
                                                d_out=cp["d_out"] if li == 0 else None, **kw)
            for li, d in enumerate(reversed(cp["layers"]))]


def run_step(lbp, cfg, cp):
    for call in step_calls(lbp, cfg, cp):
        call()


# ------------------------------------------------------------------ roofline
def kernel_profile(lbp, hip, cfg, copies, torch, nsteps):
    """Per-kernel average duration (ms) in steady state, as in the timed
    region: nsteps whole steps run back to back on the copies in rotation,
    with an event recorded right after each kernel by the library's timed
    entry points (lorabwd_*_timed) and one before each call.  A 2 GiB read
    enqueued first keeps the GPU busy while the host enqueues the steps, so
    consecutive events bracket kernels that ran back to back, not host
    launch gaps; the first step after it (cold caches, idle clocks) is not
    counted."""
    cap = 32  # kernels of one call at most
    stream = torch.cuda.current_stream().cuda_stream
    seq = [(st, call) for st in range(nsteps)
           for call in step_calls(lbp, cfg, copies[st % len(copies)])]
    evs = [hip.events(cap + 1) for _ in seq]
    recs = [(lbp.KernelRecord * cap)() for _ in seq]
    filler = torch.zeros(1 << 29, dtype=torch.float32, device="cuda:0")
    sink = torch.empty((), dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    torch.sum(filler, dim=(0,), out=sink)
    counts = []
    for (st, call), ev, rc in zip(seq, evs, recs):
        hip.record(ev[cap], stream)
        counts.append(call(timing=(ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)), rc)))
    torch.cuda.synchronize()
    stats = {}
    for (st, _), ev, rc, n in zip(seq, evs, recs, counts):
        if st == 0 and nsteps > 1:
            continue
        prev = ev[cap]
        for i in range(min(n, cap)):
            ms = hip.elapsed_ms(prev, ev[i])
            prev = ev[i]
            key = (i, rc[i].name.decode())
            e = stats.setdefault(key, {"ms": 0.0, "n": 0, "bytes": rc[i].alg_bytes,
                                       "flops": rc[i].alg_flops, "impl": rc[i].impl_bytes})
            e["ms"] += ms
            e["n"] += 1
    del filler, sink
    out = []
    for (i, name), e in sorted(stats.items()):
        out.append({"index": i, "name": name, "avg_ms": e["ms"] / e["n"], "alg_bytes": e["bytes"],
                    "alg_flops": e["flops"], "impl_bytes": e["impl"]})
    return out


# the source file of each kernel (by its record name); with the shared
# headers it decides whether a stored traffic figure is still current
KERNEL_SOURCE = (("dec_attn", "decode.hip"), ("dgemv", "decode.hip"), ("gemm", "gemm.hip"),
                 ("splitk", "gemm.hip"), ("attn", "attn.hip"), ("transpose", "attn.hip"),
                 ("lora", "lora.hip"), ("xent", "lmhead.hip"))


def kernel_source(name):
    for prefix, f in KERNEL_SOURCE:
        if name.startswith(prefix):
            return f
    return "rowwise.hip"


def source_digest(kernel):
    h = hashlib.sha256()
    for f in ("common.h", "kernels.h", kernel_source(kernel)):
        with open(os.path.join(ROOT, "layer_backward_pass_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def roofline(cfg, kernels):
    """The dominant kernel (largest time per step, launches of the same
    kernel at the same shape counted together) against its roofline."""
    groups = {}
    for k in kernels:
        key = (k["name"], k["alg_bytes"], k["alg_flops"])
        g = groups.setdefault(key, {"ms": 0.0, "launches": 0, "avg": []})
        g["ms"] += k["avg_ms"]
        g["launches"] += 1
        g["avg"].append(k["avg_ms"])
    (name, nbytes, flops), g = max(groups.items(), key=lambda kv: kv[1]["ms"])
    avg_s = sum(g["avg"]) / len(g["avg"]) / 1e3
    intensity = flops / nbytes if nbytes else float("inf")
    mfma_peak = PEAK["bf16_TFLOPs"] if "bf16" in name else PEAK["f32_TFLOPs"]
    ridge = mfma_peak * 1e12 / (PEAK["hbm_GBps"] * 1e9)
    if "mfma" in name and intensity > ridge:
        achieved = flops / avg_s / 1e12
        rl = {"bound": "mfma", "achieved": round(achieved, 2), "peak": mfma_peak,
              "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4)}
    else:
        achieved = nbytes / avg_s / 1e9
        rl = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_GBps"],
              "unit": "GB/s", "frac": round(achieved / PEAK["hbm_GBps"], 4)}
    rl.update({"kernel": name, "avg_us": round(avg_s * 1e6, 2),
               "launches_per_layer": g["launches"], "alg_bytes": nbytes, "alg_flops": flops,
               "traffic": traffic_for(cfg, name, nbytes)})
    return rl


def attn_pairs(cfg):
    """Unmasked (query, key) pairs per head (query i at key position
    kv_len - seq + i when causal)."""
    s_q, s_kv = cfg.seq, cfg.kv_len
    if cfg.causal:
        return s_q * (s_kv - s_q) + s_q * (s_q + 1) / 2.0
    return float(s_q * s_kv)


def attention_summary(cfg, kernels):
    """The attention launches of one layer (names attn_*, transpose_*, dec_attn_*)
    together: their summed event-timed duration against the three
    contractions dA = dCtx V^T, dQ = dS K, dV = P^T dCtx on unmasked pairs
    (2 flops per multiply-add), and against the single-pass bytes the
    attention must move (P over unmasked pairs, dCtx, ctx, K, V, dq, dV)."""
    names = ("attn", "transpose", "dec_attn")
    ks = [k for k in kernels if k["name"].startswith(names)]
    if not ks:
        return None
    us = sum(k["avg_ms"] for k in ks) * 1e3
    flops = 3 * 2.0 * cfg.head_dim * attn_pairs(cfg) * cfg.n_heads
    es = 2 if cfg.dtype == "bf16" else 4
    qe, kve = cfg.seq * cfg.q_dim, cfg.kv_len * cfg.kv_dim
    nbytes = (attn_pairs(cfg) * cfg.n_heads * es + qe * (4 + es + 4) + kve * (2 * es + 4))
    peak = PEAK["bf16_TFLOPs"] if cfg.dtype == "bf16" else PEAK["f32_TFLOPs"]
    tf = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"launches": [k["name"] for k in ks], "us": round(us, 2), "flops": flops,
            "TFLOPs": round(tf, 2), "mfma_peak": peak, "mfma_frac": round(tf / peak, 4),
            "alg_bytes": nbytes, "GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK["hbm_GBps"], 4)}


def traffic_for(cfg, kernel, alg_bytes):
    """Measured HBM bytes per launch of `kernel` at this shape (identified by
    its algorithmic bytes) from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(cfg.name)
    if not ent:
        return None
    for k in ent.get("kernels", []):
        if k["name"] == kernel and abs(k["alg_bytes"] - alg_bytes) <= 1e-6 * max(alg_bytes, 1.0):
            return k["traffic_bytes"] if k.get("source_digest") == source_digest(kernel) else None
    return None


CAL_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes


def pmc_pass(lbp, hip, cfg, torch, path):
    """Records of one step (kernel order, algorithmic bytes), then three eager
    steps and the calibration copy, for rocprofv3 --pmc."""
    copies = build_copies(cfg, 1, torch, lbp)
    cp = copies[0]
    cap = 128
    ev = hip.events(cap)
    recs = (lbp.KernelRecord * cap)()
    n = step_calls(lbp, cfg, cp)[0](timing=(ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)), recs))
    torch.cuda.synchronize()
    rows = [{"index": i, "name": recs[i].name.decode(), "alg_bytes": recs[i].alg_bytes,
             "alg_flops": recs[i].alg_flops} for i in range(min(n, cap))]
    for _ in range(3):
        run_step(lbp, cfg, cp)
    torch.cuda.synchronize()
    src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    with open(path, "w") as f:
        json.dump({"workload": cfg.name, "layers": getattr(cfg, "n_layers", 1),
                   "kernels_per_layer": len(rows),
                   "records": rows, "calibration_bytes": CAL_BYTES}, f)


def traffic_summary(records_json, fetch_csv, write_csv):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by the factor that maps the same counter to the known bytes
    of the calibration copy."""
    import csv
    with open(records_json) as f:
        rec = json.load(f)

    def read(path, counter):
        lbp_rows, copy_rows = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                v = float(r["Counter_Value"]) * 1024.0
                if "lbp::" in name:
                    lbp_rows.append((int(r["Dispatch_Id"]), name.split("(")[0], v))
                elif "copy" in name.lower() and v > 0.5 * rec["calibration_bytes"]:
                    copy_rows.append(v)
        lbp_rows.sort()
        return lbp_rows, copy_rows

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows, cal = read(path, counter)
        if not cal:
            raise SystemExit("no calibration copy found in %s" % path)
        factor = rec["calibration_bytes"] / (sum(cal) / len(cal))
        per = rec["kernels_per_layer"]
        # the first layer call is the recorded one; then 3 eager steps
        vals = {}
        for j, (_, name, v) in enumerate(rows):
            vals.setdefault(j % per, []).append((name, v * factor))
        out[counter] = (factor, vals)
    kernels = []
    for r in rec["records"]:
        f = out["FETCH_SIZE"][1].get(r["index"], [])
        w = out["WRITE_SIZE"][1].get(r["index"], [])
        if not f or not w:
            continue
        fb = sum(v for _, v in f) / len(f)
        wb = sum(v for _, v in w) / len(w)
        kernels.append({"index": r["index"], "name": r["name"], "symbol": f[0][0],
                        "source_digest": source_digest(r["name"]),
                        "alg_bytes": r["alg_bytes"], "fetch_bytes": round(fb),
                        "write_bytes": round(wb), "traffic_bytes": round(fb + wb),
                        "traffic_over_alg": round((fb + wb) / r["alg_bytes"], 3) if r["alg_bytes"] else None})
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[rec["workload"]] = {
        "fetch_factor": round(out["FETCH_SIZE"][0], 4), "write_factor": round(out["WRITE_SIZE"][0], 4),
        "calibration": "torch copy of %d MiB (reads and writes that many bytes)" % (rec["calibration_bytes"] >> 20),
        "kernels": kernels}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print("| # | kernel | alg MB | FETCH MB | WRITE MB | traffic / alg |")
    print("|---|---|---|---|---|---|")
    for k in kernels:
        print("| %d | %s | %.2f | %.2f | %.2f | %s |" % (k["index"], k["name"], k["alg_bytes"] / 1e6,
                                                   k["fetch_bytes"] / 1e6, k["write_bytes"] / 1e6,
                                                   k["traffic_over_alg"]))


def sq_summary(records_json, sq_csv, simds=1024, cus=256, xcds=8):
    """MFMA busy and LDS busy as shares of each kernel's cycles, and the
    bank-conflict share of the LDS cycles, averaged over the recorded call
    and the eager steps.  GRBM_GUI_ACTIVE is summed over the XCDs (its max
    is the kernel's cycle count), the SQ counters over every SIMD / CU."""
    import csv
    with open(records_json) as f:
        rec = json.load(f)
    per = rec["kernels_per_layer"]
    rows = {}
    for r in csv.DictReader(open(sq_csv)):
        if "lbp::" not in r["Kernel_Name"]:
            continue
        d = rows.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = {}
    for j, d in enumerate(sorted(rows)):
        for k, v in rows[d].items():
            agg.setdefault(j % per, {}).setdefault(k, []).append(v)
    print("| # | kernel | MFMA busy % | LDS busy % | bank-conflict share of LDS cycles |")
    print("|---|---|---|---|---|")
    for i in range(per):
        a = {k: sum(v) / len(v) for k, v in agg.get(i, {}).items()}
        cyc = a.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        if cyc <= 0:
            continue
        mf = 100.0 * a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * simds)
        lds = 100.0 * a.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cyc * cus)
        bc = a.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(a.get("SQ_LDS_IDX_ACTIVE", 0.0), 1.0)
        name = rec["records"][i]["name"] if i < len(rec["records"]) else "?"
        print("| %d | %s | %.1f | %.1f | %.2f |" % (i, name, mf, lds, bc))


# ------------------------------------------------------------------ CPU baseline
def blas_info():
    """(vendor and version, threads) of NumPy's BLAS."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            b = max(blas, key=lambda i: i.get("num_threads", 1))
            return "%s %s" % (b.get("internal_api", "?"), b.get("version", "?")), b.get("num_threads", 1)
    except Exception:  # noqa: BLE001
        pass
    return "unknown", 1


def cpu_baseline_lm(cfg, budget_s, parts=16):
    """The float64 oracle's lm_head backward on a vocabulary slice of the
    workload (all rows, hidden size as is, vocab / parts entries), repeated
    until the budget is used; every part of the step (softmax, both products,
    AdamW) scales with the vocabulary, so a whole step takes parts times a
    slice's time."""
    import numpy as np
    import synth
    from oracle import lmhead as LM
    sub = cfg.with_(vocab=cfg.vocab // parts)
    d = {k: np.asarray(v, np.int64 if k == "labels" else np.float64)
         for k, v in synth.draw_lm_head(sub).items()}
    blas, threads = blas_info()
    runs, t0 = 0, time.perf_counter()
    while True:
        LM.lm_head_bwd(d["h"], d["logits"], d["labels"], d["W"], d["m"], d["v"], cfg.lr,
                       cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay, cfg.step)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (runs + 1) / runs > 3 * budget_s:
            break
    per_step = el / runs * parts
    return {"value": round(cfg.rows / per_step, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "blas": blas,
            "sample": "%d lm_head backward(s) on a 1/%d vocabulary slice (%d rows x %d entries, "
                      "hidden %d), scaled by %d; float64 NumPy, %.1f s timed, input generation "
                      "excluded" % (runs, parts, cfg.rows, sub.vocab, cfg.hidden, parts, el)}


def cpu_baseline(cfg, budget_s):
    """The float64 oracle's backward on the host, timed on a bounded sample of
    the same workload: whole steps (for the stack, all its layers in reverse
    order, the gradient handed down from layer to layer), repeated until the
    budget is used (at least once).  Input generation and the float64
    conversion are outside the timer; the stack's layers take the inputs of
    a few drawn layers in rotation (the oracle's cost does not depend on the
    values)."""
    import numpy as np
    import synth
    from oracle import backward as OB
    one = cfg.with_(n_layers=1)
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    distinct = min(cfg.n_layers, 4)
    layers = []
    for l in range(distinct):
        t = synth.draw_timing_layer(one, l)
        w = {k: f64(v) for k, v in t.items() if k.startswith("W_") or k.startswith("gamma_")}
        saved = {k: f64(t[k]) for k in ("attn_input", "resid1", "gate", "up", "ctx", "P", "K",
                                        "V", "hidden_pre", "lora_q_h", "lora_v_h", "q_raw", "x",
                                        "q", "k_raw") if k in t}
        lora = None
        if cfg.rank > 0:
            lora = {k: f64(v) for k, v in t.items()
                    if k[:2] in ("A_", "B_") or k[:4] in ("m_A_", "m_B_", "v_A_", "v_B_")}
        layers.append((w, saved, lora))
        if l == 0:
            d_out = f64(t["d_out"])
        del t
    blas, threads = blas_info()
    runs, t0 = 0, time.perf_counter()
    while True:
        d = d_out
        for l in range(cfg.n_layers - 1, -1, -1):
            w, saved, lora = layers[l % distinct]
            d = OB.layer_bwd(one, w, saved, d, lora)["d_hidden"]
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (runs + 1) / runs > 3 * budget_s:
            break
    per_step = el / runs
    what = ("%d whole step(s) of the %s workload, each all %d layers in reverse order "
            "(inputs of %d drawn layers in rotation)" % (runs, cfg.name, cfg.n_layers, distinct)
            if cfg.n_layers > 1 else "%d whole-layer backward(s) of the %s workload" % (runs, cfg.name))
    return {"value": round(cfg.seq / per_step, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "blas": blas,
            "sample": "%s; float64 NumPy, %.1f s timed, input generation excluded" % (what, el)}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.sq_summary:
        sq_summary(*args.sq_summary)
        return 0
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return 0
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU; --gpus %d is not supported (the multi-GPU "
              "path is design-only)" % args.gpus, file=sys.stderr)
        return 2
    import torch
    import synth
    import layer_backward_pass_amd as lbp
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lbp.load_library()
    cfg = synth.get_config(args.workload)
    if args.pmc_pass:
        pmc_pass(lbp, Hip(), cfg, torch, args.pmc_pass)
        return 0
    steps = args.steps or DEFAULT_STEPS[cfg.name]
    warmup = args.warmup if args.warmup is not None else max(3, steps // 10)
    hip = Hip()
    torch.cuda.set_device(0)
    copies = build_copies(cfg, COPIES[cfg.name], torch, lbp)
    # eager warm-up: sizes the workspace, loads the code objects
    for cp in copies:
        run_step(lbp, cfg, cp)
    torch.cuda.synchronize()
    graphs, round_graph = [], None
    if not args.no_graph:
        for cp in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(lbp, cfg, cp)
            graphs.append(g)
        if len(copies) > 1:
            round_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(round_graph):
                for cp in copies:
                    run_step(lbp, cfg, cp)
        torch.cuda.synchronize()

    def run(first, count):
        """Steps first .. first+count-1 (step i on copy i mod copies)."""
        i, end = first, first + count
        while i < end:
            if round_graph is not None and i % len(copies) == 0 and end - i >= len(copies):
                round_graph.replay()
                i += len(copies)
            elif graphs:
                graphs[i % len(graphs)].replay()
                i += 1
            else:
                run_step(lbp, cfg, copies[i % len(copies)])
                i += 1

    run(0, warmup)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = hip.events(2)
    hip.record(ev[0], stream)
    run(warmup, steps)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(ev[0], ev[1])
    ms_per_step = ms / steps
    tokens = cfg.seq * steps
    value = tokens / (ms / 1e3)

    # steady-state steps for the per-kernel timings: about 40 ms of work, at
    # least two steps (the first is not counted), at most 24 (the host
    # enqueues them while the GPU reads the 2 GiB ahead of them)
    kernels = kernel_profile(lbp, hip, cfg, copies, torch,
                             nsteps=int(min(24, max(2, round(40.0 / ms_per_step)))))
    rl = roofline(cfg, kernels)
    attn = attention_summary(cfg, kernels)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = (cpu_baseline_lm if is_lm(cfg) else cpu_baseline)(cfg, args.cpu_seconds)
    if is_lm(cfg):
        config = {"workload": cfg.name, "tokens_per_step": cfg.rows, "hidden": cfg.hidden,
                  "vocab": cfg.vocab, "input_copies": len(copies), "hip_graph": bool(graphs),
                  "kernels_per_step": len(kernels)}
    else:
        config = {"workload": cfg.name, "tokens_per_step": cfg.seq, "kv_len": cfg.kv_len,
                  "hidden": cfg.hidden, "ffn": cfg.ffn, "heads": cfg.n_heads,
                  "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "act": cfg.act,
                  "sub_norms": cfg.sub_norms, "lora_rank": cfg.rank, "layers": cfg.n_layers,
                  "input_copies": len(copies), "hip_graph": bool(graphs),
                  "steps_per_graph_launch": len(copies) if round_graph is not None else 1,
                  "kernels_per_step": len(kernels) * (cfg.n_layers if cfg.n_layers > 1 else 1)}
    out = {
        "metric": "lm_head-backward tokens/s" if is_lm(cfg) else "layer-backward tokens/s",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if getattr(cfg, "dtype", "f32") == "bf16" else "f32",
        "data": "synthetic",
        "config": config,
        "roofline": rl,
        "attn": attn,
        "cpu_baseline": cpu,
        "kernels": [{"name": k["name"], "avg_us": round(k["avg_ms"] * 1e3, 2),
                     "alg_MB": round(k["alg_bytes"] / 1e6, 3), "impl_MB": round(k["impl_bytes"] / 1e6, 3),
                     "GFLOP": round(k["alg_flops"] / 1e9, 3)} for k in kernels],
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
