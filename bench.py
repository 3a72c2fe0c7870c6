"""Benchmark of the KDA recurrent-state hot path on one MI355X.

A step is one kda_decode launch over the batched decode workload (B = 64
sequences, H = 32 heads, d_k = d_v = 128, bf16 inputs, fp32 states in a
1024-slot pool addressed by a random slot table): slot resolution, conv +
SiLU, L2 norms, gates, the state read / delta update / write, RMSNorm and the
output gate.  Inputs for every step are resident in HBM before timing starts.

The timed steps rotate over 16 disjoint 64-slot sets of the pool (step t uses
set t mod 16), so every step's 128 MiB of state was last touched 15 steps
(about 2 GiB of state traffic) earlier and has left the 256 MB Infinity
Cache: each step streams its states from HBM, as a serving step over many
KDA layers does.  The decode runs with its default flags (state traffic
streamed).  The same 64 slots re-used every step (cache-resident) are timed
as a side measurement.

Prints ONE JSON line: the metric (token·heads/s over the median of 5 timed
repetitions of K steps), the roofline object of the decode kernel
(algorithmic bytes per launch over the mean launch duration from HIP events
on the launch stream, beside the rocprofv3 mean of the committed profile),
the fp64 oracle timed on the host cores on bounded samples, and side
measurements (cache-resident variant, copy ceilings, spec-verify/commit,
chunked prefill, batch-1 decode, mixed batches).

  python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--no-cpu-baseline]
                  [--no-extras]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK = 2.5e15   # MI355X dense bf16 MFMA, flop/s
METRIC = "KDA decode state updates/s (token·heads/s) + achieved HBM GB/s at B=64"

# algorithmic bytes per (token, head) of one decode step at H=32, d_k=d_v=128,
# bf16 inputs, B=64 (shared per-head parameters amortised over the batch)
def decode_bytes_per_token_head(H=32, dk=128, dv=128, B=64, in_bytes=2):
    ch = 2 * dk + dv
    state = 2 * dk * dv * 4                      # read + write
    inputs = (3 * dk + 2 * dv) * in_bytes + in_bytes   # x_q, x_k, g, x_v, z + b
    window = 2 * 3 * ch * in_bytes               # read + write
    out = dv * 4
    params = (dk + ch * 4 + dv) * 4 / B          # A, conv_wt, norm_w per head / B
    return state + inputs + window + out + params


def verify_bytes_per_seq_head(T=8, dk=128, dv=128, B=16, in_bytes=2):
    ch = 2 * dk + dv
    return (dk * dv * 4 + 3 * ch * in_bytes                  # S0 + window read
            + T * ((3 * dk + 2 * dv) * in_bytes + in_bytes)   # inputs
            + T * (dk * dv * 4 + 3 * ch * in_bytes)           # snapshots
            + T * dv * 4                                      # outputs
            + (dk + ch * 4 + dv) * 4 / B)                     # params


def verify_delta_bytes_per_seq_head(T=8, dk=128, dv=128, B=16, in_bytes=2):
    ch = 2 * dk + dv
    return (dk * dv * 4 + 3 * ch * in_bytes                  # S0 + window read
            + T * ((3 * dk + 2 * dv) * in_bytes + in_bytes)   # inputs
            + T * ch * (4 + in_bytes)                         # replay records
            + T * dv * 4                                      # outputs
            + (dk + ch * 4 + dv) * 4 / B)                     # params


def commit_delta_bytes_per_seq_head(L, dk=128, dv=128, in_bytes=2):
    ch = 2 * dk + dv
    return (2 * dk * dv * 4                  # live state read + write
            + L * (2 * dk + dv) * 4          # alpha, k^, d of the accepted tokens
            + 2 * 3 * ch * in_bytes)         # window rows read + written


# the files that define the decode kernel and its launch: the counter
# summary is stale once any of them changes
DECODE_SOURCES = ("kda_recurrent.hip", "kda_device.h", "kda_internal.h")


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "linear_attention_recurrent_kda_amd", "csrc")
    for f in DECODE_SOURCES:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill measurement (32768 tokens, H=32) and print it; "
                         "for profiling that path")
    ap.add_argument("--decode-b1-only", action="store_true",
                    help="run only the batch-1 decode latency measurement and print it; for profiling that path")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain copy of this many MiB "
                         "(a known-size kernel for calibrating memory counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU; the KDA path has no cross-GPU exchange "
              "(heads and sequences shard with no collective), so --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_recurrent_kda_amd import api, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.prefill_only:
        print(json.dumps({"chunk_prefill_t32k": prefill_extra(torch, api, synth, torch.cuda.current_stream())}),
              flush=True)
        return
    if args.decode_b1_only:
        print(json.dumps({"decode_b1": decode_b1_extra(torch, api, synth)}), flush=True)
        return
    cfg = synth.WORKLOADS["decode_b64"]
    B, H, dk, dv, n_slots = cfg["B"], cfg["H"], cfg["d_k"], cfg["d_v"], cfg["n_slots"]
    K, W = args.steps, args.warmup
    g = synth.rng(cfg["seed"])
    p = synth.layer_params(g, H, dk, dv)
    td = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    layer = api.Layer(td(p["A"]), td(p["conv_wt"]), td(p["norm_w"]))
    # pools: 2 GiB of fp32 state; slots not in the table hold seeded values
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg["seed"])
    state = (torch.randn((n_slots, H, dk, dv), generator=gen, device=dev) * 0.05)
    win = torch.randn((n_slots, H, 3, 2 * dk + dv), generator=gen, device=dev).to(torch.bfloat16)
    cache = api.Cache(state, win, torch.zeros(1, dtype=torch.int32, device=dev))
    # the random slot table of every step: a seeded permutation of the pool
    # cut into n_slots / B disjoint sets, step t on set t mod n_sets
    perm = synth.slot_table(g, n_slots, n_slots)
    n_sets = n_slots // B
    sets = td(perm.reshape(n_sets, B), torch.int32)
    # inputs of every step, resident in HBM before timing
    nsteps = W + K
    inp = synth.token_inputs(g, (nsteps, B), H, dk, dv, "bf16")
    dinp = {k: td(v, torch.bfloat16) for k, v in inp.items()}
    step_inputs = [api.Inputs(*(dinp[k][t] for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
                   for t in range(nsteps)]
    y = torch.empty((B, H, dv), device=dev)
    stream = torch.cuda.current_stream()
    # every launch's arguments are marshalled before timing starts
    calls = [api.kda_decode_prepared(layer, cache, sets[t % n_sets], step_inputs[t], y) for t in range(nsteps)]

    for t in range(W):
        calls[t]()
    torch.cuda.synchronize()
    # REPS timed regions of K back-to-back launches each, between two events
    # on the launch stream (the mean launch duration is their span / K, launch
    # gaps included) and a synchronised wall clock; the median one is reported
    reps = []
    for _ in range(REPS):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            calls[W + i]()
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append((time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3 / K))
    wall, mean_kern_s = sorted(reps)[len(reps) // 2]
    bytes_launch = decode_bytes_per_token_head(H, dk, dv, B) * B * H
    achieved = bytes_launch / mean_kern_s / 1e9
    value = B * H * K / wall

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "token·heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_b64", "B": B, "H": H, "d_k": dk, "d_v": dv,
                   "n_slots": n_slots, "input_dtype": "bf16", "state_dtype": "f32",
                   "seed": cfg["seed"], "parallelism": "single-gpu",
                   "slot_tables": f"{n_sets} disjoint {B}-slot sets of a seeded permutation of the pool, "
                                  f"step t on set t mod {n_sets}: every step's states come from HBM",
                   "flags": "default (state traffic streamed)"},
        "repetitions": {"count": REPS, "ms_per_step_wall": [r[0] / K * 1e3 for r in reps],
                        "mean_launch_us_events": [r[1] * 1e6 for r in reps], "reported": "median by wall"},
        "achieved_gbs_wall": bytes_launch * K / wall / 1e9,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "kernel": DECODE_KERNEL,
            "bytes_per_launch": bytes_launch,
            "mean_launch_us": mean_kern_s * 1e6,
            "residency": "states not cache-resident (slot sets rotated; 2 GiB pool > 256 MB Infinity Cache)",
        },
    }
    prof = load_profile("decode_b64_kernel_trace.json")
    if prof is not None:
        # the committed rocprofv3 trace of this command's decode launches
        out["roofline"]["rocprof_mean_launch_us"] = prof["mean_ns"] / 1e3
        out["roofline"]["frac_rocprof"] = bytes_launch / (prof["mean_ns"] * 1e-9) / 1e9 / HBM_PEAK_GBS
    traffic = load_profile("decode_b64_traffic.json")
    if traffic is not None:
        # counter bytes per launch over the same mean launch duration (GB/s)
        tb = traffic["fabric_bytes_per_launch"]
        out["roofline"]["traffic"] = tb / mean_kern_s / 1e9
        out["roofline"]["traffic_bytes_per_launch"] = tb
        out["roofline"]["traffic_over_algorithmic"] = tb / bytes_launch
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        api.kda_copy_probe(dst, src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_extras:
        out["extras"] = extras(torch, api, synth, layer, cache, step_inputs, y, sets, B, H, dk, dv,
                               n_slots, W, K, stream)
        # two measured ceilings: the copy probe (in place over 2 GiB) and the
        # decode itself on every slot of the pool in one call (2 GiB of state
        # read and written, the best DRAM-bound rate measured here)
        ceil = out["extras"]["inplace_probe_2gib"]["gbs"]
        out["roofline"]["inplace_ceiling_gbs"] = ceil
        out["roofline"]["frac_of_inplace_ceiling"] = achieved / ceil
        dram = out["extras"]["decode_b%d_dram" % n_slots]["algorithmic_gbs"]
        out["roofline"]["decode_dram_ceiling_gbs"] = dram
        out["roofline"]["frac_of_decode_dram_ceiling"] = achieved / dram
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth, p, inp, B, H, dk, dv)
    print(json.dumps(out), flush=True)


# the decode instance the timed steps launch (streamed state traffic)
DECODE_KERNEL = "kda::kda_recurrent_kernel<128, 128, 256, unsigned short, 1, 0, true, false>"
REPS = 5


def load_profile(name):
    """A committed profile summary (JSON under profiles/) if it was taken on
    the current decode kernel source, else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec


def timed(torch, stream, fn, reps, warm=1):
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / reps


def extras(torch, api, synth, layer, cache, step_inputs, y, sets, B, H, dk, dv, n_slots, W, K, stream):
    ex = {}
    bl = decode_bytes_per_token_head(H, dk, dv, B) * B * H
    steps = min(K, len(step_inputs) - W)
    n_sets = sets.shape[0]

    def decode_leg(lay, slot_fn, note):
        cl = [api.kda_decode_prepared(lay, cache, slot_fn(i), step_inputs[W + i], y) for i in range(steps)]
        for c in cl[:n_sets]:
            c()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for c in cl:
            c()
        b.record(stream)
        torch.cuda.synchronize()
        s = a.elapsed_time(b) / 1e3 / steps
        return {"us_per_step": s * 1e6, "token_heads_per_s": B * H / s, "algorithmic_gbs": bl / s / 1e9,
                "frac_of_8tbs": bl / s / 8e12, "residency": note}

    resident = api.Layer(layer.A, layer.conv_wt, layer.norm_w, layer.q_scale, layer.l2_eps,
                         layer.rms_eps, layer.conv_silu, state_resident=True)
    hot = sets[0]
    # the same 64 slots every step: their 128 MiB of state stays in the 256 MB
    # Infinity Cache between steps, so these figures are cache bandwidth, not HBM
    ex["decode_b64_hot_resident_flag"] = decode_leg(
        resident, lambda i: hot, "Infinity-Cache resident (same slots every step), KDA_STATE_RESIDENT")
    ex["decode_b64_hot_default"] = decode_leg(
        layer, lambda i: hot, "Infinity-Cache resident (same slots every step), default flags (streamed)")
    # the headline's rotation with the resident hint given wrongly
    ex["decode_b64_cold_resident_flag"] = decode_leg(
        resident, lambda i: sets[i % n_sets], "from HBM (rotated slot sets), KDA_STATE_RESIDENT")
    # DRAM-bound large batch: every slot of the pool in one call (n_slots
    # sequences; 2 GiB of state at H=32, d=128, eight times the Infinity Cache)
    Bl = n_slots
    gl = synth.rng(11)
    linp = synth.token_inputs(gl, (Bl,), H, dk, dv, "bf16")
    LI = api.Inputs(*(torch.from_numpy(np.ascontiguousarray(linp[k])).to("cuda:0").to(torch.bfloat16)
                      for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
    yl = torch.empty((Bl, H, dv), device="cuda:0")
    s = timed(torch, stream, api.prepared(api.kda_decode, layer, cache, sets.reshape(-1), LI, yl), 10)
    bll = decode_bytes_per_token_head(H, dk, dv, Bl) * Bl * H
    ex["decode_b%d_dram" % Bl] = {"us_per_step": s * 1e6, "token_heads_per_s": Bl * H / s,
                                  "algorithmic_gbs": bll / s / 1e9, "frac_of_8tbs": bll / s / 8e12,
                                  "state_bytes": Bl * H * dk * dv * 4}
    del LI, yl
    # memory ceilings: the probe copies n floats the way the decode moves its
    # tiles (64 KiB per workgroup, 16-byte non-temporal loads and stores).
    # In place (dst = src: read then rewrite the same bytes, the decode's
    # pattern) over 2 GiB, and as a copy between two 1 GiB buffers
    n = 1 << 29
    buf = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    s = timed(torch, stream, lambda: api.kda_copy_probe(buf, buf), 10)
    ex["inplace_probe_2gib"] = {"gbs": 2 * n * 4 / s / 1e9, "us": s * 1e6,
                                "note": "read + rewrite of 2 GiB in place (HBM)"}
    del buf
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    s = timed(torch, stream, lambda: api.kda_copy_probe(dst, src), 10)
    ex["copy_probe_1gib"] = {"gbs": 2 * n * 4 / s / 1e9, "us": s * 1e6, "note": "1 GiB copied to another 1 GiB (HBM)"}
    del src, dst
    # spec-verify B=16 x T=8 and commit
    cfg = synth.WORKLOADS["spec_verify_b16_t8"]
    Bv, T = cfg["B"], cfg["T"]
    g = synth.rng(cfg["seed"])
    vin = synth.token_inputs(g, (Bv, T), H, dk, dv, "bf16")
    td = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0").to(dt)
    vinp = api.Inputs(*(td(vin[k]) for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
    live = sets[0, :Bv].contiguous()
    rest = sets[1:1 + (Bv * T + B - 1) // B].reshape(-1)[:Bv * T].reshape(Bv, T).contiguous()
    yv = torch.empty((Bv, T, H, dv), device="cuda:0")
    acc = td(synth.accepted_lengths(g, Bv, T), torch.int32)
    sv = timed(torch, stream, api.prepared(api.kda_spec_verify, layer, cache, live, rest, vinp, yv), 100, warm=10)
    sc = timed(torch, stream, api.prepared(api.kda_spec_commit, layer, cache, live, rest, acc), 100, warm=10)
    vb = verify_bytes_per_seq_head(T, dk, dv, Bv) * Bv * H
    Lm = float(acc.float().mean().item())
    cb = Bv * H * (dk * dv * 4 + 3 * (2 * dk + dv) * 2) * 2
    ex["spec_verify_b16_t8"] = {"us_per_call": sv * 1e6, "token_heads_per_s": Bv * T * H / sv,
                                "algorithmic_gbs": vb / sv / 1e9, "frac_of_8tbs": vb / sv / 8e12}
    # the snapshots are written once and read at most once (by the commit):
    # the same call with non-temporal state traffic
    sl_layer = api.Layer(layer.A, layer.conv_wt, layer.norm_w, layer.q_scale, layer.l2_eps,
                         layer.rms_eps, layer.conv_silu, stream_state=True)
    svs = timed(torch, stream, api.prepared(api.kda_spec_verify, sl_layer, cache, live, rest, vinp, yv), 100, warm=10)
    ex["spec_verify_b16_t8_stream"] = {"us_per_call": svs * 1e6, "token_heads_per_s": Bv * T * H / svs,
                                       "algorithmic_gbs": vb / svs / 1e9, "frac_of_8tbs": vb / svs / 8e12}
    ex["spec_commit_b16"] = {"us_per_call": sc * 1e6, "mean_accepted": Lm,
                             "algorithmic_gbs": cb / sc / 1e9}
    # replayable deltas instead of snapshots (same workload, same accepted lengths)
    delta = api.new_spec_delta(layer, Bv, T, torch.bfloat16, "cuda:0")
    svd = timed(torch, stream, api.prepared(api.kda_spec_verify_delta, layer, cache, live, vinp, yv, delta), 100, warm=10)
    scd = timed(torch, stream, api.prepared(api.kda_spec_commit_delta, layer, cache, live, delta, acc), 100, warm=10)
    vdb = verify_delta_bytes_per_seq_head(T, dk, dv, Bv) * Bv * H
    cdb = sum(commit_delta_bytes_per_seq_head(int(L), dk, dv) for L in acc.cpu().tolist()) * H
    ex["spec_verify_delta_b16_t8"] = {"us_per_call": svd * 1e6, "token_heads_per_s": Bv * T * H / svd,
                                      "algorithmic_gbs": vdb / svd / 1e9, "frac_of_8tbs": vdb / svd / 8e12,
                                      "bytes_per_call": vdb}
    ex["spec_commit_delta_b16"] = {"us_per_call": scd * 1e6, "mean_accepted": Lm,
                                   "algorithmic_gbs": cdb / scd / 1e9, "bytes_per_call": cdb}
    ex["spec_step_b16_t8"] = {"snapshots_us": (sv + sc) * 1e6, "deltas_us": (svd + scd) * 1e6}
    ex["chunk_prefill_t32k"] = prefill_extra(torch, api, synth, stream)
    ex["decode_b1"] = decode_b1_extra(torch, api, synth)
    ex["mixed_batch"] = mixed_extra(torch, api, synth)
    ex["metadata_build"] = metadata_extra(torch, api, stream)
    return ex


def metadata_extra(torch, api, stream, calls=1000):
    """kda_build_metadata at batch 1, 64 and 1024 (one-token and prompt
    requests mixed): mean per call between events over `calls` back-to-back
    prepared launches, and replayed from a HIP graph of 100 launches."""
    dev = "cuda:0"
    out = {}
    g = np.random.default_rng(5)
    for n in (1, 64, 1024):
        nt = torch.from_numpy(g.choice([1, 1, 1, 500], size=n).astype(np.int32)).to(dev)
        rs = torch.from_numpy(g.permutation(4096)[:n].astype(np.int32)).to(dev)
        cu = torch.empty(n + 1, dtype=torch.int32, device=dev)
        si = torch.empty(n, dtype=torch.int32, device=dev)
        cs = torch.empty(n + 1, dtype=torch.int32, device=dev)
        ct = torch.empty(4, dtype=torch.int32, device=dev)
        call = api.prepared(api.kda_build_metadata, nt, rs, 4096, cu, si, cs, ct)
        ev = timed(torch, stream, call, calls, warm=10)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(100):
                    api.kda_build_metadata(nt, rs, 4096, cu, si, cs, ct)
        stream.wait_stream(side)
        gs = timed(torch, stream, graph.replay, 10, warm=1) / 100
        out[f"batch_{n}"] = {"us_per_call_events": ev * 1e6, "us_per_call_graph": gs * 1e6}
    return out


def mixed_extra(torch, api, synth, prompt=4096, n_one=64):
    """A mixed prefill + decode batch in one kda_chunk_prefill call: one
    `prompt`-token sequence and `n_one` one-token (decode) rows, H=32, d=128;
    beside the prompt alone and the one-token rows alone (same call), and the
    one-token rows through kda_decode; and eight `prompt`-token sequences in
    one call (the scan then takes 64-column blocks)."""
    dev = "cuda:0"
    H, dk, dv = 32, 128, 128
    g = synth.rng(106)
    p = synth.layer_params(g, H, dk, dv)
    td = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    layer = api.Layer(td(p["A"]), td(p["conv_wt"]), td(p["norm_w"]))
    stream = torch.cuda.current_stream()
    out = {}
    for name, lens in (("prompt_plus_decode_rows", [prompt] + [1] * n_one), ("prompt_only", [prompt]),
                       ("decode_rows_only", [1] * n_one), ("eight_prompts", [prompt] * 8)):
        N, total = len(lens), sum(lens)
        cache = api.Cache(torch.zeros((N, H, dk, dv), device=dev),
                          torch.zeros((N, H, 3, 2 * dk + dv), dtype=torch.bfloat16, device=dev))
        inp = synth.token_inputs(g, (total,), H, dk, dv, "bf16")
        I = api.Inputs(*(td(inp[k], torch.bfloat16) for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
        y = torch.empty((total, H, dv), device=dev)
        sl = torch.arange(N, dtype=torch.int32, device=dev)
        cu = td(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), torch.int32)
        ws = torch.empty(max(api.kda_chunk_prefill_workspace_bytes(layer, total, N), 16), dtype=torch.uint8, device=dev)
        out[name + "_us"] = timed(torch, stream, lambda: api.kda_chunk_prefill(layer, cache, sl, cu, I, y, ws), 10) * 1e6
        if name == "decode_rows_only":
            yd = torch.empty((N, H, dv), device=dev)
            out["decode_rows_via_kda_decode_us"] = timed(
                torch, stream, lambda: api.kda_decode(layer, cache, sl, I, yd), 10) * 1e6
    out["eight_prompts_tokens_per_s"] = 8 * prompt / (out["eight_prompts_us"] * 1e-6)
    out["config"] = f"{prompt}-token prompt + {n_one} one-token rows, H={H}, d={dk}, bf16; eight {prompt}-token prompts"
    return out


def decode_b1_extra(torch, api, synth, steps=1000, graph_steps=100):
    """The batch-1 decode (latency-bound) with default flags and with the
    residency hint (a single sequence's 2 MiB of state per layer can stay in
    the Infinity Cache across many layers)."""
    return {"default": decode_b1_leg(torch, api, synth, False, steps, graph_steps),
            "resident_flag": decode_b1_leg(torch, api, synth, True, steps, graph_steps)}


def decode_b1_leg(torch, api, synth, resident, steps=1000, graph_steps=100):
    """B=1, H=32, d=128, one slot of a 256-slot pool.  Times `steps`
    back-to-back launches with events (launch gaps included), and the same
    launches captured `graph_steps` at a time in a HIP graph and replayed
    (host launch cost removed)."""
    dev = "cuda:0"
    cfg = synth.WORKLOADS["decode_b1"]
    H, dk, dv, n_slots = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["n_slots"]
    g = synth.rng(cfg["seed"])
    p = synth.layer_params(g, H, dk, dv)
    td = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    layer = api.Layer(td(p["A"]), td(p["conv_wt"]), td(p["norm_w"]), state_resident=resident)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg["seed"])
    cache = api.Cache(torch.randn((n_slots, H, dk, dv), generator=gen, device=dev) * 0.05,
                      torch.zeros((n_slots, H, 3, 2 * dk + dv), dtype=torch.bfloat16, device=dev))
    slot = td(g.permutation(n_slots)[:1].astype(np.int32), torch.int32)
    inp = synth.token_inputs(g, (steps, 1), H, dk, dv, "bf16")
    dinp = {k: td(v, torch.bfloat16) for k, v in inp.items()}
    ins = [api.Inputs(*(dinp[k][t] for k in ("x_q", "x_k", "x_v", "g", "b", "z"))) for t in range(steps)]
    y = torch.empty((1, H, dv), device=dev)
    stream = torch.cuda.current_stream()
    calls = [api.kda_decode_prepared(layer, cache, slot, ins[t], y) for t in range(steps)]
    for c in calls[:10]:
        c()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for c in calls:
        c()
    b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = a.elapsed_time(b) / 1e3 / steps
    # the same launches in a graph (captured on torch's capture stream)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for t in range(graph_steps):
                api.kda_decode(layer, cache, slot, ins[t], y)
    stream.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    reps = steps // graph_steps
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    gs = a.elapsed_time(b) / 1e3 / (reps * graph_steps)
    bl = (2 * dk * dv * 4 + (3 * dk + 2 * dv) * 2 + 2 + 2 * 3 * (2 * dk + dv) * 2 + dv * 4
          + (dk + (2 * dk + dv) * 4 + dv) * 4) * H
    return {"us_per_step_events": ev * 1e6, "us_per_step_wall": wall * 1e6,
            "us_per_step_graph": gs * 1e6, "bytes_per_step": bl,
            "algorithmic_gbs_graph": bl / gs / 1e9, "steps": steps}


def prefill_mfma_flops_per_chunk_head(dk, dv, col_block=16):
    """Flops the chunked prefill issues on MFMA per (chunk, head); bf16x3 makes
    three MFMA products per fp32 product.
    intra: the 10 Gram tile pairs on or below the diagonal, A and P, d_k/32
    steps of v_mfma_f32_16x16x32_bf16 each; [W | U~] by block forward
    substitution over (d_k + d_v)/16 column tiles, 1 + 2 + 3 + 4 products of
    v_mfma_f32_16x16x16_bf16 per tile.  scan, per block of 16 state columns
    (16x16x32): W S and Q S (d_k/32 steps for each of 4 row tiles), P U (1, 1,
    2 and 2 steps for the 4 row tiles: P is lower triangular), Kd^T U (2 steps
    x d_k/16 row tiles)."""
    ks = dk // 32
    x32, x16 = 16 * 16 * 32 * 2, 16 * 16 * 16 * 2
    intra = 3 * (10 * 2 * ks) * x32 + 3 * (dk + dv) // 16 * 10 * x16
    scan = 3 * (dv // col_block) * (4 * 2 * ks + 6 + (dk // 16) * 2) * x32
    return intra + scan


def prefill_algorithmic_flops_per_chunk_head(dk, dv, C=64):
    """Dense flops of the chunk algebra, each contraction counted once: A and
    P (C x C x d_k), T = (I + A)^-1 (~C^3/3 multiply-adds), [W | U~]
    (C x C x (d_k + d_v)), W S and Q S (C x d_k x d_v), P U (C x C x d_v),
    Kd^T U (d_k x C x d_v)."""
    return 2 * (2 * C * C * dk + C ** 3 / 3 + C * C * (dk + dv) + 2 * C * dk * dv + C * C * dv + dk * C * dv)


def prefill_extra(torch, api, synth, stream):
    cfg = synth.WORKLOADS["prefill_t32k"]
    H, dk, dv, T = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["T"]
    g = synth.rng(cfg["seed"])
    p = synth.layer_params(g, H, dk, dv)
    td = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0").to(dt)
    layer = api.Layer(td(p["A"]), td(p["conv_wt"]), td(p["norm_w"]))
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    I = api.Inputs(*(td(inp[k], torch.bfloat16) for k in ("x_q", "x_k", "x_v", "g", "b", "z")))
    # slot 0 is the live slot; slots 1..4 take interval checkpoints
    cache = api.Cache(torch.zeros((5, H, dk, dv), device="cuda:0"),
                      torch.zeros((5, H, 3, 2 * dk + dv), dtype=torch.bfloat16, device="cuda:0"))
    sl = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda:0")
    y = torch.empty((T, H, dv), device="cuda:0")
    try:
        ws_n = api.kda_chunk_prefill_workspace_bytes(layer, T, 1)
        ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device="cuda:0")
        run = lambda: api.kda_chunk_prefill(layer, cache, sl, cu, I, y, ws)
        run()
    except api.KdaError as e:
        return {"status": e.status}
    s = timed(torch, stream, run, 5)
    in_b = T * H * ((3 * dk + 2 * dv) * 2 + 2)
    out_b = T * H * dv * 4
    st_b = 2 * H * dk * dv * 4
    tot = in_b + out_b + st_b
    chunk_heads = (T + 63) // 64 * H
    mfma_flops = prefill_mfma_flops_per_chunk_head(dk, dv) * chunk_heads
    alg_flops = prefill_algorithmic_flops_per_chunk_head(dk, dv) * chunk_heads
    # the same call keeping a state checkpoint every 8192 tokens (4 per call)
    ck = torch.arange(1, 5, dtype=torch.int32, device="cuda:0").reshape(1, 4)
    sck = timed(torch, stream, lambda: api.kda_chunk_prefill_ckpt(layer, cache, sl, cu, I, y, ck, 8192, ws), 5)
    return {"us_per_call": s * 1e6, "tokens_per_s": T / s, "token_heads_per_s": T * H / s,
            "algorithmic_gbs": tot / s / 1e9, "frac_of_8tbs": tot / s / 8e12,
            "mfma_flops_issued": mfma_flops, "mfma_tflops": mfma_flops / s / 1e12,
            "mfma_util_of_bf16_dense_peak": mfma_flops / s / MFMA_BF16_PEAK,
            "algorithmic_tflops": alg_flops / s / 1e12,
            "workspace_bytes": ws_n,
            "with_4_checkpoints_us": sck * 1e6}


def cpu_baseline(synth, p, inp, B, H, dk, dv):
    """The fp64 oracle (as it is, untuned) on the host cores: a bounded sample
    of the same workload (all 64 sequences x 32 heads, a few steps)."""
    from oracle import kda_oracle
    from oracle.kda_oracle_np import Layer as OLayer
    ol = OLayer(p["A"], p["conv_wt"], p["norm_w"])
    cores = kda_oracle.threads(0)
    tb = {k: np.ascontiguousarray(np.swapaxes(v, 0, 1), dtype=np.float64)
          for k, v in inp.items()}                              # [B, steps, ...]
    st = np.zeros((B, H, dk, dv))
    win = np.zeros((B, H, 3, 2 * dk + dv))
    n, el, runs = tb["x_q"].shape[1], 0.0, 0
    # repeat the staged steps (carrying the state) until ~10 s of oracle work
    while el < 10.0 and runs < 200:
        t0 = time.perf_counter()
        o = kda_oracle.run(ol, st, win, tb["x_q"], tb["x_k"], tb["x_v"], tb["g"], tb["b"], tb["z"])
        el += time.perf_counter() - t0
        st, win, runs = o["state"], o["window"], runs + 1
    # the same oracle on one core, over a quarter of the sequences
    q = max(B // 4, 1)
    sub = {k: np.ascontiguousarray(v[:q]) for k, v in tb.items()}
    t0 = time.perf_counter()
    kda_oracle.run(ol, st[:q], win[:q], sub["x_q"], sub["x_k"], sub["x_v"], sub["g"], sub["b"], sub["z"],
                   n_threads=1)
    el1 = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": B * H * n * runs / el, "unit": "token·heads/s", "cores": cores, "kind": "oracle",
            "sample": f"decode_b64: {runs} x {n} steps x {B} sequences x {H} heads (fp64, OpenMP "
                      f"over sequence x head), {el:.1f} s",
            "one_core_value": q * H * n / el1,
            "one_core_sample": f"{n} steps x {q} sequences x {H} heads on one thread, {el1:.1f} s",
            "cpu_model": model,
            "spec_verify_b16_t8": cpu_verify(synth, kda_oracle, OLayer, cores),
            "chunk_prefill_t32k": cpu_prefill(synth, kda_oracle, OLayer, cores)}


def cpu_verify(synth, kda_oracle, OLayer, cores):
    """The oracle on one spec-verify call of the verification workload
    (16 sequences x 8 draft tokens x 32 heads, a snapshot per token)."""
    cfg = synth.WORKLOADS["spec_verify_b16_t8"]
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["d_k"], cfg["d_v"]
    g = synth.rng(cfg["seed"])
    p = synth.layer_params(g, H, dk, dv)
    ol = OLayer(p["A"], p["conv_wt"], p["norm_w"])
    inp = synth.token_inputs(g, (B, T), H, dk, dv, "bf16")
    s0 = synth.random_state(g, (B, H, dk, dv), 0.05)
    w0 = synth.window_inputs(g, (B,), H, dk, dv, "bf16")
    t0 = time.perf_counter()
    kda_oracle.run(ol, s0, w0, inp["x_q"], inp["x_k"], inp["x_v"], inp["g"], inp["b"], inp["z"], snapshots=True)
    el = time.perf_counter() - t0
    return {"us_per_call": el * 1e6, "token_heads_per_s": B * T * H / el, "cores": cores, "kind": "oracle",
            "sample": f"one call: {B} sequences x {T} tokens x {H} heads with a state snapshot per token"}


def cpu_prefill(synth, kda_oracle, OLayer, cores, seg=8192):
    """The oracle's full sequential run of the long-prompt workload (1 x 32768
    tokens x 32 heads, every output and the final state), in segments of
    `seg` tokens carrying the state (to bound host memory)."""
    cfg = synth.WORKLOADS["prefill_t32k"]
    H, dk, dv, T = cfg["H"], cfg["d_k"], cfg["d_v"], cfg["T"]
    g = synth.rng(cfg["seed"])
    p = synth.layer_params(g, H, dk, dv)
    ol = OLayer(p["A"], p["conv_wt"], p["norm_w"])
    inp = synth.token_inputs(g, (T,), H, dk, dv, "bf16")
    st, win = np.zeros((1, H, dk, dv)), np.zeros((1, H, 3, 2 * dk + dv))
    el = 0.0
    for a in range(0, T, seg):
        sub = {k: v[None, a:a + seg] for k, v in inp.items()}
        t0 = time.perf_counter()
        o = kda_oracle.run(ol, st, win, sub["x_q"], sub["x_k"], sub["x_v"], sub["g"], sub["b"], sub["z"])
        el += time.perf_counter() - t0
        st, win = o["state"], o["window"]
        del o, sub
    return {"us_per_call": el * 1e6, "tokens_per_s": T / el, "token_heads_per_s": T * H / el, "cores": cores,
            "kind": "oracle",
            "sample": f"the whole workload: {T} tokens x {H} heads token by token, in {T // seg} calls of "
                      f"{seg} tokens carrying the state (each call's fp64 input conversion included)"}


if __name__ == "__main__":
    main()
