#!/usr/bin/env python3
"""Decode GEMV benchmark: effective weight GB/s and fraction of HBM peak.

One step = one decode GEMV over the workload's weights (for the routed-expert
workload: the gate, up and down grouped calls of one token).  Inputs are
seeded synthetic data already resident in HBM when the timed region starts;
the weights rotate over enough copies that the 256 MB last-level cache
cannot serve them, and every routed-expert step draws fresh expert ids.

Prints ONE JSON line.  Effective GB/s = algorithmic bytes (packed codes +
scales/mins + x + y) / time.  The CPU baseline is the fp64 oracle timed on
the host cores on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
LLC_BYTES = 256 << 20          # MI355X last-level (Infinity) cache
HOT = False                    # --hot: one weight copy / one id set (cache-resident when it fits)
STACKED = False                # --stacked: projections sharing an activation in one matrix
METRIC = "effective weight GB/s and % of HBM peak, m=1 quantized GEMV (µs/call)"


# HBM bytes per launch of the dominant kernel, from rocprofv3 --pmc FETCH_SIZE
# and WRITE_SIZE runs scaled by the same counters on a plain copy kernel of
# known size.  Valid only for the kernel sources they were taken on (and,
# for an entry with "m", for that number of activation rows).
TRAFFIC = {
    "lm_head": {"source_digest": "bf7fa25a0ebc2b57", "bytes_per_launch": 403385997},
    # mean of the merged gate+up launch (63,254,918 B) and the down launch
    # (32,023,364 B)
    "moe_experts_merged": {"source_digest": "398e6f6ceac835a6", "bytes_per_launch": 47639142},
}


# The sources that build each workload's kernels: the digest of these files
# names the kernel version a TRAFFIC entry was measured on, so an edit to an
# unrelated kernel leaves the entry valid.
_COMMON_SOURCES = ("kernel_body.h", "argmax_key.h", "launch.hip", "layout.h", "launch.h")
KERNEL_SOURCES = {
    "lm_head": _COMMON_SOURCES + ("kern_q8g64.hip",),
    "lm_head_q8g128": _COMMON_SOURCES + ("kern_q8g128.hip",),
    "moe_experts": _COMMON_SOURCES + ("kern_q4g32.hip",),
    "moe_experts_swiglu": _COMMON_SOURCES + ("kern_q4g32_swiglu.hip", "kern_q4g32.hip"),
    "moe_experts_merged": _COMMON_SOURCES + ("kern_q4g32.hip",),
    "lm_head_argmax": _COMMON_SOURCES + ("kern_q8g64.hip", "argmax.hip", "argmax.h"),
    "lm_head_argmax_fused": _COMMON_SOURCES + ("kern_argmax_epi.hip", "argmax.h"),
    "lm_head_mma": ("kern_mma.hip", "launch.hip", "layout.h", "launch.h"),
    "w8a16_qwen3_14b_tp4_mma": ("kern_mma.hip", "launch.hip", "layout.h", "launch.h"),
    "q4_k2560_mma": ("kern_mma.hip", "launch.hip", "layout.h", "launch.h"),
}


def kernel_source_digest(workload):
    import hashlib
    files = KERNEL_SOURCES.get(workload, _COMMON_SOURCES + (
        "kern_q8g64.hip", "kern_q4g32.hip", "kern_q8g128.hip", "kern_q8pc.hip"))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "weight_only_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


ROUNDS = 5


def _round_edges(steps, rounds):
    """Step indices that split K timed steps into `rounds` consecutive rounds."""
    rounds = max(1, min(rounds, steps))
    return [steps * r // rounds for r in range(rounds + 1)]


def time_steps(torch, step, warmup, steps, rounds=ROUNDS):
    """W untimed steps, then exactly K timed steps bracketed by synchronize
    and HIP events on torch's current stream (the stream the kernels use).
    The K steps are split into consecutive rounds, each between its own pair
    of events (no synchronize in between), so the same run also gives the
    per-round times.  Returns (total seconds, [seconds per step of each
    round])."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    edges = _round_edges(steps, rounds)
    ev = [torch.cuda.Event(enable_timing=True) for _ in edges]
    ev[0].record()
    for r in range(len(edges) - 1):
        for i in range(edges[r], edges[r + 1]):
            step(warmup + i)
        ev[r + 1].record()
    torch.cuda.synchronize()
    per_round = [ev[r].elapsed_time(ev[r + 1]) * 1e-3 / (edges[r + 1] - edges[r])
                 for r in range(len(edges) - 1)]
    return ev[0].elapsed_time(ev[-1]) * 1e-3, per_round


def time_steps_graph(torch, step, warmup, steps, period, rounds=ROUNDS):
    """As time_steps, but the launches of P consecutive steps are captured
    once into a HIP graph that is replayed K/P times: host launch cost leaves
    the timed region, the GPU work is the same.  P is the largest divisor of
    K up to 2000 (replaying small graphs costs more than it saves), and the
    captured steps keep the workload's rotation of weights and ids.  Rounds
    are whole replays, so fewer than `rounds` when K/P is small."""
    P = max(d for d in range(1, min(steps, 2000) + 1) if steps % d == 0)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
        for i in range(P):
            step(i)
    g.replay()                      # one untimed replay
    torch.cuda.synchronize()
    edges = _round_edges(steps // P, rounds)
    ev = [torch.cuda.Event(enable_timing=True) for _ in edges]
    ev[0].record()
    for r in range(len(edges) - 1):
        for _ in range(edges[r], edges[r + 1]):
            g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    per_round = [ev[r].elapsed_time(ev[r + 1]) * 1e-3 / ((edges[r + 1] - edges[r]) * P)
                 for r in range(len(edges) - 1)]
    return ev[0].elapsed_time(ev[-1]) * 1e-3, per_round


def read_stream_reference(torch, Q, bytes_per_launch, launches=300, warmup=50):
    """The bandwidth of a plain read (qg_read_stream: 16-byte non-temporal
    loads, as the GEMV kernels use) of the same bytes per launch, rotating
    over enough buffers that no launch finds its bytes in the last-level
    cache.  Best of a few wave counts; returns (seconds per launch, waves
    per CU)."""
    nb = (int(bytes_per_launch) + 15) // 16 * 16
    copies = 1 if HOT else max(2, -(-2 * LLC_BYTES // nb))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = Q.lib().qg_read_stream
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for wpc in (2, 4, 8, 16):
        args = [(b.data_ptr(), nb, sink.data_ptr(), wpc, stream) for b in bufs]
        for i in range(warmup):
            fn(*args[i % copies])
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(launches):
            if fn(*args[i % copies]) != Q.QG_OK:
                raise RuntimeError("qg_read_stream failed")
        end.record()
        torch.cuda.synchronize()
        t = start.elapsed_time(end) * 1e-3 / launches
        if best is None or t < best[0]:
            best = (t, wpc)
    del bufs
    torch.cuda.empty_cache()
    return best


# ------------------------------------------------------------------ lm_head

def setup_lm_head(torch, Q, synth, fmt="q8g64"):
    """The LM-head GEMV in Q8G64 (headline) or Q8G128 (one scale per 128)."""
    _, _, N, K = synth.LM_HEAD
    name = "lm_head" if fmt == "q8g64" else "lm_head_q8g128"
    rng = synth.rng_for(synth.WORKLOAD_IDS[name], 0)
    if fmt == "q8g64":
        q, s = synth.q8g64_weights(rng, N, K)
        packed, weight_bytes = Q.qpack_q8g64(q, s), synth.bytes_q8g64(N, K)
        bind, fmt_id = Q.bound_q8g64, Q.FMT_Q8G64
    else:
        q, s = synth.q8g128_weights(rng, N, K)
        packed, weight_bytes = Q.qpack_q8g128(q, s), synth.bytes_q8g128(N, K)
        bind, fmt_id = Q.bound_q8g128, Q.FMT_Q8G128
    x = synth.activations(rng, 1, K)
    copies = 1 if HOT else max(2, -(-2 * LLC_BYTES // packed.nbytes))
    w = [dev(torch, packed) for _ in range(copies)]
    del packed
    xd = dev(torch, x)
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    alg_bytes = weight_bytes + 2 * K + 4 * N

    # Each bound call holds its device buffers, so they live as long as step.
    calls = [bind(wc, xd, y, N, K) for wc in w]

    def step(i):
        calls[i % copies]()

    step.logits = y
    info = {"workload": "lm_head %s GEMV m=1, N=151936 x K=2560 (Qwen3-4B vocabulary)" % fmt.upper(),
            "format": fmt, "m": 1, "N": N, "K": K, "weight_copies": copies, "period": copies,
            "kernel": Q.variant_name(fmt_id, 1, N, K)}
    cpu = {"fmt": fmt, "q": q, "s": s, "x": x}
    return step, alg_bytes, weight_bytes, 1, info, cpu


def setup_lm_head_argmax(torch, Q, synth):
    """The LM head followed by the greedy argmax over its logits: the GEMV
    writes the fp32 logits, the argmax reads them and writes one index."""
    step0, alg, weight_bytes, _, info, cpu = setup_lm_head(torch, Q, synth, "q8g64")
    _, _, N, K = synth.LM_HEAD
    y = step0.logits                  # the GEMV's output is the argmax's input
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Q.argmax_workspace_size(1), dtype=torch.uint8, device="cuda")
    arg = Q.bound_argmax_f32(y, idx, ws, N)

    def step(i):
        step0(i)
        arg()

    info = dict(info, workload="lm_head Q8G64 GEMV m=1 (N=151936 x K=2560) + greedy argmax",
                kernel=[info["kernel"], "argmax_rows"])
    return step, alg + 4 * N + 4, weight_bytes, 2, info, cpu


def setup_lm_head_argmax_fused(torch, Q, synth):
    """The LM head with the greedy argmax in the same launch and no logits
    written: what a greedy decode step needs from the LM head."""
    _, _, N, K = synth.LM_HEAD
    rng = synth.rng_for(synth.WORKLOAD_IDS["lm_head"], 0)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, 1, K)
    packed = Q.qpack_q8g64(q, s)
    copies = 1 if HOT else max(2, -(-2 * LLC_BYTES // packed.nbytes))
    w = [dev(torch, packed) for _ in range(copies)]
    del packed
    xd = dev(torch, x)
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Q.argmax_workspace_size(1), dtype=torch.uint8, device="cuda")
    calls = [Q.bound_q8g64_argmax(wc, xd, None, idx, ws, N, K) for wc in w]

    def step(i):
        calls[i % copies]()

    weight_bytes = synth.bytes_q8g64(N, K)
    info = {"workload": "lm_head Q8G64 GEMV m=1 (N=151936 x K=2560) with the greedy argmax fused, "
                        "no logits written",
            "format": "q8g64", "m": 1, "N": N, "K": K, "weight_copies": copies, "period": copies,
            "kernel": Q.variant_name(Q.FMT_Q8G64_ARGMAX, 1, N, K)}
    return step, weight_bytes + 2 * K + 4, weight_bytes, 1, info, {"fmt": "q8g64", "q": q, "s": s, "x": x}


def setup_mma(torch, Q, synth, name, m):
    """Batched decode on the matrix cores (weights in the matrix-core
    layout): the LM head (Q8G64) or the Qwen3-14B TP4 W8A16 layer, m rows."""
    if name == "lm_head_mma":
        _, _, N, K = synth.LM_HEAD
        mats = [("lm_head", "q8g64", N, K)]
        desc = "lm_head Q8G64 matrix-core GEMV m=%d, N=151936 x K=2560" % m
        wid = synth.WORKLOAD_IDS["lm_head"]
    elif name == "q4_k2560_mma":
        mats = synth.Q4_K2560
        desc = ("Q4G32 K=2560 family on the matrix cores m=%d: gate/up 2560->9216, "
                "down 9216->2560" % m)
        wid = synth.WORKLOAD_IDS["q4_k2560"]
    else:
        mats = synth.W8A16_QWEN3_14B_TP4
        desc = ("Qwen3-14B TP4 rank-local decode layer, per-output-channel W8A16 on the matrix "
                "cores m=%d: qkv 5120->1792, o 1280->5120, gate/up 5120->8704, down 4352->5120" % m)
        wid = synth.WORKLOAD_IDS["w8a16_qwen3_14b_tp4"]
    gens = _generate(synth, name[:-len("_mma")], mats, wid, m)
    if STACKED and len(gens) < len(mats):
        mats = [(e[0], e[1], e[2], e[3]) for e in gens]
        desc += " (stacked: %s)" % ", ".join(e[0] for e in gens)
    layer, wbytes, io = [], 0, 0
    packers = {"q8g64": Q.qpack_q8g64_mma, "q4g32": Q.qpack_q4g32_mma, "q8pc": Q.qpack_q8pc_mma}
    for label, fmt, N, K, w, xh, nb in gens:
        packed = packers[fmt](*w)
        wbytes += nb
        x = dev(torch, xh)
        y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        io += m * (2 * K + 4 * N)
        layer.append((fmt, N, K, packed, x, y))
    set_bytes = sum(l[3].nbytes for l in layer)
    copies = 1 if HOT else max(2 if len(layer) == 1 else 1, -(-2 * LLC_BYTES // set_bytes))
    dev_sets = [[dev(torch, l[3]) for l in layer] for _ in range(copies)]
    calls = [[Q.bound_mma(fmt, w, x, y, N, K, m=m) for (fmt, N, K, _, x, y), w in zip(layer, ws)]
             for ws in dev_sets]

    def step(i):
        for c in calls[i % copies]:
            c()

    fid = {"q8g64": Q.FMT_Q8G64_MMA, "q8pc": Q.FMT_Q8PC_MMA, "q4g32": Q.FMT_Q4G32_MMA}
    info = {"workload": desc, "format": mats[0][1] + "_mma", "m": m, "weight_copies": copies,
            "period": copies,
            "kernel": sorted({Q.variant_name(fid[f], m, N, K) for (_, f, N, K) in mats})}
    return step, wbytes + io, wbytes, len(mats), info, None


def cpu_lm_head(oracle, cpu, threads, reps):
    fn = oracle.q8g64 if cpu["fmt"] == "q8g64" else oracle.q8g128
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn(cpu["q"], cpu["s"], cpu["x"], threads=threads)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), "one full lm_head call (151936 x 2560, m=1), median of %d" % reps


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------ small dense configs

# --stacked: projections that read the same activation become one matrix
# whose rows are the members' rows in order (rows are independent, so each
# output is the same bits as in its own call; the merged gate_up matrix of
# vllm.cpp PR #1936 is the pattern).
STACK_GROUPS = {"qwen3_0.6b": [("q", "k", "v"), ("gate", "up")],
                "q4_k2560": [("gate", "up")],
                "w8a16_qwen3_14b_tp4": [("gate", "up")]}


def _stack_group(name, label):
    for g in STACK_GROUPS.get(name, []):
        if label in g:
            return g
    return None


def _generate(synth, group_name, mats, wid, m):
    """Seeded weights and m activation rows per matrix, in layer order; with
    --stacked, the matrices of a stacking group merged into one (the first
    member's activation serves the group).  Entries: [label, fmt, N, K,
    canonical weights, x, algorithmic weight bytes]."""
    gens = []
    for j, (label, fmt, N, K) in enumerate(mats):
        rng = synth.rng_for(wid, j)
        if fmt == "q8g64":
            w, nb = synth.q8g64_weights(rng, N, K), synth.bytes_q8g64(N, K)
        elif fmt == "q8pc":
            w, nb = synth.q8pc_weights(rng, N, K), synth.bytes_q8pc(N, K)
        else:
            w, nb = synth.q4g32_weights(rng, N, K), synth.bytes_q4g32(N, K)
        gens.append([label, fmt, N, K, w, synth.activations(rng, m, K), nb])
    if not STACKED:
        return gens
    merged = []
    for e in gens:
        grp = _stack_group(group_name, e[0])
        if merged and grp is not None and _stack_group(group_name, merged[-1][0].split("+")[0]) is grp:
            prev = merged[-1]
            prev[0] += "+" + e[0]
            prev[2] += e[2]
            prev[4] = tuple(np.concatenate([a, b]) for a, b in zip(prev[4], e[4]))
            prev[6] += e[6]
        else:
            merged.append(list(e))
    return merged


def setup_dense(torch, Q, synth, name, m=1):
    """q8_small (1 GEMV), qwen3_0.6b (7 GEMVs), q4_k2560 (3 GEMVs) or
    w8a16_qwen3_14b_tp4 (5 GEMVs) per step; with --stacked, 4, 2 and 4."""
    wid = synth.WORKLOAD_IDS[name]
    if name == "q8_small":
        mats = [("w", "q8g64", 1024, 1024)]
        desc = "Q8G64 GEMV m=1, N=K=1024"
    elif name == "qwen3_0.6b":
        mats = synth.QWEN3_06B_LAYER
        desc = "Qwen3-0.6B-shaped decode layer, Q8G64 m=1: q, k, v, o, gate, up, down"
    elif name == "w8a16_qwen3_14b_tp4":
        mats = synth.W8A16_QWEN3_14B_TP4
        desc = ("Qwen3-14B TP4 rank-local decode layer, per-output-channel W8A16 m=%d: "
                "qkv 5120->1792, o 1280->5120, gate/up 5120->8704, down 4352->5120" % m)
    else:
        mats = synth.Q4_K2560
        desc = "Q4G32 K=2560 family m=%d: gate/up 2560->9216, down 9216->2560" % m
    gens = _generate(synth, name, mats, wid, m)
    if STACKED:
        mats = [(e[0], e[1], e[2], e[3]) for e in gens]
        desc += " (stacked: %s)" % ", ".join(e[0] for e in gens)
    layer, wbytes, io = [], 0, 0
    packers = {"q8g64": Q.qpack_q8g64, "q8pc": Q.qpack_q8pc, "q4g32": Q.qpack_q4g32}
    for label, fmt, N, K, w, xh, nb in gens:
        packed = packers[fmt](*w)
        wbytes += nb
        x = dev(torch, xh)
        y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        io += m * (2 * K + 4 * N)
        layer.append((fmt, N, K, packed, x, y))
    set_bytes = sum(l[3].nbytes for l in layer)
    copies = 1 if HOT else max(1, -(-2 * LLC_BYTES // set_bytes))
    dev_sets = [[dev(torch, l[3]) for l in layer] for _ in range(copies)]

    binders = {"q8g64": (Q.bound_q8g64, Q.FMT_Q8G64), "q4g32": (Q.bound_q4g32, Q.FMT_Q4G32),
               "q8pc": (Q.bound_q8pc, Q.FMT_Q8PC)}
    calls = [[binders[fmt][0](w, x, y, N, K, m=m)
              for (fmt, N, K, _, x, y), w in zip(layer, ws)] for ws in dev_sets]

    def step(i):
        for c in calls[i % copies]:
            c()

    info = {"workload": desc, "format": mats[0][1], "m": m, "weight_copies": copies,
            "period": copies,
            "kernel": sorted({Q.variant_name(binders[f][1], m, N, K) for (_, f, N, K) in mats})}
    return step, wbytes + io, wbytes, len(mats), info, None


# ----------------------------------------------------------- routed experts

def setup_moe(torch, Q, synth, id_sets=256):
    id_sets = 1 if HOT else id_sets
    n_exp, n_slots = synth.MOE["n_experts"], synth.MOE["n_slots"]
    wid = synth.WORKLOAD_IDS["moe_experts"]
    bufs, shapes = {}, {}
    cpu_experts = {}
    for pj, proj in enumerate(("gate", "up", "down")):
        N, K = synth.MOE[proj]
        stride = Q.expert_stride(N, K)
        buf = torch.empty(n_exp * stride, dtype=torch.uint8, device="cuda")
        for e in range(n_exp):
            ex = synth.q4g32_weights(synth.rng_for(wid, pj, e), N, K)
            buf[e * stride:(e + 1) * stride].copy_(torch.from_numpy(Q.qpack_q4g32(*ex)))
            if e < 8:
                cpu_experts.setdefault(proj, []).append(ex)
        bufs[proj] = (buf, stride)
        shapes[proj] = (N, K)
    ids = np.stack([synth.expert_ids(synth.rng_for(wid, 1000, t), n_exp, n_slots)
                    for t in range(id_sets)])
    ids_d = dev(torch, ids)
    rng = synth.rng_for(wid, 2000)
    x_tok = dev(torch, synth.activations(rng, 1, synth.MOE["gate"][1]))
    x_down = dev(torch, synth.activations(rng, n_slots, synth.MOE["down"][1]))
    y_gu = torch.empty((n_slots, synth.MOE["gate"][0]), dtype=torch.float32, device="cuda")
    y_dn = torch.empty((n_slots, synth.MOE["down"][0]), dtype=torch.float32, device="cuda")

    calls = []
    for t in range(id_sets):
        idv = ids_d[t]
        c = []
        for proj in ("gate", "up"):
            buf, stride = bufs[proj]
            N, K = shapes[proj]
            c.append(Q.bound_grouped_q4g32(buf, stride, n_exp, idv, x_tok, 0, y_gu, N, N, K))
        buf, stride = bufs["down"]
        N, K = shapes["down"]
        c.append(Q.bound_grouped_q4g32(buf, stride, n_exp, idv, x_down, K, y_dn, N, N, K))
        calls.append(c)

    def step(i):
        for c in calls[i % id_sets]:
            c()

    weight_bytes = sum(n_slots * synth.bytes_q4g32(*shapes[p]) for p in shapes)
    io_bytes = (2 * 2 * 4096 + 4 * 2 * n_slots * 1536) + (2 * n_slots * 1536 + 4 * n_slots * 4096)
    info = {"workload": "routed-expert decode, Q4G32, 128 experts, 8 per token: "
                        "gate/up 4096->1536 and down 1536->4096 grouped calls",
            "format": "q4g32", "m": 1, "experts": n_exp, "slots": n_slots, "period": id_sets,
            "kernel": [Q.variant_name(Q.FMT_GROUPED_Q4G32, 1, *shapes[p]) for p in ("gate", "down")]}
    return step, weight_bytes + io_bytes, weight_bytes, 3, info, {"experts": cpu_experts}


def setup_moe_merged(torch, Q, synth, id_sets=256):
    """Routed experts with each expert's gate and up rows stacked into one
    [2*1536][4096] matrix (rows are independent, so the result is the same
    bits as two calls): one grouped launch for gate+up, one for down."""
    id_sets = 1 if HOT else id_sets
    n_exp, n_slots = synth.MOE["n_experts"], synth.MOE["n_slots"]
    wid = synth.WORKLOAD_IDS["moe_experts"]
    Ng, Kg = synth.MOE["gate"]
    Nd, Kd = synth.MOE["down"]
    s_gu, s_dn = Q.expert_stride(2 * Ng, Kg), Q.expert_stride(Nd, Kd)
    buf_gu = torch.empty(n_exp * s_gu, dtype=torch.uint8, device="cuda")
    buf_dn = torch.empty(n_exp * s_dn, dtype=torch.uint8, device="cuda")
    for e in range(n_exp):
        g = synth.q4g32_weights(synth.rng_for(wid, 0, e), Ng, Kg)
        u = synth.q4g32_weights(synth.rng_for(wid, 1, e), Ng, Kg)
        stacked = [np.concatenate([a, b]) for a, b in zip(g, u)]
        buf_gu[e * s_gu:(e + 1) * s_gu].copy_(torch.from_numpy(Q.qpack_q4g32(*stacked)))
        d = synth.q4g32_weights(synth.rng_for(wid, 2, e), Nd, Kd)
        buf_dn[e * s_dn:(e + 1) * s_dn].copy_(torch.from_numpy(Q.qpack_q4g32(*d)))
    ids = np.stack([synth.expert_ids(synth.rng_for(wid, 1000, t), n_exp, n_slots)
                    for t in range(id_sets)])
    ids_d = dev(torch, ids)
    rng = synth.rng_for(wid, 2000)
    x_tok = dev(torch, synth.activations(rng, 1, Kg))
    x_down = dev(torch, synth.activations(rng, n_slots, Kd))
    y_gu = torch.empty((n_slots, 2 * Ng), dtype=torch.float32, device="cuda")
    y_dn = torch.empty((n_slots, Nd), dtype=torch.float32, device="cuda")
    calls = [(Q.bound_grouped_q4g32(buf_gu, s_gu, n_exp, ids_d[t], x_tok, 0, y_gu, 2 * Ng, 2 * Ng, Kg),
              Q.bound_grouped_q4g32(buf_dn, s_dn, n_exp, ids_d[t], x_down, Kd, y_dn, Nd, Nd, Kd))
             for t in range(id_sets)]

    def step(i):
        a, b = calls[i % id_sets]
        a()
        b()

    weight_bytes = n_slots * (synth.bytes_q4g32(2 * Ng, Kg) + synth.bytes_q4g32(Nd, Kd))
    io_bytes = (2 * Kg + 4 * n_slots * 2 * Ng) + (2 * n_slots * Kd + 4 * n_slots * Nd)
    info = {"workload": "routed-expert decode, Q4G32, 128 experts, 8 per token: merged gate+up "
                        "4096->2x1536 and down 1536->4096 grouped calls",
            "format": "q4g32", "m": 1, "experts": n_exp, "slots": n_slots, "period": id_sets,
            "kernel": [Q.variant_name(Q.FMT_GROUPED_Q4G32, 1, 2 * Ng, Kg),
                       Q.variant_name(Q.FMT_GROUPED_Q4G32, 1, Nd, Kd)]}
    return step, weight_bytes + io_bytes, weight_bytes, 2, info, None


def setup_moe_swiglu(torch, Q, synth, id_sets=256):
    """Routed experts as a decode step runs them with the fused epilogue: one
    grouped call over gate/up pair buffers that writes bf16 silu(g) * u,
    then the grouped down call reading that activation."""
    id_sets = 1 if HOT else id_sets
    n_exp, n_slots = synth.MOE["n_experts"], synth.MOE["n_slots"]
    wid = synth.WORKLOAD_IDS["moe_experts"]
    Ng, Kg = synth.MOE["gate"]
    Nd, Kd = synth.MOE["down"]
    s_gu, s_dn = Q.gate_up_expert_stride(Ng, Kg), Q.expert_stride(Nd, Kd)
    buf_gu = torch.empty(n_exp * s_gu, dtype=torch.uint8, device="cuda")
    buf_dn = torch.empty(n_exp * s_dn, dtype=torch.uint8, device="cuda")
    for e in range(n_exp):
        g = synth.q4g32_weights(synth.rng_for(wid, 0, e), Ng, Kg)
        u = synth.q4g32_weights(synth.rng_for(wid, 1, e), Ng, Kg)
        buf_gu[e * s_gu:(e + 1) * s_gu].copy_(torch.from_numpy(Q.qpack_q4g32_gate_up(g, u)))
        d = synth.q4g32_weights(synth.rng_for(wid, 2, e), Nd, Kd)
        buf_dn[e * s_dn:(e + 1) * s_dn].copy_(torch.from_numpy(Q.qpack_q4g32(*d)))
    ids = np.stack([synth.expert_ids(synth.rng_for(wid, 1000, t), n_exp, n_slots)
                    for t in range(id_sets)])
    ids_d = dev(torch, ids)
    x_tok = dev(torch, synth.activations(synth.rng_for(wid, 2000), 1, Kg))
    act = torch.empty((n_slots, Ng), dtype=torch.int16, device="cuda")
    y_dn = torch.empty((n_slots, Nd), dtype=torch.float32, device="cuda")
    calls = [(Q.bound_grouped_q4g32_swiglu(buf_gu, s_gu, n_exp, ids_d[t], x_tok, 0, act, Ng, Ng, Kg),
              Q.bound_grouped_q4g32(buf_dn, s_dn, n_exp, ids_d[t], act, Kd, y_dn, Nd, Nd, Kd))
             for t in range(id_sets)]

    def step(i):
        a, b = calls[i % id_sets]
        a()
        b()

    weight_bytes = n_slots * (2 * synth.bytes_q4g32(Ng, Kg) + synth.bytes_q4g32(Nd, Kd))
    io_bytes = (2 * Kg + 2 * n_slots * Ng) + (2 * n_slots * Kd + 4 * n_slots * Nd)
    info = {"workload": "routed-expert decode, Q4G32, 128 experts, 8 per token: gate/up "
                        "4096->2x1536 with fused SwiGLU (bf16 out), then down 1536->4096",
            "format": "q4g32", "m": 1, "experts": n_exp, "slots": n_slots, "period": id_sets,
            "kernel": [Q.variant_name(Q.FMT_GROUPED_Q4G32_SWIGLU, 1, Ng, Kg),
                       Q.variant_name(Q.FMT_GROUPED_Q4G32, 1, Nd, Kd)]}
    return step, weight_bytes + io_bytes, weight_bytes, 2, info, None


def cpu_moe(oracle, cpu, threads, reps, synth):
    # The oracle on one token's eight routed experts (gate, up, down).
    ex = cpu["experts"]
    rng = synth.rng_for(99, 5)
    xg = np.repeat(synth.activations(rng, 1, 4096), 8, axis=0)
    xd = synth.activations(rng, 8, 1536)
    ids = np.arange(8)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.grouped_q4g32(ex["gate"], ids, xg, threads=threads)
        oracle.grouped_q4g32(ex["up"], ids, xg, threads=threads)
        oracle.grouped_q4g32(ex["down"], ids, xd, threads=threads)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), "one token's 8 routed experts (gate, up, down), median of %d" % reps


# --------------------------------------------------------------------- main

def measure_setup(args, torch, Q, synth, name=None):
    """The workload's step function and its byte counts."""
    name = name or args.workload
    if name in ("lm_head_mma", "w8a16_qwen3_14b_tp4_mma", "q4_k2560_mma"):
        return setup_mma(torch, Q, synth, name, args.m)
    if name == "lm_head_argmax_fused":
        return setup_lm_head_argmax_fused(torch, Q, synth)
    if name == "lm_head_argmax":
        return setup_lm_head_argmax(torch, Q, synth)
    if name in ("lm_head", "lm_head_q8g128"):
        return setup_lm_head(torch, Q, synth, "q8g64" if name == "lm_head" else "q8g128")
    if name == "moe_experts":
        return setup_moe(torch, Q, synth)
    if name == "moe_experts_merged":
        return setup_moe_merged(torch, Q, synth)
    if name == "moe_experts_swiglu":
        return setup_moe_swiglu(torch, Q, synth)
    return setup_dense(torch, Q, synth, name, args.m)


def ab_pairs(args, step, torch):
    """Interleaved A/B pairs (the adoption rule of the vllm.cpp pull request
    #1936 commit log: a variant is taken only if it wins at least 4 of 5
    pairs).  The library reads QG_FORCE_VARIANT at every call, so switching
    it between rounds switches the launch geometry with everything else
    held fixed.  Returns per-pair us/step of each arm and B's wins."""
    a_spec, b_spec = args.ab
    a_t, b_t = [], []

    def run(spec, offset):
        if spec:
            os.environ["QG_FORCE_VARIANT"] = spec
        else:
            os.environ.pop("QG_FORCE_VARIANT", None)
        secs, _ = time_steps(torch, step, args.warmup, args.steps, rounds=1)
        return secs / args.steps * 1e6

    for p in range(args.pairs):
        order = [(a_spec, a_t), (b_spec, b_t)] if p % 2 == 0 else [(b_spec, b_t), (a_spec, a_t)]
        for spec, out in order:
            out.append(run(spec, p))
    os.environ.pop("QG_FORCE_VARIANT", None)
    wins = sum(1 for a, b in zip(a_t, b_t) if b < a)
    return {"ab": {"workload": args.workload, "m": args.m, "a": a_spec, "b": b_spec,
                   "a_us_per_step": [round(t, 3) for t in a_t], "b_us_per_step": [round(t, 3) for t in b_t],
                   "a_median": round(float(np.median(a_t)), 3), "b_median": round(float(np.median(b_t)), 3),
                   "b_wins": wins, "pairs": args.pairs}}


TRACE_MHZ = 100.0   # s_memrealtime: the GPU's constant 100 MHz clock


def _pct(v, q):
    return round(float(np.percentile(v, q)) / TRACE_MHZ, 3)


def wave_trace(args, step, torch, Q, info, trial, capacity=1 << 16):
    """Per-wave timeline of one step in the middle of a stream of steps:
    for each launch of the step, the start spread, the time from a wave's
    start until its first weights are in, wave durations and end times
    (percentiles, us from the launch's first wave start), per-XCD ends, and
    the gap from each launch's last wave end to the next launch's first
    wave start."""
    buf = torch.zeros(capacity * 8, dtype=torch.int64, device="cuda")
    for i in range(args.warmup):
        step(i)
    # The traced step is enqueued behind others, as in a steady stream.
    for i in range(200):
        step(i)
    Q.set_wave_trace(buf)
    step(1000 + trial)
    records, launches, dropped = Q.wave_trace_state()
    Q.set_wave_trace(None)
    for i in range(50):
        step(i)
    torch.cuda.synchronize()
    r = buf[:records * 8].view(-1, 8).cpu().numpy().astype(np.int64)
    out = {"workload": args.workload, "trial": trial, "kernel": info.get("kernel"), "clock_mhz": TRACE_MHZ,
           "launches": [], "dropped_launches": dropped}
    bounds = []
    for li in range(launches):
        w = r[r[:, 7] == li]
        t0, t1, t2 = w[:, 0], w[:, 1], w[:, 2]
        base = int(t0.min())
        first = (t1[t1 > 0] - t0[t1 > 0]).astype(np.float64)
        xcd = {}
        for x in sorted(set(w[:, 4].tolist())):
            sel = w[:, 4] == x
            xcd[str(int(x))] = {"waves": int(sel.sum()), "end_p50_us": _pct(t2[sel] - base, 50),
                                "end_max_us": _pct(t2[sel] - base, 100)}
        out["launches"].append({
            "waves": int(len(w)),
            "span_us": round(float(t2.max() - base) / TRACE_MHZ, 3),
            "start_spread_us": _pct(t0 - base, 100),
            "first_weights_p50_us": _pct(first, 50) if len(first) else None,
            "first_weights_max_us": _pct(first, 100) if len(first) else None,
            "wave_us_p10_p50_p90_max": [_pct(t2 - t0, q) for q in (10, 50, 90, 100)],
            "end_us_p10_p50_p90_max": [_pct(t2 - base, q) for q in (10, 50, 90, 100)],
            "xcd": xcd})
        bounds.append((base, int(t2.max())))
    out["gaps_us"] = [round((bounds[i + 1][0] - bounds[i][1]) / TRACE_MHZ, 3) for i in range(len(bounds) - 1)]
    if bounds:
        out["step_us"] = round((bounds[-1][1] - bounds[0][0]) / TRACE_MHZ, 3)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: 2000 timed steps after 500 warmup steps.  Under sustained load
    # the lm_head kernel runs fast for ~2 ms, slows by up to 30% for ~10 ms and
    # then settles (seen in kernel traces on MI355X); the warmup covers that.
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="lm_head",
                    choices=["lm_head", "lm_head_q8g128", "lm_head_argmax", "lm_head_argmax_fused",
                             "moe_experts", "moe_experts_merged",
                             "moe_experts_swiglu", "q8_small", "qwen3_0.6b", "q4_k2560", "w8a16_qwen3_14b_tp4",
                             "lm_head_mma", "w8a16_qwen3_14b_tp4_mma", "q4_k2560_mma"])
    ap.add_argument("--m", type=int, default=1,
                    help="activation rows (q4_k2560, w8a16_qwen3_14b_tp4: 1..4; *_mma: 2..16)")
    ap.add_argument("--hot", action="store_true",
                    help="one weight copy and one expert-id set, reused every step: the "
                         "cache-resident (hot) number, reported separately from the default cold one")
    ap.add_argument("--stacked", action="store_true",
                    help="qwen3_0.6b, q4_k2560, w8a16_qwen3_14b_tp4 and their *_mma forms: stack the "
                         "projections that share an activation (q+k+v, gate+up) into one matrix "
                         "per launch")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from a captured HIP graph (no host launch cost)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (for HBM counter "
                         "calibration under rocprofv3 --pmc)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="skip timing the other workload beside the headline")
    ap.add_argument("--no-read-stream", dest="read_stream", action="store_false",
                    help="skip timing a plain read of the same bytes per launch")
    ap.add_argument("--ab", nargs=2, metavar=("A", "B"),
                    help="interleaved A/B pairs instead of the benchmark line: A and B are "
                         "QG_FORCE_VARIANT values ('' = the library's own choice); each pair times "
                         "--steps steps of A then of B (the order alternates between pairs), "
                         "--pairs times, in one process on one set of inputs")
    ap.add_argument("--pairs", type=int, default=5)
    ap.add_argument("--sweep", nargs="+", metavar="SPEC",
                    help="--ab '' SPEC for each SPEC in turn on one set of inputs (one JSON line each)")
    ap.add_argument("--wave-trace", action="store_true",
                    help="instead of the benchmark line, the per-wave timelines (qg_set_wave_trace) of "
                         "three steps taken in the middle of a stream of steps, one JSON line each")
    args = ap.parse_args()
    global HOT, STACKED
    HOT = args.hot
    STACKED = args.stacked
    if args.workload.endswith("_mma") and not 2 <= args.m <= 16:
        print("--m %d: the matrix-core workloads take 2..16 rows (m = 1 is the plain kernels' "
              "case)" % args.m, file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode GEMV is single-GPU work here "
              "(--gpus %d requested). Rows of N shard across GPUs with no exchange; "
              "run with --gpus 1." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from weight_only_block_amd import qgemv as Q
    from weight_only_block_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    Q.lib()
    # Eager launches and their timing events go to the default stream: back
    # to back on a created (blocking) stream they measured about 4 us per
    # lm_head call slower on MI355X.  Graph capture needs a created stream;
    # it has default priority, and the graph is replayed on it.
    if args.graph:
        torch.cuda.set_stream(torch.cuda.Stream(device=0))

    def measure(name):
        t0 = time.time()
        step, alg, wbytes, launches, info, cpu = measure_setup(args, torch, Q, synth, name)
        log("setup %s: %.1f s" % (name, time.time() - t0))
        if args.graph:
            secs, rounds = time_steps_graph(torch, step, args.warmup, args.steps, info.get("period", 1))
        else:
            secs, rounds = time_steps(torch, step, args.warmup, args.steps)
        return dict(secs=secs, rounds=rounds, alg=alg, wbytes=wbytes, launches=launches, info=info,
                    cpu=cpu)

    if args.wave_trace:
        step, _, _, _, info, _ = measure_setup(args, torch, Q, synth)
        for trial in range(3):
            print(json.dumps({"wave_trace": wave_trace(args, step, torch, Q, info, trial)}), flush=True)
        return

    if args.ab or args.sweep:
        step = measure_setup(args, torch, Q, synth)[0]
        for pair in ([args.ab] if args.ab else [("", spec) for spec in args.sweep]):
            args.ab = list(pair)
            print(json.dumps(ab_pairs(args, step, torch)), flush=True)
        return

    head = measure(args.workload)
    secs, steps = head["secs"], args.steps
    per_step = secs / steps
    per_launch = per_step / head["launches"]
    value = head["alg"] * steps / secs / 1e9
    achieved = head["alg"] / head["launches"] / per_launch / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_step * 1e3, 5),
        "us_per_call": round(per_launch * 1e6, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; int8/4-bit codes, fp16 group scales and mins or fp32 row "
                "scales, N(0,1) bf16 x)",
        "launch": "hip_graph" if args.graph else "eager",
        "weights": ("hot: one weight copy and one id set reused every step (cache-resident when "
                    "it fits in the 256 MB last-level cache)" if HOT else
                    "cold: rotated so that no step finds its weights in the last-level cache"),
        "config": dict(head["info"], algorithmic_bytes_per_step=head["alg"]),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }
    # The timed steps in consecutive rounds (each between its own events):
    # the median round and the spread between the fastest and slowest.
    round_us = [t / head["launches"] * 1e6 for t in head["rounds"]]
    out["rounds"] = {"count": len(round_us), "steps_per_round": args.steps // max(1, len(round_us)),
                     "us_per_call": [round(u, 3) for u in round_us],
                     "median_us_per_call": round(float(np.median(round_us)), 3),
                     "min_us_per_call": round(min(round_us), 3),
                     "max_us_per_call": round(max(round_us), 3),
                     "median_pct_hbm_peak": round(100.0 * head["alg"] / head["launches"]
                                                  / (float(np.median(round_us)) * 1e-6) / 1e9
                                                  / HBM_PEAK_GBS, 2)}
    digest = kernel_source_digest(args.workload)
    entry = TRAFFIC.get(args.workload, {})
    if not HOT and entry.get("source_digest") == digest and entry.get("m", args.m) == args.m:
        out["roofline"]["traffic"] = TRAFFIC[args.workload]["bytes_per_launch"]
    out["config"]["kernel_source_digest"] = digest
    if args.read_stream:
        bpl = head["alg"] / head["launches"]
        t, wpc = read_stream_reference(torch, Q, bpl)
        out["read_stream"] = {"bytes_per_launch": int(bpl), "us_per_launch": round(t * 1e6, 3),
                              "GBs": round(bpl / t / 1e9, 2), "waves_per_cu": wpc,
                              "frac": round(achieved / (bpl / t / 1e9), 4)}
    if not args.no_cpu and head["cpu"] is not None:
        # The oracle as the parity tests run it, on the host: (i) one thread,
        # (ii) output rows split over the host cores it may use (at most 16,
        # the host's CPU share per GPU).
        import oracle
        affinity = len(os.sched_getaffinity(0))
        threads = max(1, min(16, affinity))
        run = cpu_lm_head if args.workload in ("lm_head", "lm_head_q8g128") else (
            lambda o, c, t, r: cpu_moe(o, c, t, r, synth))
        t1, sample1 = run(oracle, head["cpu"], 1, args.cpu_reps)
        tp, sample = run(oracle, head["cpu"], threads, args.cpu_reps)
        out["cpu_baseline"] = {"value": round(head["alg"] / tp / 1e9, 4), "unit": "GB/s",
                               "cores": threads, "kind": "oracle", "sample": sample,
                               "seconds_per_step": round(tp, 4),
                               "single_thread": {"value": round(head["alg"] / t1 / 1e9, 4),
                                                 "unit": "GB/s", "cores": 1, "sample": sample1,
                                                 "seconds_per_step": round(t1, 4)},
                               "affinity_cores": affinity, "cores_cap": 16,
                               "cpu_model": cpu_model()}
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst
    # The routed-expert step beside the LM head: gate and up rows stacked into
    # one grouped call (their fp32 outputs still written separately), then the
    # grouped down call.
    if args.secondary and args.workload in ("lm_head", "moe_experts", "moe_experts_merged"):
        other = "moe_experts_merged" if args.workload == "lm_head" else "lm_head"
        del head
        torch.cuda.empty_cache()
        sec = measure(other)
        ps = sec["secs"] / steps
        sec_round_us = [t / sec["launches"] * 1e6 for t in sec["rounds"]]
        out["secondary"] = {"workload": sec["info"]["workload"], "launches_per_step": sec["launches"],
                            "us_per_call": round(ps / sec["launches"] * 1e6, 3),
                            "effective_GBs": round(sec["alg"] / ps / 1e9, 2),
                            "pct_hbm_peak": round(100 * sec["alg"] / ps / 1e9 / HBM_PEAK_GBS, 2),
                            "rounds_us_per_call": [round(u, 3) for u in sec_round_us],
                            "median_us_per_call": round(float(np.median(sec_round_us)), 3)}
        if args.read_stream:
            bpl = sec["alg"] / sec["launches"]
            t, wpc = read_stream_reference(torch, Q, bpl)
            out["secondary"]["read_stream_GBs"] = round(bpl / t / 1e9, 2)
            out["secondary"]["frac_of_read_stream"] = round(sec["alg"] / ps / 1e9 / (bpl / t / 1e9), 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
