"""Benchmark: deterministic vs atomic Split-K LoRA shrink + expand on one MI355X.

Workload (one "step"): the q_proj-shaped single-adapter LoRA of an
8B-parameter Llama-3 layer - x bf16 [M x 4096] ~ N(0,1), A bf16 [16 x 4096]
and B bf16 [4096 x 16] ~ N(0, 0.02), base y bf16 [M x 4096] ~ N(0,1),
scale 2.0, Split-K 8 - run once at each batch size M in {1, 16, 64, 256}:
deterministic shrink (split partials + fixed-tree combine) then expand into y.
`value` is the mean microseconds per shrink+expand call over the four batch
sizes.  The atomic Split-K contrast (zero fill + atomic partials + expand) is
timed the same way.

Timing: steps are captured in HIP graphs, 8 consecutive steps on 8 input
copies per graph (the paper times shrink latency under CUDA graphs); the
timed region replays K / 8 graphs, i.e. exactly K steps, rotating over enough
input copies (>= 1 GiB) that no step finds its inputs in the 256 MB
last-level cache.  Inputs are resident in HBM before timing.  HIP events are
recorded on the stream the kernels run on.

Also reported: per-batch-size numbers, the roofline of the dominant kernel
(the tree + expand kernel of the deterministic pipeline, with the HBM bytes
the hardware counters recorded for it when its sources are unchanged since),
two decode bandwidth probes (32 and 128 tokens, each with its own rank-64
adapter, hidden 8192, multi-adapter shrink), the same decode shapes' expand
and shrink + expand (N = 4096), device-copy ceilings at the
probes' sizes, identical-input replay statistics of the deterministic and
atomic pipelines (1000 launches per batch size), and the CPU oracle timed on
the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --counters      # eager pass for rocprofv3 --pmc runs
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shrink+expand µs/call & HBM GB/s (% peak), deterministic vs atomic Split-K=8"
HBM_PEAK_GBS = 8000.0
M_LIST = (1, 16, 64, 256)
K_HID, RANK, N_OUT, SPLIT, SCALE = 4096, 16, 4096, 8, 2.0
ROTATE_BYTES = 1 << 30
STEPS_PER_GRAPH = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def steps_per_graph(steps: int) -> int:
    """Steps captured per HIP graph: the largest divisor of `steps` that is at
    most STEPS_PER_GRAPH, so that exactly `steps` steps run in whole graphs."""
    return max(d for d in range(1, STEPS_PER_GRAPH + 1) if steps % d == 0)


def shrink_bytes(M, K, r):
    """Algorithmic bytes of a shrink: read x and A once, write h."""
    return 2 * M * K + 2 * K * r + 4 * M * r


def expand_bytes(M, r, N):
    """Algorithmic bytes of an expand: read h and B once, read and write y."""
    return 4 * M * r + 2 * r * N + 4 * M * N


def combine_bytes(M, r, N, S):
    """Algorithmic bytes of the tree + expand kernel: read the S workspace
    slices once, write h, read B once, read and write y."""
    return 4 * S * M * r + 4 * M * r + 2 * r * N + 4 * M * N


class Bench:
    def __init__(self, args, copies=None):
        import torch
        import deterministic_split_lora_amd as dsl
        from synth import single_adapter_case
        self.t, self.dsl, self.args = torch, dsl, args
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)

        def g(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(self.dev)

        # one seeded input set per batch size, then device copies for rotation
        base = {M: single_adapter_case(M, K_HID, RANK, N_OUT, SPLIT, SCALE, seed=0) for M in M_LIST}
        self.ws_bytes = {M: dsl.lora_shrink_expand_workspace_bytes(M, RANK, SPLIT) for M in M_LIST}
        per_set = sum(2 * M * K_HID + 2 * M * N_OUT + 4 * RANK * K_HID + 4 * M * RANK * (SPLIT + 1)
                      for M in M_LIST)
        self.per_set = per_set
        self.copies = max(2, math.ceil(ROTATE_BYTES / per_set)) if not args.hot else 1
        if copies is not None:
            self.copies = copies
        self.sets = []
        for c in range(self.copies):
            s = {}
            for M in M_LIST:
                b = base[M]
                s[M] = dict(x=g(b.x), A=g(b.A), B=g(b.B), y=g(b.y),
                            h=torch.empty((M, RANK), dtype=torch.float32, device=self.dev),
                            ws=torch.empty(self.ws_bytes[M], dtype=torch.uint8, device=self.dev),
                            # the single-launch shrink's own zeroed workspace of tagged slots
                            cws=torch.zeros(dsl.lora_counted_workspace_bytes(M, RANK, SPLIT), dtype=torch.uint8,
                                            device=self.dev),
                            cnt=torch.zeros(max(1, dsl.lora_shrink_counter_bytes(M) // 4), dtype=torch.int32,
                                            device=self.dev))
            self.sets.append(s)
        # one arrival-counter buffer serves every call: the calls run one after another
        self.cnt_se = torch.zeros(dsl.lora_shrink_expand_counter_bytes(max(M_LIST)) // 4, dtype=torch.int32,
                                  device=self.dev)
        torch.cuda.synchronize()
        log(f"bench: {self.copies} input copies ({self.copies * per_set / 2**30:.2f} GiB)")

    # -- one call of each variant on one input set ---------------------------
    def det(self, s, M):
        """Deterministic shrink + expand (lora_shrink_expand: one launch for
        small M, two otherwise; the same bits either way)."""
        self.dsl.lora_shrink_expand(s["x"], s["A"], s["B"], s["y"], s["ws"], SPLIT, 1.0, SCALE, h=s["h"])

    def det_two_launch(self, s, M):
        """Split partials, then tree + expand (2 launches)."""
        d = self.dsl
        d.lora_shrink_partials(s["x"], s["A"], s["ws"], SPLIT)
        d.lora_expand_combine(s["ws"], s["B"], s["y"], SPLIT, 1.0, SCALE, h=s["h"])

    def det_counted(self, s, M):
        """Single-launch counted shrink, then expand (2 launches)."""
        d = self.dsl
        d.lora_shrink_splitk_counted(s["x"], s["A"], s["h"], s["cws"], s["cnt"], SPLIT, 1.0)
        d.lora_expand(s["h"], s["B"], s["y"], SCALE)

    def det_counted_one_launch(self, s, M):
        """Shrink and expand in one launch with arrival counters."""
        self.dsl.lora_shrink_expand_counted(s["x"], s["A"], s["B"], s["y"], s["ws"], self.cnt_se, SPLIT, 1.0, SCALE,
                                            h=s["h"])

    def det_one_launch(self, s, M):
        self.dsl.lora_shrink_expand_fused(s["x"], s["A"], s["B"], s["y"], SPLIT, 1.0, SCALE, h=s["h"])

    def det_two_call(self, s, M):
        """Deterministic shrink (partials + tree kernel) then expand (3 launches)."""
        d = self.dsl
        d.lora_shrink_splitk(s["x"], s["A"], s["h"], s["ws"], SPLIT, 1.0)
        d.lora_expand(s["h"], s["B"], s["y"], SCALE)

    def atomic(self, s, M):
        """Atomic contrast: zero fill + atomic partials, then expand (3 launches)."""
        d = self.dsl
        d.lora_shrink_splitk_atomic(s["x"], s["A"], s["h"], SPLIT, 1.0)
        d.lora_expand(s["h"], s["B"], s["y"], SCALE)

    def combine_only(self, s, M):
        self.dsl.lora_expand_combine(s["ws"], s["B"], s["y"], SPLIT, 1.0, SCALE, h=s["h"])

    def capture(self, fn, Ms, per_graph=1):
        """HIP graphs that each run fn(set, M) for M in Ms on `per_graph`
        consecutive input copies; together the graphs cover every copy."""
        t = self.t
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(side):
            for M in Ms:
                fn(self.sets[0][M], M)          # first launch outside capture
        t.cuda.current_stream().wait_stream(side)
        t.cuda.synchronize()
        C = len(self.sets)
        graphs = []
        for c0 in range(0, C, per_graph):
            gr = t.cuda.CUDAGraph()
            with t.cuda.graph(gr):
                for q in range(per_graph):
                    s = self.sets[(c0 + q) % C]
                    for M in Ms:
                        fn(s[M], M)
            graphs.append(gr)
        t.cuda.synchronize()
        return graphs

    def time_graphs(self, graphs, replays, warmup):
        t = self.t
        n = len(graphs)
        # the warm-up replays every graph at least once, so the timed region
        # never meets an input copy (or a graph) for the first time
        for i in range(max(warmup, n)):
            graphs[i % n].replay()
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(replays):
            graphs[i % n].replay()
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / replays          # ms per replay

    def per_call_us(self, fn, Ms, per_graph, calls):
        g = self.capture(fn, Ms, per_graph)
        reps = max(1, calls // per_graph)
        ms = self.time_graphs(g, reps, max(2, self.args.warmup // per_graph))
        del g
        return ms * 1000 / per_graph                  # us per pass over Ms

    def run(self):
        a = self.args
        K, W = a.steps, a.warmup
        res = {}
        # the timed steps: the four batch sizes back to back; each HIP graph
        # holds SPG consecutive steps on SPG input copies, replayed K / SPG
        # times, so exactly K steps run in the timed region
        spg = steps_per_graph(K)
        det_g = self.capture(self.det, M_LIST, spg)
        ms_det = self.time_graphs(det_g, K // spg, max(1, W // spg)) / spg
        del det_g
        res["ms_per_step"] = ms_det
        res["us_per_call"] = ms_det * 1000 / len(M_LIST)
        res["steps_per_graph"] = spg
        res["atomic_us_per_call"] = self.per_call_us(self.atomic, M_LIST, spg, K) / len(M_LIST)
        res["det_two_call_us_per_call"] = self.per_call_us(self.det_two_call, M_LIST, spg, K) / len(M_LIST)
        # per batch size: 8 calls per graph on 8 copies keep graph-launch cost out
        per_m = {}
        for M in M_LIST:
            ud = self.per_call_us(self.det, (M,), 8, K)
            ua = self.per_call_us(self.atomic, (M,), 8, K)
            u3 = self.per_call_us(self.det_two_call, (M,), 8, K)
            u2 = self.per_call_us(self.det_two_launch, (M,), 8, K)
            u1 = self.per_call_us(self.det_one_launch, (M,), 8, K)
            uc = self.per_call_us(self.det_counted, (M,), 8, K)
            uq = self.per_call_us(self.det_counted_one_launch, (M,), 8, K)
            byt = shrink_bytes(M, K_HID, RANK) + expand_bytes(M, RANK, N_OUT)
            log(f"bench: M={M} timed")
            per_m[str(M)] = {"det_us": round(ud, 3), "atomic_us": round(ua, 3),
                             "det_launches": self.dsl.lora_shrink_expand_launches(M, K_HID, RANK, N_OUT, SPLIT),
                             "det_one_launch_us": round(u1, 3), "det_two_launch_us": round(u2, 3),
                             "det_three_launch_us": round(u3, 3), "det_counted_shrink_then_expand_us": round(uc, 3),
                             "det_counted_one_launch_us": round(uq, 3),
                             "det_over_atomic": round(ud / ua, 4), "bytes": byt,
                             "workspace_bytes": 8 * SPLIT * M * RANK,
                             "det_GBps": round(byt / ud / 1e3, 1),
                             "det_pct_hbm_peak": round(100 * byt / ud / 1e3 / HBM_PEAK_GBS, 2)}
        res["per_m"] = per_m
        # roofline of the dominant kernel of the step, timed alone over the
        # batch sizes at which the step launches it, 8 launches per graph
        one = tuple(M for M in M_LIST if self.dsl.lora_shrink_expand_launches(M, K_HID, RANK, N_OUT, SPLIT) == 1)
        two = tuple(M for M in M_LIST if M not in one)
        cand = []
        if one:
            us = self.per_call_us(self.det_one_launch, one, 8, K)
            byt = sum(shrink_bytes(M, K_HID, RANK) + expand_bytes(M, RANK, N_OUT) for M in one)
            cand.append((us, len(one), byt, "k_shrink_expand_fused<2,8,8> (lora_shrink_expand_fused: Split-K "
                         "shrink recomputed per 512 columns, fixed trees, expand; r=16, N=4096, M=" +
                         "/".join(map(str, one)) + ")", None))
        if two:
            per = {M: self.per_call_us(self.combine_only, (M,), 8, K) for M in two}
            byt = sum(combine_bytes(M, RANK, N_OUT, SPLIT) for M in two)
            cand.append((sum(per.values()), len(two), byt, COMBINE_KERNEL + " (fixed tree over the Split-K "
                         "workspace + expand; M=" + "/".join(map(str, two)) + ")",
                         {str(M): round(u, 3) for M, u in per.items()}))
        res["roofline"] = pick_roofline(cand, lambda name: recorded_traffic(COMBINE_KERNEL, two)
                                        if name.startswith(COMBINE_KERNEL) else None)
        return res


def hot_step(args):
    """The step on 8 input copies that stay in the 256 MB Infinity Cache
    (warm cache) instead of >= 1 GiB of rotating copies: deterministic and
    atomic us per call, beside the cold-cache headline."""
    b = Bench(args, copies=8)
    spg = steps_per_graph(args.steps)
    det = b.per_call_us(b.det, M_LIST, spg, args.steps) / len(M_LIST)
    atom = b.per_call_us(b.atomic, M_LIST, spg, args.steps) / len(M_LIST)
    mb = 8 * b.per_set / 1e6
    del b
    return {"det_us_per_call": round(det, 3), "atomic_us_per_call": round(atom, 3),
            "det_over_atomic": round(det / atom, 4), "inputs": f"8 copies of the step's inputs ({mb:.0f} MB)"}


def pick_roofline(cand, traffic_for):
    """The roofline object for the dominant kernel of the step.  `cand` holds
    one (total us, launches, total algorithmic bytes, kernel name, per-M us or
    None) tuple per kernel the step launches; the one with the most time is
    the dominant kernel; achieved = its algorithmic bytes per launch over its
    mean launch time; traffic_for(name) gives the counter-based HBM bytes per
    launch, or None."""
    us, n, byt, name, per = max(cand, key=lambda c: c[0])
    avg_launch_us = us / n
    avg_bytes = byt / n
    ach = avg_bytes / avg_launch_us / 1e3
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_for(name),
            "avg_launch_us": round(avg_launch_us, 3), "launch_us_per_m": per,
            "algorithmic_bytes_per_launch": avg_bytes,
            "timing": "HIP events over graphs of 8 back-to-back launches: a launch's time includes "
                      "the gap to the next dispatch"}


COMBINE_KERNEL = "k_expand_combine<1,8>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_expand_combine_qproj_r16_s8_traffic.md")
KERNEL_SOURCES = ["deterministic_split_lora_amd/csrc/expand.hip", "deterministic_split_lora_amd/csrc/device.h",
                  "deterministic_split_lora_amd/csrc/kernels.h"]


def kernel_source_hash():
    """sha256 over the sources the tree + expand kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, Ms):
    """HBM bytes per launch of `kernel`, averaged over batch sizes Ms, from the
    hardware-counter summary under profiles/ (FETCH_SIZE + WRITE_SIZE, each
    scaled by the factor a plain copy of known size gives).  None when there is
    no summary or the kernel's sources have changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("source_hash:"):
                rec["hash"] = line.split(":", 1)[1].strip()
            elif line.startswith("hbm_bytes M="):
                k, v = line[len("hbm_bytes M="):].split(":")
                rec[int(k)] = float(v)
    if rec.get("hash") != kernel_source_hash() or not all(M in rec for M in Ms):
        return None
    return round(sum(rec[M] for M in Ms) / len(Ms), 1)


def counter_pass(args):
    """Driver for hardware-counter runs (rocprofv3 --pmc): the deterministic
    step at every batch size on 8 distinct input copies, eagerly, then four
    copies of 64 MiB (the plain copy of known size the counters are scaled by)."""
    import torch
    b = Bench(args, copies=8)
    for c in range(8):
        for M in M_LIST:
            b.det(b.sets[c][M], M)
    torch.cuda.synchronize()
    n = (64 << 20) // 2
    src = [torch.ones(n, dtype=torch.bfloat16, device=b.dev) for _ in range(4)]
    dst = [torch.empty_like(t) for t in src]
    torch.cuda.synchronize()
    for a, d in zip(src, dst):
        d.copy_(a)
    torch.cuda.synchronize()
    log("bench: counter pass done")


def copy_roofline(args, nbytes_list):
    """Device-to-device copy of known sizes on rotating buffers (>= 1 GiB), HIP
    graphs + events: the practical bandwidth ceiling at these sizes, and the
    plain copy of known size the hardware byte counters are calibrated with."""
    import torch
    dev = torch.device("cuda:0")
    out = {}
    for nb in nbytes_list:
        n = nb // 2
        copies = max(2, math.ceil(ROTATE_BYTES / (2 * nb)))
        src = [torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(copies)]
        dst = [torch.empty_like(t) for t in src]
        sets = [dict(s=a, d=b) for a, b in zip(src, dst)]

        def call(st):
            st["d"].copy_(st["s"])
        us = _time_rotating(call, sets, args)
        out[str(nb)] = {"us": round(us, 3), "GBps_read_plus_write": round(2 * nb / us / 1e3, 1),
                        "pct_hbm_peak": round(100 * 2 * nb / us / 1e3 / HBM_PEAK_GBS, 2)}
        del src, dst, sets
        torch.cuda.empty_cache()
    return out


def launch_floor(args):
    """Per-launch floor on this GPU and stream, timed like everything else
    (8 launches per HIP graph): an empty kernel, and a one-workgroup kernel
    that writes 64 bytes."""
    import torch
    tiny = [torch.zeros(16, dtype=torch.float32, device="cuda") for _ in range(8)]
    sets = [dict(t=t) for t in tiny]
    empty = _time_rotating(lambda st: torch.cuda._sleep(0), sets, args)
    one_wg = _time_rotating(lambda st: st["t"].zero_(), sets, args)
    return {"empty_kernel_us": round(empty, 3), "one_workgroup_kernel_us": round(one_wg, 3)}


def replay_variability(args, repeats=1000):
    """Identical-input replay (the pages' experiment that finds 97.61% of
    atomic Split-K=8 shrink comparisons differing): at the q_proj shape, each
    batch size's shrink is launched `repeats` times on the same inputs, the
    deterministic pipeline and the atomic contrast alike, and every launch's
    fp32 h (and the bf16 y its expand produces) is compared bit for bit with
    the first launch's.  Reported: fraction of comparisons with any differing
    element, fraction of differing elements, mean and max |difference| over
    the differing elements, distinct outputs."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import single_adapter_case
    dev = torch.device("cuda:0")
    out = {"workload": f"q_proj shape (K={K_HID}, r={RANK}, N={N_OUT}, Split-K {SPLIT}, scale {SCALE}), "
                       f"{repeats} launches per batch size on identical inputs, each compared with launch 0"}

    def stats(H, ref):
        """H: [n, ...] outputs as raw bits; ref: the same as values (float64)."""
        n = H.shape[0]
        flat = H.reshape(n, -1)
        diff = flat[1:] != flat[0:1]
        per = diff.any(dim=1)
        vals = ref.reshape(n, -1)
        ad = (vals[1:] - vals[0:1]).abs()[diff]
        return {"comparisons": n - 1, "differing_comparisons": int(per.sum()),
                "differing_comparisons_pct": round(100.0 * float(per.float().mean()), 2),
                "differing_elements_pct": round(100.0 * float(diff.float().mean()), 4),
                "mean_abs_diff": float(ad.mean()) if ad.numel() else 0.0,
                "max_abs_diff": float(ad.max()) if ad.numel() else 0.0,
                "distinct_outputs": distinct(flat)}

    def distinct(flat):
        """Distinct rows, by a 64-bit multiplicative hash of each row's bits."""
        g = torch.Generator(device=flat.device).manual_seed(1)
        w = torch.randint(1, 2 ** 62, (flat.shape[1],), generator=g, device=flat.device, dtype=torch.int64) | 1
        hsh = (flat.to(torch.int64) * w).sum(dim=1)
        return int(torch.unique(hsh).numel())

    for M in M_LIST:
        c = single_adapter_case(M, K_HID, RANK, N_OUT, SPLIT, SCALE, seed=0)
        x, A, B, y0 = (gpu_tensor(a, dev) for a in (c.x, c.A, c.B, c.y))
        ws = torch.empty(dsl.lora_shrink_workspace_bytes(M, RANK, SPLIT), dtype=torch.uint8, device=dev)
        row = {}
        for name in ("deterministic", "atomic"):
            H = torch.empty((repeats, M, RANK), dtype=torch.float32, device=dev)
            Y = torch.empty((repeats, M, N_OUT), dtype=torch.bfloat16, device=dev)
            for i in range(repeats):
                if name == "atomic":
                    dsl.lora_shrink_splitk_atomic(x, A, H[i], SPLIT, 1.0)
                else:
                    dsl.lora_shrink_splitk(x, A, H[i], ws, SPLIT, 1.0)
                Y[i].copy_(y0)
                dsl.lora_expand(H[i], B, Y[i], SCALE)
            torch.cuda.synchronize()
            row[name] = {"h_fp32": stats(H.view(torch.int32), H.double()),
                         "y_bf16": stats(Y.view(torch.int16), Y.double())}
            del H, Y
        out[f"M={M}"] = row
    return out


def gpu_tensor(a, dev):
    return torch_from_bf16(a).to(dev)


def torch_from_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def shrink_only_bench(args):
    """The shrink alone at the small correctness shape (M=8, K=1024, r=8,
    Split-K 8, scale 1): deterministic two launches (partials, tree),
    deterministic single launch (arrival counters) and atomic (fill + atomic
    partials)."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import single_adapter_case
    M, K, r, S = 8, 1024, 8, 8
    c = single_adapter_case(M, K, r, 0, split_k=S, scale=1.0, seed=0)
    dev = torch.device("cuda:0")
    per = 2 * M * K + 2 * K * r
    copies = max(8, math.ceil(ROTATE_BYTES / 64 / per))
    sets = [dict(x=gpu_tensor(c.x, dev), A=gpu_tensor(c.A, dev),
                 h=torch.empty((M, r), dtype=torch.float32, device=dev),
                 ws=torch.empty(dsl.lora_shrink_workspace_bytes(M, r, S), dtype=torch.uint8, device=dev),
                 cws=torch.zeros(dsl.lora_counted_workspace_bytes(M, r, S), dtype=torch.uint8, device=dev))
            for _ in range(copies)]
    cnt = torch.zeros(dsl.lora_shrink_counter_bytes(M) // 4, dtype=torch.int32, device=dev)
    out = {"workload": "shrink only: x [8 x 1024], A [8 x 1024] bf16, Split-K 8, scale 1",
           "bytes": shrink_bytes(M, K, r), "copies": copies}
    calls = {
        "det_two_launch": lambda st: dsl.lora_shrink_splitk(st["x"], st["A"], st["h"], st["ws"], S, 1.0),
        "det_one_launch": lambda st: dsl.lora_shrink_splitk_counted(st["x"], st["A"], st["h"], st["cws"], cnt, S,
                                                                    1.0),
        "atomic": lambda st: dsl.lora_shrink_splitk_atomic(st["x"], st["A"], st["h"], S, 1.0),
    }
    for name, call in calls.items():
        out[name + "_us"] = round(_time_rotating(call, sets, args), 3)
    out["det_over_atomic"] = round(min(out["det_two_launch_us"], out["det_one_launch_us"]) / out["atomic_us"], 4)
    return out


def batch_sweep_bench(args):
    """Deterministic shrink + expand vs the atomic contrast for batch sizes
    1 .. 1024 at the MLP down-projection shape (K=14336, r=32, N=4096,
    Split-K 8, scale 2): the cost of a plan that never depends on M."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import single_adapter_case
    K, r, N, S, Mmax = 14336, 32, 4096, 8, 1024
    c = single_adapter_case(Mmax, K, r, N, split_k=S, seed=0)
    dev = torch.device("cuda:0")
    per = 2 * Mmax * K + 2 * Mmax * N + 4 * K * r
    copies = max(8, math.ceil(ROTATE_BYTES / per))
    base = dict(x=gpu_tensor(c.x, dev), A=gpu_tensor(c.A, dev), B=gpu_tensor(c.B, dev), y=gpu_tensor(c.y, dev))
    sets = [dict({k: v.clone() for k, v in base.items()},
                 h=torch.empty((Mmax, r), dtype=torch.float32, device=dev),
                 ws=torch.empty(dsl.lora_shrink_expand_workspace_bytes(Mmax, r, S), dtype=torch.uint8, device=dev))
            for _ in range(copies)]
    del base
    out = {"workload": "x [b x 14336], A [32 x 14336], B [4096 x 32], y [b x 4096] bf16, Split-K 8, scale 2",
           "copies": copies, "points": {}}
    b = 1
    while b <= Mmax:
        def det(st, b=b):
            dsl.lora_shrink_expand(st["x"][:b], st["A"], st["B"], st["y"][:b], st["ws"], S, 1.0, SCALE,
                                   h=st["h"][:b])

        def atomic(st, b=b):
            dsl.lora_shrink_splitk_atomic(st["x"][:b], st["A"], st["h"][:b], S, 1.0)
            dsl.lora_expand(st["h"][:b], st["B"], st["y"][:b], SCALE)
        ud = _time_rotating(det, sets, args)
        ua = _time_rotating(atomic, sets, args)
        byt = shrink_bytes(b, K, r) + expand_bytes(b, r, N)
        out["points"][str(b)] = {"det_us": round(ud, 3), "atomic_us": round(ua, 3),
                                 "det_over_atomic": round(ud / ua, 4), "bytes": byt,
                                 "det_pct_hbm_peak": round(100 * byt / ud / 1e3 / HBM_PEAK_GBS, 2)}
        b *= 2
    return out


def split_sweep_bench(args):
    """Split count S in {1, 2, 4, 8, 16}:
    - the one-token decode shrink over three fused QKV slices (hidden 3072,
      rank 16 per slice; the slices' A rows stacked into one rank-48 operand,
      so each slice is its own 16-wide output tile: 3 x S workgroups) -
      deterministic two launches, deterministic single launch, atomic;
    - deterministic shrink + expand at the q_proj shape (M = 1, 16, 256) and
      at the MLP down-projection shape (K=14336, r=32; M = 1, 16, 256)."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import single_adapter_case
    dev = torch.device("cuda:0")
    splits = (1, 2, 4, 8, 16)
    out = {"splits": list(splits)}
    # fused QKV decode shrink
    K, r = 3072, 48
    c = single_adapter_case(1, K, r, 0, split_k=8, scale=1.0, seed=0)
    copies = 256
    sets = [dict(x=gpu_tensor(c.x, dev), A=gpu_tensor(c.A, dev), h=torch.empty((1, r), device=dev),
                 ws=torch.empty(dsl.lora_shrink_workspace_bytes(1, r, 16), dtype=torch.uint8, device=dev),
                 cws=torch.zeros(dsl.lora_counted_workspace_bytes(1, r, 16), dtype=torch.uint8, device=dev))
            for _ in range(copies)]
    cnt = torch.zeros(dsl.lora_shrink_counter_bytes(1) // 4, dtype=torch.int32, device=dev)
    qkv = {"workload": "decode shrink, 1 token, hidden 3072, 3 fused QKV slices of rank 16 (A stacked: r = 48)"}
    for S in splits:
        row = {}
        row["det_two_launch_us"] = round(_time_rotating(
            lambda st, S=S: dsl.lora_shrink_splitk(st["x"], st["A"], st["h"], st["ws"], S, 1.0), sets, args), 3)
        row["det_one_launch_us"] = round(_time_rotating(
            lambda st, S=S: dsl.lora_shrink_splitk_counted(st["x"], st["A"], st["h"], st["cws"], cnt, S, 1.0), sets,
            args), 3)
        row["atomic_us"] = round(_time_rotating(
            lambda st, S=S: dsl.lora_shrink_splitk_atomic(st["x"], st["A"], st["h"], S, 1.0), sets, args), 3)
        row["workgroups"] = 3 * S
        qkv[str(S)] = row
    best1 = min(qkv["1"]["det_two_launch_us"], qkv["1"]["det_one_launch_us"])
    for S in splits:
        b = min(qkv[str(S)]["det_two_launch_us"], qkv[str(S)]["det_one_launch_us"])
        qkv[str(S)]["det_speedup_vs_split1"] = round(best1 / b, 3)
    out["decode_qkv_shrink"] = qkv
    del sets
    # shrink + expand at two shapes
    for label, K, r, N in (("q_proj_k4096_r16_n4096", 4096, 16, 4096), ("down_k14336_r32_n4096", 14336, 32, 4096)):
        tab = {}
        for M in (1, 16, 256):
            cc = single_adapter_case(M, K, r, N, split_k=8, seed=0)
            per = 2 * M * K + 4 * M * N + 4 * K * r
            copies = max(8, math.ceil(ROTATE_BYTES / 4 / per))
            sets = [dict(x=gpu_tensor(cc.x, dev), A=gpu_tensor(cc.A, dev), B=gpu_tensor(cc.B, dev),
                         y=gpu_tensor(cc.y, dev), h=torch.empty((M, r), device=dev),
                         ws=torch.empty(dsl.lora_shrink_expand_workspace_bytes(M, r, 16), dtype=torch.uint8,
                                        device=dev))
                    for _ in range(copies)]
            tab[str(M)] = {str(S): round(_time_rotating(
                lambda st, S=S: dsl.lora_shrink_expand(st["x"], st["A"], st["B"], st["y"], st["ws"], S, 1.0, SCALE,
                                                       h=st["h"]), sets, args), 3) for S in splits}
            del sets
        out[label + "_det_us"] = tab
    torch.cuda.empty_cache()
    return out


def compensated_bench(args):
    """lora_expand vs lora_expand_compensated (two matrix-core passes, hi and
    lo of h) at N = 4096, r = 16 and 64, M = 1, 256, 4096: the cost of
    consuming 16 instead of 8 significant bits of h."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import normal_bf16
    dev = torch.device("cuda:0")
    out = {"workload": "expand only: h fp32 [M x r], B [4096 x r], y [M x 4096] bf16, scale 2"}
    N = 4096
    for r in (16, 64):
        for M in (1, 256, 4096):
            per = 4 * M * N + 2 * N * r + 4 * M * r
            copies = max(8, math.ceil(ROTATE_BYTES / 4 / per))
            Bm = gpu_tensor(normal_bf16((N, r), 0.02, 0, "cbB"), dev)
            y0 = gpu_tensor(normal_bf16((M, N), 1.0, 0, "cby"), dev)
            sets = [dict(h=torch.randn((M, r), device=dev) * 0.5, B=Bm.clone(), y=y0.clone()) for _ in range(copies)]
            up = _time_rotating(lambda st: dsl.lora_expand(st["h"], st["B"], st["y"], SCALE), sets, args)
            uc = _time_rotating(lambda st: dsl.lora_expand_compensated(st["h"], st["B"], st["y"], SCALE), sets, args)
            out[f"r{r}_m{M}"] = {"plain_us": round(up, 3), "compensated_us": round(uc, 3),
                                 "ratio": round(uc / up, 3), "bytes": per}
            del sets
    torch.cuda.empty_cache()
    return out


def sgmv_bench(args, label, M, K, N, ranks, seg_lo, seg_hi, S, replays=100, ids=None):
    """Multi-adapter shrink and expand on a prebuilt plan, cold cache.
    Compulsory bytes count only the adapters some token uses, at their own
    rank: shrink 2MK + 2K sum(r) + 4 M r_max (h), expand 4 sum_i r_(a_i) (h)
    + 2N sum(r) + 4 M' N (y read and written for the M' tokens with an
    adapter)."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import sgmv_case
    c = sgmv_case(M, K, N, ranks, seg_lo, seg_hi, S, seed=0, tag=label, ids=ids)
    dev = torch.device("cuda:0")
    n = len(c.ranks)
    valid = (c.ids >= 0) & (c.ids < n)
    touched = sorted(set(int(a) for a in c.ids[valid]))
    sum_r = sum(int(c.ranks[a]) for a in touched)
    sh_bytes = 2 * M * K + 2 * K * sum_r + 4 * M * c.r_max
    ex_bytes = 4 * int(sum(int(c.ranks[a]) for a in c.ids[valid])) + 2 * N * sum_r + 4 * int(valid.sum()) * N
    # each variant rotates over >= 1 GiB of its own operands: the shrink's
    # (x, A) and the expand's (y, B, h) copies are counted separately
    copies_sh = max(2, math.ceil(ROTATE_BYTES / sh_bytes))
    copies_ex = max(2, math.ceil(ROTATE_BYTES / ex_bytes))
    copies = max(copies_sh, copies_ex)
    base_x, base_y = gpu_tensor(c.x, dev), gpu_tensor(c.y, dev)
    base_A = [gpu_tensor(a, dev) for a in c.As]
    base_B = [gpu_tensor(b, dev) for b in c.Bs]
    ranks_g = torch.from_numpy(c.ranks).to(dev)
    scales_g = torch.from_numpy(c.scales).to(dev)
    ids_g = torch.from_numpy(c.ids).to(dev)
    plan = torch.empty(dsl.lora_sgmv_plan_bytes(M), dtype=torch.uint8, device=dev)
    dsl.lora_sgmv_plan(ids_g, n, plan)
    cnt = torch.zeros(dsl.lora_sgmv_counter_bytes(M) // 4, dtype=torch.int32, device=dev)
    xs = [base_x] + [base_x.clone() for _ in range(copies_sh - 1)]
    Ass = [base_A] + [[a.clone() for a in base_A] for _ in range(copies_sh - 1)]
    ys = [base_y] + [base_y.clone() for _ in range(copies_ex - 1)]
    Bss = [base_B] + [[b.clone() for b in base_B] for _ in range(copies_ex - 1)]
    hs = [torch.empty((M, c.r_max), dtype=torch.float32, device=dev) for _ in range(copies_ex)]
    sets = []
    for i in range(copies):
        As, Bs = Ass[i % copies_sh], Bss[i % copies_ex]
        sets.append(dict(x=xs[i % copies_sh], y=ys[i % copies_ex], A=As, B=Bs,
                         Ap=torch.tensor([a.data_ptr() for a in As], dtype=torch.int64, device=dev),
                         Bp=torch.tensor([b.data_ptr() for b in Bs], dtype=torch.int64, device=dev),
                         h=hs[i % copies_ex],
                         ws=torch.empty(dsl.lora_sgmv_workspace_bytes(M, c.r_max, S), dtype=torch.uint8,
                                        device=dev),
                         cws=torch.zeros(dsl.lora_counted_workspace_bytes(M, c.r_max, S), dtype=torch.uint8,
                                         device=dev)))
    torch.cuda.synchronize()

    def shrink(st):
        dsl.lora_sgmv_shrink(st["x"], st["Ap"], K, ranks_g, None, ids_g, n, plan, st["h"], c.r_max, S, st["ws"])

    def shrink_counted(st):
        dsl.lora_sgmv_shrink_counted(st["x"], st["Ap"], K, ranks_g, None, n, plan, st["h"], c.r_max, S,
                                     st["cws"], cnt)

    def expand(st):
        dsl.lora_sgmv_expand(st["h"], st["Bp"], ranks_g, scales_g, ids_g, n, st["y"], c.r_max)

    def both(st):
        shrink(st)
        expand(st)

    def pipeline(st):
        dsl.lora_sgmv_shrink_expand(st["x"], st["Ap"], K, st["Bp"], ranks_g, None, scales_g, ids_g, n, plan, st["y"],
                                    c.r_max, S, st["ws"], h=st["h"])

    def plan_only(st):
        dsl.lora_sgmv_plan(ids_g, n, plan)

    def atomic_shrink(st):
        dsl.lora_sgmv_shrink_atomic(st["x"], st["Ap"], K, ranks_g, None, n, plan, st["h"], c.r_max, S)

    def atomic_both(st):
        atomic_shrink(st)
        expand(st)

    layout = (f"segments {seg_lo}..{seg_hi} tokens" if ids is None
              else "ids drawn per token (interleaved, as decode tokens of many requests)")
    out = {"workload": f"M={M}, K={K}, N={N}, {n} adapters of ranks {sorted(set(int(v) for v in c.ranks))}, "
                       f"{layout}, Split-K {S}",
           "segments": len(c.segs), "touched_adapters": len(touched), "shrink_bytes": sh_bytes,
           "expand_bytes": ex_bytes, "workspace_bytes": 8 * S * M * c.r_max,
           "copies": {"x_A": copies_sh, "y_B_h": copies_ex}}
    for name, call, byt in (("shrink", shrink, sh_bytes), ("shrink_one_launch", shrink_counted, sh_bytes),
                            ("expand", expand, ex_bytes), ("shrink_expand", both, sh_bytes + ex_bytes),
                            ("shrink_expand_pipeline", pipeline, sh_bytes + ex_bytes),
                            ("atomic_shrink", atomic_shrink, sh_bytes),
                            ("atomic_shrink_expand", atomic_both, sh_bytes + ex_bytes),
                            ("plan", plan_only, 0)):
        us = _time_rotating(call, sets, args)
        out[name] = {"us": round(us, 3)}
        if byt:
            out[name]["GBps"] = round(byt / us / 1e3, 1)
            out[name]["pct_hbm_peak"] = round(100 * byt / us / 1e3 / HBM_PEAK_GBS, 2)
    out["det_over_atomic"] = round(out["shrink_expand_pipeline"]["us"] / out["atomic_shrink_expand"]["us"], 4)
    out["det_shrink_over_atomic_shrink"] = round(out["shrink"]["us"] / out["atomic_shrink"]["us"], 4)
    st0 = sets[0]
    del sets
    torch.cuda.empty_cache()
    out["replay"] = sgmv_replay(st0, pipeline, atomic_both, replays)
    return out


def _row_hashes(flat):
    """64-bit multiplicative hash of each row of an integer tensor's bits."""
    import torch
    g = torch.Generator(device=flat.device).manual_seed(1)
    w = torch.randint(1, 2 ** 62, (flat.shape[1],), generator=g, device=flat.device, dtype=torch.int64) | 1
    return (flat.to(torch.int64) * w).sum(dim=1)


def sgmv_replay(st, det_call, atomic_call, repeats):
    """Identical-input replay of a multi-adapter shrink + expand: each variant
    runs `repeats` times on the same inputs (y restored before every call);
    h is compared bit for bit with the first call's, y by a 64-bit hash of its
    bits.  Reported per variant: calls whose h (or y) differs from the first."""
    import torch
    y0 = st["y"].clone()
    out = {"repeats": repeats}
    for name, call in (("deterministic", det_call), ("atomic", atomic_call)):
        h_first = y_first = None
        dh = dy = 0
        hashes = []
        for i in range(repeats):
            st["y"].copy_(y0)
            call(st)
            hb = st["h"].view(torch.int32)
            yh = _row_hashes(st["y"].view(torch.int16).reshape(1, -1))
            if h_first is None:
                h_first, y_first = hb.clone(), yh.clone()
            else:
                dh += int(not torch.equal(hb, h_first))
                dy += int(not torch.equal(yh, y_first))
            hashes.append(_row_hashes(hb.reshape(1, -1)))
        torch.cuda.synchronize()
        out[name] = {"h_differs": dh, "y_differs": dy, "distinct_h": int(torch.unique(torch.cat(hashes)).numel())}
    st["y"].copy_(y0)
    torch.cuda.synchronize()
    return out


def decode_probe(args, M=32, mixed=False):
    """M decode tokens, each with its own adapter, hidden 8192, Split-K 8: the
    multi-adapter deterministic shrink (partials + fixed tree) on a prebuilt
    plan, cold cache, against the atomic contrast (zero h + the same partial
    kernel with fp32 atomic adds).  Adapters of rank 64, or with `mixed` the
    prefill workload's pool (ranks cycling 8, 16, 32, 64).  Algorithmic bytes:
    x, every adapter's A once at its own rank, h at each token's rank."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import normal_bf16
    dev = torch.device("cuda:0")
    K, S, n = 8192, 8, M
    rk = [(8, 16, 32, 64)[a % 4] if mixed else 64 for a in range(n)]
    r = max(rk)

    def g(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    x = normal_bf16((M, K), 1.0, 0, "probe_x")
    As = [normal_bf16((rk[a], K), 0.02, 0, f"probe_A{a}") for a in range(n)]
    byt = 2 * M * K + 2 * K * sum(rk) + 4 * sum(rk)
    copies = 1 if args.hot else max(2, math.ceil(ROTATE_BYTES / byt))
    ids = torch.arange(M, dtype=torch.int32, device=dev)
    ranks = torch.tensor(rk, dtype=torch.int32, device=dev)
    plan = torch.empty(dsl.lora_sgmv_plan_bytes(M), dtype=torch.uint8, device=dev)
    dsl.lora_sgmv_plan(ids, n, plan)
    sets = []
    for c in range(copies):
        Ag = [g(a) for a in As]
        sets.append(dict(x=g(x), A=Ag, Ap=torch.tensor([t.data_ptr() for t in Ag], dtype=torch.int64, device=dev),
                         h=torch.empty((M, r), dtype=torch.float32, device=dev),
                         ws=torch.empty(dsl.lora_sgmv_workspace_bytes(M, r, S), dtype=torch.uint8, device=dev),
                         cws=torch.zeros(dsl.lora_counted_workspace_bytes(M, r, S), dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()

    cnt = torch.zeros(dsl.lora_sgmv_counter_bytes(M) // 4, dtype=torch.int32, device=dev)

    def two_launch(s):
        dsl.lora_sgmv_shrink(s["x"], s["Ap"], K, ranks, None, ids, n, plan, s["h"], r, S, s["ws"])

    def counted(s):
        dsl.lora_sgmv_shrink_counted(s["x"], s["Ap"], K, ranks, None, n, plan, s["h"], r, S, s["cws"], cnt)

    def atomic(s):
        dsl.lora_sgmv_shrink_atomic(s["x"], s["Ap"], K, ranks, None, n, plan, s["h"], r, S)

    pool = "ranks cycling 8, 16, 32, 64" if mixed else "rank 64"
    out = {"workload": f"{M} tokens x hidden 8192, {M} adapters of {pool} (one per token), Split-K 8, "
                       "multi-adapter deterministic shrink", "bytes": byt, "copies": copies}
    for name, call in (("two_launch", two_launch), ("single_launch", counted), ("atomic", atomic)):
        us = _time_rotating(call, sets, args)
        out[name] = {"us_per_call": round(us, 3), "GBps": round(byt / us / 1e3, 1),
                     "pct_hbm_peak": round(100 * byt / us / 1e3 / HBM_PEAK_GBS, 2)}
    best = min(out["two_launch"]["us_per_call"], out["single_launch"]["us_per_call"])
    out["best_pct_hbm_peak"] = round(100 * byt / best / 1e3 / HBM_PEAK_GBS, 2)
    out["det_over_atomic"] = round(best / out["atomic"]["us_per_call"], 4)
    return out


def decode_expand_probe(args, M=32, N=4096):
    """Multi-tenant decode, expand side: M tokens, each with its own rank-64
    adapter (hidden 8192, N = 4096 outputs, Split-K 8), cold cache: the
    multi-adapter expand alone (h given), and the whole deterministic
    shrink + expand (lora_sgmv_shrink_expand: partials, then the expand that
    evaluates the fixed tree).  Algorithmic bytes: every adapter's B once, h,
    y read and written (expand); plus x and every adapter's A (pipeline)."""
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import normal_bf16
    dev = torch.device("cuda:0")
    K, r, S, n = 8192, 64, 8, M

    def g(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    x = normal_bf16((M, K), 1.0, 1, "dprobe_x")
    y = normal_bf16((M, N), 1.0, 1, "dprobe_y")
    As = [normal_bf16((r, K), 0.02, 1, f"dprobe_A{a}") for a in range(n)]
    Bs = [normal_bf16((N, r), 0.02, 1, f"dprobe_B{a}") for a in range(n)]
    ex_bytes = 2 * r * N * n + 4 * M * N + 4 * M * r
    sh_bytes = 2 * M * K + 2 * K * r * n + 4 * M * r
    copies = 1 if args.hot else max(2, math.ceil(ROTATE_BYTES / (ex_bytes + sh_bytes)))
    ids = torch.arange(M, dtype=torch.int32, device=dev)
    ranks = torch.full((n,), r, dtype=torch.int32, device=dev)
    scales = torch.full((n,), SCALE, dtype=torch.float32, device=dev)
    plan = torch.empty(dsl.lora_sgmv_plan_bytes(M), dtype=torch.uint8, device=dev)
    dsl.lora_sgmv_plan(ids, n, plan)
    h0 = torch.randn(M, r, device=dev)
    sets = []
    for c in range(copies):
        Ag, Bg = [g(a) for a in As], [g(b) for b in Bs]
        sets.append(dict(x=g(x), y=g(y), A=Ag, B=Bg, h=h0.clone(),
                         Ap=torch.tensor([t.data_ptr() for t in Ag], dtype=torch.int64, device=dev),
                         Bp=torch.tensor([t.data_ptr() for t in Bg], dtype=torch.int64, device=dev),
                         ws=torch.empty(dsl.lora_sgmv_workspace_bytes(M, r, S), dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()

    def expand(s):
        dsl.lora_sgmv_expand(s["h"], s["Bp"], ranks, scales, ids, n, s["y"], r)

    def pipeline(s):
        dsl.lora_sgmv_shrink_expand(s["x"], s["Ap"], K, s["Bp"], ranks, None, scales, ids, n, plan, s["y"], r, S,
                                    s["ws"])

    out = {"workload": f"{M} tokens, {M} adapters of rank 64 (one per token), hidden 8192 -> N = {N}, "
                       "Split-K 8, multi-adapter deterministic expand and shrink + expand",
           "expand_bytes": ex_bytes, "pipeline_bytes": ex_bytes + sh_bytes, "copies": copies}
    for name, call, byt in (("expand", expand, ex_bytes), ("shrink_expand", pipeline, ex_bytes + sh_bytes)):
        us = _time_rotating(call, sets, args)
        out[name] = {"us_per_call": round(us, 3), "GBps": round(byt / us / 1e3, 1),
                     "pct_hbm_peak": round(100 * byt / us / 1e3 / HBM_PEAK_GBS, 2)}
    return out


def _time_rotating(call, sets, args):
    """us per call: 8 calls on 8 input copies per HIP graph, graphs replayed.
    Under --counters: two eager calls, no timing (returns NaN)."""
    import torch
    copies = len(sets)
    call(sets[0])
    torch.cuda.synchronize()
    if getattr(args, "counters", False):
        call(sets[1 % copies])
        torch.cuda.synchronize()
        return float("nan")
    per_graph = 8
    graphs = []
    for c0 in range(0, copies, per_graph):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for q in range(per_graph):
                call(sets[(c0 + q) % copies])
        graphs.append(gr)
    for i in range(max(2, args.warmup // per_graph, len(graphs))):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    replays = max(args.steps // per_graph, 8)
    e0.record()
    for i in range(replays):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000 / (replays * per_graph)


def _oracle_steps(seconds: float):
    """Full steps of the CPU oracle (four batch sizes, shrink + expand each)
    for about `seconds`: (steps, elapsed seconds, threads used)."""
    import oracle
    from synth import single_adapter_case
    cases = {M: single_adapter_case(M, K_HID, RANK, N_OUT, SPLIT, SCALE, seed=0) for M in M_LIST}
    n = 0
    t0 = time.perf_counter()
    while True:
        for M, c in cases.items():
            h = oracle.shrink(c.x, c.A, 1.0)
            oracle.expand(h.astype(np.float32), c.B, c.y, SCALE)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return n, el, oracle.num_threads()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_cpu(fn, seconds):
    """Calls of fn for about `seconds` (at least one): (calls, elapsed s)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def _cpu_config_cases():
    """The oracle's work per config, as (name, sample description, callable,
    rows computed per call, rows of the config's call)."""
    import oracle
    from synth import single_adapter_case, normal_bf16, sgmv_case
    out = []
    c1 = single_adapter_case(8, 1024, 8, 0, split_k=8, scale=1.0, seed=0)
    out.append(("small_m8_k1024_r8", "whole call (fp64 shrink)", lambda: oracle.shrink(c1.x, c1.A, 1.0), 8, 8))
    c3 = sgmv_case(512, 4096, 6144, [64] * 4, 1, 64, 8, seed=0, tag="b3")

    def f3():
        h = oracle.sgmv_shrink(c3.x, c3.As, c3.ranks, None, c3.ids, c3.r_max)
        oracle.sgmv_expand(h.astype(np.float32), c3.Bs, c3.ranks, c3.scales, c3.ids, c3.y)
    out.append(("sgmv_m512_k4096_n6144_4x_r64", "whole call (fp64 multi-adapter shrink + expand)", f3, 512, 512))
    K4, r4, N4 = 14336, 32, 4096
    probe = normal_bf16((16, K4), 1.0, 0, "probe_x")
    A4 = normal_bf16((r4, K4), 0.02, 0, "probe_A")
    B4 = normal_bf16((N4, r4), 0.02, 0, "probe_B")
    y4 = normal_bf16((16, N4), 1.0, 0, "probe_y")

    def f4():
        h = oracle.shrink(probe, A4, 1.0)
        oracle.expand(h.astype(np.float32), B4, y4, SCALE)
    out.append(("down_k14336_r32_n4096_probe_rows", "the 16 probe rows of the batch sweep (shrink + expand)",
                f4, 16, 16))
    c5 = sgmv_case(4096, 8192, 28672, [8, 16, 32, 64] * 8, 32, 512, 16, seed=0, tag="b5")
    rows = np.arange(0, 4096, 32)
    x5, ids5, y5 = c5.x[rows], c5.ids[rows], c5.y[rows]

    def f5():
        h = oracle.sgmv_shrink(x5, c5.As, c5.ranks, None, ids5, c5.r_max)
        oracle.sgmv_expand(h.astype(np.float32), c5.Bs, c5.ranks, c5.scales, ids5, y5)
    out.append(("sgmv_prefill_m4096_k8192_n28672", "every 32nd token (128 of 4096; shrink + expand), "
                "scaled to the whole call", f5, len(rows), 4096))
    return out


def cpu_baseline(seconds: float):
    """The CPU oracle (fp64 C, OpenMP over rows) on the same workloads: the
    bench's step (q_proj shape, four batch sizes) timed for about `seconds`
    with the host's thread setting and for a third of that on one thread (set
    through the OpenMP runtime in this process, then restored); then each
    other config's call (sampled rows where the whole call would take long)
    for about `seconds` / 8 per thread setting, scaled to the whole call."""
    import oracle
    n, el, threads = _oracle_steps(seconds)
    prev = oracle.set_threads(1)
    try:
        n1, el1, threads1 = _oracle_steps(seconds / 3)
    finally:
        oracle.set_threads(prev)
    sample = "full steps (M = 1, 16, 64, 256; fp64 shrink + expand each)"
    configs = {}
    for name, what, fn, rows, rows_full in _cpu_config_cases():
        row = {"sample": what}
        for label, th in (("all_threads", threads), ("one_thread", 1)):
            p = oracle.set_threads(th)
            try:
                fn()                                   # warm
                calls, t = _time_cpu(fn, seconds / 8)
            finally:
                oracle.set_threads(p)
            row[label + "_us_per_call"] = round(t / calls * 1e6 * rows_full / rows, 1)
        configs[name] = row
    return {"value": round(el / (n * len(M_LIST)) * 1e6, 1), "unit": "us/call", "cores": threads,
            "kind": "oracle", "sample": f"{n} {sample} in {el:.1f} s",
            "one_thread": {"value": round(el1 / (n1 * len(M_LIST)) * 1e6, 1), "unit": "us/call",
                           "cores": threads1, "sample": f"{n1} {sample} in {el1:.1f} s"},
            "configs": configs, "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}


def _sha256_files(paths):
    import hashlib
    h = hashlib.sha256()
    for f in paths:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def provenance(b):
    """Where and on what the numbers were taken, and the bitwise evidence:
    SHA-256 of the headline's seeded inputs and of its deterministic outputs
    (h fp32 bits and y bf16 bits after one call per batch size on fresh
    copies), which any run of the same library on the same inputs reproduces."""
    import hashlib
    import subprocess
    import torch
    import deterministic_split_lora_amd as dsl
    from synth import single_adapter_case
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as fh:
            rocm = fh.read().strip()
    except OSError:
        pass
    git = None
    try:
        git = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except Exception:
        pass
    if git is None:
        # a copy of the tree without its history: the revision the library was built from
        try:
            with open(os.path.join(os.path.dirname(dsl.LIBRARY_PATH), "build_revision.txt")) as f:
                git = f.read().strip() or None
        except OSError:
            pass
    srcs = sorted(os.path.join("deterministic_split_lora_amd", "csrc", f)
                  for f in os.listdir(os.path.join(ROOT, "deterministic_split_lora_amd", "csrc")))
    hin, hout = hashlib.sha256(), hashlib.sha256()
    dev = torch.device("cuda:0")
    for M in M_LIST:
        c = single_adapter_case(M, K_HID, RANK, N_OUT, SPLIT, SCALE, seed=0)
        for a in (c.x, c.A, c.B, c.y):
            hin.update(np.ascontiguousarray(a).tobytes())
        x, A, B, y = (gpu_tensor(a, dev) for a in (c.x, c.A, c.B, c.y))
        h = torch.empty((M, RANK), dtype=torch.float32, device=dev)
        ws = torch.empty(dsl.lora_shrink_expand_workspace_bytes(M, RANK, SPLIT), dtype=torch.uint8, device=dev)
        dsl.lora_shrink_expand(x, A, B, y, ws, SPLIT, 1.0, SCALE, h=h)
        torch.cuda.synchronize()
        hout.update(h.view(torch.int32).cpu().numpy().tobytes())
        hout.update(y.view(torch.int16).cpu().numpy().tobytes())
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "hbm_gib": round(props.total_memory / 2 ** 30, 1), "torch": torch.__version__, "hip": torch.version.hip,
            "rocm": rocm, "git": git, "library_sha256": _sha256_files([os.path.relpath(dsl.LIBRARY_PATH, ROOT)]),
            "sources_sha256": _sha256_files(srcs + ["include/lora_det.h"]), "seed": 0,
            "headline_inputs_sha256": hin.hexdigest(), "headline_outputs_sha256": hout.hexdigest()}


# Workloads bench.py can time on their own (--only).
ONLY = {
    "replay": replay_variability,
    "sgmv_qkv": lambda a: sgmv_bench(a, "b3", 512, 4096, 6144, [64] * 4, 1, 64, 8, replays=200),
    "sgmv_interleaved": lambda a: sgmv_bench(a, "b3i", 512, 4096, 6144, [64] * 4, 0, 0, 8, replays=50,
                                             ids=np.random.default_rng(7).integers(0, 4, 512).astype(np.int32)),
    "sgmv_prefill": lambda a: sgmv_bench(a, "b5", 4096, 8192, 28672, [8, 16, 32, 64] * 8, 32, 512, 16,
                                         replays=50),
    "decode_probe": lambda a: decode_probe(a, 128),
    "decode_probe32": lambda a: decode_probe(a, 32),
    "decode_probe32_mixed": lambda a: decode_probe(a, 32, mixed=True),
    "decode_expand": lambda a: {"32": decode_expand_probe(a, 32), "128": decode_expand_probe(a, 128)},
    "batch_sweep": batch_sweep_bench,
    "compensated": compensated_bench,
    "small_shrink": shrink_only_bench,
    "split_sweep": split_sweep_bench,
}


def _r(v, nd=3):
    return None if v is None else round(float(v), nd)


def summarize(res, extra, probe, mixed, wide, dexp, roof, floor, replay):
    """The compact view of every measurement, small enough for one stored
    JSON line: per-config det and atomic microseconds per call with their
    ratio and HBM share, the decode probes, replay and ceiling figures."""
    out = {}
    out["per_m"] = {M: {"det_us": v["det_us"], "atomic_us": v["atomic_us"], "det_over_atomic": v["det_over_atomic"],
                        "launches": v["det_launches"], "pct_hbm_peak": v["det_pct_hbm_peak"]}
                    for M, v in res["per_m"].items()}
    cfg = {}
    if extra:
        so = extra["shrink_only_m8_k1024_r8"]
        cfg["small_m8_k1024_r8_shrink"] = {"det_us": so["det_two_launch_us"], "det_one_launch_us": so["det_one_launch_us"],
                                           "atomic_us": so["atomic_us"], "det_over_atomic": so["det_over_atomic"]}
        for key, name in (("sgmv_m512_k4096_n6144_4x_r64", "sgmv_m512_k4096_n6144_4x_r64"),
                          ("sgmv_m512_k4096_n6144_4x_r64_interleaved", "sgmv_m512_k4096_n6144_4x_r64_interleaved"),
                          ("sgmv_prefill_m4096_k8192_n28672_32_adapters", "sgmv_prefill_m4096_k8192_n28672")):
            e = extra[key]
            rp = e["replay"]
            cfg[name] = {"det_us": e["shrink_expand_pipeline"]["us"], "atomic_us": e["atomic_shrink_expand"]["us"],
                         "det_over_atomic": e["det_over_atomic"],
                         "pct_hbm_peak": e["shrink_expand_pipeline"]["pct_hbm_peak"],
                         "shrink_us": e["shrink"]["us"], "shrink_pct": e["shrink"]["pct_hbm_peak"],
                         "atomic_shrink_us": e["atomic_shrink"]["us"],
                         "shrink_one_launch_us": e["shrink_one_launch"]["us"],
                         "expand_us": e["expand"]["us"], "expand_pct": e["expand"]["pct_hbm_peak"],
                         "plan_us": e["plan"]["us"],
                         "replay": f"{rp['repeats']} calls: det h/y differ {rp['deterministic']['h_differs']}/"
                                   f"{rp['deterministic']['y_differs']}, atomic {rp['atomic']['h_differs']}/"
                                   f"{rp['atomic']['y_differs']} ({rp['atomic']['distinct_h']} distinct h)"}
        sw = extra["batch_sweep_k14336_r32_n4096"]["points"]
        cfg["down_k14336_r32_n4096_batch_sweep"] = {
            "b": {b: [v["det_us"], v["atomic_us"]] for b, v in sw.items()},
            "columns": "det_us, atomic_us",
            "det_over_atomic_max": max(v["det_over_atomic"] for v in sw.values()),
            "pct_hbm_peak_b1024": sw["1024"]["det_pct_hbm_peak"]}
        qkv = extra["split_sweep"]["decode_qkv_shrink"]
        cfg["decode_qkv_m1_k3072_3x_r16_split_sweep"] = {
            S: [qkv[S]["det_two_launch_us"], qkv[S]["det_one_launch_us"], qkv[S]["atomic_us"]]
            for S in ("1", "2", "4", "8", "16")}
        cfg["decode_qkv_m1_k3072_3x_r16_split_sweep"]["columns"] = "det two launches, det one launch, atomic (us)"
        comp = extra["compensated_expand"]
        cfg["compensated_expand_ratio"] = {k: v["ratio"] for k, v in comp.items() if isinstance(v, dict)}
    out["configs"] = cfg
    if probe:
        out["decode_probe"] = {
            M: {"bytes": p_["bytes"], "us": min(p_["two_launch"]["us_per_call"],
                                                                      p_["single_launch"]["us_per_call"]),
                                     "two_launch_us": p_["two_launch"]["us_per_call"],
                                     "single_launch_us": p_["single_launch"]["us_per_call"],
                                     "atomic_us": p_["atomic"]["us_per_call"],
                                     "det_over_atomic": p_["det_over_atomic"],
                                     "pct_hbm_peak": p_["best_pct_hbm_peak"]}
            for M, p_ in (("m32", probe), ("m32_mixed_ranks", mixed), ("m128", wide))}
        out["decode_expand_probe"] = {m: {"expand_us": v["expand"]["us_per_call"],
                                          "expand_pct": v["expand"]["pct_hbm_peak"],
                                          "shrink_expand_us": v["shrink_expand"]["us_per_call"],
                                          "shrink_expand_pct": v["shrink_expand"]["pct_hbm_peak"]}
                                      for m, v in dexp.items()}
        out["copy_ceiling_pct"] = {k: v["pct_hbm_peak"] for k, v in roof.items()}
        out["launch_floor_us"] = floor
    if replay:
        rs = {}
        for M in M_LIST:
            r = replay[f"M={M}"]
            rs[str(M)] = {"det_h": r["deterministic"]["h_fp32"]["differing_comparisons"],
                          "det_y": r["deterministic"]["y_bf16"]["differing_comparisons"],
                          "atomic_h": r["atomic"]["h_fp32"]["differing_comparisons"],
                          "atomic_y": r["atomic"]["y_bf16"]["differing_comparisons"],
                          "atomic_distinct_h": r["atomic"]["h_fp32"]["distinct_outputs"]}
        out["replay_q_proj"] = {"calls_per_m": 1000, "differing_of_999": rs}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--hot", action="store_true", help="no input rotation (inputs may sit in cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other shapes (sweep, multi-adapter)")
    ap.add_argument("--detail", help="also write every measurement, in full, to this JSON file")
    ap.add_argument("--only", choices=sorted(ONLY),
                    help="time one workload and print its JSON only (a target for a profiler run)")
    ap.add_argument("--counters", action="store_true",
                    help="only run the step eagerly for a hardware-counter profile; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the deterministic shrink/expand needs no collective; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.counters:
        if args.only:
            ONLY[args.only](args)             # eager calls, no timing (see _time_rotating)
        else:
            counter_pass(args)
        return
    if args.only:
        print(json.dumps({args.only: ONLY[args.only](args)}), flush=True)
        return
    b = Bench(args)
    res = b.run()
    log("bench: main timing done")
    hot = hot_step(args)
    log("bench: hot-cache step done")
    prov = provenance(b)
    probe = wide = mixed = roof = floor = extra = replay = dexp = None
    if not args.no_probe:
        probe = decode_probe(args, 32)
        mixed = decode_probe(args, 32, mixed=True)
        wide = decode_probe(args, 128)
        dexp = {"32": decode_expand_probe(args, 32), "128": decode_expand_probe(args, 128)}
        avg = int(res["roofline"]["algorithmic_bytes_per_launch"]) // 2 // 16 * 16
        roof = copy_roofline(args, [avg, probe["bytes"], wide["bytes"], 64 << 20])
        floor = launch_floor(args)
        log("bench: probes done")
        replay = replay_variability(args)
        log("bench: replay variability done")
    if not args.no_configs:
        extra = {"shrink_only_m8_k1024_r8": shrink_only_bench(args)}
        log("bench: shrink-only shape done")
        extra["batch_sweep_k14336_r32_n4096"] = batch_sweep_bench(args)
        log("bench: batch sweep done")
        extra["split_sweep"] = split_sweep_bench(args)
        log("bench: split sweep done")
        extra["compensated_expand"] = compensated_bench(args)
        log("bench: compensated expand done")
        extra["sgmv_m512_k4096_n6144_4x_r64"] = ONLY["sgmv_qkv"](args)
        extra["sgmv_m512_k4096_n6144_4x_r64_interleaved"] = ONLY["sgmv_interleaved"](args)
        log("bench: sgmv 512 done")
        extra["sgmv_prefill_m4096_k8192_n28672_32_adapters"] = ONLY["sgmv_prefill"](args)
        log("bench: sgmv prefill done")
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    log("bench: cpu baseline done")
    summary = summarize(res, extra, probe, mixed, wide, dexp, roof, floor, replay)
    out = {
        "metric": METRIC,
        "value": round(res["us_per_call"], 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "q_proj LoRA (8B Llama-3): x [M x 4096], A [16 x 4096], B [4096 x 16], y bf16, "
                               "s 2, Split-K 8, M 1/16/64/256",
                   "cache": "hot" if args.hot else f"cold ({b.copies} rotating copies, >= 1 GiB)",
                   "steps_per_graph": res["steps_per_graph"],
                   "det": "lora_shrink_expand", "atomic": "fill + atomic partials + lora_expand"},
        "det_over_atomic": round(res["us_per_call"] / res["atomic_us_per_call"], 4),
        "atomic_us_per_call": round(res["atomic_us_per_call"], 3),
        "det_three_launch_us_per_call": round(res["det_two_call_us_per_call"], 3),
        "hot_cache": hot,
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "provenance": prov,
    }
    out.update(summary)
    if args.detail:
        detail = dict(out, per_m_detail=res["per_m"], decode_bandwidth_probe=probe, decode_bandwidth_probe_mixed=mixed,
                      decode_bandwidth_probe_wide=wide,
                      decode_expand_probe_detail=dexp, copy_roofline=roof, replay_variability=replay,
                      other_shapes=extra)
        os.makedirs(os.path.dirname(os.path.abspath(args.detail)), exist_ok=True)
        with open(args.detail, "w") as fh:
            json.dump(detail, fh, indent=1)
    print(json.dumps(out, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
