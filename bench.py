"""Benchmark of MLA speculative-decoding verify attention on one MI355X.

Prints ONE JSON line on stdout (everything else goes to stderr).

Step = one verify call through the C ABI (plan + split kernel + combine
kernel) over one batch of seeded synthetic inputs already resident in HBM.
The headline workload is one tensor-parallel rank's share at long context:
batch 1, q_len 9 draft queries, H=8 heads, prefix 65536, bf16 latent cache
in a page_size=1 pool of 2x the tokens addressed through a random-permutation
slot table, causal draft mask. Timing is cold-cache: consecutive calls rotate
over disjoint copies of the cache (> 1 GiB in total) so neither the 4 MiB L2s
nor the 256 MiB Infinity Cache hold the next call's rows.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3_64k]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-attn µs/call + achieved TB/s & MFMA % (q_len 9, H=8/64, 16k-64k prefix)"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_64k")
    ap.add_argument("--nsplit", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--copies", type=int, default=0, help="rotation copies (0 = enough for > 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", default="c3_16k,sweep_16384,sweep_65536",
                    help="comma-separated workloads also timed (cold, warm, graph replay) and reported in the "
                         "same JSON line under 'secondary'; empty to skip")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--op", default="verify", choices=["verify", "append", "topk", "absorb"],
                    help="append: time the draft-KV append (mla_append_kv) for the workload's shape instead; "
                         "topk: time the top-k selection (mla_topk_select) feeding a sparse workload; "
                         "absorb: time the weight absorptions (mla_absorb_q + mla_project_o) for its rows")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def describe(w):
    if w.kind == "sparse":
        return (f"{w.name}: batch {w.batch}, q_len {w.q_len}, H {w.heads}, prefix {w.meta['prefix']}, "
                f"fp8 e4m3 latent + bf16 rope, top-k {w.meta['topk']}, page_size=1 random slots")
    pre = w.meta["prefixes"]
    pre_s = str(pre[0]) if len(set(pre)) == 1 else f"{min(pre)}..{max(pre)}"
    return (f"{w.name}: batch {w.batch}, q_len {w.q_len}, H {w.heads}, prefix {pre_s}, bf16 latent, "
            f"page_size=1 {LAYOUT_WORDS[w.meta['layout']]} slots, {w.mask} mask")


LAYOUT_WORDS = {"random": "random", "contiguous": "contiguous",
                "sorted": "sorted (random free rows handed out in ascending order)"}


def _replicate(host, copies, dtype=None):
    """One device tensor holding `copies` back-to-back copies of a host array."""
    import numpy as np
    import torch

    base = torch.from_numpy(np.ascontiguousarray(host))
    if dtype is not None:
        base = base.view(dtype)
    base = base.to("cuda")
    out = torch.empty((copies * base.shape[0],) + tuple(base.shape[1:]), dtype=base.dtype, device="cuda")
    for c in range(copies):
        out[c * base.shape[0]:(c + 1) * base.shape[0]].copy_(base)
    return out


class Rotation:
    """`copies` disjoint device copies of one workload's cache, each addressed by its own slot table."""

    def __init__(self, w, copies, nsplit, stage_list=("both", "split", "combine")):
        import numpy as np
        import torch

        from mla_speculative_decode_verify_amd import binding as B

        dev = "cuda"
        self.w = w
        rows = w.pool_rows
        self.q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        self.seq = torch.from_numpy(w.seq_lens).to(dev)
        self.slots = [torch.from_numpy((w.slot_table.astype(np.int64) + c * rows).astype(np.int32)).to(dev)
                      for c in range(copies)]
        self.out = torch.empty((w.batch, w.q_len, w.heads, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((w.batch, w.q_len, w.heads), dtype=torch.float32, device=dev)
        self.calls = {}
        if w.kind == "verify":
            self.pool = _replicate(w.pool_bits.view(np.int16), copies, torch.bfloat16)
            self.anc = None
            if w.mask == "tree":
                self.anc = B.build_tree_mask(torch.from_numpy(w.parents).to(dev))
            for stage in stage_list:
                self.calls[stage] = [B.PreparedCall(self.q, kv=self.pool, slot_table=s, seq_lens=self.seq,
                                                    sm_scale=w.sm_scale, mask=w.mask, tree_anc=self.anc,
                                                    out=self.out, lse=self.lse, nsplit=nsplit, stage=stage)
                                     for s in self.slots]
            p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, nsplit=nsplit, mask=w.mask)
        else:
            self.lat = _replicate(w.lat_bits, copies)
            self.rope = _replicate(w.rope_bits.view(np.int16), copies, torch.bfloat16)
            self.scale = _replicate(w.scale, copies)
            self.topk = torch.from_numpy(w.topk_idx).to(dev)
            for stage in stage_list:
                self.calls[stage] = [B.PreparedCall(self.q, latent=self.lat, rope=self.rope, scale=self.scale,
                                                    slot_table=s, seq_lens=self.seq, sm_scale=w.sm_scale,
                                                    topk_idx=self.topk, out=self.out, lse=self.lse,
                                                    nsplit=nsplit, stage=stage)
                                     for s in self.slots]
            p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, kv_dtype=B.MLA_KV_FP8_E4M3, mask="topk",
                       topk=w.meta["topk"], nsplit=nsplit)
        self.plan = p
        B.reserve_workspace(p["workspace_bytes"])


def time_calls(calls, steps, warmup, rotate=True):
    """Average µs per call over `steps` calls (events on torch's current stream)."""
    import torch

    n = len(calls)
    for i in range(warmup):
        calls[i % n if rotate else 0]()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        calls[i % n if rotate else 0]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


class TimingEvent:
    """A HIP event used for timing only, created with hipEventDisableSystemFence: recording it performs no
    system-scope fence, i.e. no L2 write-back and invalidation between the kernels it separates (a default
    event does one, which adds about 3 µs to each kernel it brackets). Called through the HIP runtime that
    torch has loaded (same soname)."""

    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes

            import torch  # noqa: F401  (loads the HIP runtime first)

            lib = ctypes.CDLL("libamdhip64.so.7")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes

        self.h = ctypes.c_void_p()
        if self.lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self.lib().hipEventRecord(self.h, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end):
        import ctypes

        ms = ctypes.c_float()
        if self.lib().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._lib is not None and self.h:
            self._lib.hipEventDestroy(self.h)


def time_stages(split_calls, combine_calls, steps, warmup):
    """Average µs of the split kernel and of the merge kernel inside a call: each step runs the split stage and
    then the merge stage of one rotation copy (as one mla_verify_attn call does), with a timing event before,
    between and after them on the stream the calls run on (torch's current stream). Every step is enqueued
    behind a GPU sleep, so the host's launch gaps never fall between two events; these are the per-dispatch
    durations a kernel trace reports. Without a merge (nsplit 1) the second figure is 0."""
    import torch

    n = len(split_calls)
    for i in range(warmup):
        split_calls[i % n]()
        if combine_calls:
            combine_calls[i % n]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    torch.cuda._sleep(int(1e5) * steps)  # ~40 µs of GPU time (shader clock) per step queued behind it
    for i in range(steps):
        ev[i][0].record(stream)
        split_calls[i % n]()
        ev[i][1].record(stream)
        if combine_calls:
            combine_calls[i % n]()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    split = sum(e[0].elapsed_ms(e[1]) for e in ev) * 1e3 / steps
    merge = sum(e[1].elapsed_ms(e[2]) for e in ev) * 1e3 / steps if combine_calls else 0.0
    return split, merge


def time_graph(rot, steps, warmup):
    """Average µs per call when the calls (one per rotation copy, in order) are captured into one HIP
    graph and the graph is replayed: no host launch gaps between the kernels. Events on the replay stream."""
    import torch

    from mla_speculative_decode_verify_amd import binding as B

    calls = rot.calls["both"]
    s = torch.cuda.Stream()
    B.reserve_workspace(rot.plan["workspace_bytes"], stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    reps = max(1, steps // len(calls))
    with torch.cuda.stream(s):
        for _ in range(max(1, warmup // len(calls))):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(calls))
    del g
    torch.cuda.synchronize()
    B.release_workspace(stream=s)
    return us


def measure(w, args, nsplit, copies=0, graph=True):
    """Cold / warm / split-kernel / merge-kernel (and graph-replay) µs per call of workload `w`."""
    from mla_speculative_decode_verify_amd import roofline as RL

    if w.kind == "sparse":
        cnt = RL.sparse_counts(w.batch, w.q_len, w.heads, w.meta["topk"])
        read_bytes = w.batch * w.q_len * w.meta["topk"] * 652
    else:
        cnt = RL.verify_counts(w.q_len, w.heads, w.seq_lens.tolist(), mask=w.mask,
                               parents=None if w.parents is None else w.parents.tolist())
        read_bytes = w.seq_lens.astype("int64").sum() * 1152
    copies = copies or max(2, int(-(-(1 << 30) // int(read_bytes))) + 1)
    log(f"[bench] {describe(w)}; copies {copies}")
    rot = Rotation(w, copies, nsplit)
    plan = rot.plan
    log(f"[bench] plan {plan}")
    r = dict(cnt=cnt, copies=copies, plan=plan)
    r["cold"] = time_calls(rot.calls["both"], args.steps, args.warmup, rotate=True)
    r["warm"] = time_calls(rot.calls["both"], args.steps, args.warmup, rotate=False)
    # the split and merge kernels of a cold call, each timed by its own event pair
    r["split"], r["combine"] = time_stages(rot.calls["split"], rot.calls["combine"] if plan["nsplit"] > 1 else None,
                                           args.steps, args.warmup)
    r["graph"] = time_graph(rot, args.steps, args.warmup) if graph else None
    log(f"[bench] cold {r['cold']:.2f} us/call, warm {r['warm']:.2f}, split kernel {r['split']:.2f}, "
        f"combine {r['combine']:.2f}, graph replay {r['graph']}")
    del rot
    return r


def roofline_entry(w, r):
    """Roofline object: achieved and frac for the whole call (cold µs, as `value`), and the same for the
    split kernel alone (the dominant kernel, whose duration the rocprofv3 summaries give)."""
    from mla_speculative_decode_verify_amd import roofline as RL

    cnt = r["cnt"]
    rf = RL.roofline_us(cnt["flops"], cnt["bytes"])
    hbm = rf["bound"] == "hbm"
    peak = RL.PEAK_HBM_GBPS if hbm else RL.PEAK_BF16_TFLOPS

    def ach(us):
        return cnt["bytes"] / (us * 1e-6) / 1e9 if hbm else cnt["flops"] / (us * 1e-6) / 1e12

    traffic = split_traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        try:
            tr = json.load(open(PROFILE_TRAFFIC))
            key = f"{w.name}/nsplit{r['plan']['nsplit']}"
            if key in tr and tr[key].get("kernel_source_hash") == kernel_hash(w.kind):
                traffic = tr[key]["bytes_per_launch"]
                split_traffic = tr[key].get("split_kernel_bytes")
        except Exception:
            traffic = split_traffic = None
    # traffic: HBM bytes of one call (split + merge kernels, FETCH_SIZE + WRITE_SIZE scaled by a calibration
    # copy, profiles/traffic.json), null once the kernel sources differ from the profiled ones
    return dict(bound=rf["bound"], achieved=round(ach(r["cold"]), 2), peak=peak,
                unit="GB/s" if hbm else "TFLOP/s", frac=round(ach(r["cold"]) / peak, 4), traffic=traffic,
                scope="whole call (split + merge kernels, cold)",
                split_kernel_us=round(r["split"], 3), split_kernel_achieved=round(ach(r["split"]), 2),
                split_kernel_frac=round(ach(r["split"]) / peak, 4), split_kernel_traffic=split_traffic,
                roofline_us=round(rf["us"], 3))


def cpu_baseline(w, reps=3):
    import numpy as np

    from oracle import mla_oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if w.kind == "sparse":
        def run():
            O.sparse_decode_attention(w.q_bits, w.lat_bits, w.rope_bits, w.scale, w.slot_table, w.topk_idx,
                                      w.sm_scale)
    else:
        anc = O.causal_masks(w.batch, w.q_len) if w.mask == "causal" else (
            O.ancestor_masks(w.parents) if w.mask == "tree" else None)

        def run():
            O.verify_attention(w.q_bits, w.pool_bits, w.slot_table, w.seq_lens, anc, w.sm_scale)
    def timed():
        ts = []
        for _ in range(reps):
            t = time.perf_counter()
            run()
            ts.append(time.perf_counter() - t)
        return statistics.median(ts) * 1e6

    out = dict(value=timed(), unit="us/call", cores=int(threads), kind="oracle",
               sample=f"the full {w.name} call (all {w.batch * w.q_len * w.heads} query rows), median of {reps}",
               cpu_model=cpu_model(), os_cpu_count=os.cpu_count())
    if w.name in ("c1", "c2", "c3_16k", "c3_64k"):
        # the same oracle with its BLAS limited to one thread
        try:
            from threadpoolctl import threadpool_limits

            with threadpool_limits(limits=1):
                out["one_thread_us"] = timed()
        except Exception:  # pragma: no cover
            out["one_thread_us"] = None
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from mla_speculative_decode_verify_amd import binding as B
    from mla_speculative_decode_verify_amd import inputs as I
    from mla_speculative_decode_verify_amd import roofline as RL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.lib()
    w = I.workload(args.workload)
    if args.op == "append":
        bench_append(args, w)
        return
    if args.op == "topk":
        bench_topk(args, w)
        return
    if args.op == "absorb":
        bench_absorb(args, w)
        return
    r = measure(w, args, args.nsplit, args.copies, graph=not args.no_graph)
    cnt, plan, cold, warm, copies = r["cnt"], r["plan"], r["cold"], r["warm"], r["copies"]
    split_us, comb_us = r["split"], r["combine"]
    rf = RL.roofline_us(cnt["flops"], cnt["bytes"])
    roof = roofline_entry(w, r)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(w)
        cpu["gpu_speedup"] = round(cpu["value"] / cold, 1)
        log(f"[bench] oracle {cpu['value']:.0f} us/call on {cpu['cores']} threads "
            f"(one thread: {cpu.get('one_thread_us')}), {cpu['gpu_speedup']}x the GPU call")
    secondary = {}
    names = [n for n in args.secondary.split(",") if n and n != w.name] if args.op == "verify" else []
    for name in names:
        torch.cuda.empty_cache()
        w2 = I.workload(name)
        r2 = measure(w2, args, 0, 0, graph=not args.no_graph)
        secondary[name] = {
            "workload": describe(w2), "us_per_call": round(r2["cold"], 3), "warm_us": round(r2["warm"], 3),
            "graph_us": None if r2["graph"] is None else round(r2["graph"], 3),
            "kernels_us": {"split": round(r2["split"], 3), "combine": round(r2["combine"], 3)},
            "nsplit": r2["plan"]["nsplit"], "row_blocks": r2["plan"]["row_blocks"],
            "row_groups": r2["plan"]["row_groups"],
            "algorithmic": {"bytes": r2["cnt"]["bytes"], "flops": r2["cnt"]["flops"]},
            "achieved_TBps": round(r2["cnt"]["bytes"] / (r2["cold"] * 1e-6) / 1e12, 4),
            "achieved_TFLOPs": round(r2["cnt"]["flops"] / (r2["cold"] * 1e-6) / 1e12, 3),
            "roofline": roofline_entry(w2, r2),
        }
        del w2, r2
    line = {
        "metric": METRIC,
        "value": round(cold, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kind == "verify" else "fp8-e4m3 cache, bf16 MFMA",
        "data": ("synthetic: seeded N(0,1) bf16 queries and latent rows, random page_size=1 slot permutation"
                 if w.kind == "verify" else
                 "synthetic: seeded N(0,1) bf16 queries, N(0,1) latent rounded to fp8 e4m3, bf16 rope, "
                 "scales U[0.5,2], top-k positions drawn without replacement, random page_size=1 slots"),
        "config": {"workload": describe(w), "batch": w.batch, "q_len": w.q_len, "heads": w.heads,
                   "prefix": (w.meta["prefix"] if w.kind == "sparse" else
                              w.meta["prefixes"][0] if len(set(w.meta["prefixes"])) == 1 else w.meta["prefixes"]),
                   "nsplit": plan["nsplit"], "balanced_splits": bool(plan["balanced"]),
                   "waves_per_group": plan["waves_per_group"],
                   "row_groups": plan["row_groups"], "grid": plan["grid"], "cold_copies": copies},
        "warm_us": round(warm, 3),
        "graph_us": None if r["graph"] is None else round(r["graph"], 3),
        "kernels_us": {"split": round(split_us, 3), "combine": round(comb_us, 3)},
        "achieved_TBps": round(cnt["bytes"] / (cold * 1e-6) / 1e12, 4),
        "achieved_TFLOPs": round(cnt["flops"] / (cold * 1e-6) / 1e12, 3),
        "mfma_frac_of_peak": round(cnt["flops"] / (cold * 1e-6) / 1e12 / RL.PEAK_BF16_TFLOPS, 5),
        "roofline_us": round(rf["us"], 3),
        "algorithmic": {"bytes": cnt["bytes"], "flops": cnt["flops"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "gpu": gpu_info(),
    }
    print(json.dumps(line), flush=True)


def gpu_info():
    """Device name, architecture and CU count as the runtime reports them."""
    import torch

    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count}


def bench_append(args, w):
    """One JSON line for the draft-KV append of the workload's batch x q_len rows into its pool."""
    import numpy as np
    import torch

    from mla_speculative_decode_verify_amd import binding as B

    assert w.kind == "verify", "the append writes a bf16 pool"
    rng = np.random.default_rng(77)
    new = rng.integers(0, 0x7F00, size=(w.batch, w.q_len, 576)).astype(np.uint16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    kv = dev(w.pool_bits.view(np.int16)).view(torch.bfloat16)
    new_t = dev(new.view(np.int16)).view(torch.bfloat16)
    slots, lens = dev(w.slot_table), dev(w.seq_lens)
    B.append_kv(kv, new_t, slots, lens)  # validates the arguments once
    L = B.lib()
    cargs = (kv.data_ptr(), int(kv.shape[0]), int(slots.shape[1]), new_t.data_ptr(), w.batch, w.q_len,
             slots.data_ptr(), lens.data_ptr(), int(torch.cuda.current_stream().cuda_stream))
    call = lambda: L.mla_append_kv(*cargs)  # noqa: E731  (no per-call Python validation)
    us = time_calls([call], args.steps, args.warmup, rotate=False)
    rows = w.batch * w.q_len
    nbytes = rows * 1152 * 2 + rows * 4 + w.batch * 4
    log(f"[bench] append {rows} rows: {us:.2f} us/call")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O

        t = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.append_kv(w.pool_bits, new, w.slot_table, w.seq_lens)
            t.append((time.perf_counter() - t0) * 1e6)
        cpu = {"value": round(statistics.median(t), 1), "unit": "us/call", "cores": 1, "kind": "oracle",
               "sample": "the full append (a copy of the pool plus the row writes), median of 3"}
    ach = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "draft-KV append µs/call", "value": round(us, 3), "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded bf16 bit patterns",
        "config": {"workload": describe(w), "rows": rows},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(ach / 8000.0, 5), "traffic": None},
        "cpu_baseline": cpu}), flush=True)


def bench_topk(args, w):
    """One JSON line for the top-k selection that would feed the sparse workload `w`: one fp32 score per
    prefix position and query, seeded N(0,1), top-k of them."""
    import numpy as np
    import torch

    from mla_speculative_decode_verify_amd import binding as B

    assert w.kind == "sparse", "the top-k selection feeds a sparse workload"
    n, k = int(w.meta["prefix"]), int(w.meta["topk"])
    rng = np.random.default_rng(78)
    scores = rng.standard_normal((w.batch, w.q_len, n)).astype(np.float32)
    lens = np.full(w.batch, n, dtype=np.int32)
    s_t, l_t = torch.from_numpy(scores).cuda(), torch.from_numpy(lens).cuda()
    out = B.topk_select(s_t, l_t, k)  # validates once
    L = B.lib()
    cargs = (s_t.data_ptr(), w.batch, w.q_len, n, l_t.data_ptr(), k, out.data_ptr(),
             int(torch.cuda.current_stream().cuda_stream))
    call = lambda: L.mla_topk_select(*cargs)  # noqa: E731
    us = time_calls([call], args.steps, args.warmup, rotate=False)
    rows = w.batch * w.q_len
    nbytes = rows * n * 4 + rows * k * 4 + w.batch * 4
    log(f"[bench] topk {rows} rows of {n}: {us:.2f} us/call")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O

        t0 = time.perf_counter()
        O.topk_select(scores[:1, :1], lens[:1], k)
        dt = (time.perf_counter() - t0) * 1e6
        cpu = {"value": round(dt * rows, 1), "unit": "us/call", "cores": 1, "kind": "oracle",
               "sample": f"one row of {n} scores, scaled by the {rows} rows of a call"}
    ach = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "top-k selection µs/call", "value": round(us, 3), "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic: seeded N(0,1) fp32 scores",
        "config": {"workload": f"top-{k} of {n} scores, {rows} rows (feeds {w.name})", "rows": rows},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(ach / 8000.0, 5), "traffic": None},
        "cpu_baseline": cpu}), flush=True)


def bench_absorb(args, w):
    """One JSON line for the query absorption plus the value projection of the workload's rows
    (seeded N(0,1) activations, N(0,1)/sqrt(fan-in) weights, per-head widths 128)."""
    import numpy as np
    import torch

    from mla_speculative_decode_verify_amd import binding as B
    from mla_speculative_decode_verify_amd import inputs as I

    T, H = w.batch * w.q_len, w.heads
    rng = np.random.default_rng(79)
    bf = lambda a: torch.from_numpy(I.f32_to_bf16_bits(a.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    qn, qr = bf(rng.standard_normal((T, H, 128))), bf(rng.standard_normal((T, H, 64)))
    w_uk = bf(rng.standard_normal((H, 512, 128)) / 128 ** 0.5)
    w_uv = bf(rng.standard_normal((H, 128, 512)) / 512 ** 0.5)
    o_lat = torch.from_numpy(rng.standard_normal((T, H, 512)).astype(np.float32)).cuda()
    q_out = B.absorb_q(qn, qr, w_uk)
    o_out = B.project_o(o_lat, w_uv)
    L = B.lib()
    st = int(torch.cuda.current_stream().cuda_stream)
    a1 = (qn.data_ptr(), qr.data_ptr(), w_uk.data_ptr(), T, H, q_out.data_ptr(), st)
    a2 = (o_lat.data_ptr(), w_uv.data_ptr(), T, H, o_out.data_ptr(), st)
    us_q = time_calls([lambda: L.mla_absorb_q(*a1)], args.steps, args.warmup, rotate=False)
    us_o = time_calls([lambda: L.mla_project_o(*a2)], args.steps, args.warmup, rotate=False)
    us = us_q + us_o
    nbytes = 2 * H * 512 * 128 * 2 + T * H * (128 * 2 + 64 * 2 + 576 * 2 + 512 * 4 + 128 * 4)
    flops = 2 * 2 * T * H * 512 * 128
    log(f"[bench] absorb {T} rows x {H} heads: q {us_q:.2f} us, o {us_o:.2f} us")
    ach = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "weight absorption µs/call (query + value projection)", "value": round(us, 3), "unit": "us/call",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations, N(0,1)/sqrt(fan-in) weights",
        "config": {"workload": f"{T} rows x {H} heads (rows of {w.name}), per-head widths 128",
                   "kernels_us": {"absorb_q": round(us_q, 3), "project_o": round(us_o, 3)}, "flops": flops},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(ach / 8000.0, 5), "traffic": None},
        "cpu_baseline": None}), flush=True)


KERNEL_SOURCES = {
    "verify": ("split_bf16.hip", "split_common.h", "split_epilogue.h", "device_common.h", "mla_internal.h",
               "combine.hip"),
    "sparse": ("split_fp8.hip", "split_epilogue.h", "device_common.h", "mla_internal.h", "combine.hip"),
}


def kernel_hash(kind="verify"):
    """Hash of the sources the split kernel of this workload kind is built from."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, "mla_speculative_decode_verify_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
