"""Benchmark of the per-decode-step sparse KV assembly path on one MI355X.

A step is one decode step of the whole hot path for every request and layer of
a workload: slot lookup + sparse diff + LRU (diff_lru), then the assembling
launch (assemble: misses fetched from pinned host memory over PCIe, written to
the compute buffer and back to the hot buffer, hits copied within HBM, and the
sparse MLA attention over every row it moves, one partial per workgroup) and
the merge of the partials (combine).  ``--separate`` times the earlier
sequence instead (gather, split-K attention over the complete compute buffer,
combine).  Inputs (host pool rows, Top-K streams, queries) are seeded and
synthetic and are resident (pool in pinned host memory, the rest in HBM)
before any timing.

Prints one JSON line.  The top-level figures are those of the headline
workload (``--workload``, default: 32 requests x 8 layers at 128K context):
``value`` is selected KV tokens gathered per second (B * L * K per decode
step) over exactly ``--steps`` timed steps after ``--warmup`` untimed ones.
``configs`` holds the same measurement protocol for every workload: R replays
of its decode steps, each from freshly freed requests, with the median
steady-state step and the cold first step reported apart, per-kernel times,
the hit copy alone (all-hit steps that cycle two disjoint Top-K sets, with
the working set stated), and a parity check of sampled requests against the
CPU oracle.  ``cpu_baseline`` is the oracle on P host processes.  A failed
parity check prints no speed line and exits 1.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import mmap
import multiprocessing as mp
import os
import statistics
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kvs_workload as W  # noqa: E402

METRIC = "selected KV tokens gathered/sec + decode steps/sec; % of HBM and PCIe peak GB/s"
HEADLINE = "ctx128k_b32_l8_zipf"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
PCIE_PEAK_GBS = 63.0             # PCIe Gen5 x16, one direction: 32 GT/s * 16 * 128/130 / 8
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MALL_BYTES = 256 << 20           # MI355X last-level (Infinity) cache
ROW = W.ROW_BYTES
KERNEL_NAMES = ("diff_lru", "gather", "attention", "combine", "assemble")
# The pages' own figures are system-level (whole models, other hardware and
# serving stacks); none is a figure for this path, so none is compared.
PAGES_CONTEXT = {
    "comparable": False,
    "device_memory_per_request": "8 GB to 200 MB with about 3x single-machine throughput "
                                 "(DeepSeek DSA scenario; SGLang/Tair hierarchical sparse "
                                 "attention summary)",
    "tpot_reduction": "49.25 % at 20 % and 63.58 % at 40 % Top-K miss, GLM-5.3 at 16K context "
                      "and per-GPU batch 192 on NVIDIA B300 decode GPUs, X-Mem against PCIe "
                      "host DRAM (XM-Sparse)",
}


def log(msg):
    print(f"# [{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20, help="timed decode steps (headline)")
    p.add_argument("--warmup", type=int, default=5,
                   help="untimed decode steps before the timed ones (step 0 is cold)")
    p.add_argument("--workload", default=HEADLINE, choices=sorted(W.WORKLOADS),
                   help="headline workload")
    p.add_argument("--configs", default="all",
                   help="comma-separated workloads measured beside the headline, 'all' "
                        "(every other workload) or 'none'")
    p.add_argument("--replays", type=int, default=5,
                   help="timed replays of each workload's decode steps, each from freed requests")
    p.add_argument("--time-budget", type=float, default=480.0,
                   help="seconds after which remaining side workloads are skipped")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle: no CPU baseline and no parity check")
    p.add_argument("--cpu-workers", type=int, default=0,
                   help="oracle processes; 0 = the host cores available, at most 16")
    p.add_argument("--parity-requests", type=int, default=2)
    p.add_argument("--fetch-blocks", type=int, default=0, help="0 = library's choice")
    p.add_argument("--attn-splits", type=int, default=0, help="0 = library's choice")
    p.add_argument("--hit-blocks", type=int, default=0, help="0 = library's choice")
    p.add_argument("--graph", action="store_true",
                   help="headline timed steps as captured HIP graphs (inputs in place)")
    p.add_argument("--hits-first", action="store_true",
                   help="hit-copy workgroups take the first grid indices of the gather")
    p.add_argument("--direct-hot", action="store_true",
                   help="attention reads the selected rows in place from the hot buffer (no "
                        "compute buffer; the gather only fetches misses)")
    p.add_argument("--separate", action="store_true",
                   help="index copy and attention as separate launches (gather, attention over "
                        "the complete compute buffer, merge) instead of one assembling launch")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy three times (the known-size "
                        "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


# ---------------------------------------------------------------- peaks and helpers

def measure_zero_copy_peak(torch, kvs, host, reps=5):
    """Best of `reps` zero-copy reads of up to 1 GiB of a pinned pool by a plain
    GPU read kernel with the fetch's load pattern (the host link's ceiling for
    GPU-initiated reads), timed with events on the stream it runs on."""
    nbytes = min(host.nbytes, 1 << 30) // 16 * 16
    sink = torch.empty(kvs.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    best = 0.0
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        kvs.probe_host_read(host.ptr, nbytes, sink)
        e1.record()
        e1.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    return best


def measure_h2d_peak(torch, nbytes=1 << 30, reps=5) -> float:
    """Best of `reps` hipMemcpyAsync copies of 1 GiB from pinned host memory, GB/s."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        e1.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


def measure_d2d_peak(torch, nbytes=1 << 30, reps=5) -> float:
    """Best of `reps` device-to-device copies of 1 GiB (torch's copy, which the
    runtime runs as its own copy kernel), GB/s counting the read and the write:
    the HBM rate a plain contiguous copy reaches on this GPU."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best = max(best, 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kvs_kernels.hip", "kvs_api.cpp", "kvs_internal.h"):
        with open(os.path.join(ROOT, "token_level_gather_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def parallel_units(fn, wl, threads=16):
    units = [(b, l) for b in range(wl.batch) for l in range(wl.layers)]
    with ThreadPoolExecutor(min(threads, len(units))) as ex:
        list(ex.map(lambda u: fn(*u), units))


def cpu_workers_count(args) -> int:
    if args.cpu_workers > 0:
        return args.cpu_workers
    # the host cores this process may use; a one-GPU share of the host is 16
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------- cpu_baseline leg
# Everything that runs the CPU oracle lives here: the multi-process throughput
# baseline and the oracle replays of sampled requests that the parity check
# compares the GPU results with.  The GPU path never calls the oracle.

def _cpu_worker(rank, wl, pool_rows, job_q, res_q, barrier):
    """Forked oracle process: numpy only, one BLAS thread, never touches the GPU."""
    from threadpoolctl import threadpool_limits

    from oracle import OracleUnit
    with threadpool_limits(limits=1):
        while True:
            job = job_q.get()
            if job is None:
                return
            reqs, steps = job
            units = [(b, l) for b in reqs for l in range(wl.layers)]
            streams = {(b, l): W.unit_topk_stream(wl, b, l, steps) for b, l in units}
            qs = {(l, t): W.queries(wl, l, t) for l in range(wl.layers) for t in range(steps)}
            barrier.wait()
            t0 = time.monotonic()
            for b, l in units:
                u = OracleUnit(wl.context, wl.slots, wl.topk)
                for t in range(steps):
                    u.step(streams[(b, l)][t], pool_rows[b, l], qs[(l, t)][b], wl.scale)
            t1 = time.monotonic()
            res_q.put((rank, t0, t1, len(units) * steps))


class CpuWorkers:
    """P oracle processes forked before the GPU is touched; they read the
    workload's pool rows through a shared mapping that the parent filled."""

    def __init__(self, wl, pool_rows, nproc):
        ctx = mp.get_context("fork")
        self.wl, self.nproc = wl, nproc
        self.barrier = ctx.Barrier(nproc)
        self.res_q = ctx.Queue()
        self.job_qs = [ctx.Queue() for _ in range(nproc)]
        self.procs = [ctx.Process(target=_cpu_worker, daemon=True,
                                  args=(r, wl, pool_rows, self.job_qs[r], self.res_q,
                                        self.barrier)) for r in range(nproc)]
        for p in self.procs:
            p.start()

    def run(self, steps, per_proc=2):
        """Each process replays whole requests (all layers, `steps` steps) through
        the oracle; the first min(B, per_proc * P) requests, split round-robin."""
        wl, P = self.wl, self.nproc
        reqs = list(range(min(wl.batch, per_proc * P)))
        for r in range(P):
            self.job_qs[r].put(([b for b in reqs if b % P == r], steps))
        res = [self.res_q.get(timeout=600) for _ in range(P)]
        t0 = min(x[1] for x in res)
        t1 = max(x[2] for x in res)
        unit_steps = sum(x[3] for x in res)
        busy = [(x[2] - x[1]) / x[3] for x in res if x[3]]
        wall = t1 - t0
        tokens = unit_steps * wl.topk
        units_per_step = wl.batch * wl.layers
        return {
            "value": round(tokens / wall, 1), "unit": "tokens/s", "cores": P, "kind": "oracle",
            "sample": f"oracle replay of requests 0..{len(reqs) - 1} x {wl.layers} layer(s) x "
                      f"{steps} steps of {wl.name} (K={wl.topk}), requests split round-robin "
                      f"over {P} processes, {wall:.2f} s wall, "
                      f"{sum(x[2] - x[1] for x in res):.1f} s of CPU work",
            "oracle_ms_per_decode_step": round(wall / steps * 1e3 * units_per_step
                                               / (unit_steps / steps), 2),
            "one_core_ms_per_unit_step": round(1e3 * statistics.mean(busy), 3),
            "unit_steps": unit_steps,
        }

    def close(self):
        for q in self.job_qs:
            q.put(None)
        for p in self.procs:
            p.join(timeout=30)


def cpu_baseline_oracle_replay(wl, host, topk_np, q_np, reqs, steps):
    """Oracle replay of the sampled requests (every layer, `steps` steps): outputs,
    log-sum-exps and final maps, the reference of the parity check."""
    from threadpoolctl import threadpool_limits

    from oracle import OracleUnit
    rec = {}
    with threadpool_limits(limits=1):
        for b in reqs:
            for l in range(wl.layers):
                u = OracleUnit(wl.context, wl.slots, wl.topk)
                for t in range(steps):
                    r = u.step(topk_np[t, l, b], host[b, l], q_np[t, l, b], wl.scale)
                    rec[(t, l, b)] = (r.out, r.lse)
                rec[("state", l, b)] = (u.tok2slot.copy(), u.slot2tok.copy(),
                                        u.last_used.copy())
    return rec


# ---------------------------------------------------------------- one workload

class Workload:
    """Device inputs, pool and the measurement phases of one workload."""

    def __init__(self, torch, kvs, wl, args, steps_total, shared_rows=None):
        self.torch, self.kvs, self.wl, self.args = torch, kvs, wl, args
        B, L, N, S, K = wl.batch, wl.layers, wl.context, wl.slots, wl.topk
        self.flags = (kvs.KVS_FLAG_HITS_FIRST if args.hits_first else 0) | \
            (kvs.KVS_FLAG_DIRECT_HOT if args.direct_hot else 0) | \
            (kvs.KVS_FLAG_SEPARATE_ATTENTION if args.separate else 0)
        self.pool = kvs.Pool(B, L, N, S, K, scale=wl.scale, attn_splits=args.attn_splits,
                             fetch_blocks=args.fetch_blocks, hit_blocks=args.hit_blocks,
                             flags=self.flags)
        host = self.pool.host.array
        if shared_rows is not None:
            parallel_units(lambda b, l: np.copyto(host[b, l], shared_rows[b, l]), wl)
        else:
            parallel_units(lambda b, l: W.fill_unit_rows(host[b, l], wl, b, l), wl)
        self.T = steps_total
        self.topk_np = W.topk_streams(wl, steps_total)                 # [T][L][B][K]
        self.q_np = np.stack([np.stack([W.queries(wl, l, t) for l in range(L)])
                              for t in range(steps_total)])            # [T][L][B][16][576]
        self.topk = torch.from_numpy(self.topk_np).cuda()
        self.q = torch.from_numpy(self.q_np.view(np.int16)).cuda().view(torch.bfloat16)
        self.out = torch.empty((steps_total, L, B, 16, 512), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((steps_total, L, B, 16), dtype=torch.float32, device="cuda")
        self.graphs = None
        self.last_t = None   # the last step run: its Top-K is all resident afterwards
        # attention partials per request of the assembling launch: hit splits +
        # fetch workgroups per request (the library's rule, restated)
        ntiles = (K + 63) // 64
        fpr = min(ntiles, -(-self.pool.sizes.fetch_blocks // B))
        self.parts = self.pool.sizes.attn_splits + fpr

    def step(self, t):
        for l in range(self.wl.layers):
            self.pool.step(l, self.topk[t, l], self.q[t, l], self.out[t, l], self.lse[t, l])
        self.last_t = t

    def sync_ok(self):
        rc, st = self.pool.sync_status()
        if rc != 0:
            raise RuntimeError(f"{self.wl.name}: device status {self.kvs.strerror(rc)}")
        return st

    def free_all(self):
        for b in range(self.wl.batch):
            self.pool.free_request(b)

    def close(self):
        if self.graphs is not None:
            for row in self.graphs:
                for g in row:
                    g.destroy()
        self.pool.release()
        self.pool.host.free()

    # -- algorithmic bytes of one kvs_step call -------------------------------
    def algorithmic(self, hits_per_call, misses_per_call):
        """Algorithmic bytes (and flops) of one kvs_step call, per kernel.

        gather and assemble are bound by the host link: their roofline bytes
        are the miss rows read over PCIe, their HBM traffic is listed beside
        them (hit rows read; rows written to the compute buffer and, for
        misses, to the victim slots; with rows read in place no compute buffer).
        """
        wl, direct = self.wl, self.args.direct_hot
        B, S, K = wl.batch, wl.slots, wl.topk
        h, m = hits_per_call, misses_per_call
        flop = B * 2 * 16 * K * (576 + 512)
        q_bytes = B * 16 * 576 * 2
        out_bytes = B * 16 * 512 * 2
        part_one = 16 * (512 + 2) * 4
        copy_hbm = ROW * m if direct else 2 * ROW * h + 2 * ROW * m
        alg = {"diff_lru": {"bound": "hbm", "bytes": B * (24 * K + 4 * S) + 40 * m}}
        if self.args.separate:
            splits = self.pool.sizes.attn_splits
            # split partials (written by attention, read by the combine); with one
            # split the attention writes the bf16 output itself and no combine runs
            part = B * splits * part_one if splits > 1 else out_bytes
            alg["gather"] = {"bound": "pcie", "bytes": ROW * m, "hbm_bytes": copy_hbm}
            alg["attention"] = {"bound": "hbm",
                                "bytes": B * K * ROW + q_bytes + part + (4 * B * K if direct
                                                                         else 0),
                                "flop": flop}
            alg["combine"] = {"bound": "hbm",
                              "bytes": part + out_bytes if splits > 1 else 0}
        else:
            part = B * self.parts * part_one
            # hit rows are read once from the hot buffer (and written to the
            # compute buffer); miss rows arrive over PCIe and are written to the
            # victim slot (and the compute buffer); then the partials
            hbm = (ROW * (h + m) if direct else 2 * ROW * (h + m)) + q_bytes + part
            alg["assemble"] = {"bound": "pcie", "bytes": ROW * m, "hbm_bytes": hbm,
                               "flop": flop}
            alg["combine"] = {"bound": "hbm", "bytes": part + out_bytes}
        return alg

    def kernel_stats(self, kt, alg, names, zc_gbs=None):
        res = {}
        calls = max(1, kt["steps"])
        for name in names:
            launches = kt["launches"][name]
            if launches == 0 or name not in alg:
                continue
            a = alg[name]
            per_call = launches / calls
            avg_ms = kt[name] / launches
            b_launch = a["bytes"] / per_call
            gbs = b_launch / (avg_ms * 1e-3) / 1e9 if avg_ms > 0 else 0.0
            peak = PCIE_PEAK_GBS if a["bound"] == "pcie" else HBM_PEAK_GBS
            k = {"avg_ms": round(avg_ms, 5), "launches_per_call": round(per_call, 3),
                 "bound": a["bound"], "bytes_per_launch": int(b_launch),
                 "achieved_gbs": round(gbs, 2), "peak_gbs": peak, "frac": round(gbs / peak, 4)}
            if a["bound"] == "pcie" and zc_gbs:
                k["frac_of_zero_copy_peak"] = round(gbs / zc_gbs, 4)
            if "flop" in a:
                tf = a["flop"] / per_call / (avg_ms * 1e-3) / 1e12 if avg_ms > 0 else 0.0
                k["tflops"] = round(tf, 2)
                k["mfma_frac"] = round(tf / BF16_MFMA_PEAK_TFLOPS, 5)
            if "hbm_bytes" in a:
                k["hbm_bytes_per_launch"] = int(a["hbm_bytes"] / per_call)
                k["hbm_gbs"] = round(a["hbm_bytes"] / per_call / (avg_ms * 1e-3) / 1e9, 2)
            res[name] = k
        return res

    # -- phases ---------------------------------------------------------------
    def contract_run(self, warmup, steps, graph=False):
        """`warmup` untimed steps from a fresh pool (the first is cold), then exactly
        `steps` timed steps bracketed by device synchronisation; HIP events on the
        launch stream bracket the dominant kernel's launches inside the timed region."""
        torch, pool, L = self.torch, self.pool, self.wl.layers
        if graph:
            self.graphs = [[pool.capture(l, self.topk[t, l], self.q[t, l], self.out[t, l],
                                         self.lse[t, l]) for l in range(L)]
                           for t in range(warmup, warmup + steps)]
        cold = None
        dominant = "gather"
        for t in range(warmup):
            probe = t == warmup - 1 and t > 0
            if probe:
                pool.profile_begin(L)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            self.step(t)
            torch.cuda.synchronize()
            if t == 0:
                cold = (time.perf_counter() - t0) * 1e3
            if probe:
                kt = pool.profile_end()
                dominant = max(KERNEL_NAMES, key=lambda k: kt[k])
        st0 = self.sync_ok()
        pool.profile_begin(steps * L, kernels=(dominant,))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(warmup, warmup + steps):
            if graph:
                for g in self.graphs[t - warmup]:
                    g.launch()
            else:
                self.step(t)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        tdom = pool.profile_end()
        st1 = self.sync_ok()
        return {"elapsed": elapsed, "cold_ms": cold, "dominant": dominant, "tdom": tdom,
                "hits": st1.hits - st0.hits, "misses": st1.misses - st0.misses}

    def replays(self, R, steps):
        """R replays of steps 0..steps-1, each from freed requests, every step
        bracketed by events on the launch stream.  Returns per-replay step times."""
        torch = self.torch
        times = []
        for _ in range(R):
            self.free_all()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            ev[0].record()
            for t in range(steps):
                self.step(t)
                ev[t + 1].record()
            ev[-1].synchronize()
            times.append([ev[t].elapsed_time(ev[t + 1]) for t in range(steps)])
        self.sync_ok()
        return times

    def breakdown(self, steps, zc_gbs):
        """One more replay from freed requests; events around every kernel of the
        steady steps 1..steps-1."""
        pool, L = self.pool, self.wl.layers
        self.free_all()
        self.step(0)
        sa = self.sync_ok()
        pool.profile_begin((steps - 1) * L)
        for t in range(1, steps):
            self.step(t)
        self.torch.cuda.synchronize()
        kt = pool.profile_end()
        sb = self.sync_ok()
        calls = (steps - 1) * L
        hits, misses = sb.hits - sa.hits, sb.misses - sa.misses
        alg = self.algorithmic(hits / calls, misses / calls)
        return self.kernel_stats(kt, alg, KERNEL_NAMES, zc_gbs), hits, misses, alg

    def hit_sets(self):
        """Two all-hit Top-K sets per unit after the last step run: A = that
        step's Top-K and B = K other resident tokens (every slot is occupied by
        then, and S >= 2K in every workload).  Every entry of either set is a
        hit, so a copy launch over it moves only HBM rows."""
        torch, pool, wl, t = self.torch, self.pool, self.wl, self.last_t
        B, L, K = wl.batch, wl.layers, wl.topk
        set_a = self.topk[t]                                     # [L][B][K]
        set_b = torch.empty_like(set_a)
        for l in range(L):
            for b in range(B):
                st = pool.read_state(b, l)
                res = st["slot2tok"][st["slot2tok"] >= 0]
                other = np.setdiff1d(res, self.topk_np[t, l, b])
                if other.size < K:
                    return None
                set_b[l, b] = torch.from_numpy(other[:K].astype(np.int32))
        return t, (set_a, set_b)

    def hit_copy(self, sets, pool=None, kname=None, reps=3):
        """The hit copy alone, with a working set well above the 256 MB Infinity
        Cache: the two all-hit sets replayed in turn, layer after layer, so
        between two reads of a hot row come the reads of every other unit's two
        sets.  `pool` / `kname`: the copy launch timed (default: this pool's
        own, the assembling launch, or the gather with separate launches)."""
        if sets is None or self.args.direct_hot:
            return None
        t, sets = sets
        wl = self.wl
        B, L, K = wl.batch, wl.layers, wl.topk
        pool = self.pool if pool is None else pool
        if kname is None:
            kname = "gather" if self.args.separate else "assemble"
        _, sa = pool.sync_status()
        pool.profile_begin(reps * 2 * L, kernels=(kname,))
        for _ in range(reps):
            for tk in sets:
                for l in range(L):
                    pool.step(l, tk[l], self.q[t, l], self.out[t, l], self.lse[t, l])
        kh = pool.profile_end()
        rc, sb = pool.sync_status()
        if rc != 0:
            raise RuntimeError(f"{wl.name}: device status {self.kvs.strerror(rc)}")
        launches = kh["launches"][kname]
        assert launches == reps * 2 * L, launches
        assert sb.misses == sa.misses, "the hit-copy replay fetched rows"
        rows = (sb.hits - sa.hits) / launches
        avg_ms = kh[kname] / launches
        gbs = 2 * ROW * rows / (avg_ms * 1e-3) / 1e9
        working_set = (2 * L * B * K + B * K) * ROW    # both sets' hot rows + the compute buffer
        note = ("two disjoint all-hit Top-K sets per unit replayed in turn over every layer; "
                "working set = both sets' hot rows + the compute buffer")
        if kname == "assemble":
            note += "; the assembling launch also attends over the rows it copies"
        return {"rows_per_launch": int(rows), "bytes_per_launch": int(2 * ROW * rows),
                "avg_ms": round(avg_ms, 5), "achieved_gbs": round(gbs, 1),
                "peak_gbs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
                "working_set_mb": round(working_set / 1e6, 1), "kernel": kname, "note": note}

    def index_copy(self, sets, reps=6):
        """The index copy of the hits alone (the copy kernel of the separate
        launches, no attention), after hit_copy: its last step was all hits, so
        kvs_probe_hit_copy copies every request's K rows.  Launched back to back,
        cycling the layers (each reads its own hot rows at the last step's
        slots), between two events: HIP events around each launch would add
        about 5 us to a 30 us kernel."""
        if sets is None or self.args.separate or self.args.direct_hot:
            return None
        torch, pool, wl = self.torch, self.pool, self.wl
        B, L, K = wl.batch, wl.layers, wl.topk
        pool.probe_hit_copy(0)   # warm-up launch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for l in range(L):
                pool.probe_hit_copy(l)
        e1.record()
        e1.synchronize()
        self.sync_ok()
        avg_ms = e0.elapsed_time(e1) / (reps * L)
        rows = B * K
        gbs = 2 * ROW * rows / (avg_ms * 1e-3) / 1e9
        working_set = (L * B * K + B * K) * ROW   # every layer's rows at the slots + the buffer
        return {"rows_per_launch": rows, "bytes_per_launch": 2 * ROW * rows,
                "avg_ms": round(avg_ms, 5), "achieved_gbs": round(gbs, 1),
                "peak_gbs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
                "working_set_mb": round(working_set / 1e6, 1), "kernel": "gather (hit copy)",
                "note": f"index copy of the hits alone (kvs_probe_hit_copy: the copy kernel of "
                        f"the separate launches), {reps} x {L} launches back to back cycling the "
                        f"layers, timed between two events; working set = every layer's rows at "
                        f"the last step's slots + the compute buffer"}

    def parity(self, steps, reqs, rec):
        """GPU outputs of steps 0..steps-1 and final maps of the sampled requests
        against the oracle replay (every layer)."""
        torch, wl = self.torch, self.wl
        out = self.out[:steps].view(torch.int16).cpu().numpy().view(np.uint16)
        lse = self.lse[:steps].cpu().numpy()
        max_abs = max_rel = max_lse = 0.0
        state_ok = True
        for b in reqs:
            for l in range(wl.layers):
                for t in range(steps):
                    ref, ref_lse = rec[(t, l, b)]
                    got = ((out[t, l, b].astype(np.uint32) << 16).view(np.float32)
                           .astype(np.float64))
                    err = got - ref
                    max_abs = max(max_abs, float(np.abs(err).max()))
                    max_rel = max(max_rel, float(np.linalg.norm(err) / np.linalg.norm(ref)))
                    max_lse = max(max_lse, float(np.abs(lse[t, l, b] - ref_lse).max()))
                st = self.pool.read_state(b, l)
                t2s, s2t, lu = rec[("state", l, b)]
                state_ok &= bool(np.array_equal(st["tok2slot"], t2s) and
                                 np.array_equal(st["slot2tok"], s2t) and
                                 np.array_equal(st["last_used"], lu))
        ok = bool(state_ok and max_abs <= 2e-2 and max_rel <= 1e-2 and max_lse <= 2e-3)
        return {"requests_checked": list(reqs), "layers_checked": wl.layers,
                "steps_checked": steps, "state_bit_exact": state_ok,
                "attn_max_abs": round(max_abs, 6), "attn_max_rel_l2": round(max_rel, 6),
                "lse_max_abs": round(max_lse, 6), "pass": ok}


def summarize(wlo, times, kernels, hits, misses, hit_copy, index_copy, parity, zc_gbs, wall):
    """Per-workload results of the measurement protocol."""
    wl = wlo.wl
    steady = [statistics.mean(r[1:]) for r in times]
    cold = [r[0] for r in times]
    ms = statistics.median(steady)
    tokens = wl.batch * wl.layers * wl.topk
    res = {
        "batch": wl.batch, "layers": wl.layers, "context": wl.context, "slots": wl.slots,
        "topk": wl.topk, "fresh_rate": wl.fresh_rate, "fresh_dist": wl.dist,
        "steps": len(times[0]), "replays": len(times),
        "attn_splits": wlo.pool.sizes.attn_splits,
        "ms_per_step": round(ms, 5),
        "ms_per_step_replays": [round(x, 5) for x in steady],
        "tokens_per_s": round(tokens / (ms * 1e-3), 1),
        "decode_steps_per_s": round(1e3 / ms, 2),
        "cold_step_ms": round(statistics.median(cold), 4),
        "miss_rate": round(misses / max(1, hits + misses), 5),
        "host_link_gbs_step": round(ROW * misses / (len(times[0]) - 1) / (ms * 1e-3) / 1e9, 3),
        "kernels": kernels,
        "hit_copy": hit_copy,
        "index_copy": index_copy,
        "parity": parity,
        "wall_s": round(wall, 1),
    }
    g = kernels.get("gather") or kernels.get("assemble")
    if g:
        res["gather_frac_of_63gbs"] = g["frac"]
        res["gather_frac_of_zero_copy_peak"] = round(g["achieved_gbs"] / zc_gbs, 4)
    a = kernels.get("attention")
    if a:
        res["attention_hbm_frac"] = a["frac"]
    a = a or kernels.get("assemble")
    if a:
        res["attention_mfma_frac"] = a.get("mfma_frac")
    link_s = ROW * misses / (len(times[0]) - 1) / (zc_gbs * 1e9)
    res["link_ceiling_frac"] = round(link_s * 1e3 / ms, 4)   # step time if only the PCIe bytes
    return res


def parity_reqs(wl, n):
    reqs = sorted({0, wl.batch - 1} if n >= 2 else {0})
    return reqs[:max(1, n)]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; run with --gpus 1 (the path "
                                   "shards by request with no exchange between GPUs, so one "
                                   "GPU's share at its real shape is the measurement)"}))
        sys.exit(2)
    t_start = time.perf_counter()
    head = W.WORKLOADS[args.workload]
    if args.configs == "all":
        side = [n for n in W.WORKLOADS if n != head.name]
    elif args.configs == "none":
        side = []
    else:
        side = [n for n in args.configs.split(",") if n and n != head.name]
        for n in side:
            if n not in W.WORKLOADS:
                raise SystemExit(f"unknown workload {n}")
    steps_head = max(head.steps, args.warmup + args.steps)

    # The headline pool is filled into a shared mapping and the oracle processes
    # are forked from it before anything touches the GPU (no torch import yet).
    workers = shared = shared_rows = None
    if not args.no_cpu_baseline and not args.copy_calibration:
        P = cpu_workers_count(args)
        log(f"filling {head.pool_bytes / 1e9:.2f} GB of pool rows for {head.name} "
            f"(shared with {P} oracle processes)")
        shared = mmap.mmap(-1, head.pool_bytes, flags=mmap.MAP_SHARED | mmap.MAP_ANONYMOUS)
        shared_rows = np.frombuffer(shared, dtype=np.uint16).reshape(
            head.batch, head.layers, head.context, head.head_dim)
        parallel_units(lambda b, l: W.fill_unit_rows(shared_rows[b, l], head, b, l), head)
        workers = CpuWorkers(head, shared_rows, P)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    import token_level_gather_amd as kvs

    torch.cuda.set_device(0)
    results = {}
    failed = []

    # ---- headline
    t0 = time.perf_counter()
    log(f"headline {head.name}: B={head.batch} L={head.layers} N={head.context} "
        f"S={head.slots} K={head.topk}; warmup {args.warmup} + timed {args.steps}")
    wo = Workload(torch, kvs, head, args, steps_head, shared_rows)
    log(f"inputs ready, pool {wo.pool.host.nbytes / 1e9:.2f} GB pinned")
    h2d = measure_h2d_peak(torch)
    zc = measure_zero_copy_peak(torch, kvs, wo.pool.host)
    d2d = measure_d2d_peak(torch)
    log(f"H2D copy peak {h2d:.1f} GB/s, zero-copy read peak {zc:.1f} GB/s, "
        f"D2D copy {d2d:.0f} GB/s")
    cr = wo.contract_run(args.warmup, args.steps, graph=args.graph)
    log(f"timed {args.steps} steps in {cr['elapsed'] * 1e3:.2f} ms")
    parity = None
    if workers is not None:
        reqs = parity_reqs(head, args.parity_requests)
        rec = cpu_baseline_oracle_replay(head, wo.pool.host.array, wo.topk_np, wo.q_np, reqs,
                                         args.warmup + args.steps)
        parity = wo.parity(args.warmup + args.steps, reqs, rec)
        del rec
        log(f"parity {parity}")
        if not parity["pass"]:
            failed.append(head.name)
    times = wo.replays(args.replays, head.steps)
    kernels, hits_b, misses_b, _ = wo.breakdown(head.steps, zc)
    sets = wo.hit_sets()
    hit_copy = wo.hit_copy(sets)
    index_copy = wo.index_copy(sets)
    results[head.name] = summarize(wo, times, kernels, hits_b, misses_b, hit_copy, index_copy,
                                   parity, zc, time.perf_counter() - t0)
    log(f"{head.name}: {results[head.name]['ms_per_step']} ms/step median of replays")

    ms_step = cr["elapsed"] * 1e3 / args.steps
    L = head.layers
    calls_timed = args.steps * L
    alg = wo.algorithmic(cr["hits"] / calls_timed, cr["misses"] / calls_timed)
    dom = wo.kernel_stats(cr["tdom"], alg, (cr["dominant"],), zc).get(cr["dominant"])
    roofline = None
    if dom is not None:
        roofline = {"kernel": cr["dominant"], "bound": dom["bound"],
                    "achieved": dom["achieved_gbs"], "peak": dom["peak_gbs"], "unit": "GB/s",
                    "frac": dom["frac"], "traffic": load_traffic(cr["dominant"], head.name),
                    "avg_ms": dom["avg_ms"], "bytes_per_launch": dom["bytes_per_launch"],
                    "avg_ms_from": "HIP events on the launch stream around every launch of "
                                   "this kernel in the timed region"}
        if dom["bound"] == "pcie":
            roofline["frac_of_measured_h2d"] = round(dom["achieved_gbs"] / h2d, 4)
            roofline["frac_of_zero_copy_peak"] = round(dom["achieved_gbs"] / zc, 4)
        if "hbm_bytes" in alg[cr["dominant"]]:
            # what the HBM counters should read if nothing is re-read: the kernel's
            # algorithmic HBM bytes plus the host rows it pulls through the L2
            a = alg[cr["dominant"]]
            roofline["algorithmic_traffic"] = int((a["hbm_bytes"] + a["bytes"])
                                                  / dom["launches_per_call"])
    misses = cr["misses"]
    hbm_bytes_step = sum(k.get("hbm_bytes", k["bytes"] if k["bound"] == "hbm" else 0)
                         for k in alg.values()) * L
    wo.close()
    del wo
    cpu = None
    if workers is not None:
        log(f"cpu baseline: {workers.nproc} oracle processes")
        cpu = workers.run(head.steps)
        workers.close()
        log(f"cpu baseline {cpu}")
    shared_rows = None
    if shared is not None:
        shared.close()

    # ---- the other workloads, same protocol
    for name in side:
        if time.perf_counter() - t_start > args.time_budget:
            results[name] = {"skipped": f"time budget of {args.time_budget:.0f} s reached"}
            log(f"{name}: skipped (time budget)")
            continue
        wl = W.WORKLOADS[name]
        t0 = time.perf_counter()
        log(f"{name}: B={wl.batch} L={wl.layers} N={wl.context} S={wl.slots} K={wl.topk} "
            f"f={wl.fresh_rate}")
        wo = Workload(torch, kvs, wl, args, wl.steps)
        pr = None
        if not args.no_cpu_baseline:
            # replay 0 from a fresh pool, outputs checked against the oracle
            for t in range(wl.steps):
                wo.step(t)
            wo.sync_ok()
            reqs = parity_reqs(wl, args.parity_requests)
            rec = cpu_baseline_oracle_replay(wl, wo.pool.host.array, wo.topk_np, wo.q_np, reqs,
                                             wl.steps)
            pr = wo.parity(wl.steps, reqs, rec)
            del rec
            if not pr["pass"]:
                failed.append(name)
        times = wo.replays(args.replays, wl.steps)
        kernels, hits_b, misses_b, _ = wo.breakdown(wl.steps, zc)
        sets = wo.hit_sets()
        hit_copy = wo.hit_copy(sets)
        index_copy = wo.index_copy(sets)
        results[name] = summarize(wo, times, kernels, hits_b, misses_b, hit_copy, index_copy,
                                  pr, zc, time.perf_counter() - t0)
        log(f"{name}: {results[name]['ms_per_step']} ms/step, parity "
            f"{None if pr is None else pr['pass']}, {results[name]['wall_s']} s")
        wo.close()
        del wo

    if failed:
        print(json.dumps({"error": "parity check failed; no speed reported", "failed": failed,
                          "parity": {n: results[n].get("parity") for n in failed}}),
              file=sys.stderr, flush=True)
        sys.exit(1)

    hr = results[head.name]
    value = head.batch * L * head.topk / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head.name, "batch": head.batch, "layers": L,
                   "context": head.context, "slots": head.slots, "topk": head.topk,
                   "fresh_rate": head.fresh_rate, "fresh_dist": head.dist, "heads": 16,
                   "head_dim": 576, "v_dim": 512, "attn_splits": hr["attn_splits"],
                   "fetch_blocks": args.fetch_blocks, "hit_blocks": args.hit_blocks,
                   "hits_first": bool(args.hits_first), "hip_graph": bool(args.graph),
                   "direct_hot": bool(args.direct_hot),
                   "separate_attention": bool(args.separate)},
        "decode_steps_per_s": round(1e3 / ms_step, 2),
        "cold_step_ms": round(cr["cold_ms"], 4),
        "miss_rate": round(misses / max(1, cr["hits"] + misses), 5),
        "host_link_gbs_step": round(ROW * misses / args.steps / (ms_step * 1e-3) / 1e9, 3),
        "hbm_gbs_step": round(hbm_bytes_step / (ms_step * 1e-3) / 1e9, 2),
        "h2d_peak_measured_gbs": round(h2d, 2),
        "zero_copy_read_peak_gbs": round(zc, 2),
        "hbm_copy_peak_measured_gbs": round(d2d, 1),
        # decode steps/s if the step were only its miss bytes at the link's rate
        "steps_per_s_link_ceiling": {
            "pcie_gen5_x16_63gbs": round(63.0e9 / max(1.0, ROW * misses / args.steps), 1),
            "measured_zero_copy": round(zc * 1e9 / max(1.0, ROW * misses / args.steps), 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "kernels": hr["kernels"],
        # the index copy of the hits alone (gather kernel), and the assembling
        # launch that copies and attends over them in one pass (the default step)
        "hit_gather": hr["index_copy"] or hr["hit_copy"],
        "hit_gather_fused": hr["hit_copy"] if hr["index_copy"] else None,
        "protocol": {k: hr[k] for k in ("steps", "replays", "ms_per_step", "ms_per_step_replays",
                                        "cold_step_ms", "miss_rate")},
        "configs": results,
        "pages_context": PAGES_CONTEXT,
        "wall_s": round(time.perf_counter() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
