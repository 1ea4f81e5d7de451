"""Benchmark: ReplaySSM SSM-layer decode on one MI355X vs the same-GPU conventional kernel.

Default workload (the one the headline metric is quoted on): the
Nemotron-style Mamba-2 layer at serving batch 256 (128 heads, headdim 64,
dstate 128, 8 groups, bf16 inputs, fp32 checkpoint, 4 MiB of state per
sequence), seeded synthetic inputs resident in HBM.

One "step" is one full buffer window: 15 non-flush steps (append + output
from checkpoint and buffer) and one flush step (fold, one checkpoint write),
i.e. 16 decode tokens for all 256 sequences; `value` is decode tokens/s over
the K timed windows. The conventional read-modify-write kernel is timed on
the same windows for comparison. The JSON line carries the roofline of the
dominant kernel (the non-flush step) measured with HIP events on the launch
stream, beside two plain streams of the same tiles (read only, and with the
step's writes per tile) timed in the same process, and the fp64 CPU oracle
timed on a bounded sample of the workload.

Other workloads (each one more JSON line, only when asked with --workload):
  gdn       Qwen3.5-style Gated DeltaNet layer, batch 256 (UT-form non-flush)
  kda       the same shapes with Kimi Delta Attention's per-key-channel gate
  spec      speculative decode on 120B-class Mamba-2 shapes, batch 512, 4 drafts
            per round: ReplaySSM append + commit vs snapshot / restore
  gdn_spec  speculative decode on the Gated DeltaNet layer, batch 256, 4 drafts
  kda_spec  the same for Kimi Delta Attention
  lowprec   Nemotron shapes at batch 64 (or --lowprec-batch): fp32 / fp16 / fp8
            checkpoints with and without the NVFP4 read copy, and the uniform
            NVFP4 checkpoint; optionally (--lowprec-error-steps) y error vs fp64
            over length
  serve     continuous batching (staggered buffer fills, one self-scheduling
            launch per step) and prefix-cache save / restore of 64 sequences
  block     the Mamba-2 block per token: short convolution, SSM step, gated norm
  sweep     the Nemotron layer at batch 1 .. 512, ReplaySSM vs conventional
  copy      a 1 GiB device copy, a read-only sum and the tile probes (the
            references the HBM counters and the roofline are read against)
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

import workloads as W  # noqa: E402

RING = 16
HBM_PEAK_GBS = 8000.0
POOL_MAX = 16            # worker processes of the CPU oracle leg (the host's CPU share per GPU)
METRIC = "SSM-layer decode tokens/s at batch 256 + achieved HBM GB/s (% of peak) vs conventional"
PROFILES = os.path.join(ROOT, "profiles")
# What the fp32 non-flush kernel (the bench line's roofline kernel) is built
# from: the shared headers and flags whole, and from the Mamba-2 kernel header
# only the kernel's own text (its shared-memory struct through its body), so
# that work on the other kernels there leaves its committed counters valid.
KERNEL_HEADERS = ["ssm_decode_checkpoint_amd/csrc/rs_tile.h", "ssm_decode_checkpoint_amd/csrc/rs_device.h",
                  "ssm_decode_checkpoint_amd/csrc/rs_internal.h", "ssm_decode_checkpoint_amd/build.py"]
NONFLUSH_SOURCE = "ssm_decode_checkpoint_amd/csrc/rs_mamba2_kernels.h"


def nonflush_kernel_text(src: str) -> str:
    """The fp32 non-flush kernel's text in the Mamba-2 kernel header: from its
    shared-memory struct to the end of m2_nonflush_kernel."""
    start = src.index("struct alignas(16) M2NfSmem")
    body = src.index("void m2_nonflush_kernel(M2Args a) {", start)
    return src[start:src.index("\n}\n", body) + 3]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_HEADERS:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, NONFLUSH_SOURCE)) as f:
        h.update(nonflush_kernel_text(f.read()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes per sequence (what the method must move; cache effects not counted)
# ---------------------------------------------------------------------------

def m2_bytes(w: W.Mamba2Workload, ckpt_bytes_per_elem: float = 4.0, read_bytes_per_elem: float = None):
    """Per-sequence bytes of each Mamba-2 step. The checkpoint element costs
    ckpt_bytes_per_elem when written or folded from, and read_bytes_per_elem
    when a non-flush step reads it through a read copy (the flush then also
    writes the copy)."""
    s_in = 2 if w.in_dtype == "bf16" else 4
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    rd = ckpt_bytes_per_elem if read_bytes_per_elem is None else read_bytes_per_elem
    S = H * P * N * ckpt_bytes_per_elem
    S_read = H * P * N * rd
    E_in = (H * P + 2 * G * N + H) * s_in      # x, B, C, dt of the current token
    E_old = (H * P + G * N + H) * s_in         # x, B, dt of a held entry (C is not re-read)
    Y = H * P * 4
    rc_write = 0.0 if read_bytes_per_elem is None else H * P * N * rd
    nonflush = {j: S_read + (j - 1) * E_old + 2 * E_in + Y for j in range(1, RING)}
    flush = 2 * S + (RING - 1) * E_old + E_in + Y + rc_write
    conv = 2 * H * P * N * 4 + E_in + Y
    return {"state": S, "E_in": E_in, "E_old": E_old, "Y": Y, "nonflush": nonflush, "flush": flush, "conv": conv}


def gdn_bytes(w: W.GDNWorkload):
    """Per-sequence bytes of each Gated DeltaNet step. A held entry is re-read
    as its k, its decay g and its solved row u (fp32); each non-flush step
    appends the record (q, k, v, g, beta) and the new entry's u. A per-channel
    gate (Kimi Delta Attention) is dk floats per value head instead of one."""
    s_in = 2 if w.in_dtype == "bf16" else 4
    gw = w.dk if w.gate == "channel" else 1
    S = w.n_v * w.dv * w.dk * 4
    E_in = 2 * w.n_qk * w.dk * s_in + w.n_v * w.dv * s_in + w.n_v * gw * 4 + w.n_v * 4   # q, k, v, g, beta
    Urow = w.n_v * w.dv * 4
    E_old = w.n_qk * w.dk * s_in + Urow + w.n_v * gw * 4                    # k, u, g of a held entry
    O = w.n_v * w.dv * 4
    nonflush = {j: S + (j - 1) * E_old + 2 * E_in + Urow + O for j in range(1, RING)}
    flush = 2 * S + (RING - 1) * E_old + E_in + O
    conv = 2 * S + E_in + O
    # with the NVFP4 read copy: non-flush steps read the copy (4.5 bits per element and a
    # tensor scale); the flush re-solves the held entries' rows from the fp32 checkpoint
    # (re-reading their k, v, g and beta instead of u), folds, and writes the checkpoint
    # and, from the same registers, the copy
    S_rc = w.n_v * w.dv * w.dk * (0.5 + 1 / 16) + w.n_v * 4
    E_old_rc = w.n_qk * w.dk * s_in + w.n_v * w.dv * s_in + w.n_v * gw * 4 + w.n_v * 4
    nonflush_rc = {j: S_rc + (j - 1) * E_old + 2 * E_in + Urow + O for j in range(1, RING)}
    flush_rc = 2 * S + (RING - 1) * E_old_rc + E_in + O + S_rc
    # FP16 / FP8 checkpoints: the state in 2 or 1 bytes per element (FP8 with a
    # 4-byte scale per matrix), read by every step and written by the flush
    lp = {}
    for fmt, es, extra in (("f16", 2, 0), ("fp8", 1, 4)):
        S_lp = w.n_v * w.dv * w.dk * es + w.n_v * extra
        lp[fmt] = {"state": S_lp,
                   "nonflush": {j: S_lp + (j - 1) * E_old + 2 * E_in + Urow + O for j in range(1, RING)},
                   "flush": 2 * S_lp + (RING - 1) * E_old + E_in + O}
    return {"state": S, "E_in": E_in, "E_old": E_old, "O": O, "nonflush": nonflush, "flush": flush, "conv": conv,
            "state_rc": S_rc, "nonflush_rc": nonflush_rc, "flush_rc": flush_rc, "lowprec": lp}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def _conv_window(w: W.Mamba2Workload, seqs, steps: int) -> float:
    """Seconds the fp64 conventional recurrence (the oracle) takes for `steps`
    decode steps of the listed sequences, one thread; inputs drawn beforehand."""
    from oracle import decode
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        p = W.m2_params(w)
        ref = decode.M2Conventional(W.m2_init_states(w, seqs), p["A"], p["D"])
        toks = [W.m2_step(w, t, seqs) for t in range(steps)]
        t0 = time.perf_counter()
        for tk in toks:
            ref.step(tk)
        return time.perf_counter() - t0


def _pool_worker(w, seqs, steps, ready, go, out):
    """One shard of the pool leg: draw inputs, wait for every shard, then time."""
    from oracle import decode
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        p = W.m2_params(w)
        ref = decode.M2Conventional(W.m2_init_states(w, seqs), p["A"], p["D"])
        toks = [W.m2_step(w, t, seqs) for t in range(steps)]
        ready.wait()
        go.wait()
        t0 = time.perf_counter()
        for tk in toks:
            ref.step(tk)
        out.put(time.perf_counter() - t0)


def cpu_baseline(w: W.Mamba2Workload, single_seqs: int = 48, replay_seqs: int = 64):
    """The fp64 CPU oracle timed on this host's cores on one 16-step window of
    the workload: the conventional recurrence single-process (a sample of
    sequences) and as a process pool over every core this process may run on,
    one shard of sequences per core, the whole batch (the value); and, as a
    separate figure, the oracle's ReplaySSM form on one thread. A reported
    baseline, not the target. Runs before the GPU is touched (the pool forks)."""
    import multiprocessing as mp
    from oracle import decode
    from threadpoolctl import threadpool_limits
    host = len(os.sched_getaffinity(0))
    n = min(host, POOL_MAX)
    # single process, one thread
    single = _conv_window(w, list(range(single_seqs)), RING)
    # pool: one process per core, sequences dealt round-robin
    ctx = mp.get_context("fork")
    ready, go, out = ctx.Barrier(n + 1), ctx.Barrier(n + 1), ctx.Queue()
    shards = [list(range(i, w.batch, n)) for i in range(n)]
    procs = [ctx.Process(target=_pool_worker, args=(w, sh, RING, ready, go, out)) for sh in shards if sh]
    for pr in procs:
        pr.start()
    ready.wait()
    t0 = time.perf_counter()
    go.wait()
    times = [out.get() for _ in procs]
    pool_wall = time.perf_counter() - t0
    for pr in procs:
        pr.join()
    # ReplaySSM form of the oracle, one thread
    p = W.m2_params(w)
    seqs = list(range(replay_seqs))
    with threadpool_limits(1):
        rep = decode.M2Replay(W.m2_init_states(w, seqs), p["A"], p["D"])
        toks = [W.m2_step(w, t, seqs) for t in range(RING)]
        t1 = time.perf_counter()
        for tk in toks:
            rep.step(tk)
        rwall = time.perf_counter() - t1
    return {"value": w.batch * RING / pool_wall, "unit": "tokens/s", "cores": len(procs), "kind": "oracle",
            "label": "baseline, not target", "host_cores": host,
            "sample": (f"fp64 conventional recurrence (the oracle, plain numpy, one thread per process) on all "
                       f"{w.batch} sequences x {RING} decode steps (one window) of the {w.name} workload, "
                       f"{len(procs)} processes ({host} cores in os.sched_getaffinity(0), at most {POOL_MAX} used), "
                       f"sequences dealt "
                       f"round-robin; {pool_wall:.1f} s wall (slowest shard {max(times):.1f} s)"),
            "single_process": {"value": single_seqs * RING / single, "unit": "tokens/s", "cores": 1,
                               "sample": f"{single_seqs} sequences x {RING} steps, conventional recurrence; "
                                         f"{single:.1f} s"},
            "replay_oracle_one_thread": {"value": replay_seqs * RING / rwall, "unit": "tokens/s", "cores": 1,
                                         "sample": f"fp64 ReplaySSM form of the oracle (checkpoint + buffer), "
                                                   f"{replay_seqs} sequences x {RING} steps; {rwall:.1f} s"}}


# ---------------------------------------------------------------------------
# GPU helpers
# ---------------------------------------------------------------------------

def traffic_from_profile(name: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources."""
    path = os.path.join(PROFILES, "counters_" + name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


class Timer:
    """HIP-event timing of a sequence of launches on torch's current stream
    (the stream every library call here is enqueued on)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def run(self, fn, K, warm, nmarks, reset=None):
        """Total time of K steps with nothing but the launches in the timed
        region, then a second pass of K steps with events around each marked
        call for the per-call breakdown (those events add their own gaps, so
        the total never comes from that pass). `reset` runs before each pass."""
        torch = self.torch
        for _ in range(warm):
            fn(None)
        if reset is not None:
            reset()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(self.stream)
        for k in range(K):
            fn(None)
        t1.record(self.stream)
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1)
        if reset is not None:
            reset()
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nmarks)] for _ in range(K)]
        torch.cuda.synchronize()
        for k in range(K):
            fn(evs[k])
        torch.cuda.synchronize()
        per = np.array([[evs[k][i][0].elapsed_time(evs[k][i][1]) for i in range(nmarks)] for k in range(K)])
        return total, per


def _marked(ev, i, stream, call):
    if ev is not None:
        ev[i][0].record(stream)
    call()
    if ev is not None:
        ev[i][1].record(stream)


def _bf16_dev(torch, arr, dev):
    return torch.from_numpy(W.bf16_bits(arr).view(np.int16).copy()).view(torch.bfloat16).to(dev)


def _m2_layer(rs, w, B, mode, dev, ckpt=None, read_copy=None, fuse=1, max_draft=0):
    cfg = rs.make_config(rs.RS_MAMBA2, B, mode=mode, nheads=w.nheads, headdim=w.headdim, dstate=w.dstate,
                         ngroups=w.ngroups, in_dtype=rs.RS_BF16 if w.in_dtype == "bf16" else rs.RS_F32,
                         ckpt_dtype=rs.RS_F32 if ckpt is None else ckpt,
                         read_copy=rs.RS_NONE if read_copy is None else read_copy, fuse_requant=fuse,
                         max_draft=max_draft)
    _, layer = rs.rs_init(cfg)
    return layer, rs.alloc_buffers(layer, dev)


def _m2_load_init(torch, rs, w, layer, bufs, dev):
    ck = rs.ckpt_f32_view(layer, bufs)
    for b in range(layer.cfg.batch):
        ck[b].copy_(torch.from_numpy(np.ascontiguousarray(W.m2_init_state(w, b).transpose(0, 2, 1))).to(dev))


def _m2_pool(torch, w, B, dev, t0=0, n=RING):
    pool = []
    for t in range(t0, t0 + n):
        tk = W.m2_step(w, t, range(B))
        pool.append({k: (_bf16_dev(torch, v, dev) if w.in_dtype == "bf16" else torch.from_numpy(v).to(dev))
                     for k, v in tk.items()})
    return pool


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def bench_mamba2(args, torch, rs):
    w = W.M2_NEMOTRON
    dev = "cuda"
    B = w.batch
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    rl, rb = _m2_layer(rs, w, B, rs.RS_REPLAY, dev)
    cl, cb = _m2_layer(rs, w, B, rs.RS_CONVENTIONAL, dev)
    _m2_load_init(torch, rs, w, rl, rb, dev)
    rs.ckpt_f32_view(cl, cb).copy_(rs.ckpt_f32_view(rl, rb))
    pool = _m2_pool(torch, w, B, dev)
    y = torch.empty(B, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    tm = Timer(torch)

    def replay_window(ev):
        for t in range(RING):
            fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
            _marked(ev, t, tm.stream, lambda: fn(rl, rb, pool[t], A, D, y))

    def conv_window(ev):
        for t in range(RING):
            _marked(ev, t, tm.stream, lambda: rs.rs_step_conventional(cl, cb, pool[t], A, D, y))

    K, warm = args.steps, args.warmup
    total_r, per_r = tm.run(replay_window, K, warm, RING)
    total_c, per_c = tm.run(conv_window, K, warm, RING)
    byt = m2_bytes(w)
    ntok = B * RING * K
    value = ntok / (total_r * 1e-3)
    conv_value = ntok / (total_c * 1e-3)
    nf_ms = per_r[:, : RING - 1]
    nf_bytes = sum(byt["nonflush"][j] for j in range(1, RING)) * B
    nf_avg_ms = float(nf_ms.mean())
    nf_gbs = nf_bytes / (nf_ms.sum(axis=1).mean() * 1e-3) / 1e9
    fl_ms = float(per_r[:, RING - 1].mean())
    cv_ms = float(per_c.mean())
    win_bytes = nf_bytes + byt["flush"] * B
    # what a plain stream of the same 32 KiB tiles reaches on this chip, after the timed
    # runs: read only, and with the step's writes per tile (y and the appended record)
    probe_gbs = probe_read_gbs(torch, tm)
    wtile = m2_writes_per_tile(w)
    probe_rw_gbs = probe_read_gbs(torch, tm, write_bytes=wtile)
    win_ms = total_r / K
    return {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": warm,
        "ms_per_step": win_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                   "ngroups": w.ngroups, "inputs": "bf16", "checkpoint": "f32", "ring": RING,
                   "step": "one 16-token window: 15 non-flush + 1 flush", "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": nf_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nf_gbs / HBM_PEAK_GBS, "traffic": traffic_from_profile("m2_nonflush_b256"),
                     "kernel": "m2_nonflush_kernel", "avg_launch_ms": nf_avg_ms,
                     "alg_bytes_per_launch": nf_bytes / (RING - 1),
                     "read_stream_gbs": probe_gbs, "frac_of_read_stream": nf_gbs / probe_gbs,
                     "read_write_stream_gbs": probe_rw_gbs, "write_bytes_per_tile": wtile,
                     "frac_of_read_write_stream": nf_gbs / probe_rw_gbs},
        "replay": {"tokens_per_s": value, "window_ms": win_ms, "window_alg_bytes": win_bytes,
                   "window_gbs": win_bytes / (win_ms * 1e-3) / 1e9,
                   "nonflush_avg_ms": nf_avg_ms, "nonflush_gbs": nf_gbs,
                   "nonflush_by_fill_ms": [float(x) for x in nf_ms.mean(axis=0)],
                   "flush_ms": fl_ms, "flush_gbs": byt["flush"] * B / (fl_ms * 1e-3) / 1e9},
        "conventional": {"tokens_per_s": conv_value, "step_ms": cv_ms,
                         "gbs": byt["conv"] * B / (cv_ms * 1e-3) / 1e9,
                         "window_ms": total_c / K, "window_alg_bytes": byt["conv"] * B * RING},
        "speedup_vs_conventional": value / conv_value,
        "bytes_ratio_conventional_over_replay": byt["conv"] * B * RING / win_bytes,
    }


SWEEP_BATCHES = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


def _graph_window_ms(torch, window, K, warm):
    """Milliseconds per window when the window's launches are captured once in a
    HIP graph (torch.cuda.CUDAGraph) and replayed K times. The library calls
    allocate, synchronise and memset nothing, and the buffer counters advance on
    the device, so each replay continues the window sequence; a graph's first
    replays are warm-up."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        window()
    for _ in range(max(1, warm)):
        g.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(K):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    del g
    return ms


def bench_sweep(args, torch, rs):
    """Conventional vs ReplaySSM decode over batch sizes on the Nemotron-style
    Mamba-2 layer shapes (128 heads, 64 x 128 fp32 state, bf16 inputs). Each
    batch times whole 16-token windows of both paths; the inputs are the first
    B sequences of one resident 16-step pool. Below about 64 sequences the
    checkpoint (4 MiB per sequence) fits the 256 MB last-level cache, so GB/s
    there are effective rather than HBM rates."""
    w = W.M2_NEMOTRON
    dev = "cuda"
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    bmax = max(SWEEP_BATCHES)
    pool = _m2_pool(torch, w, bmax, dev)
    byt = m2_bytes(w)
    tm = Timer(torch)
    rows = []
    for B in SWEEP_BATCHES:
        sub = [{k: v[:B] for k, v in tk.items()} for tk in pool]
        rl, rb = _m2_layer(rs, w, B, rs.RS_REPLAY, dev)
        cl, cb = _m2_layer(rs, w, B, rs.RS_CONVENTIONAL, dev)
        y = torch.empty(B, w.nheads, w.headdim, dtype=torch.float32, device=dev)

        def replay_window(ev):
            for t in range(RING):
                fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
                _marked(ev, t, tm.stream, lambda: fn(rl, rb, sub[t], A, D, y))

        def conv_window(ev):
            for t in range(RING):
                _marked(ev, t, tm.stream, lambda: rs.rs_step_conventional(cl, cb, sub[t], A, D, y))

        total_r, per_r = tm.run(replay_window, args.steps, args.warmup, RING)
        total_c, _ = tm.run(conv_window, args.steps, args.warmup, RING)
        # the same windows captured once as HIP graphs and replayed (no host launch cost)
        graph_r = _graph_window_ms(torch, lambda: replay_window(None), args.steps, args.warmup)
        graph_c = _graph_window_ms(torch, lambda: conv_window(None), args.steps, args.warmup)
        ntok = B * RING * args.steps
        win_bytes = (sum(byt["nonflush"].values()) + byt["flush"]) * B
        rows.append({"batch": B,
                     "replay_tokens_per_s": ntok / (total_r * 1e-3),
                     "conventional_tokens_per_s": ntok / (total_c * 1e-3),
                     "speedup": total_c / total_r,
                     "replay_window_ms": total_r / args.steps,
                     "conventional_window_ms": total_c / args.steps,
                     "replay_nonflush_ms": float(per_r[:, :RING - 1].mean()),
                     "replay_flush_ms": float(per_r[:, RING - 1].mean()),
                     "replay_window_gbs": win_bytes / (total_r / args.steps * 1e-3) / 1e9,
                     "conventional_gbs": byt["conv"] * B * RING / (total_c / args.steps * 1e-3) / 1e9,
                     "graph_replay_tokens_per_s": B * RING / (graph_r * 1e-3),
                     "graph_conventional_tokens_per_s": B * RING / (graph_c * 1e-3),
                     "graph_speedup": graph_c / graph_r})
        print(f"sweep: batch {B} done", file=sys.stderr, flush=True)
        del rl, rb, cl, cb, y
        torch.cuda.empty_cache()
    best = max(rows, key=lambda r: r["replay_tokens_per_s"])
    return {"metric": "SSM-layer decode tokens/s over batch size, ReplaySSM vs conventional (Mamba-2)",
            "value": best["replay_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": best["replay_window_ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "mamba2_nemotron_batch_sweep", "batches": list(SWEEP_BATCHES),
                       "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                       "inputs": "bf16", "checkpoint": "f32",
                       "step": "one 16-token window per path: 15 non-flush + 1 flush vs 16 conventional"},
            "rows": rows}


def bench_serve(args, torch, rs):
    """Continuous-batching schedule on the Nemotron-style Mamba-2 layer at batch
    256: slots are reused at staggered times (rs_reset_slots) so that the buffer
    fills differ, then every step is one self-scheduling call (rs_step) in which
    the sequences whose buffers are full (1/16 of them) flush and the others take
    a non-flush step. Reports throughput and the per-step time spread, beside the
    lockstep schedule (15 non-flush calls, then one flush call for everyone)."""
    w = W.M2_NEMOTRON
    dev = "cuda"
    B = w.batch
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    layer, bufs = _m2_layer(rs, w, B, rs.RS_REPLAY, dev)
    _m2_load_init(torch, rs, w, layer, bufs, dev)
    pool = _m2_pool(torch, w, B, dev)
    y = torch.empty(B, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    groups = [torch.tensor([b for b in range(B) if b % RING == t], dtype=torch.int32, device=dev) for t in range(RING)]
    for t in range(RING):                      # stagger: group t starts t steps later
        rs.rs_reset_slots(layer, bufs, groups[t], len(groups[t]))
        rs.rs_step(layer, bufs, pool[t], A, D, y)
    torch.cuda.synchronize()
    tm = Timer(torch)

    def window(ev):
        for t in range(RING):
            _marked(ev, t, tm.stream, lambda: rs.rs_step(layer, bufs, pool[t], A, D, y))

    total, per = tm.run(window, args.steps, args.warmup, RING)
    ntok = B * RING * args.steps
    steps_ms = per.reshape(-1)
    # prefix cache: save 64 mid-window sequences into a 64-slot cache of the same
    # layer and restore them into other slots (checkpoint rows + ring + counters)
    nc = 64
    cl, cb = _m2_layer(rs, w, nc, rs.RS_REPLAY, dev)
    src = torch.arange(0, B, B // nc, dtype=torch.int32, device=dev)[:nc]
    slots = torch.arange(nc, dtype=torch.int32, device=dev)
    dst = (src + 1) % B

    def cache_pass(ev):
        _marked(ev, 0, tm.stream, lambda: rs.rs_copy_slots(layer, bufs, src, cl, cb, slots, nc))
        _marked(ev, 1, tm.stream, lambda: rs.rs_copy_slots(cl, cb, slots, layer, bufs, dst, nc))

    ctot, cper = tm.run(cache_pass, 4, 1, 2)
    per_seq = (layer.ckpt_bytes + layer.ring_bytes) / B
    copy_ms = float(cper.mean())
    return {"metric": "continuous-batching decode tokens/s at batch 256, staggered fills (self-scheduling step)",
            "value": ntok / (total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": total / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "mamba2_nemotron_b256_staggered", "batch": B, "nheads": w.nheads,
                       "headdim": w.headdim, "dstate": w.dstate, "fills": "sequence b at fill (15 - b mod 16) "
                       "after the staggering phase", "step": "16 self-scheduling steps per timed window"},
            "step_ms": {"mean": float(steps_ms.mean()), "max": float(steps_ms.max()), "min": float(steps_ms.min()),
                        "p99": float(np.percentile(steps_ms, 99))},
            "prefix_cache": {"seqs_per_copy": nc, "bytes_per_seq": per_seq, "save_ms": float(cper[:, 0].mean()),
                             "restore_ms": float(cper[:, 1].mean()),
                             "copy_gbs": 2 * nc * per_seq / (copy_ms * 1e-3) / 1e9,
                             "note": "one call copies the sequences' checkpoint rows, 16 ring slots and counters; "
                                     "GB/s counts read + write"}}


def bench_block(args, torch, rs):
    """The Nemotron-style Mamba-2 layer's per-token path at batch 256 beyond the
    SSM step: short causal convolution (ring of recent inputs) -> self-scheduling
    SSM step -> gated RMS norm, 16 tokens per window, vs the SSM step alone."""
    w = W.M2_NEMOTRON
    dev = "cuda"
    B = w.batch
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    layer, bufs = _m2_layer(rs, w, B, rs.RS_REPLAY, dev)
    _m2_load_init(torch, rs, w, layer, bufs, dev)
    bp = W.block_params(w)
    ch = rs.conv_channels(layer)
    ring = torch.zeros(rs.conv_ring_bytes(layer), dtype=torch.uint8, device=dev)
    cw = torch.from_numpy(bp["conv_w"]).to(dev)
    cbias = torch.from_numpy(bp["conv_b"]).to(dev)
    nw = torch.from_numpy(bp["norm_w"]).to(dev)
    d = w.nheads * w.headdim
    xbc, z = [], []
    for t in range(RING):
        bt = W.block_step(w, t, range(B))
        xbc.append(_bf16_dev(torch, bt["xbc"], dev))
        z.append(_bf16_dev(torch, bt["z"], dev))
    dts = [_bf16_dev(torch, W.m2_step(w, t, range(B))["dt"], dev) for t in range(RING)]
    x = torch.empty(B, w.nheads, w.headdim, dtype=torch.bfloat16, device=dev)
    Bm = torch.empty(B, w.ngroups, w.dstate, dtype=torch.bfloat16, device=dev)
    Cm = torch.empty(B, w.ngroups, w.dstate, dtype=torch.bfloat16, device=dev)
    y = torch.empty(B, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    out = torch.empty(B, d, dtype=torch.bfloat16, device=dev)
    tm = Timer(torch)

    def window(ev):
        for t in range(RING):
            _marked(ev, 3 * t, tm.stream,
                    lambda: rs.rs_conv_step(layer, bufs, ring, xbc[t], 1, cw, cbias, 4, x, Bm, Cm))
            _marked(ev, 3 * t + 1, tm.stream,
                    lambda: rs.rs_step(layer, bufs, {"x": x, "B": Bm, "C": Cm, "dt": dts[t]}, A, D, y))
            _marked(ev, 3 * t + 2, tm.stream, lambda: rs.rs_gated_norm(layer, 1, y, z[t], nw, w.ngroups, 1e-5, out))

    total, per = tm.run(window, args.steps, args.warmup, 3 * RING)
    conv_ms, ssm_ms, norm_ms = (float(per[:, i::3].mean()) for i in range(3))
    conv_bytes = B * ch * 2 * 6          # 3 history reads, input, ring write, output (bf16)
    norm_bytes = B * d * (4 + 2 + 2)     # y fp32, z and out bf16
    ntok = B * RING * args.steps
    return {"metric": "Mamba-2 layer per-token path (conv + SSM step + gated norm) tokens/s at batch 256",
            "value": ntok / (total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": total / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "mamba2_nemotron_b256_block", "batch": B, "conv_channels": ch, "conv_width": 4,
                       "norm_groups": w.ngroups, "step": "16 tokens of conv -> rs_step -> gated norm"},
            "per_call_ms": {"conv": conv_ms, "ssm_step": ssm_ms, "gated_norm": norm_ms},
            "conv_gbs": conv_bytes / (conv_ms * 1e-3) / 1e9, "norm_gbs": norm_bytes / (norm_ms * 1e-3) / 1e9}


def bench_gdn(args, torch, rs, w=W.GDN_QWEN):
    """A delta-rule layer (Gated DeltaNet, or Kimi Delta Attention for a per-channel
    gate) at batch 256: ReplaySSM windows vs the conventional kernel."""
    dev = "cuda"
    B = w.batch
    gp = W.gdn_params(w)
    kda_layer = w.gate == "channel"

    def mk(mode, rc=False, ckpt=rs.RS_F32):
        cfg = rs.make_config(rs.RS_KDA if kda_layer else rs.RS_GDN, B, mode=mode, n_qk_heads=w.n_qk,
                             n_v_heads=w.n_v, head_k_dim=w.dk, head_v_dim=w.dv, in_dtype=rs.RS_BF16,
                             read_copy=rs.RS_NVFP4 if rc else rs.RS_NONE, ckpt_dtype=ckpt)
        _, layer = rs.rs_init(cfg)
        return layer, rs.alloc_buffers(layer, dev)

    rl, rb = mk(rs.RS_REPLAY)
    cl, cb = mk(rs.RS_CONVENTIONAL)
    ql, qb = mk(rs.RS_REPLAY, rc=True)
    ck = rs.ckpt_f32_view(rl, rb)
    for b in range(B):
        ck[b].copy_(torch.from_numpy(np.ascontiguousarray(W.gdn_init_state(w, b).transpose(0, 2, 1))).to(dev))
    rs.ckpt_f32_view(cl, cb).copy_(ck)
    rs.ckpt_f32_view(ql, qb).copy_(ck)
    rs.rs_requant_read_copy(ql, qb)
    pool = []
    for t in range(RING):
        tk = W.gdn_step(w, t, range(B), gp)
        d = {k: _bf16_dev(torch, tk[k], dev) for k in ("q", "k", "v")}
        d["g"] = torch.from_numpy(tk["g"]).to(dev)
        d["beta"] = torch.from_numpy(tk["beta"]).to(dev)
        pool.append(d)
    o = torch.empty(B, w.n_v, w.dv, dtype=torch.float32, device=dev)
    tm = Timer(torch)

    def replay_window(ev):
        for t in range(RING):
            fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
            _marked(ev, t, tm.stream, lambda: fn(rl, rb, pool[t], None, None, o))

    def conv_window(ev):
        for t in range(RING):
            _marked(ev, t, tm.stream, lambda: rs.rs_step_conventional(cl, cb, pool[t], None, None, o))

    def rc_window(ev):
        for t in range(RING):
            fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
            _marked(ev, t, tm.stream, lambda: fn(ql, qb, pool[t], None, None, o))

    # FP16 / FP8 checkpoints, from a zero state (the warm-up windows fold real
    # entries into it before the timed ones)
    lp_layers = {"f16": mk(rs.RS_REPLAY, ckpt=rs.RS_F16), "fp8": mk(rs.RS_REPLAY, ckpt=rs.RS_FP8E4M3)}

    def lp_window(fmt):
        ll, lb = lp_layers[fmt]

        def run(ev):
            for t in range(RING):
                fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
                _marked(ev, t, tm.stream, lambda: fn(ll, lb, pool[t], None, None, o))
        return run

    K, warm = args.steps, args.warmup
    total_r, per_r = tm.run(replay_window, K, warm, RING)
    total_c, per_c = tm.run(conv_window, K, warm, RING)
    total_q, per_q = tm.run(rc_window, K, warm, RING)
    lp_runs = {fmt: tm.run(lp_window(fmt), K, warm, RING) for fmt in lp_layers}
    byt = gdn_bytes(w)
    ntok = B * RING * K
    nf_ms = per_r[:, : RING - 1]
    nf_bytes = sum(byt["nonflush"][j] for j in range(1, RING)) * B
    nf_gbs = nf_bytes / (nf_ms.sum(axis=1).mean() * 1e-3) / 1e9
    fl_ms = float(per_r[:, RING - 1].mean())
    cv_ms = float(per_c.mean())
    win_bytes = nf_bytes + byt["flush"] * B
    value = ntok / (total_r * 1e-3)
    conv_value = ntok / (total_c * 1e-3)
    q_nf = per_q[:, : RING - 1]
    q_nf_bytes = sum(byt["nonflush_rc"][j] for j in range(1, RING)) * B
    q_win_bytes = q_nf_bytes + byt["flush_rc"] * B
    q_fl = float(per_q[:, RING - 1].mean())
    q_value = ntok / (total_q * 1e-3)
    read_copy = {"tokens_per_s": q_value, "window_ms": total_q / K, "window_alg_bytes": q_win_bytes,
                 "window_gbs": q_win_bytes / (total_q / K * 1e-3) / 1e9, "nonflush_avg_ms": float(q_nf.mean()),
                 "nonflush_gbs": q_nf_bytes / (q_nf.sum(axis=1).mean() * 1e-3) / 1e9,
                 "flush_ms": q_fl, "flush_gbs": byt["flush_rc"] * B / (q_fl * 1e-3) / 1e9,
                 "speedup_vs_fp32_replay": q_value / value, "speedup_vs_conventional": q_value / conv_value,
                 "bytes_ratio_conventional_over_read_copy": byt["conv"] * B * RING / q_win_bytes,
                 "note": "fp32 checkpoint, NVFP4 read copy; the flush re-solves, folds and writes both"}
    lowprec = {}
    for fmt, (total_l, per_l) in lp_runs.items():
        lb_ = byt["lowprec"][fmt]
        l_nf = per_l[:, : RING - 1]
        l_nf_bytes = sum(lb_["nonflush"][j] for j in range(1, RING)) * B
        l_win = l_nf_bytes + lb_["flush"] * B
        l_fl = float(per_l[:, RING - 1].mean())
        l_value = ntok / (total_l * 1e-3)
        lowprec[fmt] = {"tokens_per_s": l_value, "window_ms": total_l / K, "window_alg_bytes": l_win,
                        "window_gbs": l_win / (total_l / K * 1e-3) / 1e9, "nonflush_avg_ms": float(l_nf.mean()),
                        "nonflush_gbs": l_nf_bytes / (l_nf.sum(axis=1).mean() * 1e-3) / 1e9, "flush_ms": l_fl,
                        "flush_gbs": lb_["flush"] * B / (l_fl * 1e-3) / 1e9,
                        "speedup_vs_fp32_replay": l_value / value, "speedup_vs_conventional": l_value / conv_value}
    return {
        "metric": ("KDA" if kda_layer else "GDN") + "-layer decode tokens/s at batch 256 + achieved HBM GB/s vs conventional",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": warm, "ms_per_step": total_r / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_qk": w.n_qk, "n_v": w.n_v, "dk": w.dk, "dv": w.dv,
                   "inputs": "bf16", "checkpoint": "f32", "step": "one 16-token window: 15 non-flush + 1 flush"},
        "roofline": {"bound": "hbm", "achieved": nf_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nf_gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "gdn_nonflush_kernel",
                     "avg_launch_ms": float(nf_ms.mean()), "alg_bytes_per_launch": nf_bytes / (RING - 1)},
        "replay": {"tokens_per_s": value, "window_ms": total_r / K, "window_alg_bytes": win_bytes,
                   "window_gbs": win_bytes / (total_r / K * 1e-3) / 1e9, "nonflush_avg_ms": float(nf_ms.mean()),
                   "nonflush_by_fill_ms": [float(x) for x in nf_ms.mean(axis=0)],
                   "flush_ms": fl_ms, "flush_gbs": byt["flush"] * B / (fl_ms * 1e-3) / 1e9},
        "conventional": {"tokens_per_s": conv_value, "step_ms": cv_ms,
                         "gbs": byt["conv"] * B / (cv_ms * 1e-3) / 1e9},
        "speedup_vs_conventional": value / conv_value,
        "bytes_ratio_conventional_over_replay": byt["conv"] * B * RING / win_bytes,
        "read_copy": read_copy,
        "lowprec_checkpoints": lowprec,
    }


def bench_spec(args, torch, rs):
    w = W.M2_SPEC
    dev = "cuda"
    B, K = w.batch, w.max_draft
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    rl, rb = _m2_layer(rs, w, B, rs.RS_REPLAY, dev, max_draft=K)
    cl, cb = _m2_layer(rs, w, B, rs.RS_CONVENTIONAL, dev, max_draft=K)
    _m2_load_init(torch, rs, w, rl, rb, dev)
    rs.ckpt_f32_view(cl, cb).copy_(rs.ckpt_f32_view(rl, rb))
    rounds = args.spec_rounds
    # a pool of 8 rounds of draft inputs (reused cyclically) and the seeded acceptance of every round
    npool = min(rounds, 8)
    drafts = []
    for r in range(npool):
        toks = [W.m2_step(w, r * K + d, range(B)) for d in range(K)]
        drafts.append({k: _bf16_dev(torch, np.stack([t[k] for t in toks]), dev) for k in ("x", "B", "C", "dt")})
    accs_np = [W.accepted_counts(w.seed, r, B, K) for r in range(rounds)]
    accs = [torch.from_numpy(a).to(dev) for a in accs_np]
    committed = int(sum(a.sum() for a in accs_np))
    y = torch.empty(K, B, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    tm = Timer(torch)
    st = tm.stream

    def replay_all(ev):
        for r in range(rounds):
            _marked(ev, 2 * r, st, lambda: rs.rs_spec_append(rl, rb, drafts[r % npool], K, A, D, y))
            _marked(ev, 2 * r + 1, st, lambda: rs.rs_spec_commit(rl, rb, accs[r], A, D))

    def snap_all(ev):
        for r in range(rounds):
            _marked(ev, 2 * r, st, lambda: rs.rs_spec_append(cl, cb, drafts[r % npool], K, A, D, y))
            _marked(ev, 2 * r + 1, st, lambda: rs.rs_spec_commit(cl, cb, accs[r], A, D))

    # one timed "step" = all rounds; the buffer counters restart from empty for the timed pass
    total_r, per_r = tm.run(replay_all, 1, 1, 2 * rounds, reset=lambda: rb.meta.zero_())
    total_c, per_c = tm.run(snap_all, 1, 1, 2 * rounds)
    S = w.nheads * w.headdim * w.dstate * 4
    return {
        "metric": "speculative decode committed tokens/s at batch 512, 4 drafts (ReplaySSM vs snapshot/restore)",
        "value": committed / (total_r * 1e-3), "unit": "committed tokens/s", "n_gpus": 1, "steps": 1,
        "warmup": 1, "ms_per_step": total_r, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "drafts": K, "rounds": rounds, "accepted": "U{0..4} per round",
                   "mean_accepted": committed / (rounds * B), "step": f"{rounds} rounds of append + commit"},
        "replay": {"append_ms": float(per_r[0, 0::2].mean()), "commit_ms": float(per_r[0, 1::2].mean()),
                   "round_ms": total_r / rounds,
                   "append_ckpt_read_gbs": S * B / (per_r[0, 0::2].mean() * 1e-3) / 1e9},
        "snapshot_baseline": {"committed_tokens_per_s": committed / (total_c * 1e-3),
                              "append_ms": float(per_c[0, 0::2].mean()), "restore_ms": float(per_c[0, 1::2].mean()),
                              "round_ms": total_c / rounds},
        "speedup_vs_snapshot": total_c / total_r,
    }


def bench_gdn_spec(args, torch, rs, w=None):
    """Speculative decoding on the Qwen-style GDN layer (or KDA on its shapes):
    batch 256, 4 drafts per round, seeded acceptance U{0..4}; ReplaySSM (append
    with cached u rows, commit by pointer move, folds when room runs short) vs the
    snapshot/restore baseline."""
    w = W.GDN_SPEC if w is None else w
    layer_name = "KDA" if w.gate == "channel" else "GDN"
    dev = "cuda"
    B, K = w.batch, w.max_draft
    gp = W.gdn_params(w)

    def mk(mode):
        cfg = rs.make_config(rs.RS_KDA if w.gate == "channel" else rs.RS_GDN, B, mode=mode, n_qk_heads=w.n_qk, n_v_heads=w.n_v, head_k_dim=w.dk,
                             head_v_dim=w.dv, in_dtype=rs.RS_BF16, max_draft=K)
        _, layer = rs.rs_init(cfg)
        return layer, rs.alloc_buffers(layer, dev)

    rl, rb = mk(rs.RS_REPLAY)
    cl, cb = mk(rs.RS_CONVENTIONAL)
    ck = rs.ckpt_f32_view(rl, rb)
    for b in range(B):
        ck[b].copy_(torch.from_numpy(np.ascontiguousarray(W.gdn_init_state(w, b).transpose(0, 2, 1))).to(dev))
    rs.ckpt_f32_view(cl, cb).copy_(ck)
    rounds = args.spec_rounds
    npool = min(rounds, 8)
    drafts = []
    for r in range(npool):
        toks = [W.gdn_step(w, r * K + d, range(B), gp) for d in range(K)]
        d = {k: _bf16_dev(torch, np.stack([t[k] for t in toks]), dev) for k in ("q", "k", "v")}
        for k in ("g", "beta"):
            d[k] = torch.from_numpy(np.stack([t[k] for t in toks]).astype(np.float32)).to(dev)
        drafts.append(d)
    accs_np = [W.accepted_counts(w.seed, r, B, K) for r in range(rounds)]
    accs = [torch.from_numpy(a).to(dev) for a in accs_np]
    committed = int(sum(a.sum() for a in accs_np))
    o = torch.empty(K, B, w.n_v, w.dv, dtype=torch.float32, device=dev)
    tm = Timer(torch)
    st = tm.stream

    def replay_all(ev):
        for r in range(rounds):
            _marked(ev, 2 * r, st, lambda: rs.rs_spec_append(rl, rb, drafts[r % npool], K, None, None, o))
            _marked(ev, 2 * r + 1, st, lambda: rs.rs_spec_commit(rl, rb, accs[r], None, None))

    def snap_all(ev):
        for r in range(rounds):
            _marked(ev, 2 * r, st, lambda: rs.rs_spec_append(cl, cb, drafts[r % npool], K, None, None, o))
            _marked(ev, 2 * r + 1, st, lambda: rs.rs_spec_commit(cl, cb, accs[r], None, None))

    total_r, per_r = tm.run(replay_all, 1, 1, 2 * rounds, reset=lambda: rb.meta.zero_())
    total_c, per_c = tm.run(snap_all, 1, 1, 2 * rounds)
    S = w.n_v * w.dv * w.dk * 4
    return {
        "metric": f"{layer_name} speculative decode committed tokens/s at batch {B}, {K} drafts "
                  "(ReplaySSM vs snapshot/restore)",
        "value": committed / (total_r * 1e-3), "unit": "committed tokens/s", "n_gpus": 1, "steps": 1,
        "warmup": 1, "ms_per_step": total_r, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_qk": w.n_qk, "n_v": w.n_v, "dk": w.dk, "dv": w.dv,
                   "drafts": K, "rounds": rounds, "accepted": "U{0..4} per round",
                   "mean_accepted": committed / (rounds * B), "step": f"{rounds} rounds of append + commit"},
        "replay": {"append_ms": float(per_r[0, 0::2].mean()), "commit_ms": float(per_r[0, 1::2].mean()),
                   "round_ms": total_r / rounds,
                   "append_ckpt_read_gbs": S * B / (per_r[0, 0::2].mean() * 1e-3) / 1e9},
        "snapshot_baseline": {"committed_tokens_per_s": committed / (total_c * 1e-3),
                              "append_ms": float(per_c[0, 0::2].mean()), "restore_ms": float(per_c[0, 1::2].mean()),
                              "round_ms": total_c / rounds},
        "speedup_vs_snapshot": total_c / total_r,
    }


LOWPREC_VARIANTS = [("f32", None), ("f32", "nvfp4"), ("f16", "nvfp4"), ("fp8", "nvfp4"), ("f16", None),
                    ("fp8", None), ("nvfp4", None)]


def bench_lowprec(args, torch, rs):
    w = W.M2_LOWPREC
    if args.lowprec_batch:
        # the same layer at another batch (256: the step is HBM-bound there, the 256 MB
        # last-level cache no longer holds the state)
        w = w.with_(name=f"mamba2_lowprec_b{args.lowprec_batch}", batch=args.lowprec_batch)
    dev = "cuda"
    B = w.batch
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    code = {"f32": rs.RS_F32, "f16": rs.RS_F16, "fp8": rs.RS_FP8E4M3, "nvfp4": rs.RS_NVFP4}
    ebytes = {"f32": 4.0, "f16": 2.0, "fp8": 1.0 + 4.0 / 8192, "nvfp4": 0.5 + 1.0 / 16 + 4.0 / 8192}
    pool = _m2_pool(torch, w, B, dev)
    y = torch.empty(B, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    tm = Timer(torch)
    out = {"metric": f"low-precision-read decode tokens/s, Mamba-2 batch {B} (per checkpoint / read-copy format)",
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "batch": B, "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                      "note": (f"fp32 state {B * 4} MiB" + ("; fits the 256 MB last-level cache, GB/s are effective"
                                                             if B <= 64 else ""))},
           "variants": {}}
    for fmt, rc in LOWPREC_VARIANTS:
        layer, bufs = _m2_layer(rs, w, B, rs.RS_REPLAY, dev, ckpt=code[fmt],
                                read_copy=rs.RS_NVFP4 if rc else None, fuse=1)

        def window(ev):
            for t in range(RING):
                fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
                _marked(ev, t, tm.stream, lambda: fn(layer, bufs, pool[t], A, D, y))

        total, per = tm.run(window, args.steps, args.warmup, RING)
        byt = m2_bytes(w, ebytes[fmt], ebytes["nvfp4"] if rc else None)
        win_bytes = sum(byt["nonflush"].values()) * B + byt["flush"] * B
        name = fmt + ("+nvfp4_reads" if rc else "")
        out["variants"][name] = {"tokens_per_s": B * RING * args.steps / (total * 1e-3),
                                 "window_ms": total / args.steps, "window_alg_bytes": win_bytes,
                                 "window_gbs": win_bytes / (total / args.steps * 1e-3) / 1e9,
                                 "nonflush_avg_ms": float(per[:, :RING - 1].mean()),
                                 "flush_ms": float(per[:, RING - 1].mean())}
        del layer, bufs
        torch.cuda.empty_cache()
    out["value"] = out["variants"]["f32+nvfp4_reads"]["tokens_per_s"]
    out["ms_per_step"] = out["variants"]["f32+nvfp4_reads"]["window_ms"]
    if args.lowprec_error_steps:
        out["error_over_length"] = lowprec_error(args, torch, rs)
    return out


def lowprec_error(args, torch, rs):
    """Relative L2 error of y vs the fp64 recurrence over length, per format, on a
    few sequences of the low-precision workload (inputs drawn step by step).
    The GPU runs every head; the fp64 reference and the error cover every 8th
    head (heads are independent; head 8k keeps its B/C group k div 2 under the
    contiguous head-to-group map, so the sampled heads form a layer of their own)."""
    from oracle import decode
    w = W.M2_LOWPREC
    if args.lowprec_slow_decay:
        # stress run outside the C5 configuration: |A| in (0.002, 0.02) keeps ~99% of the
        # checkpoint across a 16-token window, so an error stored in it is carried over
        w = w.with_(name="mamba2_lowprec_b64_slow_decay", a_range=(0.002, 0.02))
    nb = args.lowprec_error_seqs
    dev = "cuda"
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    code = {"f32": rs.RS_F32, "f16": rs.RS_F16, "fp8": rs.RS_FP8E4M3, "nvfp4": rs.RS_NVFP4}
    layers = {}
    for fmt, rc in LOWPREC_VARIANTS:
        layers[fmt + ("+nvfp4_reads" if rc else "")] = _m2_layer(rs, w, nb, rs.RS_REPLAY, dev, ckpt=code[fmt],
                                                                 read_copy=rs.RS_NVFP4 if rc else None, fuse=1)
    hs = np.arange(0, w.nheads, 8)
    assert w.nheads % 8 == 0 and (w.nheads // w.ngroups) % 8 == 0
    exact = decode.M2Conventional(W.m2_init_states(w, range(nb))[:, hs], p["A"][hs], p["D"][hs])
    y = torch.empty(nb, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    steps = args.lowprec_error_steps
    every = max(1, steps // 16)
    curve = {k: [] for k in layers}
    acc = {k: [0.0, 0.0] for k in layers}
    for t in range(steps):
        tk = W.m2_step(w, t, range(nb))
        dtk = {k: _bf16_dev(torch, v, dev) for k, v in tk.items()}
        ye = exact.step({**tk, "x": tk["x"][:, hs], "dt": tk["dt"][:, hs]})
        for name, (layer, bufs) in layers.items():
            fn = rs.rs_step_flush if t % RING == RING - 1 else rs.rs_step_nonflush
            fn(layer, bufs, dtk, A, D, y)
            yg = y[:, hs].cpu().numpy().astype(np.float64)
            acc[name][0] += float(np.sum((yg - ye) ** 2))
            acc[name][1] += float(np.sum(ye ** 2))
        if (t + 1) % every == 0:
            for name in layers:
                curve[name].append([t + 1, (acc[name][0] / acc[name][1]) ** 0.5])
                acc[name] = [0.0, 0.0]
            print(f"lowprec error: step {t + 1} of {steps}", file=sys.stderr, flush=True)
    return {"workload": w.name, "a_range": list(w.a_range), "sequences": nb, "heads": [int(h) for h in hs],
            "steps": steps, "bucket_steps": every, "rel_l2_by_bucket": curve}


def delta_readcopy_error(args, torch, rs, w):
    """Relative L2 error of o vs the fp64 recurrence over length for a delta-rule
    layer (Qwen-style shapes, a few sequences, every head), with an fp32
    checkpoint, with and without the NVFP4 read copy (sitech.ge ReplaySSM page,
    "Bounding quantization error": 4-bit reads over a full-precision recurrence)."""
    from oracle import decode, gdn, kda
    nb, steps = args.delta_error_seqs, args.delta_error_steps
    w = w.with_(batch=nb)
    dev = "cuda"
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(nb))
    kind = rs.RS_KDA if w.gate == "channel" else rs.RS_GDN
    layers = {}
    for name, rc in (("f32", rs.RS_NONE), ("f32+nvfp4_reads", rs.RS_NVFP4)):
        cfg = rs.make_config(kind, nb, n_qk_heads=w.n_qk, n_v_heads=w.n_v, head_k_dim=w.dk, head_v_dim=w.dv,
                             in_dtype=rs.RS_BF16, read_copy=rc)
        _, layer = rs.rs_init(cfg)
        bufs = rs.alloc_buffers(layer, dev)
        rs.ckpt_f32_view(layer, bufs).copy_(torch.from_numpy(np.ascontiguousarray(
            S0.transpose(0, 1, 3, 2)).astype(np.float32)).to(dev))
        if rc:
            rs.rs_requant_read_copy(layer, bufs)
        layers[name] = (layer, bufs)
    exact = decode.GDNConventional(S0, rule=kda if w.gate == "channel" else gdn)
    o = torch.empty(nb, w.n_v, w.dv, dtype=torch.float32, device=dev)
    every = max(1, steps // 16)
    curve = {k: [] for k in layers}
    acc = {k: [0.0, 0.0] for k in layers}
    for t in range(steps):
        tk = W.gdn_step(w, t, range(nb), gp)
        d = {k: _bf16_dev(torch, tk[k], dev) for k in ("q", "k", "v")}
        d["g"] = torch.from_numpy(tk["g"]).to(dev)
        d["beta"] = torch.from_numpy(tk["beta"]).to(dev)
        oe = exact.step(tk)
        for name, (layer, bufs) in layers.items():
            fn = rs.rs_step_flush if t % RING == RING - 1 else rs.rs_step_nonflush
            fn(layer, bufs, d, None, None, o)
            og = o.cpu().numpy().astype(np.float64)
            acc[name][0] += float(np.sum((og - oe) ** 2))
            acc[name][1] += float(np.sum(oe ** 2))
        if (t + 1) % every == 0:
            for name in layers:
                curve[name].append([t + 1, (acc[name][0] / acc[name][1]) ** 0.5])
                acc[name] = [0.0, 0.0]
            print(f"{w.name} read-copy error: step {t + 1} of {steps}", file=sys.stderr, flush=True)
    return {"workload": w.name, "sequences": nb, "steps": steps, "bucket_steps": every, "rel_l2_by_bucket": curve}


def probe_read_gbs(torch, tm, nbytes=1 << 30, threads=256, per=8, steps=10, warmup=2, write_bytes=0):
    """Bandwidth of a plain stream of the decode kernels' 32 KiB tiles over
    nbytes of device memory (librs_probe.so): read only (rs_probe_read), or
    with write_bytes written per tile after its sum (rs_probe_read_write),
    counting the bytes read plus the bytes written."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "ssm_decode_checkpoint_amd", "librs_probe.so"))
    probe.rs_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p]
    probe.rs_probe_read.restype = ctypes.c_int32
    probe.rs_probe_read_write.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    probe.rs_probe_read_write.restype = ctypes.c_int32
    tiles = nbytes // (16 * threads * per)
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    if write_bytes:
        dst = torch.empty(tiles * write_bytes, dtype=torch.uint8, device="cuda")
    else:
        dst = torch.empty(tiles, dtype=torch.float32, device="cuda")

    def call():
        if write_bytes:
            st = probe.rs_probe_read_write(src.data_ptr(), dst.data_ptr(), nbytes, threads, per, write_bytes,
                                           tm.stream.cuda_stream)
        else:
            st = probe.rs_probe_read(src.data_ptr(), dst.data_ptr(), nbytes, threads, per, tm.stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"librs_probe returned {st}")

    _, per_ms = tm.run(lambda ev: _marked(ev, 0, tm.stream, call), steps, warmup, 1)
    return (nbytes + tiles * write_bytes) / (float(per_ms.mean()) * 1e-3) / 1e9


PROBE_VARIANTS = ("reg_256x8_nt", "reg_256x8_plain", "reg_256x16_nt", "lds_256x8", "lds_256x16",
                  "persistent_256x8_pairs")


def probe_variant_gbs(torch, tm, nbytes, variant, steps=10, warmup=2):
    """Read bandwidth of one rs_probe_read_variant scheme over nbytes."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "ssm_decode_checkpoint_amd", "librs_probe.so"))
    probe.rs_probe_read_variant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32,
                                            ctypes.c_void_p]
    probe.rs_probe_read_variant.restype = ctypes.c_int32
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    out = torch.empty(nbytes // (32 << 10), dtype=torch.float32, device="cuda")

    def call():
        st = probe.rs_probe_read_variant(src.data_ptr(), out.data_ptr(), nbytes, variant, tm.stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"librs_probe returned {st}")

    _, per_ms = tm.run(lambda ev: _marked(ev, 0, tm.stream, call), steps, warmup, 1)
    return nbytes / (float(per_ms.mean()) * 1e-3) / 1e9


def m2_writes_per_tile(w, s_in=2):
    """Bytes a Mamba-2 non-flush step writes per (sequence, head) tile: y in
    fp32, the appended x row and dt, and the head's share of the group's B and
    C rows; rounded to a whole number of 16-byte stores."""
    b = w.headdim * 4 + w.headdim * s_in + s_in + 2 * w.ngroups * w.dstate * s_in // w.nheads
    return 16 * max(1, round(b / 16))


def bench_copy(args, torch, rs):
    """A plain 1 GiB device copy (torch's copy kernel): the known-size reference
    that HBM traffic counters are scaled by."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    tm = Timer(torch)
    total, per = tm.run(lambda ev: _marked(ev, 0, tm.stream, lambda: dst.copy_(src)), args.steps, args.warmup, 1)
    ms = float(per.mean())
    # a plain read of the same 1 GiB (torch's sum over fp32): a reference for what a
    # read-only stream reaches on this chip
    srcf = src.view(torch.float32)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    rtot, rper = tm.run(lambda ev: _marked(ev, 0, tm.stream, lambda: torch.sum(srcf, dim=0, out=acc)), args.steps,
                        args.warmup, 1)
    rms = float(rper.mean())
    # the read-only stream with the decode kernels' tile shapes (librs_probe.so)
    del dst
    tiles = {}
    for threads, per in ((256, 8), (256, 4), (128, 16)):
        tiles[f"{threads}x{per}"] = {"tile_kib": threads * per * 16 // 1024,
                                     "gbs": probe_read_gbs(torch, tm, n, threads, per, args.steps, args.warmup)}
    # other ways to stream the same bytes (rs_probe_read_variant): larger tiles,
    # global-to-LDS loads, persistent workgroups, cached loads
    variants = {}
    for v, name in enumerate(PROBE_VARIANTS):
        variants[name] = probe_variant_gbs(torch, tm, n, v, args.steps, args.warmup)
    # the 32 KiB tile stream with a write per tile after its sum, as a decode step
    # writes its output and appended record: what those writes cost in a read stream
    writes = {}
    for wb in (128, 256, 416, 1024, 4096):
        writes[str(wb)] = probe_read_gbs(torch, tm, n, 256, 8, args.steps, args.warmup, write_bytes=wb)
    return {"metric": "device copy GB/s (read + write)", "value": 2 * n / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "config": {"workload": "copy_1GiB", "bytes_read": n, "bytes_written": n},
            "read_reference": {"what": "torch.sum over the same 1 GiB (read only)", "ms": rms,
                               "gbs": n / (rms * 1e-3) / 1e9},
            "read_probe": {"what": "1 GiB read as tiles of threads x 16-byte non-temporal loads per workgroup "
                                   "(rs_probe_read); 256x8 is the decode kernels' 32 KiB state tile",
                           "tiles": tiles,
                           "variants_gbs": variants},
            "read_write_probe": {"what": "the 256x8 tile read with write_bytes written per tile after its sum "
                                         "(rs_probe_read_write); GB/s of bytes read plus written",
                                 "gbs_by_write_bytes": writes}}


# legs the default run times after the headline, and the figures of each that its line carries
OTHER_LEGS = ("gdn", "kda", "spec", "gdn_spec", "kda_spec", "lowprec")
SUMMARY_KEYS = ("value", "unit", "speedup_vs_conventional", "speedup_vs_snapshot", "roofline.frac",
                "replay.nonflush_avg_ms", "replay.flush_ms", "replay.append_ms", "read_copy.tokens_per_s",
                "read_copy.speedup_vs_fp32_replay", "lowprec_checkpoints.f16.tokens_per_s",
                "lowprec_checkpoints.fp8.tokens_per_s")


def leg_summary(out: dict) -> dict:
    """The figures of one leg's output that the headline line repeats."""
    summ = {"workload": out.get("config", {}).get("workload")}
    for key in SUMMARY_KEYS:
        v = out
        for part in key.split("."):
            v = v.get(part) if isinstance(v, dict) else None
        if v is not None:
            summ[key] = v
    for name, var in out.get("variants", {}).items():
        summ[f"variants.{name}.tokens_per_s"] = var.get("tokens_per_s")
    return summ


def other_workloads(args, torch, fns, rs) -> dict:
    """Run the other layers' legs (Gated DeltaNet, KDA, speculative, low precision) after the
    headline, with the same step counts, and return a summary of each."""
    res = {}
    for wl in OTHER_LEGS:
        torch.cuda.empty_cache()
        t0 = time.time()
        res[wl] = leg_summary(fns[wl](args, torch, rs))
        res[wl]["wall_s"] = round(time.time() - t0, 1)
        print(f"bench: {wl} leg done in {res[wl]['wall_s']} s", file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed windows")
    ap.add_argument("--warmup", type=int, default=3, help="untimed windows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--workload", action="append",
                    choices=["mamba2", "gdn", "kda", "spec", "gdn_spec", "kda_spec", "lowprec", "copy", "sweep",
                             "serve", "block"],
                    help="workloads to run, one JSON line each; repeat for several (default: mamba2, whose line "
                         "also summarises the gdn, kda, spec, gdn_spec, kda_spec and lowprec legs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="default run: skip the other layers' legs that the headline line summarises")
    ap.add_argument("--spec-rounds", type=int, default=64)
    ap.add_argument("--lowprec-error-steps", type=int, default=0)
    ap.add_argument("--lowprec-error-seqs", type=int, default=2)
    ap.add_argument("--lowprec-batch", type=int, default=0, help="batch of the low-precision workload (0: 64)")
    ap.add_argument("--delta-error-steps", type=int, default=0,
                    help="gdn / kda: error over length with and without the NVFP4 read copy")
    ap.add_argument("--delta-error-seqs", type=int, default=2)
    ap.add_argument("--lowprec-slow-decay", action="store_true",
                    help="error run with slowly decaying heads (outside the C5 configuration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode step needs no "
              f"collective, so N GPUs would each run this single-GPU workload on their own batch shard.",
              file=sys.stderr)
        sys.exit(2)
    wls = args.workload or ["mamba2"]
    # the CPU oracle leg forks worker processes: before anything touches the GPU
    cpu = cpu_baseline(W.M2_NEMOTRON) if ("mamba2" in wls and not args.no_cpu) else None
    import torch
    import ssm_decode_checkpoint_amd as rs
    torch.cuda.set_device(0)
    fns = {"mamba2": bench_mamba2, "gdn": bench_gdn, "spec": bench_spec, "lowprec": bench_lowprec,
           "sweep": bench_sweep, "gdn_spec": bench_gdn_spec, "serve": bench_serve, "block": bench_block,
           "kda": lambda a, t, r: bench_gdn(a, t, r, W.KDA_B256),
           "kda_spec": lambda a, t, r: bench_gdn_spec(a, t, r,
                                                      W.KDA_B256.with_(name="kda_spec_b256", max_draft=4)),
           "copy": bench_copy}
    for wl in wls:
        out = fns[wl](args, torch, rs)
        if wl in ("gdn", "kda") and args.delta_error_steps:
            out["read_copy_error_over_length"] = delta_readcopy_error(args, torch, rs,
                                                                      W.GDN_QWEN if wl == "gdn" else W.KDA_B256)
        if wl == "mamba2":
            out["cpu_baseline"] = cpu
            if args.workload is None and not args.headline_only:
                out["other_workloads"] = other_workloads(args, torch, fns, rs)
        print(json.dumps(out), flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
