"""Benchmark: ReplaySSM SSM-layer decode on one MI355X vs the same-GPU conventional kernel.

Default workload: the Nemotron-style Mamba-2 layer at serving batch 256
(128 heads, headdim 64, dstate 128, 8 groups, bf16 inputs, fp32 checkpoint,
4 MiB of state per sequence), seeded synthetic inputs resident in HBM.

One "step" is one full buffer window: 15 non-flush steps (append + output
from checkpoint and buffer) and one flush step (fold, one checkpoint write),
i.e. 16 decode tokens for all 256 sequences; `value` is decode tokens/s over
the K timed windows. The conventional read-modify-write kernel is timed on
the same windows for comparison.

Prints one JSON line with the roofline of the dominant kernel (the non-flush
step) measured with HIP events on the launch stream, and the fp64 CPU oracle
timed on a bounded sample of the same workload.
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
METRIC = "SSM-layer decode tokens/s at batch 256 + achieved HBM GB/s (% of peak) vs conventional"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["ssm_decode_checkpoint_amd/csrc/rs_mamba2_kernels.h", "ssm_decode_checkpoint_amd/csrc/rs_tile.h",
                  "ssm_decode_checkpoint_amd/csrc/rs_device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes per sequence (what the method must move; cache effects not counted)
# ---------------------------------------------------------------------------

def m2_bytes(w: W.Mamba2Workload):
    s_in = 2 if w.in_dtype == "bf16" else 4
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    S = H * P * N * 4
    E_in = (H * P + 2 * G * N + H) * s_in      # x, B, C, dt of the current token
    E_old = (H * P + G * N + H) * s_in         # x, B, dt of a held entry (C is not re-read)
    Y = H * P * 4
    nonflush = {j: S + (j - 1) * E_old + 2 * E_in + Y for j in range(1, RING)}
    flush = 2 * S + (RING - 1) * E_old + E_in + Y
    conv = 2 * S + E_in + Y
    return {"state": S, "E_in": E_in, "E_old": E_old, "Y": Y, "nonflush": nonflush, "flush": flush, "conv": conv}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(w: W.Mamba2Workload, nseq: int, windows: int = 1):
    from oracle import decode
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    p = W.m2_params(w)
    seqs = list(range(nseq))
    H0 = W.m2_init_states(w, seqs)
    toks = [W.m2_step(w, t, seqs) for t in range(RING * windows)]
    rep = decode.M2Replay(H0, p["A"], p["D"])
    c0, t0 = time.process_time(), time.perf_counter()
    for tk in toks:
        rep.step(tk)
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    if limiter is not None:
        limiter.unregister()
    ntok = nseq * RING * windows
    return {"value": ntok / wall, "unit": "tokens/s", "cores": max(1, int(round(cpu / wall))), "kind": "oracle",
            "sample": f"fp64 ReplaySSM oracle (checkpoint + buffer, plain numpy) on {nseq} of {w.batch} sequences "
                      f"x {RING * windows} decode steps ({windows} window) of the {w.name} workload; "
                      f"{wall:.1f} s wall, {cpu:.1f} s CPU"}


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------

def traffic_from_profile(name: str, launch_bytes_alg: float):
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


def run_gpu(args):
    import torch
    import ssm_decode_checkpoint_amd as rs
    from ssm_decode_checkpoint_amd import RS_CONVENTIONAL, RS_REPLAY

    w = W.M2_NEMOTRON
    dev = "cuda"
    torch.cuda.set_device(0)
    B = w.batch
    p = W.m2_params(w)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)

    def mk(mode):
        cfg = rs.make_config(rs.RS_MAMBA2, B, mode=mode, nheads=w.nheads, headdim=w.headdim, dstate=w.dstate,
                             ngroups=w.ngroups, in_dtype=rs.RS_BF16, ckpt_dtype=rs.RS_F32)
        _, layer = rs.rs_init(cfg)
        return layer, rs.alloc_buffers(layer, dev)

    rl, rb = mk(RS_REPLAY)
    cl, cb = mk(RS_CONVENTIONAL)
    # initial checkpoint N(0, 0.1^2) from the seeded generator, stored [b][h][N][P]
    ck = rs.ckpt_f32_view(rl, rb)
    for b in range(B):
        ck[b].copy_(torch.from_numpy(np.ascontiguousarray(W.m2_init_state(w, b).transpose(0, 2, 1))))
    rs.ckpt_f32_view(cl, cb).copy_(ck)
    # one window of seeded step inputs, resident in HBM, reused every window
    pool = []
    for t in range(RING):
        tk = W.m2_step(w, t, range(B))
        pool.append({k: torch.from_numpy(W.bf16_bits(v).view(np.int16).copy()).view(torch.bfloat16).to(dev)
                     for k, v in tk.items()})
    y = torch.empty(B, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def replay_window(ev=None):
        for t in range(RING):
            if ev is not None:
                ev[t][0].record(stream)
            if t == RING - 1:
                rs.rs_step_flush(rl, rb, pool[t], A, D, y)
            else:
                rs.rs_step_nonflush(rl, rb, pool[t], A, D, y)
            if ev is not None:
                ev[t][1].record(stream)

    def conv_window(ev=None):
        for t in range(RING):
            if ev is not None:
                ev[t][0].record(stream)
            rs.rs_step_conventional(cl, cb, pool[t], A, D, y)
            if ev is not None:
                ev[t][1].record(stream)

    def timed(fn, K, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(RING)] for _ in range(K)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for k in range(K):
            fn(evs[k])
        t1.record(stream)
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1)
        per = np.array([[evs[k][t][0].elapsed_time(evs[k][t][1]) for t in range(RING)] for k in range(K)])
        return total, per

    K, warm = args.steps, args.warmup
    wall0 = time.perf_counter()
    total_r, per_r = timed(replay_window, K, warm)
    total_c, per_c = timed(conv_window, K, warm)
    wall = time.perf_counter() - wall0

    byt = m2_bytes(w)
    ntok = B * RING * K
    value = ntok / (total_r * 1e-3)
    conv_value = ntok / (total_c * 1e-3)
    # dominant kernel: the non-flush step (15 of 16 launches per window)
    nf_ms = per_r[:, : RING - 1]
    nf_bytes = sum(byt["nonflush"][j] for j in range(1, RING)) * B      # one window of non-flush launches
    nf_avg_ms = float(nf_ms.mean())
    nf_avg_bytes = nf_bytes / (RING - 1)
    nf_gbs = nf_bytes / (nf_ms.sum(axis=1).mean() * 1e-3) / 1e9
    fl_ms = float(per_r[:, RING - 1].mean())
    fl_gbs = byt["flush"] * B / (fl_ms * 1e-3) / 1e9
    cv_ms = float(per_c.mean())
    cv_gbs = byt["conv"] * B / (cv_ms * 1e-3) / 1e9
    win_bytes = nf_bytes + byt["flush"] * B
    win_ms = total_r / K
    traffic = traffic_from_profile("m2_nonflush_b256", nf_avg_bytes)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm,
        "ms_per_step": win_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                   "ngroups": w.ngroups, "inputs": "bf16", "checkpoint": "f32", "ring": RING,
                   "step": "one 16-token window: 15 non-flush + 1 flush", "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": nf_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nf_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "m2_nonflush_kernel", "avg_launch_ms": nf_avg_ms,
                     "alg_bytes_per_launch": nf_avg_bytes},
        "replay": {"tokens_per_s": value, "window_ms": win_ms, "window_alg_bytes": win_bytes,
                   "window_gbs": win_bytes / (win_ms * 1e-3) / 1e9,
                   "nonflush_avg_ms": nf_avg_ms, "nonflush_gbs": nf_gbs,
                   "flush_ms": fl_ms, "flush_gbs": fl_gbs},
        "conventional": {"tokens_per_s": conv_value, "step_ms": cv_ms, "gbs": cv_gbs,
                         "window_ms": total_c / K, "window_alg_bytes": byt["conv"] * B * RING},
        "speedup_vs_conventional": value / conv_value,
        "bytes_ratio_conventional_over_replay": byt["conv"] * B * RING / win_bytes,
        "gpu_wall_s": wall,
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed windows")
    ap.add_argument("--warmup", type=int, default=3, help="untimed windows")
    ap.add_argument("--cpu-seqs", type=int, default=256, help="sequences in the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode step needs no "
              f"collective, so N GPUs would each run this single-GPU workload on their own batch shard.",
              file=sys.stderr)
        sys.exit(2)
    out = run_gpu(args)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(W.M2_NEMOTRON, args.cpu_seqs, windows=2)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
