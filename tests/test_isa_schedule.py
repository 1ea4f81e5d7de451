"""The step kernels' load order, checked on the gfx950 assembly hipcc emits
(CPU only: hipcc cross-compiles, nothing runs).

The kernels are written so that a workgroup issues its buffer-record and
parameter loads first and the state tile's non-temporal loads after them:
vector loads return in issue order, so the state-independent work (staging,
dots, decay weights) can run while the tile streams in. A load placed, or
scheduled, behind the tile makes the first wait on it a wait for the whole
tile, and the workgroup barrier after the staging then holds every wave until
the tile has arrived. Here: between the first non-temporal load and the first
s_barrier of each step kernel there is no `s_waitcnt vmcnt(0)`.

The exception, by measurement: the Mamba-2 flushes that fold on the matrix
cores (FP8 and NVFP4 checkpoints, FP16 with the read copy, on 64-multiple
shapes) issue the checkpoint tile before the counters and records, so their
first barrier does wait for it; that is checked too.

Also pinned: the occupancy the dominant kernels were tuned for (8 waves per
SIMD for the fp32-read non-flush and flush kernels, 6 for the wave-per-head
kernel on FP8 and NVFP4 reads), from the compiler's resource-usage remarks.
"""
import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from ssm_decode_checkpoint_amd import build as B  # noqa: E402

SOURCES = ["rs_m2_128x64.hip", "rs_gdn.hip"]
# kernels whose first barrier follows the record staging (replay step kernels
# and the baselines that load their inputs first)
STEP_KERNELS = ("m2_nonflush_kernel", "m2_nonflush_wave_kernel", "m2_flush_kernel", "m2_auto_kernel",
                "m2_spec_append_kernel", "m2_commit_fold_kernel", "m2_conv_kernel", "m2_conv_spec_kernel",
                "gdn_nonflush_kernel", "gdn_flush_kernel", "gdn_auto_kernel", "gdn_spec_append_kernel",
                "gdn_commit_fold_kernel", "gdn_conv_kernel", "gdn_conv_spec_kernel")


def _compile(src, out_dir):
    s = os.path.join(out_dir, src + ".s")
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           "-Rpass-analysis=kernel-resource-usage", os.path.join(B.CSRC, src), "-o", s]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(s).read(), r.stderr


@pytest.fixture(scope="module")
def isa():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="rs_isa_")
    try:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            outs = list(ex.map(lambda s: _compile(s, d), SOURCES))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    kernels, usage = {}, {}
    for asm, remarks in outs:
        cur = None
        for line in asm.split("\n"):
            m = re.match(r"^(_Z\w+):", line)
            if m:
                cur = m.group(1)
                kernels[cur] = []
            elif cur is not None:
                kernels[cur].append(line)
        cur = None
        for line in remarks.split("\n"):
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = m.group(1)
                continue
            m = re.search(r"(VGPRs|Occupancy \[waves/SIMD\]|VGPRs Spill): (\d+)", line)
            if m and cur:
                usage.setdefault(cur, {})[m.group(1)] = int(m.group(2))
    return kernels, usage


def _first_barrier_waits_all(lines):
    loads = [i for i, l in enumerate(lines) if "global_load" in l and " nt" in l]
    if not loads:
        return None
    bars = [i for i in range(loads[0], len(lines)) if "s_barrier" in lines[i]]
    if not bars:
        return None
    return any(re.search(r"s_waitcnt vmcnt\(0\)", lines[i]) for i in range(loads[0], bars[0]))


def _tile_first(name):
    """Mamba-2 flush (or self-scheduling) kernels whose fold runs on the matrix cores."""
    m = re.search(r"m2_(?:flush|auto)_kernelI(?:NS_4bf16E|f)Li(\d)ELb([01])ELi(\d+)ELi(\d+)E", name)
    if not m:
        return False
    ckf, rc, nr, nc = (int(x) for x in m.groups())
    return nr % 64 == 0 and nc % 64 == 0 and (ckf in (2, 3) or (ckf == 1 and rc == 1))


def test_records_stay_ahead_of_the_state_tile(isa):
    kernels, _ = isa
    checked, bad, first = 0, [], 0
    for name, lines in kernels.items():
        if not any(k in name for k in STEP_KERNELS):
            continue
        r = _first_barrier_waits_all(lines)
        if r is None:
            continue
        checked += 1
        if _tile_first(name) and "m2_flush_kernel" in name:
            first += 1
            if not r:
                bad.append(("tile not first", name))
        elif _tile_first(name):
            continue   # the self-scheduling kernel holds both orders behind its branch
        elif r:
            bad.append(name)
    assert checked >= 40, checked
    assert first == 10, first   # ({fp8, NVFP4} x {copy, none} + fp16 with the copy) x {bf16, fp32 inputs}
    assert not bad, bad


def _usage(usage, pattern):
    hits = {k: v for k, v in usage.items() if re.search(pattern, k)}
    assert hits, pattern
    return hits


def test_dominant_kernels_keep_their_occupancy(isa):
    _, usage = isa
    # m2_nonflush_kernel / m2_flush_kernel <bf16, FMT_F32 (0), 128, 64>
    for pat in (r"m2_nonflush_kernelINS_4bf16ELi0ELi128ELi64E", r"m2_flush_kernelINS_4bf16ELi0ELb[01]ELi128ELi64E"):
        for k, v in _usage(usage, pat).items():
            assert v["Occupancy [waves/SIMD]"] == 8, (k, v)
    # wave-per-head kernel, FP8 (2) and NVFP4 (3) reads with bf16 records
    for k, v in _usage(usage, r"m2_nonflush_wave_kernelINS_4bf16ELi[23]ELi128ELi64E").items():
        assert v["Occupancy [waves/SIMD]"] >= 6, (k, v)


def test_fold_layout_per_format(isa):
    """The rank-16 fold runs on the matrix cores (v_mfma_f32_16x16x4_f32) for the
    FP8 and NVFP4 checkpoints and for FP16 with the read copy, and on the
    streaming layout's VALU FMAs for fp32 checkpoints (traffic-bound there)."""
    kernels, _ = isa

    def has_mfma(pat):
        hits = [k for k in kernels if re.search(pat, k)]
        assert hits, pat
        return all(any("v_mfma_f32_16x16x4" in l for l in kernels[k]) for k in hits), \
            any(any("v_mfma_f32_16x16x4" in l for l in kernels[k]) for k in hits)

    for fmt_rc in ("Li2ELb0", "Li2ELb1", "Li3ELb0", "Li1ELb1"):
        for kern in ("m2_flush_kernel", "m2_commit_fold_kernel"):
            every, _ = has_mfma(rf"{kern}INS_4bf16E{fmt_rc}ELi128ELi64E")
            assert every, (kern, fmt_rc)
    for fmt_rc in ("Li0ELb0", "Li0ELb1", "Li1ELb0"):
        _, some = has_mfma(rf"m2_flush_kernelINS_4bf16E{fmt_rc}ELi128ELi64E")
        assert not some, fmt_rc
