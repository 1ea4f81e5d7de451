"""The committed profile summaries are reproducible from committed files: every
rocprofv3 command in profiles/ profiles `bench.py` at the repository root
(nothing under a working directory), names an output directory under
gpurun_out/, and asks for at most one hardware counter block's worth of
counters per pass (FETCH_SIZE and WRITE_SIZE each in a pass of their own)."""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _commands():
    out = []
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(p):
            if line.startswith("cd /tmp") and "rocprofv3" in line:
                out.append((os.path.basename(p), line.strip()))
    return out


def test_every_summary_gives_its_command():
    names = {n for n, _ in _commands()}
    mds = {os.path.basename(p) for p in glob.glob(os.path.join(ROOT, "profiles", "*.md"))}
    assert mds and names == mds, mds - names


def test_commands_run_committed_files_only():
    for name, cmd in _commands():
        prog = cmd.split(" -- ", 1)
        assert len(prog) == 2, (name, cmd)
        assert re.match(r"python3 \$REPO/bench\.py( |$)", prog[1]), (name, cmd)
        assert "_work" not in cmd, (name, cmd)
        assert re.search(r"-d \$REPO/gpurun_out/\w+", cmd), (name, cmd)
        for flag in re.findall(r"--workload (\w+)", prog[1]):
            assert flag in ("mamba2", "gdn", "kda", "spec", "gdn_spec", "kda_spec", "lowprec", "copy", "sweep",
                            "serve", "block"), (name, flag)


def test_counter_passes_fit_the_hardware():
    for name, cmd in _commands():
        m = re.search(r"--pmc ((?:[A-Z_0-9]+ ?)+)", cmd)
        if not m:
            continue
        ctrs = m.group(1).split()
        if "FETCH_SIZE" in ctrs or "WRITE_SIZE" in ctrs:
            assert ctrs in (["FETCH_SIZE"], ["WRITE_SIZE"]), (name, ctrs)
        assert sum(c.startswith("SQ_") for c in ctrs) <= 8, (name, ctrs)
        assert sum(c.startswith("GRBM_") for c in ctrs) <= 2, (name, ctrs)
