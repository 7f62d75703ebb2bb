"""FMOE_LOG=1: every layer call prints its plan to stderr (read once per process, so the call
runs in a child process), and the output is the same as without the log."""
import os
import subprocess
import sys

import pytest

from gpu_common import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import torch
import mixture_experts_layer_sigmoid_amd as fm
from mixture_experts_layer_sigmoid_amd import synth
T, H, I, E, k = 40, 256, 128, 8, 2
L = synth.tiny_layer(T, H, E, I, seed=3)
logits = synth.routed_logits(5, T, E, k, "uniform").cuda()
shape = fm.make_shape(T, H, I, E, k)
w = fm.ExpertWeights(L["wg"].cuda(), L["wu"].cuda(), L["wd"].cuda())
out = fm.fmoe_forward(shape, L["x"].cuda(), logits, w)
torch.cuda.synchronize()
torch.save(out.cpu(), OUT)
"""


def run_child(log: str, out_path: str):
    env = dict(os.environ, FMOE_LOG=log, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    code = SCRIPT.replace("OUT", repr(out_path))
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)


def test_fmoe_log_prints_the_plan(tmp_path):
    announce("FMOE_LOG=1 plan print (child processes)")
    import torch
    on = run_child("1", str(tmp_path / "on.pt"))
    assert on.returncode == 0, on.stderr[-2000:]
    lines = [l for l in on.stderr.splitlines() if l.startswith("[fmoe] fmoe_forward:")]
    assert len(lines) == 1, on.stderr[-2000:]
    for field in ("T=40", "H=256", "I=128", "E=8", "k=2", "bf16", "rows_estimate=10", "tile_rows=32",
                  "heavy5=", "split_gate_up=", "workspace="):
        assert field in lines[0], lines[0]
    off = run_child("0", str(tmp_path / "off.pt"))
    assert off.returncode == 0, off.stderr[-2000:]
    assert "[fmoe]" not in off.stderr
    assert torch.equal(torch.load(tmp_path / "on.pt", weights_only=True),
                       torch.load(tmp_path / "off.pt", weights_only=True))
