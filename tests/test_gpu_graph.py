"""A grouped step captured into a HIP graph and replayed equals the same
steps run eagerly, bit for bit: every Muon weight and momentum buffer and
every AdamW weight and moment, after each of several replays, with eager
work and synchronisations between the replays.  AdamW's bias correction
follows the plan's device step count, so each replay takes the correction
of its own step (a host count would stay at the captured step's)."""
import pytest
import torch

import workloads as wl
from adamw_optimizer_step_amd import api
from gpu_common import build_entries, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _workload():
    # Gram-space GEMM, plain GEMM and slice-resident slices (the step's three
    # Newton-Schulz chains, on two streams) beside AdamW params
    ps = [wl.ParamSpec("embed", (256, 64), "bf16", wl.ROLE_EMBEDDING, no_decay=True),
          wl.ParamSpec("norm", (64,), "bf16", wl.ROLE_NORM, no_decay=True),
          wl.ParamSpec("square", (384, 384), "bf16"),
          wl.ParamSpec("wide", (256, 640), "bf16"),
          wl.ParamSpec("head", (128, 512), "bf16")]
    return wl.Workload("graph_replay", 17, tuple(ps), grad_std=1e-3)


def _state(ents):
    return [e[k].clone() for e in ents
            for k in ("param", "momentum", "exp_avg", "exp_avg_sq") if k in e]


def _run(w, graph: bool, replays: int):
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(muon_wd=0.1))
    ws = plan.workspace(torch.device("cuda"))
    # the same gradients at every step: a graph reads the tensors it captured
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(wl.grad(w, i, 1), p.dtype))
    plan.step(workspace=ws)   # uploads the tables and creates the side streams
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
            plan.step(workspace=ws)   # recorded, not run
        torch.cuda.synchronize()
    states = []
    for _ in range(replays):
        if graph:
            g.replay()
        else:
            plan.step(workspace=ws)
        torch.cuda.synchronize()
        states.append(_state(ents))
        # unrelated eager work between the replays
        torch.randn(1 << 20, device="cuda").square().sum().item()
        torch.cuda.synchronize()
    return states


def test_graph_replay_equals_eager_steps():
    require_gpu()
    w = _workload()
    print("[graph] eager steps", flush=True)
    eager = _run(w, graph=False, replays=3)
    print("[graph] replays", flush=True)
    replayed = _run(w, graph=True, replays=3)
    for k, (a, b) in enumerate(zip(eager, replayed)):
        assert len(a) == len(b)
        for j, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"step {k + 2}, tensor {j}"
