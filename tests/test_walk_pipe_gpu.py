"""The walk's one-launch forms against the walk in three launches (walk_prep,
the walk, walk_keys): the same arithmetic, so every output agrees bit for bit.

osdn_precond_scan runs in one launch (walk_prep, the walk and walk_keys, the
records and the walk's results handed over through two flags per chunk in
the workspace) with the workspace of osdn_precond_scan_workspace_bytes, and
in three launches with 16 bytes per (b, h, chunk) less; its d_all and k_tilde
expose the walk's result for every chunk.  osdn_forward runs walk_prep and the
walk in one launch.  Also calls that reuse one workspace, whose flags then
hold earlier calls' values, and repeated calls (a race between the launch's
workgroups would show as a difference between them)."""
import pytest
import torch

import delta_rule_recurrent_precond_amd as osdn
from delta_rule_recurrent_precond_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    osdn.load()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _inputs(B, H, T, seed, apf=True):
    w = W.custom(B, H, T, 128, 128, 64, dtype="bf16", eta=0.05, apf=apf, seed=seed)
    return W.generate(w).to("cuda")


def _scan(dev, one_launch, want=True, ws=None):
    B, H, T, dk = dev.k.shape
    if ws is None:
        full = osdn.precond_scan_workspace_bytes(B, H, T, dk, 0)
        n = full if one_launch else full - 16 * B * H * ((T + 63) // 64)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    return osdn.precond_scan(dev.k, dev.beta, dev.r, eta=0.05, want_d_all=want,
                             want_log_ratio=want, workspace=ws)


def _equal(a, b, label):
    for key in ("k_tilde", "d_final", "d_all", "log_ratio"):
        if key in a or key in b:
            assert torch.equal(a[key], b[key]), (label, key)


# (B, H, T): one chunk, a single token, ragged tails, fewer chunks than the
# walk keeps in flight, the workloads' shapes, head counts at the one-launch
# limit (B*H = half of MI355X's 256 compute units: as many preparing workgroups
# as walks) and past it, which take the walk in three launches
SHAPES = [(1, 1, 64), (1, 1, 1), (1, 3, 65), (2, 2, 200), (1, 4, 257), (2, 3, 1000),
          (4, 16, 4096), (8, 8, 2048), (2, 16, 16384), (8, 16, 700), (8, 20, 300)]


@pytest.mark.parametrize("B,H,T", SHAPES)
def test_one_launch_walk_matches_two_launch_bitwise(B, H, T):
    _log("walk pipe B=%d H=%d T=%d" % (B, H, T))
    dev = _inputs(B, H, T, seed=B * 1000 + H * 10 + T)
    a = _scan(dev, True)
    b = _scan(dev, False)
    torch.cuda.synchronize()
    _equal(a, b, (B, H, T))


@pytest.mark.parametrize("B,H,T", [(4, 16, 4096), (2, 3, 1000), (1, 1, 1)])
def test_one_launch_scan_without_optional_outputs(B, H, T):
    """k_tilde and d_final alone (no d_all, no log rho_t), as the bench calls it."""
    _log("scan pipe, no optional outputs, B=%d H=%d T=%d" % (B, H, T))
    dev = _inputs(B, H, T, seed=3 + T)
    _equal(_scan(dev, True, want=False), _scan(dev, False, want=False), (B, H, T))
    torch.cuda.synchronize()


def test_one_launch_scan_reused_workspace():
    """Three inputs through one precond_scan workspace, then the first again:
    every call equals the three-launch walk (stale flags never pass)."""
    shape = (2, 8, 1000)
    n = osdn.precond_scan_workspace_bytes(*shape, 128, 0)
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    devs = [_inputs(*shape, seed=s) for s in (15, 16, 17)]
    for i in (0, 1, 2, 0, 2):
        _equal(_scan(devs[i], True, ws=ws), _scan(devs[i], False), i)
    torch.cuda.synchronize()


def test_one_launch_walk_repeated():
    """The metric workload's walk five times over: every call bitwise equal
    to the two-launch walk."""
    dev = _inputs(4, 16, 4096, seed=11)
    ref = _scan(dev, False)
    for i in range(5):
        _equal(_scan(dev, True), ref, i)
    torch.cuda.synchronize()


@pytest.mark.parametrize("B,H,T", [(4, 16, 4096), (2, 3, 1000), (1, 1, 1), (8, 16, 700)])
def test_forward_walk_matches_precond_scan(B, H, T):
    """osdn_forward runs the one-launch walk inside its pipeline: its d_final
    equals the scan's."""
    dev = _inputs(B, H, T, seed=7 + T)
    f = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=0.05, chunk=64)
    s = _scan(dev, False)
    torch.cuda.synchronize()
    assert torch.equal(f["d_final"], s["d_final"])
    assert torch.isfinite(f["o"]).all() and torch.isfinite(f["S_final"]).all()


def test_reused_workspace_across_inputs():
    """Three inputs through one workspace, then the first again: every call
    equals a call with a fresh workspace (stale flags and records of earlier
    calls are never taken for this call's)."""
    shape = (2, 8, 1000)
    need = osdn.forward_workspace_bytes(*shape, 128, 128, 64, 0, True)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
    devs = [_inputs(*shape, seed=s) for s in (5, 6, 7)]
    for i in (0, 1, 2, 0, 2):
        d = devs[i]
        a = osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=0.05, chunk=64, workspace=ws)
        b = osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=0.05, chunk=64)
        torch.cuda.synchronize()
        for key in ("o", "S_final", "d_final", "log_ratio_sum"):
            assert torch.equal(a[key], b[key]), (i, key)
