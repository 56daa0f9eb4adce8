"""bench.py's counter-pass mode runs every extended op it offers (the figures in the
committed traffic summary of the extended rows come from it), and its ceiling mode runs every
probe (the committed ceiling summary comes from it)."""
import json

import pytest
import torch

import bench
import block_scaled_precision_mxfp8_amd as bsq
import workloads
from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("op", bench.PROFILE_OPS)
def test_profile_op_runs(op, capsys):
    log("bench --profile-op %s" % op)
    bench.profile_op(torch, bsq, workloads, torch.device("cuda:0"), op)
    torch.cuda.synchronize()
    out = capsys.readouterr().out.strip().splitlines()
    assert json.loads(out[-1]) == {"profile_op": op}
    torch.cuda.empty_cache()


def test_hbm_ceiling_runs(capsys):
    log("bench --hbm-ceiling, one timed launch per probe")
    bench.hbm_ceiling(torch, bsq, torch.device("cuda:0"), reps=1)
    torch.cuda.synchronize()
    lines = [json.loads(l) for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 17
    assert all(l["alone_us"] > 0 and l["bytes"] > 0 for l in lines)
    torch.cuda.empty_cache()
