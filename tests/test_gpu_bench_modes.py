"""bench.py's counter-pass mode runs every extended op it offers (the figures in the
committed traffic summary of the extended rows come from it)."""
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
