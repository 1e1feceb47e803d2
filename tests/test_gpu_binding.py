"""The binding's argument checks and the library's device-plan check on a
GPU: short or misshapen caller buffers raise ValueError before any launch,
and a device plan is accepted only from an upload of the same plan."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import prefix_tree_packed_plan_amd as ptp
from prefix_tree_packed_plan_amd import _lib
from workloads import make_conv_inputs, make_scan_inputs, make_ssd_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PARENTS = np.array([-1, 0, 0, 1], np.int32)
LENS = np.array([40, 17, 9, 33], np.int32)
N = int(LENS.sum())


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_misshapen_caller_buffers_raise_before_launch():
    say("binding shape checks")
    plan = ptp.tree_plan(PARENTS, LENS, 4)
    c = make_conv_inputs(N, 64, 4, "bf16", DEV, seed=1, with_bias=True)
    with pytest.raises(ValueError, match="out"):
        ptp.tree_conv(c["x"], c["w"], plan, out=torch.empty(N - 1, 64, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="bias"):
        ptp.tree_conv(c["x"], c["w"], plan, bias=c["bias"][:32].contiguous())
    dy = torch.randn_like(c["x"])
    with pytest.raises(ValueError, match="bias"):
        ptp.tree_conv_backward(c["x"], c["w"], dy, plan, bias=c["bias"][:32].contiguous())
    with pytest.raises(ValueError, match="dx"):
        ptp.tree_conv_backward(c["x"], c["w"], dy, plan, dx=torch.empty(N, 32, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="workspace"):
        ptp.tree_conv_backward(c["x"], c["w"], dy, plan, workspace=torch.empty(4, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="device tensor"):
        ptp.tree_conv_backward(c["x"], c["w"], dy, plan, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    t = make_scan_inputs(N, 2, 4, 128, 128, "bf16", DEV, seed=2)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], plan)
    with pytest.raises(ValueError, match="out"):
        ptp.tree_gdn_scan(*args, out=torch.empty(N, 2, 128, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="states"):
        ptp.tree_gdn_scan(*args, states=torch.empty(3, 4, 128, 128, device=DEV))
    with pytest.raises(ValueError, match="workspace"):
        ptp.tree_gdn_scan(*args, schedule="level", workspace=torch.empty(8, dtype=torch.uint8, device=DEV))
    s = make_ssd_inputs(N, 1, 4, 64, 32, "bf16", DEV, seed=3)
    sargs = (s["x"], s["dt"], s["A"], s["B"], s["C"], plan)
    with pytest.raises(ValueError, match="out"):
        ptp.tree_ssd_scan(*sargs, out=torch.empty(N, 4, 16, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="states"):
        ptp.tree_ssd_scan(*sargs, states=torch.empty(4, 4, 32, 64, device=DEV))
    # a workspace counted in bytes whatever its element type
    o_ref = ptp.tree_gdn_scan(*args, schedule="level")
    need = int(_lib.load().tree_scan_workspace_bytes(plan.handle, 4, 128, 128, 0))
    ws32 = torch.empty((need + 3) // 4, dtype=torch.float32, device=DEV)
    o = ptp.tree_gdn_scan(*args, schedule="level", workspace=ws32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_device_plan_identity_checked_on_the_host():
    """The library runs with the buffer the plan was uploaded into and
    rejects a same-sized buffer uploaded from another plan, a buffer never
    uploaded, and a short byte count, before launching anything."""
    say("device plan identity")
    lib = _lib.load()
    plan = ptp.tree_plan(PARENTS, LENS, 4)
    other = ptp.tree_plan(PARENTS, np.array([40, 9, 17, 33], np.int32), 4)  # same size, other rows
    assert plan.device_bytes() == other.device_bytes()
    c = make_conv_inputs(N, 64, 4, "bf16", DEV, seed=4)
    y = torch.empty_like(c["x"])
    dplan = plan.on_device(DEV)
    foreign = other.on_device(DEV)
    blank = torch.zeros(plan.device_bytes(), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    db = plan.device_bytes()

    def conv(buf, nbytes):
        return lib.tree_conv(c["x"].data_ptr(), c["w"].data_ptr(), None, y.data_ptr(), None, None, N, 64, 1, 0,
                             plan.handle, buf.data_ptr(), nbytes, stream)

    assert conv(dplan, db) == 0
    torch.cuda.synchronize()
    want = ptp.tree_conv(c["x"], c["w"], plan)
    torch.cuda.synchronize()
    assert torch.equal(y, want)
    y.zero_()
    assert conv(foreign, db) == -1
    assert b"not an upload of this plan" in lib.tree_last_error()
    assert conv(blank, db) == -1
    assert conv(dplan, db - 1) == -5
    assert conv(dplan, db + 64) == -1  # more bytes than the upload had
    torch.cuda.synchronize()
    assert not y.any()  # nothing was launched by the rejected calls
