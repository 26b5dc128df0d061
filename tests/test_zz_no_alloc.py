"""The no-allocation pulse-group entry point, sarbp_backproject_split_noalloc, through the C ABI:
its image must equal sarbp_backproject_split's with a caller workspace (the same kernels, so bit
for bit) on two calls in a row, the second with a smaller grid and fewer pulses, and stay within
the oracle's bar; device memory in use must not change across its calls."""
import numpy as np
import pytest

import oracle
import synth
from _parity import REL_L2, rel_l2

pytestmark = pytest.mark.gpu


def _case(sb, s, accumulate=False):
    import torch

    with sb.Plan.for_scene(s) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(s.echo).cuda()
        need = plan.split_workspace_bytes(s.na)
        assert 0 < need <= sb.SARBP_STATIC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        base = torch.from_numpy((0.5 * s.echo[0, 0] * np.ones(plan.image_shape)).astype(np.complex64)).cuda()
        ref = base.clone() if accumulate else plan.new_image()
        sb.sarbp_backproject_split(plan.handle, pos, ech, ref, ws, accumulate=int(accumulate))
        torch.cuda.synchronize()
        got = base.clone() if accumulate else torch.full(plan.image_shape, 7.0, dtype=torch.complex64, device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        sb.sarbp_backproject_split_noalloc(plan.handle, pos, ech, got, accumulate=int(accumulate))
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        print(f"[noalloc] {s.nx}x{s.ny} px, {s.na} pulses, workspace {need} B, accumulate {accumulate}: "
              f"equal {torch.equal(got, ref)}, device memory free before/after {free0}/{free1}", flush=True)
        assert free1 == free0
        assert torch.equal(got, ref)
        out = got.cpu().numpy().astype(np.complex128)
    want = oracle.scene_backproject(s)
    if accumulate:
        want = want + (0.5 * s.echo[0, 0]).astype(np.complex128)
    assert rel_l2(out, want) <= REL_L2, rel_l2(out, want)


def test_noalloc_matches_the_workspace_call_twice(gpu_device):
    from domain_backprojection_amd import sarbp as sb

    big = synth.make_scene("std", na=512, nr=1024, nx=256, ny=200, n_targets=3)
    small = synth.make_scene("hifi", na=200, nr=1024, nx=100, ny=70, interp="nearest", n_targets=1)
    _case(sb, big)
    _case(sb, small)  # smaller grid and fewer pulses: the array still holds the first call's partials
    _case(sb, small, accumulate=True)


def test_noalloc_arguments(gpu_device):
    import torch

    from domain_backprojection_amd import sarbp as sb

    s = synth.make_scene("tiny", na=64, nx=64, ny=64)
    with sb.Plan.for_scene(s, n_pulses=s.na - 8) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(s.echo).cuda()
        img = plan.new_image()
        with pytest.raises(sb.SarbpError, match="invalid"):  # more pulses than the plan takes
            sb.sarbp_backproject_split_noalloc(plan.handle, pos, ech, img, n=s.na)
        with pytest.raises(sb.SarbpError, match="invalid"):
            sb.sarbp_backproject_split_noalloc(plan.handle, pos, ech, img, n=s.na - 8, accumulate=2)
        sb.sarbp_backproject_split_noalloc(plan.handle, pos, ech, img, n=s.na - 8)
        ref = plan.backproject(pos, ech, n=s.na - 8, split=True)
        torch.cuda.synchronize()
        assert torch.equal(img, ref)
