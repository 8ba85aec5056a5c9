"""Every entry point captured in a HIP graph gives the eager result on every replay (GPU).

The kernels clear nothing with memset nodes (each launch writes its whole
output itself), so a captured launch must reproduce the eager bytes no matter
what the output held before. Between replays the outputs are overwritten by
eager fills and the host synchronises; each replay is compared with the eager
result. The benchmark times exactly such graph replays.
"""

import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def env():
    import torch

    from group_scale_factor_amd import _build

    if not os.path.exists(_build.LIBRARY):
        _build.build()
    import group_scale_factor_amd as gsf

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return gsf, torch


def check_graph(torch, label, launch, outs):
    """Eager launch, then a graph of the same launch replayed REPLAYS times over poisoned outputs."""
    print("case graph", label, flush=True)
    for o in outs:
        o.fill_(0x5A)
    launch()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            launch()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(0xA5 ^ rep)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o, w), "%s: replay %d differs from the eager launch (output %d)" % (label, rep, k)


def test_rearrange_M_and_K(env):
    import workloads

    gsf, torch = env
    for name in ("m_groups_tiny", "m_groups_experts", "k_groups"):
        w = workloads.make(name)
        s = torch.from_numpy(np.ascontiguousarray(w.scales)).cuda()
        o = torch.from_numpy(w.offs).cuda()
        fn = gsf.mx_block_rearrange_M_groups if w.kind == "M" else gsf.mx_block_rearrange_K_groups
        size = (gsf.mx_rearrange_M_groups_out_bytes if w.kind == "M" else gsf.mx_rearrange_K_groups_out_bytes)(
            w.rows, w.cols, w.num_groups)
        out = torch.empty(size, dtype=torch.uint8, device="cuda")
        check_graph(torch, name, lambda: fn(s, o, out=out), [out])


def test_rearrange_3d(env):
    import workloads

    gsf, torch = env
    w = workloads.make("experts_3d_small")
    s = torch.from_numpy(np.ascontiguousarray(w.scales)).cuda()
    out = torch.empty(gsf.mx_rearrange_3d_out_bytes(w.experts, w.rows, w.cols), dtype=torch.uint8, device="cuda")
    check_graph(torch, "experts_3d_small", lambda: gsf.mx_block_rearrange_3d(s, out=out), [out])


def test_quantize_dim0_dim1_and_experts(env):
    import workloads

    gsf, torch = env
    w = workloads.make("quant_m_groups_small")
    x = torch.from_numpy(w.x.view(np.int16)).cuda().view(torch.bfloat16)
    o = torch.from_numpy(w.offs).cuda()
    q = torch.empty((w.rows, w.K), dtype=torch.uint8, device="cuda")
    sc = torch.empty(gsf.mx_quantize_dim0_M_groups_scale_bytes(w.rows, w.K, w.num_groups), dtype=torch.uint8,
                     device="cuda")
    check_graph(torch, "quant_m_groups_small", lambda: gsf.mx_quantize_dim0_M_groups(x, o, q=q, scales=sc), [q, sc])

    w = workloads.make("quant_k_groups_small")
    x = torch.from_numpy(w.x.view(np.int16)).cuda().view(torch.bfloat16)
    o = torch.from_numpy(w.offs).cuda()
    qT = torch.empty((w.K, w.rows), dtype=torch.uint8, device="cuda")
    sc = torch.empty(gsf.mx_quantize_dim1_K_groups_scale_bytes(w.rows, w.K, w.num_groups), dtype=torch.uint8,
                     device="cuda")
    check_graph(torch, "quant_k_groups_small", lambda: gsf.mx_quantize_dim1_K_groups(x, o, qT=qT, scales=sc),
                [qT, sc])

    w = workloads.make("quant_3d_small")
    ld = (w.N + 7) // 8 * 8                  # rows padded to a multiple of 8 elements (16 bytes)
    padded = np.zeros((w.experts, w.K, ld), np.uint16)
    padded[:, :, :w.N] = w.w
    wt = torch.from_numpy(padded.view(np.int16)).cuda().view(torch.bfloat16)[:, :, :w.N]
    q3 = torch.empty((w.experts, w.N, w.K), dtype=torch.uint8, device="cuda")
    s3 = torch.empty(gsf.mx_quantize_dim1_3d_scale_bytes(w.experts, w.K, w.N), dtype=torch.uint8, device="cuda")
    check_graph(torch, "quant_3d_small", lambda: gsf.mx_quantize_dim1_3d(wt, q=q3, scales=s3), [q3, s3])

    # K a multiple of 128: two feature blocks per workgroup (the kernel whose LDS allowance the host raises)
    import pins

    rng = np.random.default_rng(91)
    E, K, N = 3, 256, 300
    wb = np.zeros((E, K, 304), np.uint16)    # rows padded to 304 elements (16-byte strides)
    for e in range(E):
        wb[e, :, :N] = pins.random_bf16_rows(rng, K, N)
    wp = torch.from_numpy(wb.view(np.int16)).cuda().view(torch.bfloat16)[:, :, :N]
    qp = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    sp = torch.empty(gsf.mx_quantize_dim1_3d_scale_bytes(E, K, N), dtype=torch.uint8, device="cuda")
    check_graph(torch, "quant_3d paired blocks", lambda: gsf.mx_quantize_dim1_3d(wp, q=qp, scales=sp), [qp, sp])


def test_pad_unpad_and_inverse(env):
    import workloads

    gsf, torch = env
    w = workloads.make("pad_m_groups_small")
    d = torch.from_numpy(w.data).cuda()
    o = torch.from_numpy(w.offs).cuda()
    padded = torch.empty((w.rows + 128 * w.num_groups, w.cols), dtype=torch.uint8, device="cuda")
    check_graph(torch, "pad", lambda: gsf.mx_pad_M_groups(d, o, out=padded), [padded])
    back = torch.empty((w.rows, w.cols), dtype=torch.uint8, device="cuda")
    check_graph(torch, "unpad", lambda: gsf.mx_unpad_M_groups(padded, w.rows, o, out=back), [back])

    for name in ("m_groups_experts", "k_groups"):
        f = workloads.make(name)
        kind = f.kind
        s = torch.from_numpy(np.ascontiguousarray(f.scales)).cuda()
        o = torch.from_numpy(f.offs).cuda()
        fwd = gsf.mx_block_rearrange_M_groups if kind == "M" else gsf.mx_block_rearrange_K_groups
        blocked = fwd(s, o)
        inv = gsf.mx_block_unrearrange_M_groups if kind == "M" else gsf.mx_block_unrearrange_K_groups
        out = torch.empty((f.rows, f.cols), dtype=torch.uint8, device="cuda")
        check_graph(torch, "inverse " + name, lambda: inv(blocked, f.rows, f.cols, o, out=out), [out])


FIRST_CALL_CAPTURED = r"""
import numpy as np, torch
import group_scale_factor_amd as gsf
rng = np.random.default_rng(5)
rows, cols = 7168, 4096          # a shape whose grid takes the 512-column windows on MI355X
scales = torch.from_numpy(rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)).cuda()
offs = torch.from_numpy(np.array([1, 700, 701, 2049, 2050, 3000, 4001, 4096], np.int32)).cuda()
out = torch.empty(gsf.mx_rearrange_K_groups_out_bytes(rows, cols, 8), dtype=torch.uint8, device="cuda")
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
g = torch.cuda.CUDAGraph()
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        gsf.mx_block_rearrange_K_groups(scales, offs, out=out)   # the process's first K-groups call
torch.cuda.current_stream().wait_stream(s)
out.fill_(0x5A)
g.replay()
torch.cuda.synchronize()
got = out.clone()
out.fill_(0xA5)
gsf.mx_block_rearrange_K_groups(scales, offs, out=out)
torch.cuda.synchronize()
assert torch.equal(got, out), "captured first call differs from the eager call"
print("first call captured: ok")
"""


def test_first_k_call_inside_a_capture():
    """The library's first K-groups call in a process (which asks the runtime, once per device, how many
    workgroups of each window kernel fit and raises the 512-column kernel's LDS allowance) may itself be
    inside a graph capture: the captured launch replays to the eager result. Run in a fresh process of its
    own, since this test process has made K-groups calls already."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("case graph: first K-groups call of a fresh process inside a capture", flush=True)
    res = subprocess.run([sys.executable, "-c", FIRST_CALL_CAPTURED], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0 and "ok" in res.stdout, res.stdout[-2000:] + res.stderr[-4000:]
