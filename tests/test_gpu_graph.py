"""HIP-graph capture of the library's entry points: each call is captured
once on a side stream and replayed several times, with eager work and fresh
input data between the replays; every replay must equal the eager call on
the same data bit for bit (the kernels are deterministic).  The split-K path
runs with a caller-owned workspace (the form documented for capture); its
arrival counters must be left zeroed by every replay.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_gemm_amd as fbg
import workloads
from tests._gpu import to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def replay_and_check(capture, eager, refill, replays=4):
    """capture(): the captured call writing into fixed buffers, returns them;
    eager(): the same call made eagerly, returns fresh outputs; refill(i):
    writes new input data into the captured input buffers."""
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up outside the graph
        capture()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = capture()
    torch.cuda.synchronize()
    for i in range(replays):
        refill(i)
        torch.cuda.synchronize()
        # unrelated eager work between replays
        x = torch.randn(512, 512, device=DEV)
        (x @ x).sum().item()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {i} differs from the eager call"


def test_split_k_gemm_with_caller_workspace_in_a_graph(gpu):
    M, N, K = 32, 512, 16384
    p = fbg.plan(M, N, K)
    assert p["variant_name"] == "swap_ab_splitk"
    dd = to_dev(workloads.make_inputs(M, N, K, seed=31))
    ws = torch.zeros(fbg.workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def capture():
        fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], out=C, workspace=ws, stream=torch.cuda.current_stream())
        return [C]

    def eager():
        return [fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"])]

    def refill(i):
        d = to_dev(workloads.make_inputs(M, N, K, seed=40 + i))
        for k in dd:
            dd[k].copy_(d[k])

    replay_and_check(capture, eager, refill)
    off = p["workspace_bytes"] - 4 * (-(-M // p["tile_m"]) * -(-N // p["tile_n"]))
    assert int(ws[off:].count_nonzero()) == 0, "arrival counters not left zeroed"


def test_grouped_gemm_in_a_graph(gpu):
    counts = [3, 0, 17, 1, 40, 0, 9]
    d0 = workloads.make_grouped_inputs(counts, 300, 1024, seed=5)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in d0.items() if k != "offsets"}
    dev["A"] = dev["A"].view(torch.float8_e4m3fn)
    dev["B"] = dev["B"].view(torch.float8_e4m3fn)
    off = torch.from_numpy(d0["offsets"].astype(np.int32)).to(DEV)
    C = torch.empty((int(d0["offsets"][-1]), 300), dtype=torch.bfloat16, device=DEV)

    def capture():
        fbg.grouped_gemm(dev["A"], dev["a_s"], dev["B"], dev["b_s"], off, out=C, stream=torch.cuda.current_stream())
        return [C]

    def eager():
        return [fbg.grouped_gemm(dev["A"], dev["a_s"], dev["B"], dev["b_s"], off)]

    def refill(i):
        # new routing of the same rows: the offsets are device data, read at replay time
        c = np.random.default_rng(i).permutation(counts)
        off.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(c)]).astype(np.int32)))

    replay_and_check(capture, eager, refill)


def test_quantizers_in_a_graph(gpu):
    x = torch.randn(96, 1024, device=DEV).to(torch.bfloat16)
    w = (torch.randn(300, 512, device=DEV) * 0.02).to(torch.bfloat16)
    A = torch.empty((96, 1024), dtype=torch.float8_e4m3fn, device=DEV)
    a_s = torch.empty((96, 8), dtype=torch.float32, device=DEV)
    B = torch.empty((300, 512), dtype=torch.float8_e4m3fn, device=DEV)
    b_s = torch.empty((3, 4), dtype=torch.float32, device=DEV)

    def capture():
        s = torch.cuda.current_stream()
        fbg.quantize_rows(x, A, a_s, stream=s)
        fbg.quantize_blocks(w, B, b_s, stream=s)
        return [A, a_s, B, b_s]

    def eager():
        return list(fbg.quantize_rows(x)) + list(fbg.quantize_blocks(w))

    def refill(i):
        x.copy_(torch.randn(96, 1024, device=DEV) * (i + 1))
        w.copy_(torch.randn(300, 512, device=DEV) * 0.01 * (i + 1))

    replay_and_check(capture, eager, refill)


def test_split_k_gemm_with_library_workspace_in_a_graph(gpu):
    """A split forced without a caller workspace: the library's own
    stream-ordered workspace (allocate, zero the counters with a kernel,
    launch, free) captured as graph nodes."""
    M, N, K = 64, 512, 4096
    dd = to_dev(workloads.make_inputs(M, N, K, seed=32))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def capture():
        fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], out=C, stream=torch.cuda.current_stream(),
                 variant="swap_ab_splitk", split_k=4, workspace="library")
        return [C]

    def eager():
        return [fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], variant="swap_ab_splitk", split_k=4,
                         workspace="library")]

    def refill(i):
        d = to_dev(workloads.make_inputs(M, N, K, seed=50 + i))
        for k in dd:
            dd[k].copy_(d[k])

    replay_and_check(capture, eager, refill)


def test_plain_entry_point_in_a_graph(gpu):
    """fp8_block_gemm with no workspace (the unsplit plan: nothing to
    allocate) captured and replayed."""
    M, N, K = 64, 512, 4096
    dd = to_dev(workloads.make_inputs(M, N, K, seed=34))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def capture():
        fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], out=C, stream=torch.cuda.current_stream(),
                 workspace="library")
        return [C]

    def eager():
        return [fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], workspace="library")]

    def refill(i):
        d = to_dev(workloads.make_inputs(M, N, K, seed=70 + i))
        for k in dd:
            dd[k].copy_(d[k])

    replay_and_check(capture, eager, refill)


def test_split_k_gemm_with_default_workspace_in_a_graph(gpu):
    """The binding's default workspace (a zeroed torch tensor on the call's
    stream) captured into the graph's memory pool."""
    M, N, K = 16, 512, 16384
    assert fbg.plan(M, N, K)["split_k"] > 1
    dd = to_dev(workloads.make_inputs(M, N, K, seed=33))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def capture():
        fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], out=C, stream=torch.cuda.current_stream())
        return [C]

    def eager():
        return [fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"])]

    def refill(i):
        d = to_dev(workloads.make_inputs(M, N, K, seed=60 + i))
        for k in dd:
            dd[k].copy_(d[k])

    replay_and_check(capture, eager, refill)
