"""GPU test of gemm355_gemm_noalloc, the entry point for callers that cannot
allocate device memory: through the C ABI, its output equals
gemm355_gemm_ex's (same plan, same kernels: bit for bit) and lies within the
oracle's tolerance, on calls in a row whose scratch use shrinks: a split-K
product with a split tail (partial sums in the fixed array), then a smaller
product with both operands repacked and a uniform split, then a smaller
block-scaled product (scales regrouped in the array).  The array keeps the
previous call's contents, so a stale partial sum or row would show."""
import numpy as np
import pytest
import torch

from dense_tiled_gemm_fp8_amd import gemm355 as g
from dense_tiled_gemm_fp8_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _call(ops, entry, layout=g.A_ROW_B_COL, A_dev=None, B_dev=None, lda=None, ldb=None, **knobs):
    M, N, K = ops.M, ops.N, ops.K
    C = H.empty_c(1, M, N, "f32")
    bsa = bsb = None
    if ops.mx:
        bsa, bsb = H.dev(ops.bsa), H.dev(ops.bsb)
    args = g.make_args(M, N, K, A=A_dev if A_dev is not None else H.dev(ops.A), lda=lda,
                       B=B_dev if B_dev is not None else H.dev(ops.B), ldb=ldb, C=C,
                       dtype=H.out_dtype(ops.fmt, "f32"), layout=layout, block_scale_a=bsa, block_scale_b=bsb,
                       **knobs)
    p = g.gemm355_plan(args)
    entry(args)
    torch.cuda.synchronize()
    return C.double().cpu().numpy(), p


def test_no_alloc_matches_gemm_ex_on_shrinking_calls():
    cases = []
    # 1: the long-K workload 256 x 256 x 65536 (automatic plan: persistent grid, split tail)
    w = inputs.WORKLOADS[3]
    cases.append(("split tail 256x256x65536", inputs.workload_operands(w, 0), {}))
    # 2: smaller, A column-major and B row-major (both repacked), 4-way split
    ops2 = inputs.make_operands(300, 200, 3000, "bf16", "normal", 61, 62)
    At = np.ascontiguousarray(ops2.A.T)
    Br = np.ascontiguousarray(ops2.B.T)
    cases.append(("repacked, split 4, 300x200x3000", ops2,
                  dict(layout=g.A_COL_B_ROW, A_dev=H.dev(At), B_dev=H.dev(Br), lda=300, ldb=200, split_k=4)))
    # 3: smaller still, block-scaled E4M3 with a 2-way split
    ops3 = inputs.make_operands(190, 130, 512, "mxe4m3", "normal", 63, 64)
    cases.append(("block-scaled, split 2, 190x130x512", ops3, dict(split_k=2)))
    used = []
    for name, ops, kn in cases:
        C_ex, p = _call(ops, g.gemm355_gemm_ex, **kn)
        C_na, p2 = _call(ops, g.gemm355_gemm_noalloc, **kn)
        H.say("no-alloc", name, "plan tile", p["tile"], "split", p["split"], "tail", p["tail_tiles"],
              p["tail_split"], "repack", p["repack"], "scratch bytes", p["workspace_bytes"])
        assert p == p2
        assert p["workspace_bytes"] > 0
        used.append(p["workspace_bytes"])
        assert np.array_equal(C_na, C_ex), name
        C_ref, W = H.oracle_full(ops)
        H.check(C_na, C_ref, W, ops.fmt, name)
    assert used[0] > used[1] > used[2]


def test_no_alloc_rejects_workspace_and_oversized_plans():
    ops = inputs.make_operands(64, 64, 64, "bf16", "normal", 65, 66)
    A, B = H.dev(ops.A), H.dev(ops.B)
    C = H.empty_c(1, 64, 64, "f32")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    a = g.make_args(64, 64, 64, A=A, B=B, C=C, workspace=ws, workspace_bytes=1 << 20, split_k=2)
    with pytest.raises(g.Gemm355Error) as e:
        g.gemm355_gemm_noalloc(a)
    assert e.value.status == g.EINVAL
    # 4096^3 cut into 8 slices: 512 MiB of partial sums, beyond the 64 MiB
    # array (real operands of that size, so the call is well-formed)
    Ab = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    Bb = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    Cb = torch.full((4096, 4096), float("nan"), dtype=torch.float32, device="cuda")
    big = g.make_args(4096, 4096, 4096, A=Ab, B=Bb, C=Cb, split_k=8, tile=0)
    assert g.gemm355_plan(big)["workspace_bytes"] > 64 << 20
    with pytest.raises(g.Gemm355Error) as e:
        g.gemm355_gemm_noalloc(big)
    assert e.value.status == g.ETOOBIG
    torch.cuda.synchronize()
    assert torch.isnan(C).all() and torch.isnan(Cb).all()   # nothing was launched


def test_no_alloc_replays_in_a_captured_graph():
    """The callers this entry point is for include code under HIP graph
    capture.  A product that uses the fixed array twice over (A repacked
    into it, then a 4-way split whose partial sums it holds and a combine
    pass) is captured once and replayed three times, with an eager call of
    another shape on the same array before each replay; every replay's C
    equals the eager call's bit for bit.  The library records no memset and
    makes no allocation while captured."""
    M, N, K = 300, 200, 3000
    ops = inputs.make_operands(M, N, K, "bf16", "normal", 67, 68)
    At = H.dev(np.ascontiguousarray(ops.A.T))
    B = H.dev(ops.B)
    kn = dict(layout=g.A_COL_B_COL, split_k=4)
    C_e = H.empty_c(1, M, N, "f32")
    C_g = H.empty_c(1, M, N, "f32")
    a_e = g.make_args(M, N, K, A=At, lda=M, B=B, C=C_e, **kn)
    a_g = g.make_args(M, N, K, A=At, lda=M, B=B, C=C_g, **kn)
    p = g.gemm355_plan(a_g)
    assert p["repack"] == 1 and p["split"] == 4
    # the first call on the device looks up the array's address: before the capture
    g.gemm355_gemm_noalloc(a_e)
    torch.cuda.synchronize()
    other = inputs.make_operands(190, 130, 640, "bf16", "normal", 69, 70)
    C_o = H.empty_c(1, 190, 130, "f32")
    a_o = g.make_args(190, 130, 640, A=H.dev(other.A), B=H.dev(other.B), C=C_o, split_k=3)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        g.gemm355_gemm_noalloc(a_g, torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        C_g.fill_(float("nan"))
        g.gemm355_gemm_noalloc(a_o)
        torch.cuda.synchronize()
        H.say("graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C_g, C_e), r
    C_ref, W = H.oracle_full(ops)
    H.check(C_g.double().cpu().numpy(), C_ref, W, "bf16", "captured graph")
