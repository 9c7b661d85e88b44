"""The arn:: torch custom ops on the GPU: eager results equal the binding's,
and a function using them compiles with fullgraph=True (no graph breaks)
and gives the same results."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import assert_codes_close, bits, codes, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import residual_add_rmsnorm_amd.torch_ops  # noqa: F401


def _inputs(rows=48, hidden=2048, seed=70):
    rng = np.random.default_rng(seed)
    x = W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16")
    r = W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16")
    w = W.to_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), "bf16")
    g = W.to_bits(rng.standard_normal((rows, 2 * hidden)).astype(np.float32), "bf16")
    return x, r, w, g


def block_tail(x, residual, weight, gate_up):
    """residual += x; h = norm(residual) as dynamic e4m3; a = SwiGLU(gate_up)
    as dynamic e4m3 -- the two fused kernels of one decoder block."""
    q, s = torch.ops.arn.fused_add_rmsnorm_fp8_dynamic(x, residual, weight, 1e-6)
    a, sa = torch.ops.arn.silu_and_mul_fp8_dynamic(gate_up)
    return q, s, a, sa


@pytest.mark.parametrize("compiled", [False, True])
def test_block_tail(orc, compiled):
    x, r, w, g = _inputs()
    xd, rd, wd, gd = dev(x, "bf16"), dev(r, "bf16"), dev(w, "bf16"), dev(g, "bf16")
    fn = torch.compile(block_tail, backend="aot_eager", fullgraph=True) if compiled else block_tail
    q, s, a, sa = fn(xd, rd, wd, gd)
    torch.cuda.synchronize()
    ref = orc.add_rmsnorm("bf16", x, r, w, 1e-6, fp8_mode=O.FP8_DYNAMIC)
    ref_g = orc.silu_and_mul("bf16", g, fp8_mode=O.FP8_DYNAMIC)
    assert np.array_equal(bits(rd), ref["r16"]), "residual not updated in place"
    assert_codes_close(codes(q), ref["q"])
    assert_codes_close(codes(a), ref_g["q"])


def test_ops_equal_binding():
    import residual_add_rmsnorm_amd as arn

    x, r, w, g = _inputs(seed=71)
    xd, wd, gd = dev(x, "bf16"), dev(w, "bf16"), dev(g, "bf16")
    r1, r2 = dev(r, "bf16"), dev(r, "bf16")
    assert torch.equal(torch.ops.arn.fused_add_rmsnorm(xd, r1, wd, 1e-5),
                       arn.fused_add_rmsnorm(xd, r2, wd, 1e-5))
    assert torch.equal(r1, r2)
    assert torch.equal(torch.ops.arn.rmsnorm(xd, wd, 1e-5), arn.rmsnorm(xd, wd, 1e-5))
    assert torch.equal(torch.ops.arn.silu_and_mul(gd), arn.silu_and_mul(gd))
    s = torch.tensor([0.02], device="cuda")
    assert torch.equal(torch.ops.arn.silu_and_mul_fp8_static(gd, s).view(torch.uint8),
                       arn.silu_and_mul_fp8(gd, scale=s)[0].view(torch.uint8))


def decode_mlp(x, residual, weight, w_gate_up, s_gate_up, w_down, s_down, n_gate_up, k):
    """residual += x; h = e4m3(norm(residual)); gate_up = h @ W1^T;
    a = e4m3(SwiGLU(gate_up)); out = a @ W2^T -- the decode MLP of one block
    through the library's ops, with pre-shuffled weights."""
    h, sh = torch.ops.arn.fused_add_rmsnorm_fp8_dynamic(x, residual, weight, 1e-6)
    gu = torch.ops.arn.fp8_gemm_preshuffled(h, sh, w_gate_up, n_gate_up, k, s_gate_up,
                                            torch.bfloat16)
    a, sa = torch.ops.arn.silu_and_mul_fp8_dynamic(gu)
    return torch.ops.arn.fp8_gemm_preshuffled(a, sa, w_down, k, n_gate_up // 2, s_down,
                                              torch.bfloat16)


@pytest.mark.parametrize("compiled", [False, True])
def test_decode_mlp(compiled):
    """The same chain compiled (fullgraph, no breaks) and eager gives the
    same bits as the binding called step by step."""
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(72)
    rows, hidden, inter = 4, 1024, 1536
    x = dev(W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16"), "bf16")
    r = dev(W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16"), "bf16")
    w = dev(W.to_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), "bf16"), "bf16")
    w1 = torch.from_numpy(W.e4m3_codes(rng.standard_normal((2 * inter, hidden)) * 4)).cuda()
    w2 = torch.from_numpy(W.e4m3_codes(rng.standard_normal((hidden, inter)) * 4)).cuda()
    s1 = torch.full((2 * inter,), 0.01, device="cuda")
    s2 = torch.full((hidden,), 0.01, device="cuda")
    w1s = torch.ops.arn.fp8_weight_preshuffle(w1)
    w2s = torch.ops.arn.fp8_weight_preshuffle(w2)
    fn = torch.compile(decode_mlp, backend="aot_eager", fullgraph=True) if compiled else decode_mlp
    r_op = r.clone()
    out = fn(x, r_op, w, w1s, s1, w2s, s2, 2 * inter, hidden)
    # step by step through the binding
    r_b = r.clone()
    h, sh = arn.fused_add_rmsnorm_fp8(x, r_b, w, 1e-6, dynamic=True)
    gu = arn.fp8_gemm(h, sh, arn.fp8_weight_preshuffle(w1), s1)
    a, sa = arn.silu_and_mul_fp8(gu, dynamic=True)
    ref = arn.fp8_gemm(a, sa, arn.fp8_weight_preshuffle(w2), s2)
    torch.cuda.synchronize()
    assert torch.equal(r_op, r_b)
    assert torch.equal(out, ref)
    assert torch.isfinite(out.float()).all()


def tp_block_tail(parts, residual, weight):
    """The step after a tensor-parallel block: all-reduce reduction of the
    ranks' partial outputs, residual add, norm to dynamic e4m3."""
    return torch.ops.arn.sum_add_rmsnorm_fp8_dynamic(parts, residual, weight, 1e-6)


@pytest.mark.parametrize("compiled", [False, True])
def test_tp_block_tail(orc, compiled):
    rng = np.random.default_rng(73)
    rows, hidden, g = 12, 2048, 4
    ph = [W.to_bits((rng.standard_normal((rows, hidden)) * 0.5).astype(np.float32), "bf16")
          for _ in range(g)]
    r = W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16")
    w = W.to_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), "bf16")
    pd, rd, wd = [dev(p, "bf16") for p in ph], dev(r, "bf16"), dev(w, "bf16")
    fn = torch.compile(tp_block_tail, backend="aot_eager", fullgraph=True) if compiled \
        else tp_block_tail
    q, s = fn(pd, rd, wd)
    torch.cuda.synchronize()
    ref = orc.sum_add_rmsnorm("bf16", ph, r, w, 1e-6, fp8_mode=O.FP8_DYNAMIC)
    assert np.array_equal(bits(rd), ref["r16"])
    assert_codes_close(codes(q), ref["q"])


def test_decode_mlp_captured_in_a_graph():
    """The decode MLP through torch.ops (outputs allocated inside each op)
    captured in one CUDA graph: every replay, with eager work between the
    replays, equals the eager chain on the same inputs."""
    rng = np.random.default_rng(73)
    rows, hidden, inter = 8, 1024, 1536
    x = dev(W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16"), "bf16")
    r0 = dev(W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16"), "bf16")
    w = dev(W.to_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), "bf16"), "bf16")
    w1 = torch.ops.arn.fp8_weight_preshuffle(
        torch.from_numpy(W.e4m3_codes(rng.standard_normal((2 * inter, hidden)) * 4)).cuda())
    w2 = torch.ops.arn.fp8_weight_preshuffle(
        torch.from_numpy(W.e4m3_codes(rng.standard_normal((hidden, inter)) * 4)).cuda())
    s1 = torch.full((2 * inter,), 0.01, device="cuda")
    s2 = torch.full((hidden,), 0.01, device="cuda")

    r_eager = r0.clone()
    want = decode_mlp(x, r_eager, w, w1, s1, w2, s2, 2 * inter, hidden)
    torch.cuda.synchronize()

    r_graph = r0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the allocator outside the capture
        decode_mlp(x, r0.clone(), w, w1, s1, w2, s2, 2 * inter, hidden)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = decode_mlp(x, r_graph, w, w1, s1, w2, s2, 2 * inter, hidden)
    for rep in range(4):
        r_graph.copy_(r0)  # each replay starts from the same residual
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), rep
        assert torch.equal(r_graph, r_eager), rep
        torch.ops.arn.rmsnorm(x, w, 1e-6)  # eager work between replays
        torch.cuda.synchronize()
