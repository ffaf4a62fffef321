"""The C ABI under HIP graph capture: the fused products, the two-operand
quantizer, the GEMM and the workspace-free error statistics, captured once
on torch's capture stream and replayed. The library allocates nothing and
never synchronizes, so every call is capturable; each replay must give the
eager results bit for bit (all kernels are deterministic), including after
the inputs are overwritten in place between replays. Between replays the
outputs are poisoned eagerly (NaN / 0xAB), so a replay that skipped a
kernel would show."""
import numpy as np
import pytest

from tests.gpu_util import to_dev_bf16
from tests.test_gpu_quant import heavy

pytestmark = pytest.mark.gpu

# (op, T, N, K): GEMM shapes on the persistent LDS-DMA path (reduction
# length % 2048 == 0) with several tiles
PRODUCTS = [("fprop", 512, 768, 2048), ("dgrad", 512, 2048, 640), ("wgrad", 2048, 256, 512)]


def _operands(op, T, N, K, seed):
    if op == "fprop":
        return heavy(T, K, seed), heavy(N, K, seed + 1)
    if op == "dgrad":
        return heavy(T, N, seed), heavy(N, K, seed + 1)
    return heavy(T, N, seed), heavy(T, K, seed + 1)


def _out_shape(op, T, N, K):
    return {"fprop": (T, N), "dgrad": (T, K), "wgrad": (N, K)}[op]


class Work:
    """Device buffers of one captured sequence and the calls that fill them."""

    def __init__(self, seed):
        import torch
        import mxfp4_quantized_gemm_amd as mx
        self.mx = mx
        self.prods = []
        for i, (op, T, N, K) in enumerate(PRODUCTS):
            P, Q = _operands(op, T, N, K, seed + 10 * i)
            opc = {"fprop": mx.OP_FPROP, "dgrad": mx.OP_DGRAD, "wgrad": mx.OP_WGRAD}[op]
            self.prods.append(dict(
                op=op, T=T, N=N, K=K, P=to_dev_bf16(P), Q=to_dev_bf16(Q),
                ws=torch.empty(mx.mxfp4_workspace_bytes(opc, T, N, K), dtype=torch.uint8,
                               device="cuda"),
                Y=torch.empty(_out_shape(op, T, N, K), dtype=torch.float32, device="cuda")))
        # the fprop operands once more through the two-operand launch and the GEMM
        p0 = self.prods[0]
        T, N, K = p0["T"], p0["N"], p0["K"]
        self.an = torch.empty(mx.packed_shapes(T, K, 0)[0], dtype=torch.uint8, device="cuda")
        self.asc = torch.empty(mx.packed_shapes(T, K, 0)[1], dtype=torch.uint8, device="cuda")
        self.bn = torch.empty(mx.packed_shapes(N, K, 0)[0], dtype=torch.uint8, device="cuda")
        self.bsc = torch.empty(mx.packed_shapes(N, K, 0)[1], dtype=torch.uint8, device="cuda")
        self.C = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        self.stats = torch.empty(mx.ERROR_STATS_COUNT, dtype=torch.float64, device="cuda")

    def run(self, stream=None):
        mx = self.mx
        for p in self.prods:
            fn = {"fprop": mx.mxfp4_fprop, "dgrad": mx.mxfp4_dgrad, "wgrad": mx.mxfp4_wgrad}[p["op"]]
            fn(p["P"], p["Q"], p["T"], p["N"], p["K"], 16, 0, p["ws"], p["Y"], mx.OUT_F32, stream)
        p0 = self.prods[0]
        T, N, K = p0["T"], p0["N"], p0["K"]
        mx.mxfp4_quantize_pair(p0["P"], T, K, 0, self.an, self.asc, p0["Q"], N, K, 0, self.bn,
                               self.bsc, 32, 1, stream)
        mx.mxfp4_gemm(self.an, self.asc, self.bn, self.bsc, T, N, K, self.C, mx.OUT_BF16, stream)
        mx.mxfp4_error_stats_noalloc(p0["Q"], N, K, 0, 16, 1, self.stats, stream)

    def outputs(self):
        outs = [p["Y"] for p in self.prods] + [p["ws"] for p in self.prods]
        return outs + [self.an, self.asc, self.bn, self.bsc, self.C, self.stats]

    def poison(self):
        import torch
        for t in self.outputs():
            if t.dtype == torch.uint8:
                t.fill_(0xAB)
            else:
                t.fill_(float("nan"))

    def snapshot(self):
        import torch
        torch.cuda.synchronize()
        return [t.cpu().view(torch.uint8).numpy().copy() if t.dtype != torch.float64 else
                t.cpu().numpy().view(np.uint64).copy() for t in self.outputs()]


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), f"{what}: output {i} differs"


def test_captured_sequence_replays_bit_exact():
    import torch
    w = Work(seed=900)
    w.run()                      # eager first: also resolves the static array's address
    eager = w.snapshot()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            w.run()              # the binding passes torch's current (capturing) stream
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        w.poison()               # eager work between replays
        g.replay()
        _same(w.snapshot(), eager, f"replay {rep}")
    # new inputs written in place: the graph reads them at replay time
    for i, p in enumerate(w.prods):
        P, Q = _operands(p["op"], p["T"], p["N"], p["K"], 1900 + 10 * i)
        p["P"].copy_(to_dev_bf16(P))
        p["Q"].copy_(to_dev_bf16(Q))
    w.run()
    eager2 = w.snapshot()
    assert any(not np.array_equal(a, b) for a, b in zip(eager, eager2))
    for rep in range(2):
        w.poison()
        g.replay()
        _same(w.snapshot(), eager2, f"replay {rep} after new inputs")
