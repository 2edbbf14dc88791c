"""GPU parity of the W8A8 linear through the C ABI against oracle/w8a8.py:
quantization codes and scales bit-exact, int32 accumulators bit-exact, bf16
outputs within bf16 rounding of the exact value; ragged M and N, several K,
the 1.3B QKV shape on sampled rows."""
import numpy as np
import pytest
import torch

import roundlib as RL
from oracle import w8a8 as OW
from workloads import make_linear_inputs

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8  # bf16 rounding of the output (2^-9) plus the fp32 epilogue, with margin


def _dev(a, dt):
    return RL.to_dev(a, dt)


def _quantized(wf, x, w):
    xq, sx = wf.quant_rows_i8(_dev(x, torch.bfloat16))
    wq, sw = wf.quant_rows_i8(_dev(w, torch.bfloat16))
    return xq, sx, wq, sw


# K picks the register pieces per lane of the quantizer: 1, 2, 3, 4, 8, 10, and past 16 the second read
@pytest.mark.parametrize("M,K", [(1, 64), (70, 1024), (300, 1536), (65, 2048), (40, 4096), (257, 5120), (33, 8960)])
def test_quant_rows_bit_exact(M, K):
    wf = RL.require_gpu()
    x, _, _ = make_linear_inputs(M, 8, K, seed=M + K)
    x[0] = 0.0  # zero row: scale 1, codes 0
    if M > 2:
        x[2] *= 37.0  # another magnitude
        x[2] = RL.round_like("bf16")(x[2])
    codes, scales = wf.quant_rows_i8(_dev(x, torch.bfloat16))
    torch.cuda.synchronize()
    rq, rs = OW.quantize_rows(x)
    assert np.array_equal(codes.cpu().numpy(), rq)
    assert np.array_equal(scales.cpu().numpy(), rs)


# K = 64 and 192 take the 64-byte-stage kernel; 128 .. 5120 the 128-byte-stage kernel with 1, 2, 3, 12, 40 stages
@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (300, 264, 128), (260, 8, 256), (100, 520, 384), (70, 264, 192),
                                   (513, 520, 1536), (77, 1536, 5120), (256, 256, 64)])
def test_int32_accumulators_bit_exact(M, N, K):
    wf = RL.require_gpu()
    print(f"[case] gemm int32 M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * N + K)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    xq[0] = 127  # extremes
    wq[0] = -127
    acc = wf.gemm_w8a8(torch.from_numpy(xq).cuda(), None, torch.from_numpy(wq).cuda(), None,
                       out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), OW.int8_matmul(xq, wq))


@pytest.mark.parametrize("M,N,K,with_bias", [(300, 264, 1536, True), (1000, 1536, 1536, False), (129, 512, 5120, True)])
def test_bf16_output_matches_oracle(M, N, K, with_bias):
    wf = RL.require_gpu()
    x, w, b = make_linear_inputs(M, N, K, seed=7 + M)
    xq, sx, wq, sw = _quantized(wf, x, w)
    bias = _dev(b, torch.bfloat16) if with_bias else None
    y = wf.gemm_w8a8(xq, sx, wq, sw, bias)
    torch.cuda.synchronize()
    rq, rsx = OW.quantize_rows(x)
    wq_ref, rsw = OW.quantize_rows(w)
    ref = OW.w8a8_linear(rq, rsx, wq_ref, rsw, b if with_bias else None)
    got = y.float().cpu().numpy()
    err = np.abs(got - ref)
    print(f"[parity] w8a8 bf16 M={M} N={N} K={K}: max rel {np.max(err / (np.abs(ref) + 1e-30)):.3e}", flush=True)
    assert (err <= BF16_REL * np.abs(ref) + 1e-6).all()
    # and the W8A8 result stays close to the unquantized float linear
    fl = x.astype(np.float64) @ w.astype(np.float64).T + (b if with_bias else 0)
    assert np.abs(got - fl).mean() / np.abs(fl).mean() < 2e-2


def test_qkv_shape_sampled_rows():
    """Wan2.1-1.3B QKV projection of a 4-step round: 23400 tokens x 1536 -> 4608."""
    wf = RL.require_gpu()
    M, N, K = 23400, 4608, 1536
    x, w, b = make_linear_inputs(M, N, K, seed=11)
    xq, sx, wq, sw = _quantized(wf, x, w)
    y = wf.gemm_w8a8(xq, sx, wq, sw, _dev(b, torch.bfloat16))
    acc = wf.gemm_w8a8(xq, None, wq, None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = RL.boundary_rows(M, 1, 64, seed=3)
    rq, rsx = OW.quantize_rows(x[rows])
    wq_ref, rsw = OW.quantize_rows(w)
    assert np.array_equal(xq[torch.from_numpy(rows).cuda()].cpu().numpy(), rq)
    assert np.array_equal(acc[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.int64), OW.int8_matmul(rq, wq_ref))
    ref = OW.w8a8_linear(rq, rsx, wq_ref, rsw, b)
    got = y[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    assert (np.abs(got - ref) <= BF16_REL * np.abs(ref) + 1e-6).all()


def _narrow_tiles(M, N):
    """The launch rule of the 128-byte-stage GEMM (w8a8.hip): 256 x 192 tiles when their
    waves of workgroups, weighted by the tile width and a 10 % efficiency penalty, cost no
    more than 256 x 256 tiles'."""
    tm = -(-M // 256)
    w256 = -(-(tm * -(-N // 256)) // 256)
    w192 = -(-(tm * -(-N // 192)) // 256)
    return w192 * 0.75 * 1.10 <= w256


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (23400, 1536, 1536), (700, 200, 384)])
def test_tile_widths_sampled_rows(M, N, K):
    """Both tile widths of the 128-byte-stage GEMM: 4096 x 4096 runs on 256 x 256 tiles, the
    Wan2.1-1.3B O projection (23400 x 1536 x 1536) and a ragged small shape on 256 x 192
    tiles. int32 accumulators bit-exact and bf16 outputs within rounding on sampled rows
    (every column, so every column tile and the ragged last one are checked)."""
    wf = RL.require_gpu()
    print(f"[case] gemm M={M} N={N} K={K} narrow={_narrow_tiles(M, N)}", flush=True)
    assert _narrow_tiles(M, N) == (N != 4096)
    x, w, b = make_linear_inputs(M, N, K, seed=M + N + K)
    xq, sx, wq, sw = _quantized(wf, x, w)
    y = wf.gemm_w8a8(xq, sx, wq, sw, _dev(b, torch.bfloat16))
    acc = wf.gemm_w8a8(xq, None, wq, None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = RL.boundary_rows(M, 1, 48, seed=5)
    rows = rows[rows < M]
    rq, rsx = OW.quantize_rows(x[rows])
    wq_ref, rsw = OW.quantize_rows(w)
    sel = torch.from_numpy(rows).cuda()
    assert np.array_equal(acc[sel].cpu().numpy().astype(np.int64), OW.int8_matmul(rq, wq_ref))
    ref = OW.w8a8_linear(rq, rsx, wq_ref, rsw, b)
    got = y[sel].float().cpu().numpy()
    assert (np.abs(got - ref) <= BF16_REL * np.abs(ref) + 1e-6).all()


def test_deterministic_and_bias_optional():
    wf = RL.require_gpu()
    x, w, b = make_linear_inputs(300, 520, 1536, seed=12)
    xq, sx, wq, sw = _quantized(wf, x, w)
    y1 = wf.gemm_w8a8(xq, sx, wq, sw, None)
    y2 = wf.gemm_w8a8(xq, sx, wq, sw, None)
    yb = wf.gemm_w8a8(xq, sx, wq, sw, torch.zeros(520, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, yb)
