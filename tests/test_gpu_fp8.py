"""GPU parity of the block-scaled FP8 path (quantisers and product) against
the float64 oracle in oracle/fp8_oracle.py.

Codes and scale bytes are integer results of one float decision per element,
taken in the same precision on both sides (exact power-of-two scaling, then
round to nearest even into E4M3), so they must match bit for bit.  The
product's terms are exactly representable (fp8 x fp8 x 2^e), but the matrix
core does not return their exactly rounded sum: within one 64-term step its
dot product keeps fewer bits than fp32 (errors near 2^-16 of sum_k |a_k b_k|
were measured at K = 128), and the steps are then summed in fp32.  The bound
checked element by element is (K * 2^-24 + 2^-13) * sum_k |a_k b_k| (plus
half a bf16 step of the result when C is bf16): a wrong scale, a dropped
k-step or a misplaced row gives errors of the order of the sum itself."""

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as f8
from tests.gpu_util import gpu, require_gpu, si

pytestmark = gpu


def _m():
    require_gpu()
    import head_latent_attention_08_amd as m
    return m


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def _act_bytes(e, rows, pitch):
    # oracle exponents [rows, K/128] -> E8M0 bytes [K/128, pitch]
    out = np.zeros((e.shape[1], pitch), dtype=np.uint8)
    out[:, :rows] = (e.T + 127).astype(np.uint8)
    return out


def _weight_bytes(e, rows, pitch):
    # oracle block exponents [ceil(rows/128), K/128] -> one byte per row
    per_row = np.repeat(e, 128, axis=0)[:rows]
    return _act_bytes(per_row, rows, pitch)


def _ties_tile():
    # a 1 x 128 tile (amax 448, so e = 0) holding exact midpoints of the E4M3
    # grid, normal and subnormal, both signs: round-half-to-even decides them
    table = f8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (table[1:] + table[:-1]) / 2
    mids = mids[si.round_bf16(mids.astype(np.float32)) == mids]   # bf16-representable ones
    v = np.concatenate([[448.0], mids, -mids])[:128]
    return np.pad(v, (0, 128 - len(v)), constant_values=0.5)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (300, 512), (64, 7168)])
def test_quantize_rows_matches_oracle_bitwise(dtype, rows, cols):
    m = _m()
    x, _ = si.make_fp8_operands(rows, 8, cols, seed=100 + rows)
    if rows > 2:
        x[1, :128] = _ties_tile()
        x[2, 128:256] = 0.0                      # all-zero tile: e = 0
        x[2, :128] *= np.float32(2.0 ** -60)      # tiny tile
        x = si.round_bf16(x)
    q, s = m.mla_fp8_quantize_rows(_dev(x, dtype))
    torch.cuda.synchronize()
    qo, eo = f8.quantize_act_tiles(x.astype(np.float64))
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    sb = s.cpu().numpy()
    assert sb.shape == (cols // 128, m.mla_fp8_scale_pitch(rows))
    np.testing.assert_array_equal(sb[:, :rows], (eo.T + 127).astype(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,cols", [(128, 128), (300, 384), (2112, 1024)])
def test_quantize_blocks_matches_oracle_bitwise(dtype, rows, cols):
    m = _m()
    _, w = si.make_fp8_operands(8, rows, cols, seed=200 + rows)
    q, s = m.mla_fp8_quantize_blocks(_dev(w, dtype))
    torch.cuda.synchronize()
    qo, eo = f8.quantize_weight_blocks(w.astype(np.float64))
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy()[:, :rows],
                                  _weight_bytes(eo, rows, m.mla_fp8_scale_pitch(rows))[:, :rows])


def _check_product(c, qa, ea, qb, eb, bf16_out):
    ref = f8.fp8_gemm(qa, ea, qb, eb)
    mag = np.abs(f8.dequant_act(qa, ea)) @ np.abs(f8.dequant_weight(qb, eb)).T
    K = qa.shape[1]
    bound = (K * 2.0 ** -24 + 2.0 ** -13) * mag + 1e-30
    if bf16_out:
        bound = bound + np.abs(ref) * 2.0 ** -8
    err = np.abs(c - ref)
    worst = np.max(err / bound)
    rel = np.max(err / (mag + 1e-30))
    print(f"fp8 product K={K} bf16={bf16_out}: max |err| / sum|ab| = {rel:.3g} (2^{np.log2(rel + 1e-300):.1f})")
    assert worst <= 1.0, f"max error / bound = {worst:.3g}"


@pytest.mark.parametrize("out", ["fp32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (64, 256, 128), (257, 264, 256), (1, 8, 384),
                                   (520, 1032, 2048)])
def test_gemm_matches_oracle(out, M, N, K):
    # oracle codes in, so the product alone is under test; K = 128 and 256
    # leave the main loop empty (fewer slabs than stages), the others run it
    m = _m()
    x, w = si.make_fp8_operands(M, N, K, seed=300 + M + N + K)
    qa, ea = f8.quantize_act_tiles(x.astype(np.float64))
    qb, eb = f8.quantize_weight_blocks(w.astype(np.float64))
    pa, pb = m.mla_fp8_scale_pitch(M), m.mla_fp8_scale_pitch(N)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    c = m.mla_fp8_gemm(dev(qa), dev(_act_bytes(ea, M, pa)), dev(qb), dev(_weight_bytes(eb, N, pb)),
                       out_dtype=torch.float32 if out == "fp32" else torch.bfloat16)
    torch.cuda.synchronize()
    _check_product(c.float().cpu().numpy().astype(np.float64), qa, ea, qb, eb, out == "bf16")


def test_gemm_padded_pitches_and_views():
    # row pitches above K and scale pitches above the minimum
    m = _m()
    M, N, K = 200, 136, 512
    x, w = si.make_fp8_operands(M, N, K, seed=7)
    qa, ea = f8.quantize_act_tiles(x.astype(np.float64))
    qb, eb = f8.quantize_weight_blocks(w.astype(np.float64))
    A = torch.zeros((M, K + 64), dtype=torch.uint8); A[:, :K] = torch.from_numpy(qa)
    B = torch.zeros((N, K + 32), dtype=torch.uint8); B[:, :K] = torch.from_numpy(qb)
    pa, pb = m.mla_fp8_scale_pitch(M) + 256, m.mla_fp8_scale_pitch(N) + 4
    C = torch.full((M, N + 8), float("nan"), dtype=torch.float32, device="cuda")
    m.mla_fp8_gemm(A.cuda()[:, :K], torch.from_numpy(_act_bytes(ea, M, pa)).cuda(), B.cuda()[:, :K],
                   torch.from_numpy(_weight_bytes(eb, N, pb)).cuda(), c=C[:, :N])
    torch.cuda.synchronize()
    Cn = C.cpu().numpy()
    assert np.all(np.isnan(Cn[:, N:]))            # nothing written past N
    _check_product(Cn[:, :N].astype(np.float64), qa, ea, qb, eb, False)


def test_quantize_then_gemm_end_to_end():
    # the device quantisers feed the device product; codes equal the oracle's
    m = _m()
    M, N, K = 384, 512, 1536
    x, w = si.make_fp8_operands(M, N, K, seed=11)
    qa, sa = m.mla_fp8_quantize_rows(_dev(x, "bf16"))
    qb, sb = m.mla_fp8_quantize_blocks(_dev(w, "bf16"))
    c = m.mla_fp8_gemm(qa, sa, qb, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qao, eao = f8.quantize_act_tiles(x.astype(np.float64))
    qbo, ebo = f8.quantize_weight_blocks(w.astype(np.float64))
    np.testing.assert_array_equal(qa.cpu().numpy(), qao)
    np.testing.assert_array_equal(qb.cpu().numpy(), qbo)
    _check_product(c.cpu().numpy().astype(np.float64), qao, eao, qbo, ebo, False)
    # and the block-scaled product stays close to the unquantised one
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.abs(c.cpu().numpy() - exact).max() / np.abs(exact).max()
    assert rel < 0.05


def test_gemm_is_deterministic():
    m = _m()
    M, N, K = 512, 768, 2048
    x, w = si.make_fp8_operands(M, N, K, seed=12)
    qa, sa = m.mla_fp8_quantize_rows(_dev(x, "bf16"))
    qb, sb = m.mla_fp8_quantize_blocks(_dev(w, "bf16"))
    c1 = m.mla_fp8_gemm(qa, sa, qb, sb)
    c2 = m.mla_fp8_gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_rows_unaligned_view(dtype):
    # a column window starting two elements in: element-wise loads and stores
    m = _m()
    rows, cols = 70, 640
    x, _ = si.make_fp8_operands(rows, 8, cols + 128, seed=21)
    xd = _dev(x, dtype)[:, 2:2 + cols]
    q, s = m.mla_fp8_quantize_rows(xd)
    torch.cuda.synchronize()
    qo, eo = f8.quantize_act_tiles(x[:, 2:2 + cols].astype(np.float64))
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy()[:, :rows], (eo.T + 127).astype(np.uint8))


def test_v3_out_projection_shape_sampled_rows():
    # the product at the output projection's full size (4096 tokens,
    # 7168 x 16384 weight), launched as the bench launches it (bf16 C): every
    # weight code and scale byte against the oracle, activation codes and
    # products on sampled rows
    m = _m()
    M, N, K = 4096, 7168, 16384
    x, w = si.make_fp8_operands(M, N, K, seed=13)
    qa, sa = m.mla_fp8_quantize_rows(_dev(x, "bf16"))
    qb, sb = m.mla_fp8_quantize_blocks(_dev(w, "bf16"))
    c = m.mla_fp8_gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    qbo, ebo = f8.quantize_weight_blocks(w.astype(np.float64))
    del w
    np.testing.assert_array_equal(qb.cpu().numpy(), qbo)
    np.testing.assert_array_equal(sb.cpu().numpy()[:, :N],
                                  _weight_bytes(ebo, N, m.mla_fp8_scale_pitch(N))[:, :N])
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 2047, 4095],
                                     np.random.default_rng(14).integers(0, M, 6)]))
    qao, eao = f8.quantize_act_tiles(x[rows].astype(np.float64))
    np.testing.assert_array_equal(qa.cpu().numpy()[rows], qao)
    np.testing.assert_array_equal(sa.cpu().numpy()[:, rows], (eao.T + 127).astype(np.uint8))
    _check_product(c.float().cpu().numpy()[rows].astype(np.float64), qao, eao, qbo, ebo, True)
