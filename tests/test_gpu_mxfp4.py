"""GPU parity of the mxfp4 mode (E2M1 codes, one E8M0 scale byte per 32
columns, no bias: the mode the ml-explore/mlx issue #3856 repro runs beside
affine) against the oracle.

Acceptance: qdequant codes and values bit-exact (subnormal and overflowing
products included); qmatvec rel-L2 <= 1e-5 (fp32); gather_qmm and
moe_gather_qmm per-row rel-L2 <= 2e-2 (bf16 MFMA), at K with and without a
half-step tail, unsorted = sorted, and zero bad rows at the issue's mxfp4
seam row count.
"""

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_unpack_amd import moeq, synth
from tests.gpu_util import bf16_bits_to_f32, bf16_dev, dev, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.mark.parametrize("batch,rows,cols,e_lo,e_hi", [(3, 37, 256, 118, 124), (1, 5, 96, 1, 254),
                                                       (2, 1, 32, 0, 3)])
def test_qdequant_bit_exact(batch, rows, cols, e_lo, e_hi):
    say(f"mxfp4 qdequant ({batch},{rows},{cols}) scale bytes {e_lo}..{e_hi}")
    host = synth.draw_mxfp4((81, rows, cols, e_lo), batch, rows, cols, e_lo, e_hi)
    codes, deq = moeq.qdequant(moeq.QTensor.from_host(host, dev()))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack_codes(host["q"], 4, cols))
    ref = oracle.dequantize(host)
    got = deq.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cols", [2048, 96])
def test_qmatvec(cols):
    host = synth.draw_mxfp4((82, cols), 1, 53, cols)
    h1 = dict(host, q=host["q"][0], scales=host["scales"][0], batch=1)
    x = np.random.default_rng(cols).standard_normal((6, cols)).astype(np.float32)
    y = moeq.qmatvec(moeq.QTensor.from_host(h1, dev()), to_dev(x))
    assert rel_l2_rows(y.cpu().numpy(), oracle.qmatvec(h1, x)).max() <= 1e-5


def _case(n, E, N, Kd, seed):
    host = synth.draw_mxfp4((83, E, N, Kd), E, N, Kd)
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits((rng.standard_normal((n, Kd)) * 0.5).astype(np.float32))
    ridx = np.sort(rng.integers(0, E, n)).astype(np.int32)
    return host, x, ridx


@pytest.mark.parametrize("n,E,N,Kd", [(1000, 8, 200, 2048), (700, 4, 96, 96), (300, 16, 64, 64),
                                      (1, 2, 256, 512)])
def test_gather_qmm(n, E, N, Kd):
    say(f"mxfp4 gather_qmm n={n} E={E} N={N} K={Kd} (K % 64 = {Kd % 64})")
    host, xb, ridx = _case(n, E, N, Kd, seed=n + Kd)
    W = moeq.QTensor.from_host(host, dev())
    out = moeq.gather_qmm(W, bf16_dev(xb), to_dev(ridx), sorted_indices=True)
    ref = oracle.gather_qmm(host, bf16_bits_to_f32(xb), ridx)
    err = rel_l2_rows(out.cpu().numpy(), ref)
    say(f"  max rel-L2 {err.max():.3e}")
    assert np.isfinite(out.cpu().numpy()).all() and err.max() <= TOL
    perm = np.random.default_rng(1).permutation(n)
    out_u = moeq.gather_qmm(W, bf16_dev(xb[perm]), to_dev(ridx[perm]), sorted_indices=False)
    assert torch.equal(out[perm], out_u)


def test_gather_qmm_seam_row_count_has_no_bad_rows():
    # the issue's mxfp4 trial: 32802 rows (n % 64 = 34), group size 32
    n = 32802
    host, xb, ridx = _case(n, 8, 64, 64, seed=5)
    W = moeq.QTensor.from_host(host, dev())
    outs = []
    for p in (float("nan"), 3.0e38):
        out = torch.full((n, 64), p, dtype=torch.float32, device=dev())
        moeq.gather_qmm(W, bf16_dev(xb), to_dev(ridx), sorted_indices=True, out=out)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    ref = oracle.gather_qmm(host, bf16_bits_to_f32(xb), ridx)
    rel = rel_l2_rows(outs[0].cpu().numpy(), ref)
    bad = int((~np.isfinite(rel) | (rel > TOL)).sum())
    say(f"  mxfp4 seam n={n}: max rel-L2 {np.nanmax(rel):.2e} bad rows {bad}")
    assert bad == 0


@pytest.mark.parametrize("H,I,m", [(512, 256, 500), (2048, 768, 64), (160, 96, 33)])
def test_moe_gather_qmm_with_mxfp4_experts(H, I, m):
    cfg = synth.scaled(synth.CONFIGS["c4"], hidden=H, inter=I, experts=16, top_k=4, tokens=m,
                       seed=84 + H)
    host = synth.mxfp4_experts(cfg, 0)
    L = moeq.MoELayer.from_host(host, dev())
    say(f"mxfp4 moe_gather_qmm H={H} I={I} M={m}")
    xb = synth.prefill_x_bf16(cfg, m)
    lg = synth.zipf_logits(cfg, m)
    idx, w = moeq.moe_route(None, to_dev(lg), cfg.experts, cfg.top_k)
    y = moeq.moe_gather_qmm(L, bf16_dev(xb), idx, w)
    torch.cuda.synchronize()
    ridx, rw, _ = oracle.route(lg.astype(np.float64), cfg.top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = oracle.moe_experts(host, bf16_bits_to_f32(xb), ridx, rw)
    err = rel_l2_rows(y.cpu().numpy(), ref)
    say(f"  max rel-L2 {err.max():.3e}")
    assert np.isfinite(y.cpu().numpy()).all() and err.max() <= TOL
