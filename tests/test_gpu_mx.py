"""GPU parity of the MXFP4 routed experts (FP8 activations with 64-element
blocks, FP4 weights with 32-element blocks) against the CPU oracle.

Quantisers: codes and scales bit-exact (the same exact decisions on both
sides: power-of-two scaling and round-to-nearest-even on the E2M1 / E4M3
grids).  Expert FFN, step-wise on the GPU's own routing, every row of every
expert: the GPU's quantised activation is compared with the oracle's
quantisation of the exact activation (computed in fp64 from the dequantised x
and weights): equal block scales away from power-of-two boundaries, codes
equal or one grid step apart plus what the activation's own error can move
(the instruction's accumulation error of h, bounded as for the output below,
carried through the activation's slope), at most 0.5% differing; the fp32
output must equal the oracle's down
projection of the GPU's quantised activation within 2e-4 of the sum of
absolute terms (the matrix instruction's internal accumulation, measured at
~1e-4 of it, plus fp32 rounding).
"""

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle as orc
from top_routing_expert_amd import binding as B, presets, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _w_oracle(codes_u8, scales_u8):
    """Device MXFP4 layout of one expert (codes [K/64, N, 32], scales [K/32, N])
    -> oracle codes [N, K] and scales [N, K/32]."""
    c = codes_u8.transpose(1, 0, 2).reshape(codes_u8.shape[1], -1).astype(np.int64)
    lo, hi = c & 15, c >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(c.shape[0], -1)
    return codes, scales_u8.T.astype(np.int64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_quantizers_bit_exact(dtype):
    p = presets.get("c4", dtype=dtype)
    rng = np.random.default_rng(60)
    G, N, K = 3, 256, 512
    w = (rng.normal(size=(G, N, K)) * np.exp(rng.uniform(-6, 6, size=(G, N, 1)))).astype(np.float32)
    w[0, 0, :32] = 0.0
    w[1, 1, 5] = 1e30
    if dtype == "bf16":
        w = synth.bf16_round(w)
    wt = torch.from_numpy(w).to(DEV).to(B.TORCH_DTYPE[dtype])
    codes, scales = B.mx_quantize_weights(p, wt)
    x = (rng.normal(size=(300, K)) * np.exp(rng.uniform(-10, 10, size=(300, 1)))).astype(np.float32)
    x[7] = 0.0
    x[8, 3] = -0.0
    if dtype == "bf16":
        x = synth.bf16_round(x)
    xq, xs = B.mx_quantize_act(p, torch.from_numpy(x).to(DEV).to(B.TORCH_DTYPE[dtype]), stride=320)
    torch.cuda.synchronize()
    for g in range(G):
        rc, rs = orc.mx_quantize(w[g], 32, "e2m1")
        gc, gs = _w_oracle(codes[g].cpu().numpy(), scales[g].cpu().numpy())
        np.testing.assert_array_equal(gs, rs)
        np.testing.assert_array_equal(gc, rc)
    rc, rs = orc.mx_quantize(x, 64, "e4m3")
    np.testing.assert_array_equal(_act_rows(xq.cpu().numpy())[:300].astype(np.int64), rc)
    np.testing.assert_array_equal(xs.cpu().numpy()[:, :300].T.astype(np.int64), rs)


def _act_rows(codes_u8):
    """Device FP8 activation codes [K/64, stride, 64] -> rows [stride, K]."""
    return codes_u8.transpose(1, 0, 2).reshape(codes_u8.shape[1], -1)


def _grid_step(v, sc):
    """FP8 E4M3 grid step at |v| under the block scale code sc."""
    X = sc.astype(np.float64) - 127
    a = np.abs(v) / np.exp2(X)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    return np.exp2(e - 3 + X)


def _act_error(h, dh, F, act):
    """Bound of |act(h + e) - act(h)| for |e| <= dh elementwise: the slope
    term plus the second-order ones (|silu'| <= 1.1, |silu''| <= 0.5,
    |gelu''| <= 0.8)."""
    if act == "swiglu":
        hg, hu = h[:, :F], h[:, F:]
        dg, du = dh[:, :F], dh[:, F:]
        sg = 1.0 / (1.0 + np.exp(-hg))
        ds = sg * (1 + hg * (1 - sg))
        return (np.abs(ds * hu) * dg + np.abs(hg * sg) * du + 1.1 * dg * du
                + 0.25 * (np.abs(hu) + du) * dg * dg)
    dgelu = 0.5 * (1 + sps.erf(h / np.sqrt(2))) + h * np.exp(-0.5 * h * h) / np.sqrt(2 * np.pi)
    return np.abs(dgelu) * dh + 0.4 * dh * dh


@pytest.mark.parametrize("name", ["c4", "c2"])
def test_expert_ffn_mx_parity(name):
    p = presets.get(name)
    inp = synth.make_inputs(p, seed=0)
    x = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16).contiguous()
    w = B.weights_to_device(p, inp, DEV)
    r = B.route(p, x, w.Wg, w.offset, w.sel_bias)
    pm = B.permute(p, x, r["idx"])
    R_max = p.T * p.k
    xq, xs = B.mx_quantize_act(p, pm["x_perm"], stride=B.mx_stride(R_max))
    W13q, W13s = B.mx_quantize_weights(p, w.W13)
    W2q, W2s = B.mx_quantize_weights(p, w.W2)
    res = B.expert_ffn_mx(p, xq, xs, pm["offsets"], W13q, W13s, W2q, W2s, max_rows=R_max)
    torch.cuda.synchronize()
    offsets = pm["offsets"].cpu().numpy().astype(np.int64)
    sizes = np.diff(offsets)
    experts = [e for e in range(p.E) if sizes[e] > 0]
    xq_h, xs_h = _act_rows(xq.cpu().numpy()), xs.cpu().numpy()
    aq_h, aqs_h = _act_rows(res["aq"].cpu().numpy()), res["aqs"].cpu().numpy()
    out_h = res["out"].cpu().numpy()
    W13q_h, W13s_h = W13q.cpu().numpy(), W13s.cpu().numpy()
    W2q_h, W2s_h = W2q.cpu().numpy(), W2s.cpu().numpy()
    worst_out, near_boundary, codes_off = 0.0, 0, 0
    print(f"[mx] {name}: oracle on all {int(offsets[-1])} rows of {len(experts)} experts", flush=True)
    for e in experts:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rows = np.arange(r0, r1)
        xd = orc.mx_dequantize(xq_h[rows].astype(np.int64), xs_h[:, rows].T.astype(np.int64), 64, "e4m3")
        c13, s13 = _w_oracle(W13q_h[e], W13s_h[e])
        W13d = orc.mx_dequantize(c13, s13, 32, "e2m1")
        h = xd @ W13d.T
        a = orc.silu(h[:, :p.F]) * h[:, p.F:] if p.act == "swiglu" else orc.gelu(h)
        sc_gpu = aqs_h[:, rows].T.astype(np.int64)
        ad = orc.mx_dequantize(aq_h[rows].astype(np.int64), sc_gpu, 64, "e4m3")
        # the oracle's quantisation of the exact activation (saturation at 448
        # included): block scales equal unless the block maximum sits at a
        # power-of-two boundary
        rc, sc_ref = orc.mx_quantize(a, 64, "e4m3")
        rd = orc.mx_dequantize(rc, sc_ref, 64, "e4m3")
        amax = np.abs(a.reshape(len(rows), -1, 64)).max(axis=2)
        frac = np.log2(np.maximum(amax, 1e-300)) % 1.0
        boundary = (frac < 1e-3) | (frac > 1 - 1e-3)
        assert np.all((sc_gpu == sc_ref) | boundary), f"expert {e}: scale mismatch away from boundaries"
        near_boundary += int(boundary.sum())
        # codes: equal, or apart by one grid step (the fp32 activation fell on
        # the other side of a rounding midpoint) plus what the activation's own
        # error can move: h carries the scaled instruction's accumulation
        # error, at most 2e-4 of its sum of absolute terms (the bound the
        # output check below uses), carried through the activation's slope
        same = np.repeat(sc_gpu == sc_ref, 64, axis=1)
        step = _grid_step(np.maximum(np.abs(rd), np.abs(ad)), np.repeat(sc_gpu, 64, axis=1))
        dh = 2e-4 * (np.abs(xd) @ np.abs(W13d.T))
        da = _act_error(h, dh, p.F, p.act)
        off = np.abs(ad - rd)[same] - step[same] * 1.0001 - da[same]
        assert np.all(off <= 0), f"expert {e}: {int((off > 0).sum())} activation codes off by more than one step plus the activation's error"
        n_diff = int((ad != rd)[same].sum())
        assert n_diff <= 0.005 * same.sum(), f"expert {e}: {n_diff} activation codes differ"
        codes_off += n_diff
        c2, s2 = _w_oracle(W2q_h[e], W2s_h[e])
        W2d = orc.mx_dequantize(c2, s2, 32, "e2m1")
        ref = ad @ W2d.T
        cond = np.abs(ad) @ np.abs(W2d.T)
        err = np.abs(out_h[rows] - ref)
        worst_out = max(worst_out, float(np.max(err / (cond + 1e-30))))
        assert np.all(err <= 2e-4 * cond + 1e-6 * np.sqrt(np.mean(ref ** 2))), f"expert {e}: output"
    print(f"{name}: every row of {len(experts)} experts, output err/sum|terms| {worst_out:.2e}, "
          f"boundary blocks {near_boundary}, codes one step off {codes_off}")


def test_fp8_activation_codes_at_every_rounding_midpoint():
    """E4M3 activation codes bit-exact against the oracle on crafted values:
    every positive grid point (subnormals included), every midpoint between
    neighbouring grid points (exact ties, which go to the even code), both fp32
    neighbours of each midpoint, values that saturate to 448, both signs and
    both zeros.  Each 64-element block leads with 480, so its scale is 2^0
    (largest magnitude in [256, 512)) and the element values are coded as
    they stand."""
    p = presets.get("c4", dtype="f32")
    grid = [m * 2.0 ** -9 for m in range(1, 8)]
    grid += [(8 + m) * 2.0 ** (e - 3) for e in range(-6, 9) for m in range(8) if (8 + m) * 2.0 ** (e - 3) <= 448]
    grid = np.array(sorted(set([0.0] + grid)), dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    m32 = mids.astype(np.float32)
    assert np.all(m32.astype(np.float64) == mids)      # the ties are exact in fp32
    vals = np.concatenate([grid.astype(np.float32), m32,
                           np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0)),
                           np.array([448.5, 449, 460, 464, 470, 479.9, 480], np.float32)])
    vals = np.concatenate([vals, -vals, np.array([0.0, -0.0], np.float32)])
    n_per = 63
    rows = -(-len(vals) // n_per)
    x = np.zeros((rows, 64), np.float32)
    x[:, 0] = 480.0
    flat = np.zeros(rows * n_per, np.float32)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(rows, n_per)
    K = 512                                             # eight 64-blocks per row
    x = np.tile(x, (1, K // 64))
    xq, xs = B.mx_quantize_act(p, torch.from_numpy(x).to(DEV), stride=B.mx_stride(rows))
    torch.cuda.synchronize()
    rc, rs = orc.mx_quantize(x, 64, "e4m3")
    assert np.all(rs == 127)
    np.testing.assert_array_equal(xs.cpu().numpy()[:, :rows].T.astype(np.int64), rs)
    np.testing.assert_array_equal(_act_rows(xq.cpu().numpy())[:rows].astype(np.int64), rc)
