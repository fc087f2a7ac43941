"""GPU parity of activation ordering and static groups ([P1] "GPTQ：基于近似二阶信息的
大模型权重量化", GPTQ 的高级技巧: 激活排序（desc_act）, 静态与动态分组), through the C ABI,
against the float64 oracle (oracle.activation_order, oracle.gptq_ordered)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import ETA, check_row_losses, compare_quant
from post_weight_quantization_syrk_amd import gptq, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    gptq.lib()


def dev(a, dtype=np.float32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to(DEV)


def rand_x(n, d, seed, ld=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, ld or d), dtype=np.float32) * np.exp(
        rng.standard_normal(ld or d)).astype(np.float32)
    b = synth.f32_to_bf16_bits(x)
    return b, synth.as_f64(b, "bf16")[:, :d]


def spd(d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3 * d, d)) @ (np.eye(d) + 0.3 * rng.standard_normal((d, d)) / np.sqrt(d))
    x *= np.exp(0.5 * rng.standard_normal(d))
    return (2.0 * x.T @ x).astype(np.float32)


def gpu_ordered(W, H32, perm_np, *, bits, g, sym, static):
    perm = dev(perm_np, np.int32) if perm_np is not None else None
    H = dev(H32)
    U, dead, _ = gptq.gptq_prepare_hinv_perm(H, perm)
    codes, scales, zeros, g_idx, loss = gptq.gptq_quantize_layer_perm(
        dev(W), U, dead, perm, static_groups=static, bits=bits, group_size=g, sym=sym)
    torch.cuda.synchronize()
    return dict(codes=codes.cpu().numpy(), scales=scales.cpu().numpy(),
                zeros=zeros.cpu().numpy(), g_idx=g_idx.cpu().numpy(), loss=loss.cpu().numpy())


# ---------------------------------------------------------------- the order
@pytest.mark.parametrize("n,d,ld", [(1000, 256, None), (777, 37, None), (3000, 520, 528),
                                    (64, 1000, None)])
def test_act_order_matches_oracle(n, d, ld):
    print(f"[act_order] n={n} d={d} ld={ld}", flush=True)
    xb, x64 = rand_x(n, d, seed=n + d, ld=ld)
    X = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    a = torch.empty(d, dtype=torch.float64, device=DEV)
    perm, _ = gptq.gptq_act_order(X, d, act_sum=a)
    torch.cuda.synchronize()
    ref, ra = oracle.activation_order([x64])
    np.testing.assert_allclose(a.cpu().numpy(), ra, rtol=1e-12)
    np.testing.assert_array_equal(perm.cpu().numpy(), ref)


def test_act_order_fp32_ties_and_no_tokens():
    X = np.array([[1.0, -3.0, 0.5, 2.0, 0.0], [2.0, 1.0, -0.5, -1.0, 0.0]], dtype=np.float32)
    perm, _ = gptq.gptq_act_order(dev(X))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(perm.cpu().numpy(), [4, 2, 0, 3, 1])
    empty = torch.empty((0, 6), dtype=torch.float32, device=DEV)
    perm0, _ = gptq.gptq_act_order(empty)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(perm0.cpu().numpy(), np.arange(6))


# ---------------------------------------------------------------- prepare
@pytest.mark.parametrize("d", [100, 256, 1000])
def test_prepare_perm(d):
    print(f"[prepare_perm] d={d}", flush=True)
    H32 = spd(d, 21 + d)
    H32 = np.tril(H32) + np.tril(H32, -1).T  # exactly symmetric
    H32[7, :] = 0.0
    H32[:, 7] = 0.0   # a dead channel
    perm_np = np.random.default_rng(d).permutation(d).astype(np.int32)
    Hd = dev(H32)
    U, dead, _ = gptq.gptq_prepare_hinv_perm(Hd, dev(perm_np, np.int32))
    # the same kernels on the matrix permuted on the host give the same bits
    Hp = dev(H32[np.ix_(perm_np, perm_np)])
    U2, _, _ = gptq.gptq_prepare_hinv(Hp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(U.cpu().numpy(), U2.cpu().numpy())
    dn = dead.cpu().numpy().astype(bool)
    assert dn[7] and dn.sum() == 1
    ref = oracle.prepare(oracle.act_order._lower_to_symmetric(H32)[np.ix_(perm_np, perm_np)])
    Ur = ref["U"]
    bar = max(2e-6, np.sqrt(d) * 2.0 ** -24) * np.abs(Ur).max()
    assert np.abs(U.cpu().numpy() - Ur).max() <= bar
    # H is damped and mirrored in natural order
    Hn = Hd.cpu().numpy()
    np.testing.assert_allclose(Hn, Hn.T, rtol=0, atol=0)


# ---------------------------------------------------------------- quantize
QC = [(4, 128, False), (3, 64, True), (2, 32, False), (4, -1, False)]


@pytest.mark.parametrize("bits,g,sym", QC)
@pytest.mark.parametrize("static", [False, True])
def test_diagonal_hessian_exact(bits, g, sym, static):
    # no feedback between columns: bit-exact against round-to-nearest
    d_out, d_in = 48, 256
    print(f"[act_order diag] bits={bits} g={g} sym={sym} static={static}", flush=True)
    rng = np.random.default_rng(31)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    H32 = np.diag(np.linspace(1.0, 3.0, d_in)).astype(np.float32)
    perm = rng.permutation(d_in).astype(np.int32)
    out = gpu_ordered(W, H32, perm, bits=bits, g=g, sym=sym, static=static)
    ref = oracle.gptq_ordered(W, H32, perm, bits=bits, group_size=g, sym=sym, block=128,
                              static_groups=static)
    np.testing.assert_array_equal(out["codes"], ref["codes"])
    np.testing.assert_array_equal(out["scales"], ref["scales"])
    np.testing.assert_array_equal(out["zeros"], ref["zeros"])
    np.testing.assert_array_equal(out["g_idx"], ref["g_idx"])


@pytest.mark.parametrize("bits,g,sym", QC[:3])
def test_dynamic_groups_correlated(bits, g, sym):
    d_out, d_in = 96, 384
    print(f"[act_order dyn] bits={bits} g={g} sym={sym}", flush=True)
    H32 = spd(d_in, 41)
    rng = np.random.default_rng(42)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    perm = rng.permutation(d_in).astype(np.int32)
    out = gpu_ordered(W, H32, perm, bits=bits, g=g, sym=sym, static=False)
    ref = oracle.gptq_ordered(W, H32, perm, bits=bits, group_size=g, sym=sym, block=128)
    np.testing.assert_array_equal(out["g_idx"], ref["g_idx"])
    # groups are runs in processing order: compare there
    gpu_p = dict(codes=out["codes"][:, perm], scales=out["scales"], zeros=out["zeros"])
    ref_p = dict(codes=ref["codes_p"], scales=ref["scales"], zeros=ref["zeros"],
                 raw_scales=ref["raw_scales"], raw_zeros=ref["raw_zeros"], raw_q=ref["raw_q_p"],
                 What=ref["What_p"])
    Hs = oracle.act_order._lower_to_symmetric(H32)
    rep = compare_quant(gpu_p, ref_p, group_size=g, bits=bits, W=W.astype(np.float64)[:, perm],
                        H0=Hs[np.ix_(perm, perm)])
    print(f"[act_order dyn] {rep}", flush=True)
    check_row_losses(out["loss"], gpu_p, dict(ref_p, loss_damped=ref["loss_damped"]))


@pytest.mark.parametrize("bits,g,sym", QC[:3])
def test_static_groups_correlated(bits, g, sym):
    d_out, d_in = 96, 384
    print(f"[act_order static] bits={bits} g={g} sym={sym}", flush=True)
    H32 = spd(d_in, 51)
    rng = np.random.default_rng(52)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    perm = rng.permutation(d_in).astype(np.int32)
    out = gpu_ordered(W, H32, perm, bits=bits, g=g, sym=sym, static=True)
    ref = oracle.gptq_ordered(W, H32, perm, bits=bits, group_size=g, sym=sym, block=128,
                              static_groups=True)
    # parameters come from the original weights on both sides: exact
    np.testing.assert_array_equal(out["scales"], ref["scales"])
    np.testing.assert_array_equal(out["zeros"], ref["zeros"])
    np.testing.assert_array_equal(out["g_idx"], np.arange(d_in) // g)
    # codes: in processing order each row matches up to its first difference,
    # which must be a near-tie of the quotient; few codes differ
    cg = out["codes"][:, perm].astype(np.int64)
    cr = ref["codes_p"].astype(np.int64)
    zk = ref["zeros"][:, perm // g]
    for r in np.nonzero((cg != cr).any(axis=1))[0]:
        k = int(np.nonzero(cg[r] != cr[r])[0][0])
        lo = min(cg[r, k], cr[r, k])
        assert abs(cg[r, k] - cr[r, k]) == 1, (r, k)
        assert abs(ref["raw_q_p"][r, k] - ((lo - zk[r, k]) + 0.5)) <= ETA, (r, k)
    assert (cg != cr).mean() <= 0.005
    check_row_losses(out["loss"], dict(codes=cg, scales=out["scales"], zeros=out["zeros"]),
                     dict(codes=cr, scales=ref["scales"], zeros=ref["zeros"],
                          loss_damped=ref["loss_damped"]))


def test_null_perm_is_the_plain_path():
    d_out, d_in = 64, 256
    H32 = spd(d_in, 61)
    W = (0.02 * np.random.default_rng(62).standard_normal((d_out, d_in))).astype(np.float32)
    U, dead, _ = gptq.gptq_prepare_hinv(dev(H32))
    c1, s1, z1, _ = gptq.gptq_quantize_layer(dev(W), U, dead, bits=4, group_size=64)
    U2, dead2, _ = gptq.gptq_prepare_hinv_perm(dev(H32), None)
    c2, s2, z2, gi, _ = gptq.gptq_quantize_layer_perm(dev(W), U2, dead2, None, bits=4,
                                                      group_size=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(U.cpu().numpy(), U2.cpu().numpy())
    np.testing.assert_array_equal(c1.cpu().numpy(), c2.cpu().numpy())
    np.testing.assert_array_equal(s1.cpu().numpy(), s2.cpu().numpy())
    np.testing.assert_array_equal(gi.cpu().numpy(), np.arange(d_in) // 64)


def test_end_to_end_small_workload_ordered():
    # X -> H -> order -> factor -> quantize (static groups), against the oracle's pipeline
    wl = synth.scaled(synth.ATTN7B, d_out=64, d_in=256, n_tokens=4096, chunk_tokens=4096)
    print(f"[act_order e2e] {wl.name}", flush=True)
    xb = synth.x_chunk(wl, 0)
    x64 = synth.as_f64(xb, "bf16")
    X = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    W32 = synth.bf16_bits_to_f32(synth.w_matrix(wl)).astype(np.float32)
    H = torch.zeros((256, 256), dtype=torch.float32, device=DEV)
    gptq.gptq_hessian_accumulate(H, X)
    perm, _ = gptq.gptq_act_order(X)
    U, dead, _ = gptq.gptq_prepare_hinv_perm(H, perm)
    codes, scales, zeros, g_idx, _ = gptq.gptq_quantize_layer_perm(
        dev(W32), U, dead, perm, static_groups=True, bits=4, group_size=128)
    torch.cuda.synchronize()
    ref_perm, _ = oracle.activation_order([x64])
    np.testing.assert_array_equal(perm.cpu().numpy(), ref_perm)
    H0 = oracle.hessian([x64])
    ref = oracle.gptq_ordered(W32, H0, ref_perm, bits=4, group_size=128, block=128,
                              static_groups=True)
    np.testing.assert_array_equal(scales.cpu().numpy(), ref["scales"])
    cg, cr = codes.cpu().numpy(), ref["codes"]
    assert (cg != cr).mean() <= 0.005
    What = scales.cpu().numpy()[:, g_idx.cpu().numpy()] * (cg - zeros.cpu().numpy()[:, g_idx.cpu().numpy()])
    lg = oracle.layer_loss(W32.astype(np.float64), What, H0)
    lr = oracle.layer_loss(W32.astype(np.float64), ref["What"], H0)
    assert abs(lg - lr) <= 1e-3 * lr
