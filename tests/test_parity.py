"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances of the operator: |d logp| <= 1e-3 per row, relative d entropy <=
1e-3 per row, relative (Frobenius) d gradient <= 5e-3 per tensor. Small cases
are compared element by element; the full-size cases (T = 512, 5208, 7168 at
H = 4096, V = 151936) run the GPU on the whole batch, in the launch
configuration the benchmark times, and compare sampled rows, plus the
dW column-sum invariant (sum_v dW[v, :] = 0) on the whole output.
"""

import math

import numpy as np
import pytest
import torch

import rollout_rlk_linear_amd as rlk
import workloads as wl
from oracle import backward, decode_bf16, forward, slice_partials
from tests._util import (bits_equal, case_to_device, check_entropy, check_grad,
                         check_grad_elements, check_logp, dev, f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rlk.load_library()


# sum_v G[t, v] = 0 for every row, so the columns of dW sum to zero in exact
# arithmetic. The kernels multiply the bf16-rounded logit gradient, whose
# rounding errors do not cancel: per row their sum over v is a sum of
# independent errors, each uniform over half a bf16 ulp either side, and half
# an ulp is at most 2^-8 of the value, so its RMS is at most 2^-8 / sqrt(3) of
# ||G_t||; the same fraction of ||dW|| carries over to the column sum. (The
# float64 oracle's G rounded to bf16 gives 1.6e-3 to 1.7e-3 on these inputs.)
COLSUM_REL = 2.0 ** -8 / math.sqrt(3)


def check_column_sum(dw, what):
    colsum = dw.double().sum(dim=0)
    ratio = float(colsum.norm()) / float(dw.double().norm())
    assert ratio <= COLSUM_REL, f"{what}: ||sum_v dW[v]|| / ||dW|| = {ratio:.3e} > {COLSUM_REL:.3e}"


def n_dh(V):
    """fp32 additions on the longest path of a dH element: the MFMA chain
    over the vocabulary in steps of 32, the 32 products inside a step and the
    split partials (a generous count)."""
    return (V + 31) // 32 + 64


def n_dw(T):
    """The same for a dW element: the chain over the batch in steps of 32."""
    return (T + 31) // 32 + 64


def check_backward(dh, dw, rb, T, V, what):
    """Norm-wise, per-row and per-element checks of dH and dW against the
    oracle's rows (rb from backward(..., with_abs=True))."""
    check_grad(f64(dh), rb["dH"], f"{what} dH")
    check_grad(f64(dw), rb["dW"], f"{what} dW")
    check_grad_elements(dh, rb["dH"], rb["dH_abs"], n_dh(V), f"{what} dH elements")
    check_grad_elements(f64(dw), rb["dW"], rb["dW_abs"], n_dw(T), f"{what} dW elements")


def run_fwd(d, **kw):
    o = rlk.fwd(d["hidden"], d["weight"], d["targets"], **kw)
    torch.cuda.synchronize()
    return o


# ------------------------------------------------------------------ tiny

def test_tiny_forward():
    c = wl.tiny()
    d = case_to_device(c)
    o = run_fwd(d)
    ref = forward(c.hidden, c.weight, c.targets)
    check_logp(o["logp"].cpu().numpy(), ref["logp"], "tiny logp")
    check_entropy(o["entropy"].cpu().numpy(), ref["entropy"], "tiny entropy")
    st = o["stats"].cpu().double().numpy()
    np.testing.assert_allclose(st[:, 0], ref["m"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(np.log1p(st[:, 1]), np.log1p(ref["R"]), rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("with_dent", [True, False])
@pytest.mark.parametrize("dh_f32", [False, True])
def test_tiny_backward(with_dent, dh_f32):
    c = wl.tiny()
    d = case_to_device(c)
    o = run_fwd(d)
    de = d["dentropy"] if with_dent else None
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], de,
                     dhidden_f32=dh_f32)
    torch.cuda.synchronize()
    ref = backward(c.hidden, c.weight, c.targets, c.dlogp, c.dentropy if with_dent else None,
                   with_abs=True)
    assert dh.dtype == (torch.float32 if dh_f32 else torch.bfloat16)
    check_backward(dh, dw, ref, c.T, c.V, "tiny")


# ---------------------------------------------------- ragged / edge shapes

RAGGED = [(1, 64, 1), (1, 64, 2), (2, 64, 31), (3, 128, 33), (64, 64, 257), (65, 192, 1000),
          (70, 128, 4099), (300, 64, 777), (257, 256, 2304), (33, 320, 5000),
          (20, 256, 3001), (27, 192, 2000)]


@pytest.mark.parametrize("T,H,V", RAGGED)
def test_ragged_shapes(T, H, V):
    c = wl.make_case("ragged", T, H, V, seed=1000 + T + V, rms=True)
    c.weight = wl.to_bf16(c.weight.float() * 20)  # logits of spread ~ 1.3
    d = case_to_device(c)
    o = run_fwd(d)
    ref = forward(c.hidden, c.weight, c.targets)
    check_logp(o["logp"].cpu().numpy(), ref["logp"], f"logp {T,H,V}")
    check_entropy(o["entropy"].cpu().numpy(), np.maximum(ref["entropy"], 0), f"entropy {T,H,V}")
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], d["dentropy"])
    torch.cuda.synchronize()
    rb = backward(c.hidden, c.weight, c.targets, c.dlogp, c.dentropy, with_abs=True)
    if V > 1:
        check_backward(dh, dw, rb, T, V, f"{T,H,V}")
    else:  # one vocabulary entry: every gradient is exactly zero
        assert float(dh.float().abs().max()) == 0.0 and float(dw.abs().max()) == 0.0


@pytest.mark.parametrize("T,V", [(20, 1100), (64, 300), (70, 1100)])
def test_backward_ignores_stale_workspace(T, V):
    # The logit-gradient buffer in the workspace is written tile by tile; a
    # 256-row dW v-tile may read columns past V that no tile of a small batch
    # wrote (V = 1100: columns 1152..1279). Those feed only dW rows past V,
    # which are never stored. A workspace full of NaN bytes must give the
    # same bits as a zeroed one.
    H = 128
    c = wl.make_case("stale", T, H, V, seed=41 + T, rms=True)
    d = case_to_device(c)
    o = run_fwd(d)
    nws = max(rlk.bwd_workspace_bytes(T, H, V), 256)
    res = []
    for fill in (0x00, 0xFF):  # 0xFF bytes: every bf16 and fp32 value a NaN
        ws = torch.full((nws,), fill, dtype=torch.uint8, device="cuda")
        dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"],
                         d["dentropy"], out={"_ws_bwd": ws})
        torch.cuda.synchronize()
        res.append((dh.clone(), dw.clone()))
    assert torch.isfinite(res[1][0].float()).all() and torch.isfinite(res[1][1]).all()
    assert bits_equal(res[1][0], res[0][0]), f"dH depends on stale workspace bytes (T={T}, V={V})"
    assert bits_equal(res[1][1], res[0][1]), f"dW depends on stale workspace bytes (T={T}, V={V})"


# ------------------------------------------------------- maximum sizes

@pytest.mark.parametrize("T", [3, 70])
def test_max_hidden_size(T):
    # H = 65536 (RLK_MAX_H): the largest operand rows; T = 3 takes the
    # streaming forward (natural and packed W), T = 70 the tile kernels
    H, V = 65536, 300
    c = wl.make_case("maxH", T, H, V, seed=70 + T, rms=True)
    d = case_to_device(c)
    o = run_fwd(d)
    ref = forward(c.hidden, c.weight, c.targets)
    check_logp(o["logp"].cpu().numpy(), ref["logp"], f"logp T={T} H={H}")
    check_entropy(o["entropy"].cpu().numpy(), ref["entropy"], f"entropy T={T} H={H}")
    op = rlk.fwd_packed(d["hidden"], rlk.pack_weight(d["weight"]), d["targets"])
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], d["dentropy"])
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "stats"):
        assert torch.equal(op[k].view(torch.int32), o[k].view(torch.int32)), f"packed {k}"
    rb = backward(c.hidden, c.weight, c.targets, c.dlogp, c.dentropy, with_abs=True)
    check_backward(dh, dw, rb, T, V, f"T={T} H={H}")
    check_column_sum(dw, f"dW T={T} H={H}")


def test_max_batch_size():
    # T = 2^21 (RLK_MAX_T) rows: every row tile and dW's 2^21-long reduction;
    # sampled rows and vocabulary entries against the oracle
    T, H, V = 1 << 21, 64, 256
    c = wl.make_case("maxT", T, H, V, seed=77, rms=False)
    d = case_to_device(c)
    o = run_fwd(d)
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], None)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, T, 4099), [T - 1]]))
    ref = forward(c.hidden[rows], c.weight, c.targets[rows])
    check_logp(o["logp"].cpu().numpy()[rows], ref["logp"], "logp T=2^21")
    check_entropy(o["entropy"].cpu().numpy()[rows], ref["entropy"], "entropy T=2^21")
    vrows = np.array([0, 5, 100, 255])
    rb = backward(c.hidden, c.weight, c.targets, c.dlogp, None, dh_rows=rows, dw_rows=vrows,
                  with_abs=True)
    check_backward(dh[torch.from_numpy(rows).cuda()], dw[torch.from_numpy(vrows).cuda()], rb, T,
                   V, "rows T=2^21")
    check_column_sum(dw, "dW T=2^21")


def test_single_entry_vocabulary():
    c = wl.make_case("v1", 5, 64, 1, seed=3)
    o = run_fwd(case_to_device(c))
    assert torch.all(o["logp"] == 0).item() and torch.all(o["entropy"] == 0).item()


# ------------------------------------------------------------ closed forms

def test_uniform_logits_on_gpu():
    T, H, V = 40, 128, 3000
    hidden = wl.to_bf16(torch.randn(T, H, generator=torch.Generator().manual_seed(1)))
    tg = torch.randint(0, V, (T,), generator=torch.Generator().manual_seed(2), dtype=torch.int32)
    for W in (torch.zeros(V, H, dtype=torch.bfloat16),
              wl.to_bf16(torch.randn(1, H, generator=torch.Generator().manual_seed(3))).repeat(V, 1)):
        o = rlk.fwd(dev(hidden), dev(W), dev(tg))
        torch.cuda.synchronize()
        np.testing.assert_allclose(o["logp"].cpu().numpy(), -math.log(V), rtol=2e-6)
        np.testing.assert_allclose(o["entropy"].cpu().numpy(), math.log(V), rtol=2e-6)
        # every column ties at the max: R counts them exactly
        assert torch.all(o["stats"][:, 1] == V - 1).item()


@pytest.mark.parametrize("c_val", [64.0, 4.0])
def test_one_hot_dominant_on_gpu(c_val):
    V, H = 1024, 64
    a = math.sqrt(c_val)
    ys = [0, 31, 32, 255, 256, 1023]
    hidden = torch.zeros(len(ys), H)
    hidden[:, 0] = a
    outs_l, outs_e = [], []
    for i, y in enumerate(ys):
        W = torch.zeros(V, H)
        W[y, 0] = a
        o = rlk.fwd(dev(wl.to_bf16(hidden[i:i + 1])), dev(wl.to_bf16(W)),
                    dev(torch.tensor([y], dtype=torch.int32)))
        torch.cuda.synchronize()
        outs_l.append(o["logp"].item())
        outs_e.append(o["entropy"].item())
    ab = float(wl.to_bf16(torch.tensor(a)).float()) ** 2  # the exact bf16 logit
    q = (V - 1) * math.exp(-ab)
    np.testing.assert_allclose(outs_l, -math.log1p(q), rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(outs_e, math.log1p(q) + ab * q / (1 + q), rtol=1e-4)


def test_out_of_range_target_gives_nan():
    c = wl.make_case("oor", 4, 64, 100, seed=9)
    c.targets[1] = 100
    c.targets[2] = -1
    o = run_fwd(case_to_device(c))
    lp = o["logp"].cpu()
    assert torch.isnan(lp[1]) and torch.isnan(lp[2]) and torch.isfinite(lp[[0, 3]]).all()


def test_autograd_wrapper_matches_bwd():
    c = wl.tiny()
    d = case_to_device(c)
    h = d["hidden"].clone().requires_grad_(True)
    W = d["weight"].clone().requires_grad_(True)
    logp, ent = rlk.linear_logp(h, W, d["targets"])
    (logp * d["dlogp"] + ent * d["dentropy"]).sum().backward()
    o = run_fwd(d)
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], d["dentropy"])
    torch.cuda.synchronize()
    assert torch.equal(h.grad, dh)
    assert torch.equal(W.grad, dw.to(torch.bfloat16))


# ----------------------------------------------- full size: T = 512 (bench)

@pytest.fixture(scope="module")
def qwen():
    c = wl.qwen512()
    return c, case_to_device(c)


def test_qwen512_forward_all_rows(qwen):
    c, d = qwen
    o = run_fwd(d)
    ref = forward(c.hidden, c.weight, c.targets)
    check_logp(o["logp"].cpu().numpy(), ref["logp"], "qwen512 logp")
    check_entropy(o["entropy"].cpu().numpy(), ref["entropy"], "qwen512 entropy")


def test_qwen512_backward_sampled(qwen):
    c, d = qwen
    o = run_fwd(d)
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], None)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(11)
    rows = torch.randperm(c.T, generator=g)[:64].sort().values.numpy()
    vrows = np.unique(np.concatenate([torch.randperm(c.V, generator=g)[:192].numpy(),
                                      c.targets[:64].numpy(), [0, c.V - 1]]))
    ref = backward(c.hidden, c.weight, c.targets, c.dlogp, None, dh_rows=rows, dw_rows=vrows,
                   with_abs=True)
    check_backward(dh[torch.from_numpy(rows).cuda()], dw[torch.from_numpy(vrows).cuda()], ref,
                   c.T, c.V, "qwen512 rows")
    check_column_sum(dw, "qwen512")


def test_qwen512_backward_entropy_sampled(qwen):
    # the entropy-regularised objective: dlogp and dentropy both N(0,1)
    c, d = qwen
    dent_cpu = torch.randn(c.T, generator=torch.Generator().manual_seed(14), dtype=torch.float32)
    o = run_fwd(d)
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"],
                     dent_cpu.cuda())
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(15)
    rows = torch.randperm(c.T, generator=g)[:48].sort().values.numpy()
    vrows = np.unique(np.concatenate([torch.randperm(c.V, generator=g)[:128].numpy(),
                                      c.targets[:48].numpy()]))
    ref = backward(c.hidden, c.weight, c.targets, c.dlogp, dent_cpu, dh_rows=rows, dw_rows=vrows,
                   with_abs=True)
    check_backward(dh[torch.from_numpy(rows).cuda()], dw[torch.from_numpy(vrows).cuda()], ref,
                   c.T, c.V, "qwen512 rows (entropy term)")
    check_column_sum(dw, "qwen512 (entropy term)")


def test_persistent_recompute_whole_and_partial_tiles():
    # T = 600 gives T-tiles of 256, 256 and 88 rows and V = 40000 gives 480
    # recompute items for a grid of 256 workgroups, so a workgroup's two tiles
    # are of different T-tiles: a whole tile after a partial one and the other
    # way round. The next mainloop may start with the previous tile's G stores
    # still in flight only after a whole tile; every path must give the
    # oracle's gradients, and dH rows the bits of a 256-row call.
    c = wl.make_case("recompute_mix", 600, 128, 40000, seed=77, rms=True)
    d = case_to_device(c)
    o = run_fwd(d)
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], None)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(78)
    drow = np.unique(np.concatenate([torch.randperm(c.T, generator=g)[:40].numpy(),
                                     np.array([0, 255, 256, 511, 512, 599])]))
    vrows = np.unique(np.concatenate([torch.randperm(c.V, generator=g)[:96].numpy(),
                                      c.targets[drow].numpy(), np.array([0, c.V - 1])]))
    rb = backward(c.hidden, c.weight, c.targets, c.dlogp, None, dh_rows=drow, dw_rows=vrows,
                  with_abs=True)
    check_backward(dh[torch.from_numpy(drow).cuda()], dw[torch.from_numpy(vrows).cuda()], rb,
                   c.T, c.V, "T600 V40000 rows")
    check_column_sum(dw, "T600 V40000")
    sub = {k: v[:256].contiguous() for k, v in d.items() if k in ("hidden", "targets", "dlogp")}
    o2 = rlk.fwd(sub["hidden"], d["weight"], sub["targets"])
    dh2, _ = rlk.bwd(sub["hidden"], d["weight"], sub["targets"], o2["stats"], sub["dlogp"], None)
    torch.cuda.synchronize()
    assert bits_equal(dh2, dh[:256]), "dH rows of the first 256 tokens differ from a 256-row call"


# ------------------------------------------ full size: T = 5208 (full step)

@pytest.mark.slow
def test_step5208_sampled():
    c = wl.step5208()
    d = case_to_device(c)
    o = run_fwd(d)
    dh, dw = rlk.bwd(d["hidden"], d["weight"], d["targets"], o["stats"], d["dlogp"], None)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(12)
    rows = torch.randperm(c.T, generator=g)[:256].sort().values
    ref = forward(c.hidden[rows], c.weight, c.targets[rows])
    check_logp(o["logp"].cpu()[rows].numpy(), ref["logp"], "step5208 logp")
    check_entropy(o["entropy"].cpu()[rows].numpy(), ref["entropy"], "step5208 entropy")
    drow = rows[:32].numpy()
    vrows = np.unique(np.concatenate([torch.randperm(c.V, generator=g)[:96].numpy(),
                                      c.targets[drow].numpy()]))
    rb = backward(c.hidden, c.weight, c.targets, c.dlogp, None, dh_rows=drow, dw_rows=vrows,
                  with_abs=True)
    check_backward(dh[torch.from_numpy(drow).cuda()], dw[torch.from_numpy(vrows).cuda()], rb,
                   c.T, c.V, "step5208 rows")
    check_column_sum(dw, "step5208")


# --------------------------------- full size: T = 7168, TP=4 vocabulary slices

@pytest.mark.slow
def test_slice7168_partials_combine_and_backward():
    c = wl.slice7168()
    hd, td = dev(c.hidden), dev(c.targets)
    g = torch.Generator().manual_seed(13)
    rows = torch.randperm(c.T, generator=g)[:192].sort().values
    parts = []
    for (a, b) in c.meta["slices"]:
        Ws = dev(c.weight[a:b])
        o = rlk.fwd(hd, Ws, td, vocab_start=a, vocab_total=c.V)
        torch.cuda.synchronize()
        assert o["logp"] is None and o["entropy"] is None
        st = o["stats"].cpu()
        parts.append(st)
        m, R, B, zy = slice_partials(c.hidden[rows], c.weight[a:b], c.targets[rows], a)
        np.testing.assert_allclose(st[rows, 0].double().numpy(), m, rtol=1e-5, atol=1e-4)
        in_slice = np.isfinite(zy)
        assert np.array_equal(np.isfinite(st[rows, 3].numpy()), in_slice)
        np.testing.assert_allclose(st[rows, 3].double().numpy()[in_slice], zy[in_slice], atol=2e-4)
        del Ws
    logp, ent, stats = rlk.combine_host(parts)
    ref = forward(c.hidden[rows], c.weight, c.targets[rows])
    check_logp(logp[rows].numpy(), ref["logp"], "slice7168 logp")
    check_entropy(ent[rows].numpy(), ref["entropy"], "slice7168 entropy")
    # backward per slice with the combined statistics
    stats_d = dev(stats)
    drow = rows[:24].numpy()
    vsel = []
    dh_sum = None
    dw_rows = []
    for s, (a, b) in enumerate(c.meta["slices"]):
        Ws = dev(c.weight[a:b])
        dh, dw = rlk.bwd(hd, Ws, td, stats_d, dev(c.dlogp), None, vocab_start=a,
                         vocab_total=c.V, dhidden_f32=True)
        torch.cuda.synchronize()
        dh_s = dh[torch.from_numpy(drow).cuda()].double().cpu()
        dh_sum = dh_s if dh_sum is None else dh_sum + dh_s
        loc = torch.randperm(b - a, generator=g)[:24].sort().values
        vsel.append(loc.numpy() + a)
        dw_rows.append(dw[loc.cuda()].double().cpu())
        assert float(dw.double().sum(dim=0).norm()) > 0
        del Ws, dh, dw
    vsel = np.concatenate(vsel)
    rb = backward(c.hidden, c.weight, c.targets, c.dlogp, None, dh_rows=drow, dw_rows=vsel,
                  with_abs=True)
    check_grad(dh_sum.numpy(), rb["dH"], "slice7168 dH (sum of slices)")
    check_grad(torch.cat(dw_rows).numpy(), rb["dW"], "slice7168 dW rows")
    check_grad_elements(dh_sum.numpy(), rb["dH"], rb["dH_abs"], n_dh(c.V) + 4,
                        "slice7168 dH elements")
    check_grad_elements(torch.cat(dw_rows).numpy(), rb["dW"], rb["dW_abs"], n_dw(c.T),
                        "slice7168 dW elements")
