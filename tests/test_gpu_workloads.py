"""Parity at the workloads' full layer shapes (GPU, through the C ABI).

The workloads are the five synthetic layer configurations of gptq_inputs.
Every expected value comes from the float64 oracle run on the same input bytes:

* Hessian of the q_proj workload over all 262,144 calibration tokens, in one
  call (the benchmark's launch) and streamed as eight 32,768-token calls:
  sampled entries and the whole fp64 diagonal.
* Every layer at its full (d_out, d_in): both sides build H from the
  workload's first 32,768-token chunk (the GPU with the SYRK kernel, the
  oracle in float64); H is compared entry by entry, the factor as a whole,
  and the column loop on sampled rows (rows are independent given H), for
  every quantizer setting of the workload.
* The 70B down_proj (d_in = 28,672) is beyond a float64 factor in test time:
  sampled Hessian entries and the whole diagonal, the order, the factor's
  defining property U^T U H_d = I on sampled columns (H_d from the H the
  factor was given), and on sampled rows the codes' range,
  Q = scale * (code - zero), the packing, and GPTQ <= round-to-nearest.
"""
from __future__ import annotations

import numpy as np
import pytest

import gptq_inputs as gi
from oracle import gptq_ref as o

from gpu_helpers import compare_quant, gpu_hessian, say, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu
CHUNK = 32768


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import post_weight_quantization_29_amd as P
    P.lib()
    yield


def _diag_ref(chunks, dtype, d):
    """2 * sum_t x_t^2 per channel in float64, summed in blocks of 256 tokens."""
    acc = np.zeros(d)
    for x in chunks:
        for c0 in range(0, d, 2048):
            x64 = gi.to_float64(x[:, c0:c0 + 2048], dtype)
            n = x64.shape[0] - x64.shape[0] % 256
            sq = x64 * x64
            acc[c0:c0 + 2048] += sq[:n].reshape(-1, 256, sq.shape[1]).sum(axis=1).sum(axis=0)
            acc[c0:c0 + 2048] += sq[n:].sum(axis=0)
    return 2.0 * acc


def _check_h_sampled(Hg, idx, cols64, hd, diag_ref, tol=1e-4):
    ti = torch.as_tensor(idx, device=Hg.device)
    Hs = Hg.index_select(0, ti).index_select(1, ti).cpu().numpy().astype(np.float64)
    ref = 2.0 * cols64.T @ cols64
    dg = np.sqrt(np.diag(ref))
    err = np.abs(Hs - ref) / np.outer(dg, dg)
    say(f"  sampled H: max |dH|/sqrt(Hii Hjj) = {err.max():.2e}")
    assert err.max() <= tol
    hdn = hd.cpu().numpy()
    rel = np.abs(hdn - diag_ref) / diag_ref
    say(f"  fp64 diagonal: max rel = {rel.max():.2e}")
    assert rel.max() <= 1e-12


def _sample(n, k, seed, must=()):
    rng = np.random.default_rng(seed)
    s = set(int(v) for v in must)
    s.update(int(v) for v in rng.choice(n, size=min(n, k), replace=False))
    return np.array(sorted(s))


def test_q_proj_hessian_full_tokens():
    """All 262,144 tokens: one call (as timed) and eight streamed calls."""
    wl = gi.workload("c2_llama7b_q_proj")
    cal = wl.calib[0]
    d = cal.d_in
    say(f"[workload] c2 q_proj Hessian, N={cal.n_tokens} d={d}")
    X = gi.x_full(cal, wl.config)
    idx = _sample(d, 60, 11, must=gi.outlier_channels(cal, wl.config)[:4])
    cols64 = gi.to_float64(X[:, idx], cal.dtype)
    diag_ref = _diag_ref([X], cal.dtype, d)
    H1, hd1 = gpu_hessian([X], cal.dtype, d, with_diag=True)
    _check_h_sampled(H1, idx, cols64, hd1, diag_ref)
    del H1, hd1
    H2, hd2 = gpu_hessian([X[c:c + CHUNK] for c in range(0, X.shape[0], CHUNK)], cal.dtype, d,
                          with_diag=True)
    _check_h_sampled(H2, idx, cols64, hd2, diag_ref)


LAYERS = [("c2_llama7b_q_proj", 0), ("c3_llama7b_mlp", 0), ("c3_llama7b_mlp", 2),
          ("c4_13b_desc_act", 0), ("c4_13b_desc_act", 1)]

# Code agreement bar.  North star: >= 99.9 %, disagreements only at rounding
# ties.  GPTQ's error feedback makes a row's codes after its first tie flip
# diverge (the two sides then compensate different errors), so agreement is
# (rows with a flip) x (length of the divergence).  The kernels keep the
# column loop's running weights in fp64 like the oracle (with the oracle's
# own factor given to the GPU loop, no row flips at the 13B down_proj shape);
# what remains is H's fp32 accumulation (about 1e-6 relative after 2048
# accumulation steps), and in the oracle a 1e-6 relative perturbation of H
# alone moves 61 % of that layer's rows.  At d_in = 13824 with 4-bit groups of
# 64 this leaves 99.8-99.9 %; that one layer is held to 99.8 %, with every row's
# first disagreement at a tie and the objective within 1e-3 like the others.
AGREE = {("c4_13b_desc_act", 1): 0.998}


@pytest.mark.parametrize("key,li", LAYERS, ids=[f"{k.split('_')[0]}-{gi.workload(k).layers[i].name}"
                                                for k, i in LAYERS])
def test_workload_layer(key, li):
    import post_weight_quantization_29_amd as P
    wl = gi.workload(key)
    layer = wl.layers[li]
    cal = wl.calib_for(layer.d_in)
    d, d_out = layer.d_in, layer.d_out
    say(f"[workload] {key} {layer.name}: W {d_out}x{d}, H from {CHUNK} tokens, "
        f"{len(wl.quant)} quantizer setting(s)")
    x0 = gi.x_chunk(cal, wl.config, 0)
    W = gi.weight(layer, wl.config)
    W64 = gi.to_float64(W, layer.dtype)
    Hg, hd = gpu_hessian([x0], cal.dtype, d, with_diag=True)
    H64 = o.hessian([gi.to_float64(x0, cal.dtype)], d)
    # H entry by entry (fp32 accumulation of exact products)
    Hn = Hg.cpu().numpy().astype(np.float64)
    dg = np.sqrt(np.diag(H64))
    err = float((np.abs(Hn - H64) / np.outer(dg, dg)).max())
    say(f"  H: max |dH|/sqrt(Hii Hjj) = {err:.2e}")
    assert err <= 1e-4 and np.array_equal(Hn, Hn.T)
    assert np.max(np.abs(hd.cpu().numpy() - np.diag(H64)) / np.diag(H64)) <= 1e-12
    del Hn

    q0 = wl.quant[0]
    prep = o.prepare(H64, q0.damp_percent, bool(q0.desc_act))
    U = torch.empty((d, d), dtype=torch.float32, device="cuda")
    perm = torch.empty((d,), dtype=torch.int32, device="cuda")
    P.gptq_prepare_hinv(Hg, q0.damp_percent, q0.desc_act, U, perm, hd)
    assert np.array_equal(perm.cpu().numpy(), prep.perm)
    Un = U.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(Un - prep.U) / np.linalg.norm(prep.U)
    say(f"  U: rel Frobenius = {rel:.2e}")
    assert rel <= 1e-3 and np.all(np.tril(Un, -1) == 0)
    del Un

    rows = _sample(d_out, 62, 5, must=(0, d_out - 1))
    Wg = to_dev(W, layer.dtype)
    tr = torch.as_tensor(rows, device="cuda")
    bar = AGREE.get((key, li), 0.999)
    failures = []
    for q in wl.quant:
        assert q.damp_percent == q0.damp_percent and q.desc_act == q0.desc_act
        cfg = P.make_config(bits=q.bits, group_size=q.group_size, block_size=q.block_size,
                            damp_percent=q.damp_percent, desc_act=q.desc_act)
        res = P.quantize_layer_outputs(Wg, Hg, cfg, with_q=True, pack=True, U=U, perm=perm, hdiag=hd)
        ref = o.gptq(W64[rows], H64, bits=q.bits, group_size=q.group_size,
                     block_size=q.block_size, damp_percent=q.damp_percent,
                     desc_act=bool(q.desc_act), prepared=prep)
        G = d if q.group_size == -1 else q.group_size
        codes = res.codes.index_select(0, tr).cpu().numpy()
        par = compare_quant(ref, W64[rows], H64, codes, res.scales.index_select(0, tr).cpu().numpy(),
                            res.zeros.index_select(0, tr).cpu().numpy(),
                            res.Q.index_select(0, tr).cpu().numpy(), G)
        say(f"  {q.bits}-bit G{q.group_size}: {par}")
        ok = (np.array_equal(res.g_idx.cpu().numpy(), ref.g_idx)
              and codes.min() >= 0 and codes.max() <= (1 << q.bits) - 1
              and par.agree >= bar and par.first_not_tie == 0
              and par.scale_rel <= 1e-3 and par.zero_mismatch == 0 and par.q_bad == 0
              and par.obj_rel <= 1e-3)
        if res.packed is not None:
            pk = res.packed.index_select(0, tr).cpu().numpy().view(np.uint32)
            ok = ok and np.array_equal(pk, o.pack_int4(codes))
        if not ok:
            failures.append((q.bits, q.group_size))
        del res
    assert not failures, failures


def test_70b_down_proj_properties():
    import post_weight_quantization_29_amd as P
    wl = gi.workload("c5_70b_down_proj")
    layer, q = wl.layers[0], wl.quant[0]
    cal = wl.calib_for(layer.d_in)
    d, d_out = layer.d_in, layer.d_out
    say(f"[workload] c5 down_proj: W {d_out}x{d}, H from {CHUNK} tokens")
    x0 = gi.x_chunk(cal, wl.config, 0)
    Hg, hd = gpu_hessian([x0], cal.dtype, d, with_diag=True)
    idx = _sample(d, 48, 17)
    diag_ref = _diag_ref([x0], cal.dtype, d)
    _check_h_sampled(Hg, idx, gi.to_float64(x0[:, idx], cal.dtype), hd, diag_ref)
    del x0

    U = torch.empty((d, d), dtype=torch.float32, device="cuda")
    perm = torch.empty((d,), dtype=torch.int32, device="cuda")
    P.gptq_prepare_hinv(Hg, q.damp_percent, q.desc_act, U, perm, hd)
    pn = perm.cpu().numpy()
    assert np.array_equal(pn, o.order_from_keys(diag_ref, bool(q.desc_act)))
    # U^T U H_d = I on sampled columns of H_d = H[perm][:, perm] + lambda I
    lam = q.damp_percent * float(np.mean(diag_ref))
    S = _sample(d, 16, 23, must=(0, d - 1))
    tp = perm.long()
    HdS = Hg.index_select(0, tp).index_select(1, tp[torch.as_tensor(S, device="cuda")]).double()
    HdS[torch.as_tensor(S, device="cuda"), torch.arange(len(S), device="cuda")] += lam
    U64 = U.double()
    Z = (U64.t() @ (U64 @ HdS)).cpu().numpy()
    E = np.zeros_like(Z)
    E[S, np.arange(len(S))] = 1.0
    say(f"  U^T U H_d - I on {len(S)} columns: max {np.abs(Z - E).max():.2e}")
    assert np.abs(Z - E).max() <= 1e-2
    assert bool((torch.tril(U, -1) == 0).all()) and bool((torch.diagonal(U) > 0).all())
    del U64, HdS

    W = gi.weight(layer, wl.config)
    W64 = gi.to_float64(W, layer.dtype)
    cfg = P.make_config(bits=q.bits, group_size=q.group_size, block_size=q.block_size,
                        damp_percent=q.damp_percent, desc_act=q.desc_act)
    res = P.quantize_layer_outputs(to_dev(W, layer.dtype), Hg, cfg, with_q=True, pack=True,
                                   U=U, perm=perm, hdiag=hd)
    rows = _sample(d_out, 14, 29, must=(0, d_out - 1))
    tr = torch.as_tensor(rows, device="cuda")
    codes = res.codes.index_select(0, tr).cpu().numpy().astype(np.int64)
    scales = res.scales.index_select(0, tr).cpu().numpy()
    zeros = res.zeros.index_select(0, tr).cpu().numpy()
    Qg = res.Q.index_select(0, tr).cpu().numpy()
    g_idx = res.g_idx.cpu().numpy()
    assert np.array_equal(g_idx[pn], np.arange(d) // q.group_size)
    assert codes.min() >= 0 and codes.max() <= (1 << q.bits) - 1
    # Q = scale * (code - zero) in fp32, group by g_idx
    sc = scales[:, g_idx].astype(np.float32)
    zc = zeros[:, g_idx].astype(np.float32)
    assert np.array_equal(Qg, (sc * (codes.astype(np.float32) - zc)).astype(np.float32))
    pk = res.packed.index_select(0, tr).cpu().numpy().view(np.uint32)
    assert np.array_equal(pk, o.pack_int4(codes))
    # GPTQ does not do worse than round-to-nearest on H's objective
    Hn = Hg.cpu().numpy().astype(np.float64)
    _, Qr = o.rtn(W64[rows], bits=q.bits, group_size=q.group_size, perm=pn)
    og = o.objective(W64[rows], Qg.astype(np.float64), Hn)
    orr = o.objective(W64[rows], Qr, Hn)
    say(f"  objective on {len(rows)} rows: GPTQ {og:.4g}  RTN {orr:.4g}")
    assert og <= orr


_LARGE = {}


def _large_inputs(desc):
    """H (fp32, shared by both sides), W and the oracle's factor for desc_act."""
    if "H32" not in _LARGE:
        rng = np.random.default_rng(8192)
        X = rng.standard_normal((12288, 8192), dtype=np.float32)
        _LARGE["H32"] = 2.0 * (X.T @ X)
        _LARGE["W"] = (rng.standard_normal((4096, 8192)) * 0.02).astype(np.float16)
    if desc not in _LARGE:
        _LARGE[desc] = o.prepare(_LARGE["H32"].astype(np.float64), 0.01, bool(desc))
    return _LARGE["H32"], _LARGE["W"], _LARGE[desc]


@pytest.mark.parametrize("G,desc", [(-1, 0), (256, 1), (128, 1)])
def test_large_layer_wide_groups(G, desc):
    """A 4096 x 8192 layer (2^25 weights: the column loop's trailing updates
    overlap the next panel on a second stream) with one group per row, groups
    wider than the 128-column block, and in-block groups.  Both sides get the
    same fp32 H (2 X^T X of 12,288 normal tokens, more than the 8192
    channels, so that H is well conditioned like the workloads'), so only the
    factor and the loop are compared; sampled rows."""
    import post_weight_quantization_29_amd as P
    say(f"[large layer] 4096x8192 G{G} desc_act={desc}")
    H32, W, prep = _large_inputs(desc)
    d_out, d = W.shape
    H64 = H32.astype(np.float64)
    W64 = W.astype(np.float64)
    cfg = P.make_config(bits=4, group_size=G, desc_act=desc)
    res = P.quantize_layer_outputs(torch.from_numpy(W).cuda(), torch.from_numpy(H32).cuda(), cfg,
                                   with_q=True)
    rows = _sample(d_out, 16, 31, must=(0, d_out - 1))
    ref = o.gptq(W64[rows], H64, bits=4, group_size=G, damp_percent=0.01, desc_act=bool(desc),
                 prepared=prep)
    tr = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(res.perm.cpu().numpy(), ref.perm)
    assert np.array_equal(res.g_idx.cpu().numpy(), ref.g_idx)
    Ge = d if G == -1 else G
    codes = res.codes.index_select(0, tr).cpu().numpy()
    par = compare_quant(ref, W64[rows], H64, codes, res.scales.index_select(0, tr).cpu().numpy(),
                        res.zeros.index_select(0, tr).cpu().numpy(),
                        res.Q.index_select(0, tr).cpu().numpy(), Ge)
    say(f"  {par}")
    assert par.agree >= 0.999 and par.first_not_tie == 0
    assert par.scale_rel <= 1e-3 and par.zero_mismatch == 0 and par.q_bad == 0
    assert par.obj_rel <= 1e-3
