"""Per-element error bounds for the FP8 forward, derived from its arithmetic.

Test infrastructure: it takes the oracle's dequantised inputs, L and O (the
exact answer for the very codes the kernel reads) and bounds, element by
element, how far the FP8 kernel's O and L may lie from them. Nothing here
runs on the GPU or shares code with the kernels.

The kernel ("1.8x Faster Attention on an RTX 5080", section "P goes through
shared memory, then P.V"; "Kernels and Memory in LLM Inference", section
"FlashAttention-4" for the lagging reference) computes, per row i,
    p_j = 2^(s_j c - m_ref)    (m_ref within tau = 0.75 below the running max,
                                so p_j <= 2^tau),
    l   = sum_j p_j in fp32,
    O   = sum_j e4m3(256 p_j) v_j / (256 l), rounded to bf16,
    L   = ln 2 (m_ref + log2 l).
Writing P_ij = exp(S_ij - L_i) for the exact weights (rows sum to 1), the
error sources and their bounds are:
  * P's e4m3 rounding. A normal e4m3 value carries a relative error of at most
    2^-4 (three mantissa bits, round to nearest), so O moves by at most
    A_wc = 2^-4 sum_j P_ij |v_jd|. Rounding errors of different keys are
    unbiased and, for values that are not chosen adversarially, independent:
    their sum has a standard deviation of at most 2^-3 / sqrt(12) times
    sqrt(sum_j P_ij^2 v_jd^2). A_st = 7 of those standard deviations. The
    bound takes min(A_wc, A_st): a row dominated by one key gets the worst
    case, a row that averages many keys the statistical one.
  * Subnormal P. Below 2^-6 e4m3 is uniform with spacing 2^-9, so
    e4m3(256 p) is off by at most 2^-10 absolute, i.e. p by 2^-18 against the
    reference, which lies at most at the row's final max: B = 2^-18 exp(max_j S_ij
    - L_i) sum_j |v_jd|.
  * The FP8 MFMA does not sum in full fp32: its error is at most
    EPS_FP8_ACC * sum |a b| (pinned on the hardware by the MFMA probe test).
    On QK^T this moves score j by D_ij = EPS_FP8_ACC scale sum_d |q_id k_jd|;
    with D_i = max_j D_ij the weights change by a factor within
    exp(+-2 D_i), so O moves by at most (exp(2 D_i) - 1) sum_j P_ij |v_jd| and L by
    at most D_i. On P V it adds EPS_FP8_ACC (1 + 2^-4) sum_j P_ij |v_jd|.
  * fp32 sums. l adds n_i terms (n_i valid keys) in fp32, so its relative
    error is at most n_i 2^-24 (plus 2^-23 for exp2); that moves L and,
    through the division by l, O by the same relative amount.
  * bf16 output: at most 2^-8 of |O| (round to nearest with 8 significant
    bits: 1 + 2^-8 rounds to 1).
"""
from __future__ import annotations

import numpy as np

EPS_E4M3 = 2.0 ** -4
SIGMA_E4M3 = 2.0 ** -3 / np.sqrt(12.0)
K_SIGMA = 7.0


def fp8_bounds(ref_in, scale: float, L_ref, O_ref, causal: bool = False, rows=None,
               eps_acc: float = 2.0 ** -10, key_range=None, chunk: int = 256):
    """Per-element bound on |O_gpu - O_ref| and per-row bound on |L_gpu - L_ref|.

    ref_in: the dequantised (q, k, v) the oracle was fed, [B, H, N, d] (k and v
    may have fewer heads: grouped-query attention). L_ref [B, H, R] and
    O_ref [B, H, R, d] are the oracle's answers on the R compared rows (rows, or
    all N). key_range = (k0, k1) restricts the keys (a split-KV chunk); a row
    with no valid key gets bounds of 0. Returns (bound_O like O_ref, bound_L
    like L_ref, n_valid [B, H, R]): the bounds and each row's number of keys."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in ref_in)
    B, H, N, d = q.shape
    group = H // k.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    R = len(rows)
    bO = np.zeros((B, H, R, d))
    bL = np.zeros((B, H, R))
    nv = np.zeros((B, H, R))
    k0, k1 = (0, N) if key_range is None else key_range
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // group], v[b, h // group]
            ak, av, av2 = np.abs(kh), np.abs(vh), vh * vh
            for r0 in range(0, R, chunk):
                rr = rows[r0:r0 + chunk]
                qr = q[b, h, rr]
                S = scale * (qr @ kh.T)                        # [r, N]
                Dq = eps_acc * abs(scale) * (np.abs(qr) @ ak.T)
                keys = np.arange(N)[None, :]
                valid = np.broadcast_to((keys >= k0) & (keys < k1), (len(rr), N))
                if causal:
                    valid = valid & (keys <= rr[:, None])
                has = valid.any(axis=1)
                Lr = np.where(has, L_ref[b, h, r0:r0 + len(rr)], 0.0)
                P = np.where(valid, np.exp(np.where(valid, S, 0.0) - Lr[:, None]), 0.0)
                Di = np.max(np.where(valid, Dq, 0.0), axis=1)
                smax = np.where(has, np.max(np.where(valid, S, -np.inf), axis=1), 0.0)
                n_valid = valid.sum(axis=1).astype(np.float64)
                PV = P @ av                                     # sum_j P_ij |v_jd|
                A_wc = EPS_E4M3 * PV
                A_st = K_SIGMA * SIGMA_E4M3 * np.sqrt((P * P) @ av2)
                A = np.minimum(A_wc, A_st)
                Bsub = 2.0 ** -18 * np.exp(smax - Lr)[:, None] * (valid.astype(np.float64) @ av)
                C = np.expm1(2.0 * Di)[:, None] * PV
                F = eps_acc * (1.0 + EPS_E4M3) * PV
                rel_l = (n_valid + 2.0) * 2.0 ** -24
                Or = O_ref[b, h, r0:r0 + len(rr)]
                # the exponent argument s c - m: fp32 rounding of c and of the fma
                rel_l = rel_l + 2.0 ** -21 * (np.abs(smax) + np.abs(Lr) + 1.0)
                G = rel_l[:, None] * np.abs(Or)
                core = A + Bsub + C + F + G
                bO[b, h, r0:r0 + len(rr)] = np.where(has[:, None], core + 2.0 ** -8 * (np.abs(Or) + core) + 1e-6, 0.0)
                bL[b, h, r0:r0 + len(rr)] = np.where(has, Di + rel_l + 1e-6, 0.0)
                nv[b, h, r0:r0 + len(rr)] = n_valid
    return bO, bL, nv


def p_weighted_abs_v(ref_in, scale: float, L_ref, causal: bool = False, rows=None, chunk: int = 256):
    """sum_j P_ij |v_jd| for every compared element, with P_ij = exp(S_ij - L_i)
    the exact weights (rows without keys give 0). The bf16 forward rounds each
    p to bf16 before P V (relative error at most 2^-8: 8 significant bits,
    round to nearest) and its largest weight is exactly 1 (exact running max),
    so its O moves by at most 2^-8 times this; the bf16 stress checks of the
    parity tests add that term to their tolerance."""
    # bf16 inputs may come as torch tensors: widen them exactly first
    q, k, v = (x.double().numpy() if hasattr(x, "double") and not isinstance(x, np.ndarray)
               else np.asarray(x, dtype=np.float64) for x in ref_in)
    B, H, N, d = q.shape
    group = H // k.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.zeros((B, H, len(rows), d))
    for b in range(B):
        for h in range(H):
            kh, av = k[b, h // group], np.abs(v[b, h // group])
            for r0 in range(0, len(rows), chunk):
                rr = rows[r0:r0 + chunk]
                S = scale * (q[b, h, rr] @ kh.T)
                valid = np.ones_like(S, dtype=bool)
                if causal:
                    valid = np.arange(N)[None, :] <= rr[:, None]
                Lr = np.where(valid.any(axis=1), L_ref[b, h, r0:r0 + len(rr)], 0.0)
                P = np.where(valid, np.exp(np.where(valid, S, 0.0) - Lr[:, None]), 0.0)
                out[b, h, r0:r0 + len(rr)] = P @ av
    return out


def assert_fp8(O_gpu, L_gpu, O_ref, L_ref, ref_in, scale: float, causal: bool = False, rows=None,
               key_range=None, label: str = "", iid: bool = True, floor: float = 0.0,
               tol_o: float = 6e-2, tol_l: float = 1e-3):
    """The FP8 parity check, element by element: every element of O and every
    L within the bound derived above; cosine(O_gpu, O_ref) >= 0.999 over the
    rows that have keys; and, for iid inputs (iid=True), the stated FP8
    tolerances (tol_o + floor on O, tol_l on L) on every row that averages at
    least 64 keys. A row without keys (a split-KV chunk above its diagonal)
    must come out as O = 0, L = -inf. Prints the largest error, the largest
    error-to-bound ratio and the rows they come from."""
    from test_mfma_layout_gpu import EPS_FP8_ACC

    rows_i = np.arange(O_ref.shape[2]) if rows is None else np.asarray(rows)
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    L_gpu = np.asarray(L_gpu, dtype=np.float64)
    bO, bL, nv = fp8_bounds(ref_in, scale, L_ref, O_ref, causal=causal, rows=rows, eps_acc=EPS_FP8_ACC,
                            key_range=key_range)
    empty = nv == 0
    assert np.all(O_gpu[empty] == 0.0) and np.all(L_gpu[empty] == -np.inf), (label, "rows without keys")
    full = ~empty
    assert np.all(np.isfinite(O_gpu[full])) and np.all(np.isfinite(L_gpu[full])), (label, "non-finite")
    eO = np.where(full[..., None], np.abs(O_gpu - np.where(full[..., None], O_ref, 0.0)), 0.0)
    eL = np.where(full, np.abs(np.where(full, L_gpu, 0.0) - np.where(full, L_ref, 0.0)), 0.0)
    rO = np.where(full[..., None], eO / np.where(bO > 0, bO, 1.0), 0.0)
    rL = np.where(full, eL / np.where(bL > 0, bL, 1.0), 0.0)
    iO = np.unravel_index(np.argmax(rO), rO.shape)
    iE = np.unravel_index(np.argmax(eO), eO.shape)
    iL = np.unravel_index(np.argmax(rL), rL.shape)
    at = lambda i: (int(i[0]), int(i[1]), int(rows_i[i[2]])) + ((int(i[3]),) if len(i) > 3 else ())
    print(f"    fp8 bounds{(' ' + label) if label else ''}: max|dO| {eO[iE]:.3e} at (b,h,row,d)={at(iE)} "
          f"(bound there {bO[iE]:.3e}, {int(nv[iE[:3]])} keys); largest dO/bound {rO[iO]:.3f} at {at(iO)} "
          f"(bound {bO[iO]:.3e}); O bounds {bO[full].min():.3e}..{bO[full].max():.3e}; "
          f"max|dL| {eL.max():.3e}, largest dL/bound {rL[iL]:.3f} at {at(iL)} (bound {bL[iL]:.3e})", flush=True)
    assert rO[iO] <= 1.0, (label, "O beyond its derived bound", at(iO), eO[iO], bO[iO])
    assert rL[iL] <= 1.0, (label, "L beyond its derived bound", at(iL), eL[iL], bL[iL])
    a, b = O_gpu[full].ravel(), O_ref[full].ravel()
    if np.linalg.norm(b) > 0:
        cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
        assert cos >= 0.999, (label, cos)
    if iid:
        many = full & (nv >= 64)
        if many.any():
            e_o = float(np.max(eO[many]))
            e_l = float(np.max(eL[many]))
            print(f"    rows with >= 64 keys: max|dO| {e_o:.3e} (tol {tol_o + floor:.3e}) "
                  f"max|dL| {e_l:.3e} (tol {tol_l:.1e})", flush=True)
            assert e_o <= tol_o + floor and e_l <= tol_l, (label, e_o, e_l)
