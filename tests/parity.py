"""Helpers for GPU-vs-oracle parity tests: device upload/download and the
acceptance rule for the draft head's picks and probabilities.

Acceptance (the method's contract, restated):
  * counts, n_invalid, t2f, f2t, sums and W_trim: bit-exact;
  * picks: at every rank the GPU id equals the oracle's, or the two ids'
    fp64 logits differ by at most 1e-3; every GPU id is a kept id whose
    logit is within 1e-3 of the oracle's k-th or above, and ids in a row
    are distinct;
  * probabilities: each GPU probability is within 2e-3 absolute of the
    oracle's fp64 subset-softmax probability of the same id; as a stricter
    diagnostic also within 1e-4 relative (bf16 inputs, fp32 sums give
    about 1e-6).
"""
import numpy as np
import torch

DEV = torch.device("cuda:0")
Z_TIE = 1e-3
P_ABS = 2e-3
P_REL = 1e-4


def to_dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def to_dev_u32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV).view(torch.uint32)


def to_dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def u32_host(t):
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def u64_scalar(t):
    return int(t.view(torch.int64).item())


def bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def inverse_map(t2f):
    inv = {}
    for j, f in enumerate(np.asarray(t2f).tolist()):
        inv[f] = j
    return inv


def check_picks(ids_g, probs_g, z_o, t2f, k, ids_o=None):
    """Checks GPU picks against fp64 oracle logits z_o[M, V_high]."""
    ids_g = np.asarray(ids_g)
    probs_g = np.asarray(probs_g, dtype=np.float64)
    M = z_o.shape[0]
    inv = inverse_map(t2f)
    t2f = np.asarray(t2f)
    worst = {"p_abs": 0.0, "p_rel": 0.0, "swaps": 0}
    for m in range(M):
        z = z_o[m]
        mu = z.max()
        e = np.exp(z - mu)
        p = e / e.sum()
        order = np.lexsort((t2f, -z))[:k]
        want = t2f[order]
        if ids_o is not None:
            np.testing.assert_array_equal(want, ids_o[m])
        zk = z[order[-1]]
        row = ids_g[m]
        assert len(set(row.tolist())) == k, f"row {m}: repeated ids {row}"
        for r in range(k):
            g = int(row[r])
            assert g in inv, f"row {m} rank {r}: id {g} is not a kept id"
            zg = z[inv[g]]
            if g != int(want[r]):
                worst["swaps"] += 1
                assert abs(zg - z[order[r]]) <= Z_TIE, (m, r, g, int(want[r]), zg, z[order[r]])
            assert zg >= zk - Z_TIE, (m, r, zg, zk)
            pa = abs(probs_g[m, r] - p[inv[g]])
            assert pa <= P_ABS, (m, r, probs_g[m, r], p[inv[g]])
            pr = pa / p[inv[g]]
            assert pr <= P_REL, (m, r, probs_g[m, r], p[inv[g]], pr)
            worst["p_abs"] = max(worst["p_abs"], pa)
            worst["p_rel"] = max(worst["p_rel"], pr)
    return worst


def logit_bound(h, W):
    """Elementwise bound gamma_d * sum_t |h_t W_t| for fp32 summation of d
    exact products (Higham's bound, u = 2^-24), as fp64 [M, rows]."""
    import synth
    hf = np.abs(synth.f32_from_bf16_bits(h).astype(np.float64))
    Wf = np.abs(synth.f32_from_bf16_bits(W).astype(np.float64))
    d = h.shape[1]
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    return gamma * (hf @ Wf.T)


def check_draws(ids_g, probs_g, h, W, t2f, seed, offset, bias=None):
    """Checks GPU draws (one per row) against the oracle's Gumbel-max draws
    on the same (seed, offset). A different pick is accepted only where the
    two candidates' perturbed logits z + G are within the fp32 error of the
    GPU's z (Higham's bound) and of G and the sum (a few ulp of |z + G|);
    probs are the oracle's subset-softmax value of the GPU's pick to 2e-3
    absolute and 1e-4 relative. Returns the number of accepted near-ties."""
    import oracle
    ids_g = np.asarray(ids_g).ravel()
    probs_g = np.asarray(probs_g, dtype=np.float64).ravel()
    ids_o, probs_o, ti_o, z = oracle.draft_sample(h, W, t2f, seed, offset, want_logits=True,
                                                  bias=bias)
    M, n = z.shape
    G = oracle.gumbel(seed, offset, M, n)
    v = z + G
    bound = logit_bound(h, W)
    inv = inverse_map(t2f)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    near = 0
    for m in range(M):
        jg = inv[int(ids_g[m])]
        jo = int(ti_o[m])
        assert jg >= 0, f"row {m}: GPU drew a full id outside t2f"
        if jg != jo:
            tol = bound[m, jg] + bound[m, jo] + 4e-6 * (1.0 + abs(v[m, jo]))
            assert v[m, jo] - v[m, jg] <= tol, (m, jo, jg, v[m, jo] - v[m, jg], tol)
            near += 1
        assert abs(probs_g[m] - p[m, jg]) <= 2e-3 + 1e-4 * p[m, jg], (m, probs_g[m], p[m, jg])
    return near
