"""Pins for the CPU fp64 oracle: each checks it against something other than
itself -- finite differences, an independent library autograd, the pages' worked
example, closed forms, invariants and special cases -- so that a dropped term, a
wrong sign or index, a transposed operand or an off-by-one causal mask fails at
least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = line.split("=", 1)
                out[k.strip()] = v.strip()
    return out


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(Q, K, V, G, scale, causal):
    O, _ = oracle.attn_fwd(Q, K, V, scale, causal)
    return float(np.sum(O * G))


# --------------------------------------------------------------------------
# finite differences (CS349E lecture 11, demo 1; 1point3acres closing check)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_fd_demo1_recipe(causal):
    """The demo-1 gradient check: N=48, d=16, seed 0, Q,K,V,G standard normal,
    loss = sum(O*G), central differences eps=1e-6 at 6 random points per tensor."""
    g = _golden("gradcheck_levels.txt")
    N, d = int(g["demo1_N"]), int(g["demo1_d"])
    eps = float(g["demo1_eps"])
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    G = rng.standard_normal((N, d))
    scale = 1.0 / math.sqrt(d)
    dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, G, scale, causal)
    grads = {"Q": dQ, "K": dK, "V": dV}
    worst = 0.0
    for name in ("Q", "K", "V"):
        for _ in range(int(g["demo1_fd_points_per_tensor"])):
            r, c = int(rng.integers(N)), int(rng.integers(d))
            args_p = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            args_m = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            args_p[name][r, c] += eps
            args_m[name][r, c] -= eps
            fp = _loss(args_p["Q"], args_p["K"], args_p["V"], G, scale, causal)
            fm = _loss(args_m["Q"], args_m["K"], args_m["V"], G, scale, causal)
            worst = max(worst, abs((fp - fm) / (2 * eps) - grads[name][r, c]))
    # the page reports agreement of about 1e-9; allow a factor of 100
    assert worst < 100 * float(g["demo1_fd_agreement"]), worst


@pytest.mark.parametrize("causal", [False, True])
def test_fd_every_element_tiny(causal):
    """Central differences of EVERY element of Q, K, V on a tiny two-head case:
    catches any index, transpose or masking slip the sampled check could miss."""
    B, H, N, d = 1, 2, 7, 3
    Q, K, V, G = (_rand((B, H, N, d), s) for s in (11, 12, 13, 14))
    scale = 0.7
    dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, G, scale, causal)
    eps = 1e-6
    for name, grad in (("Q", dQ), ("K", dK), ("V", dV)):
        for idx in np.ndindex(*Q.shape):
            args_p = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            args_m = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            args_p[name][idx] += eps
            args_m[name][idx] -= eps
            fd = (_loss(args_p["Q"], args_p["K"], args_p["V"], G, scale, causal)
                  - _loss(args_m["Q"], args_m["K"], args_m["V"], G, scale, causal)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-8, (name, idx, fd, grad[idx])


def test_fd_pins_forward_lse():
    """L is the log of the softmax denominator: dL_i/ds_ij = P_ij, so a finite
    difference of L with respect to Q_i reproduces scale * sum_j P_ij K_j."""
    N, d = 9, 4
    Q, K, V = (_rand((N, d), s) for s in (1, 2, 3))
    scale = 0.5
    for causal in (False, True):
        O, L = oracle.attn_fwd(Q, K, V, scale, causal)
        i = N - 2
        eps = 1e-6
        for c in range(d):
            Qp, Qm = Q.copy(), Q.copy()
            Qp[i, c] += eps
            Qm[i, c] -= eps
            fd = (oracle.attn_fwd(Qp, K, V, scale, causal)[1][i]
                  - oracle.attn_fwd(Qm, K, V, scale, causal)[1][i]) / (2 * eps)
            n = i + 1 if causal else N
            s = scale * K[:n] @ Q[i]
            p = np.exp(s - L[i])
            assert abs(fd - scale * p @ K[:n, c]) < 1e-8
        # rows of P sum to one, so O_i is a convex combination of visible V rows
        p_sum = [np.exp(scale * K[: (r + 1 if causal else N)] @ Q[r] - L[r]).sum() for r in range(N)]
        assert np.allclose(p_sum, 1.0, atol=1e-14)


# --------------------------------------------------------------------------
# independent library: torch autograd in float64 on the CPU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 33, 16), (1, 2, 100, 64)])
def test_against_torch_autograd_f64(causal, shape):
    B, H, N, d = shape
    Q, K, V, G = (_rand(shape, s) for s in (21, 22, 23, 24))
    scale = 1.0 / math.sqrt(d)
    dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, G, scale, causal)
    O, L = oracle.attn_fwd(Q, K, V, scale, causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        mask = torch.ones(N, N, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    to = torch.matmul(p, tv)
    to.backward(torch.tensor(G))
    for a, b in ((O, to), (L, lse), (dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        b = b.detach().numpy()
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


# --------------------------------------------------------------------------
# identities and the tiled formulation (FA2 ch.16, sec 16.1, 16.2, 16.4, 16.8)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_D_identity(causal):
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i with no extra coefficient."""
    Q, K, V, G = (_rand((2, 2, 57, 24), s) for s in (31, 32, 33, 34))
    scale = 1.0 / math.sqrt(24)
    _, _, _, D = oracle.attn_bwd(Q, K, V, G, scale, causal)
    O, _ = oracle.attn_fwd(Q, K, V, scale, causal)
    D2 = np.sum(O * G, axis=-1)
    assert np.abs(D - D2).max() <= 1e-13 * np.abs(D2).max()


def _tiled_cases():
    w = si.draw(si.WORKLOADS["n48_d16_fp32"])
    yield "n48_d16_fp32", w.Q, w.K, w.V, w.dO, 16, 12
    big = si.draw_custom(1, 2, 50, 16, "fp32", seed=7, q_mult=4.0)
    yield "ragged_q4", big.Q, big.K, big.V, big.dO, 16, 12
    tiny = si.draw_custom(1, 1, 5, 8, "fp32", seed=8)
    yield "smaller_than_tile", tiny.Q, tiny.K, tiny.V, tiny.dO, 16, 12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", list(_tiled_cases()), ids=lambda c: c[0])
def test_tiled_matches_definition(case, causal):
    """The tiled online-softmax forward and the key-outer backward from L agree
    with the plain definition (pages: ~1e-15 and 4.44e-16 in fp64)."""
    _, Q, K, V, G, Br, Bc = case
    scale = 1.0 / math.sqrt(Q.shape[-1])
    O, L = oracle.attn_fwd(Q, K, V, scale, causal)
    O2, L2 = oracle.flash_fwd_tiled(Q, K, V, scale, causal, Br, Bc)
    assert np.abs(O - O2).max() < 1e-13
    assert np.abs(L - L2).max() < 1e-13
    dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, G, scale, causal)
    tQ, tK, tV = oracle.flash_bwd_tiled(Q, K, V, O2, G, L2, scale, causal, Br, Bc)
    for a, b in ((dQ, tQ), (dK, tK), (dV, tV)):
        assert np.abs(a - b).max() < 1e-12 * max(1.0, np.abs(a).max())


def test_tiled_new_max_in_last_block():
    """A row whose maximum score appears only in the last key block (the case
    the 1point3acres post says to test): keys of the last block are parallel to
    the queries and scaled up."""
    N, d = 40, 8
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((N, d))
    K = rng.standard_normal((N, d)) * 0.1
    K[-8:] = Q[-8:] * 3.0
    V = rng.standard_normal((N, d))
    scale = 1.0
    O, L = oracle.attn_fwd(Q, K, V, scale, False)
    O2, L2 = oracle.flash_fwd_tiled(Q, K, V, scale, False, 8, 8)
    assert np.abs(O - O2).max() < 1e-13 and np.abs(L - L2).max() < 1e-12


# --------------------------------------------------------------------------
# the pages' four-number worked example and its negative control
# --------------------------------------------------------------------------

def _example(values):
    k = np.array([0.0, 0.0, 10.0, 10.0]).reshape(4, 1)
    q = np.ones((4, 1))
    v = np.array(values, dtype=np.float64).reshape(4, 1)
    return q, k, v


def test_worked_example_split_softmax():
    g = _golden("split_softmax_example.txt")
    assert g["scores"] == "0 0 | 10 10" and g["values"] == "0 0 | 1 1"
    q, k, v = _example([0, 0, 1, 1])
    exact = 2 * math.exp(10) / (2 + 2 * math.exp(10))      # full_attention_closed_form
    O, L = oracle.attn_fwd(q, k, v, 1.0, False)
    O2, L2 = oracle.flash_fwd_tiled(q, k, v, 1.0, False, 4, int(g["block_size"]))
    for o in (O, O2):
        assert np.abs(o - exact).max() < 1e-13
        assert np.abs(o - float(g["full_attention_printed"])).max() < 0.5 * 10 ** -int(g["printed_digits"]) + 1e-12
    assert np.abs(L - (10 + math.log(2 + 2 * math.exp(-10)))).max() < 1e-13
    assert np.abs(L - L2).max() < 1e-13
    # the page's wrong approach: attention on each block alone, then average
    avg = np.mean([oracle.attn_fwd(q[:2], k[b:b + 2], v[b:b + 2], 1.0, False)[0][0, 0] for b in (0, 2)])
    assert avg == float(g["per_block_average"])


def test_alpha_pitfall_negative_control():
    """Forgetting alpha on the accumulator (1point3acres: numerator and
    denominator must both be rebased) must be caught.  With values all one the
    correct result is exactly 1 and the planted bug gives about 1.99991; with
    the page's own values, or with the maximum in the first block, the bug hides
    -- which is why the control uses these inputs."""
    q, k, v = _example([1, 1, 1, 1])
    good, _ = oracle.flash_fwd_tiled(q, k, v, 1.0, False, 4, 2)
    bad, _ = oracle.flash_fwd_tiled(q, k, v, 1.0, False, 4, 2, flags=oracle.FLAG_FORGET_ALPHA_ON_ACC)
    assert np.abs(good - 1.0).max() < 1e-14
    a = math.exp(-10)
    assert np.abs(bad - 4 / (2 * a + 2)).max() < 1e-12 and np.abs(bad - 1.0).min() > 0.9
    q, k, v = _example([0, 0, 1, 1])
    hidden, _ = oracle.flash_fwd_tiled(q, k, v, 1.0, False, 4, 2, flags=oracle.FLAG_FORGET_ALPHA_ON_ACC)
    assert np.abs(hidden - 2 * math.exp(10) / (2 + 2 * math.exp(10))).max() < 1e-13
    kr = k[::-1].copy()
    hidden2, _ = oracle.flash_fwd_tiled(q, kr, np.ones((4, 1)), 1.0, False, 4, 2,
                                        flags=oracle.FLAG_FORGET_ALPHA_ON_ACC)
    assert np.abs(hidden2 - 1.0).max() < 1e-14


def test_worked_example_backward_closed_form():
    """Backward of the worked example with dO = 1 and scale 1: the reduction is
    delta = g . o = o, dS_j = P_j (v_j - o), dV_j = sum_i P_ij, dK_j = sum_i dS_ij q_i,
    dQ_i = sum_j dS_j k_j; P = [1, 1, e^10, e^10] / (2 + 2 e^10)."""
    q, k, v = _example([0, 0, 1, 1])
    g = np.ones((4, 1))
    dQ, dK, dV, D = oracle.attn_bwd(q, k, v, g, 1.0, False)
    e = math.exp(10)
    P = np.array([1, 1, e, e]) / (2 + 2 * e)
    o = 2 * e / (2 + 2 * e)
    dS = P * (np.array([0, 0, 1, 1]) - o)
    assert np.abs(D - o).max() < 1e-13
    assert np.abs(dV[:, 0] - 4 * P).max() < 1e-13
    assert np.abs(dK[:, 0] - 4 * dS).max() < 1e-15
    assert np.abs(dQ[:, 0] - 10 * (dS[2] + dS[3])).max() < 1e-13
    assert abs(dS[0] - (-2.2697904e-5)) < 1e-11


# --------------------------------------------------------------------------
# invariants and special cases (exact in real arithmetic)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, N, d = 2, 2, 37, 8
    Q, K, V, G = (_rand((B, H, N, d), s) for s in (41, 42, 43, 44))
    scale = 1.0 / math.sqrt(d)
    dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, G, scale, causal)
    # rows of dS sum to zero, so the key gradients sum to zero
    assert np.abs(dK.sum(axis=2)).max() < 1e-12
    # rows of P sum to one, so the value gradients sum to the output gradients
    assert np.abs(dV.sum(axis=2) - G.sum(axis=2)).max() < 1e-12
    if causal:
        # row 0 sees only key 0: P = 1, dS = 0, so dQ_0 = 0
        assert np.abs(dQ[:, :, 0]).max() == 0.0
        # the last key is seen only by the last row: dV_{N-1} = P_{N-1,N-1} dO_{N-1}
        _, L = oracle.attn_fwd(Q, K, V, scale, causal)
        p = np.exp(scale * np.sum(Q[:, :, -1] * K[:, :, -1], -1) - L[:, :, -1])
        assert np.abs(dV[:, :, -1] - p[..., None] * G[:, :, -1]).max() < 1e-13


def test_special_cases():
    d = 6
    # N = 1: O = V, dV = dO, dQ = dK = 0
    Q, K, V, G = (_rand((1, 1, 1, d), s) for s in (51, 52, 53, 54))
    for causal in (False, True):
        O, L = oracle.attn_fwd(Q, K, V, 0.3, causal)
        dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, G, 0.3, causal)
        assert np.abs(O - V).max() < 1e-15 and np.abs(dV - G).max() < 1e-15
        assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
        assert abs(L[0, 0, 0] - 0.3 * float(Q.ravel() @ K.ravel())) < 1e-15
    # all keys equal: P uniform over visible keys and dQ = 0
    N = 11
    Q, V, G = (_rand((1, 1, N, d), s) for s in (55, 56, 57))
    K = np.repeat(_rand((1, 1, 1, d), 58), N, axis=2)
    for causal in (False, True):
        O, _ = oracle.attn_fwd(Q, K, V, 0.4, causal)
        ref = np.cumsum(V, axis=2) / np.arange(1, N + 1)[:, None] if causal else \
            np.repeat(V.mean(axis=2, keepdims=True), N, axis=2)
        assert np.abs(O - ref).max() < 1e-14
        dQ, _, _, _ = oracle.attn_bwd(Q, K, V, G, 0.4, causal)
        assert np.abs(dQ).max() < 1e-14
    # Q = 0: scores are zero and dK = scale * dS^T Q = 0
    Q0 = np.zeros((1, 1, N, d))
    K = _rand((1, 1, N, d), 59)
    for causal in (False, True):
        _, dK, _, _ = oracle.attn_bwd(Q0, K, V, G, 0.4, causal)
        assert np.abs(dK).max() == 0.0


# --------------------------------------------------------------------------
# sampled functions agree with the whole-tensor definitions
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_sampled_functions_match_full(causal):
    N, d = 131, 32
    Q, K, V, G = (_rand((N, d), s) for s in (61, 62, 63, 64))
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attn_fwd(Q, K, V, scale, causal)
    dQ, dK, dV, D = oracle.attn_bwd(Q, K, V, G, scale, causal)
    L2, D2 = oracle.row_stats(Q, K, V, G, scale, causal)
    assert np.abs(L - L2).max() < 1e-14 and np.abs(D - D2).max() < 1e-13
    rows = [0, 1, 64, 129, 130]
    O3, L3 = oracle.fwd_rows(Q, K, V, scale, causal, rows)
    assert np.abs(O3 - O[rows]).max() < 1e-14 and np.abs(L3 - L[rows]).max() < 1e-14
    assert np.abs(oracle.dq_rows(Q, K, V, G, scale, causal, rows) - dQ[rows]).max() < 1e-13
    dk, dv = oracle.dkdv_rows(Q, K, V, G, L2, D2, scale, causal, rows)
    assert np.abs(dk - dK[rows]).max() < 1e-13 and np.abs(dv - dV[rows]).max() < 1e-13


def test_thread_count_does_not_change_result():
    Q, K, V, G = (_rand((1, 1, 64, 16), s) for s in (71, 72, 73, 74))
    n0 = oracle.max_threads()
    try:
        oracle.set_threads(1)
        a = oracle.attn_bwd(Q, K, V, G, 0.25, True)
        oracle.set_threads(max(2, n0))
        b = oracle.attn_bwd(Q, K, V, G, 0.25, True)
    finally:
        oracle.set_threads(n0)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() < 1e-14
