"""Pins of the oracle's GEMMs and routing (no GPU).

What pins them, besides themselves:
  * a pure-Python triple loop for the exact integer parts on tiny inputs;
  * a second route through the mathematics: dequantise both operands, then
    one fp64 matrix product, must equal the block/channel formulas;
  * the quantised product must approximate the unquantised X . W^T within the
    round-trip bound of each factor (a wrong scale index, sign or transposed
    operand breaks it);
  * exact rational evaluation of y on tiny inputs bounds y64 and y32;
  * identity of the two schemes when one K block spans all of K;
  * routing properties (each token k times; picked logits dominate the rest).
"""

from fractions import Fraction

import numpy as np

import synth
from oracle import formats, gemm, quant, routing


def _tiny(M=5, K=256, N=7, seed=0):
    x = synth.to_numpy(synth.activations(M, K, seed=seed, outlier_frac=0.01, outlier_factor=20.0))
    w = synth.to_numpy(synth.weights(N, K, seed=seed + 100))
    return x, w


def test_partials_and_acc_equal_pure_python_loops():
    x, w = _tiny(M=3, K=256, N=5)
    Aq, _ = quant.quant_act_group(x)
    Wq, _ = quant.quant_weight_block(w)
    P = gemm.block_partials(Aq, Wq)
    ACC, _, _ = gemm.gemm_channel(Aq, np.ones(3, np.float32), Wq, np.ones(5, np.float32))
    for m in range(3):
        for n in range(5):
            tot = 0
            for kb in range(2):
                s = 0
                for k in range(kb * 128, kb * 128 + 128):
                    s += int(Aq[m, k]) * int(Wq[n, k])
                assert P[kb, m, n] == s
                tot += s
            assert ACC[m, n] == tot


def test_extreme_codes_are_exact():
    K = 18432
    Aq = np.full((2, K), 127, np.int8)
    Aq[1] = -127
    Wq = np.full((3, K), 127, np.int8)
    ACC, _, _ = gemm.gemm_channel(Aq, np.ones(2, np.float32), Wq, np.ones(3, np.float32))
    assert ACC[0, 0] == K * 127 * 127 and ACC[1, 2] == -K * 127 * 127
    P = gemm.block_partials(Aq, Wq)
    assert np.all(P[:, 0] == 128 * 127 * 127)


def _deq_rows(q, s_rows_blocks):
    """Dequantise q[R, K] with per-(row, 128-block) scales [R, KB] in fp64."""
    return q.astype(np.float64) * np.repeat(s_rows_blocks.astype(np.float64), 128, axis=1)


def test_block_gemm_equals_dequantise_then_matmul_and_approximates_xw():
    x, w = _tiny(M=9, K=384, N=200, seed=3)        # ragged last weight tile
    Aq, sa = quant.quant_act_group(x)
    Wq, sw = quant.quant_weight_block(w)
    _, y64, y32 = gemm.gemm_block(Aq, sa, Wq, sw)
    A_deq = _deq_rows(Aq, sa)
    W_deq = _deq_rows(Wq, sw[np.arange(200) // 128])
    y_route = A_deq @ W_deq.T
    assert np.allclose(y64, y_route, rtol=1e-12, atol=1e-12 * np.abs(y_route).max())
    # quantised product vs unquantised product: |err| <= sum_k |x||dw| + |dx||w| + |dx||dw|
    X = formats.bf16_bits_to_f32(x).astype(np.float64)
    Wf = formats.bf16_bits_to_f32(w).astype(np.float64)
    dx = np.repeat(sa.astype(np.float64), 128, axis=1) * 0.5 * (1 + 2.0 ** -16)
    dw = np.repeat(sw[np.arange(200) // 128].astype(np.float64), 128, axis=1) * 0.5 * (1 + 2.0 ** -16)
    bound = np.abs(X) @ dw.T + dx @ np.abs(Wf).T + dx @ dw.T
    err = np.abs(y64 - X @ Wf.T)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-300)
    assert err.max() > 0          # the bound is not vacuous
    assert gemm.normwise_rel_err(y32, y64) < 1e-5


def test_channel_gemm_equals_dequantise_then_matmul_and_approximates_xw():
    x, w = _tiny(M=6, K=512, N=33, seed=4)
    Aq, sa = quant.quant_act_token(x)
    Wq, sw = quant.quant_act_token(w)
    ACC, y64, y32 = gemm.gemm_channel(Aq, sa, Wq, sw)
    y_route = (Aq.astype(np.float64) * sa[:, None]) @ (Wq.astype(np.float64) * sw[:, None]).T
    assert np.allclose(y64, y_route, rtol=1e-12, atol=1e-12 * np.abs(y_route).max())
    X = formats.bf16_bits_to_f32(x).astype(np.float64)
    Wf = formats.bf16_bits_to_f32(w).astype(np.float64)
    dx = np.broadcast_to(sa[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -16), X.shape)
    dw = np.broadcast_to(sw[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -16), Wf.shape)
    bound = np.abs(X) @ dw.T + dx @ np.abs(Wf).T + dx @ dw.T
    assert np.all(np.abs(y64 - X @ Wf.T) <= bound * (1 + 1e-9))
    assert gemm.normwise_rel_err(y32, y64) < 1e-6


def test_y64_and_y32_against_exact_rational_value():
    x, w = _tiny(M=2, K=384, N=3, seed=6)
    Aq, sa = quant.quant_act_group(x)
    Wq, sw = quant.quant_weight_block(w)
    P, y64, y32 = gemm.gemm_block(Aq, sa, Wq, sw)
    KB = 3
    for m in range(2):
        for n in range(3):
            terms = [Fraction(float(sa[m, kb])) * Fraction(float(sw[0, kb])) * int(P[kb, m, n])
                     for kb in range(KB)]
            exact = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(float(y64[m, n])) - exact) <= (KB + 2) * Fraction(1, 2 ** 53) * mag
            assert abs(Fraction(float(y32[m, n])) - exact) <= (KB + 2) * Fraction(1, 2 ** 24) * mag


def test_block_equals_channel_when_one_block_spans_k():
    x, w = _tiny(M=7, K=128, N=256, seed=8)
    Aq_g, sa_g = quant.quant_act_group(x)
    Aq_t, sa_t = quant.quant_act_token(x)
    assert np.array_equal(Aq_g, Aq_t) and np.array_equal(sa_g[:, 0], sa_t)
    Wq, sw = quant.quant_weight_block(w)
    sw_ch = sw[np.arange(256) // 128, 0]
    P, yb64, yb32 = gemm.gemm_block(Aq_g, sa_g, Wq, sw)
    ACC, yc64, yc32 = gemm.gemm_channel(Aq_t, sa_t, Wq, sw_ch)
    assert np.array_equal(P[0], ACC)
    assert np.array_equal(yb64, yc64)
    assert np.array_equal(yb32, yc32)


def test_partials_sum_to_channel_accumulator():
    x, w = _tiny(M=4, K=1024, N=17, seed=10)
    Aq, _ = quant.quant_act_token(x)
    Wq, _ = quant.quant_act_token(w)
    P = gemm.block_partials(Aq, Wq)
    ACC, _, _ = gemm.gemm_channel(Aq, np.ones(4, np.float32), Wq, np.ones(17, np.float32))
    assert np.array_equal(P.astype(np.int64).sum(axis=0), ACC.astype(np.int64))


def test_w8a16_equals_dequantised_weights_product():
    M, K, N = 3, 384, 20
    x = synth.activations(M, K, seed=2, dtype=__import__("torch").float16).numpy()
    w = synth.weights(N, K, seed=21, dtype=__import__("torch").float16).numpy()
    Wq, s = quant.quant_act_group(w)
    y64, y32 = gemm.gemm_w8a16_group(x, Wq, s)
    W_deq = _deq_rows(Wq, s)
    X = x.astype(np.float64)
    assert np.allclose(y64, X @ W_deq.T, rtol=1e-12, atol=1e-12 * np.abs(y64).max())
    # vs the unquantised fp16 weights: |err| <= sum_k |x| * s/2
    bound = np.abs(X) @ (np.repeat(s.astype(np.float64), 128, axis=1) * 0.5 * (1 + 2.0 ** -16)).T
    assert np.all(np.abs(y64 - X @ w.astype(np.float64).T) <= bound * (1 + 1e-9))
    assert gemm.normwise_rel_err(y32, y64) < 1e-5
    # brute force on a few entries
    for (m, n) in [(0, 0), (2, 19), (1, 7)]:
        tot = Fraction(0)
        for g in range(3):
            part = sum(Fraction(float(x[m, k])) * int(Wq[n, k]) for k in range(g * 128, g * 128 + 128))
            tot += Fraction(float(s[n, g])) * part
        assert abs(Fraction(float(y64[m, n])) - tot) <= Fraction(1, 2 ** 40) * (abs(tot) + 1)


def test_routing_properties():
    logits = synth.router_logits(64, 16, seed=4).numpy()
    rows, exps, offs = routing.topk_route(logits, 4)
    assert offs[-1] == 64 * 4 and np.all(np.diff(offs) >= 0)
    assert np.array_equal(np.bincount(rows, minlength=64), np.full(64, 4))
    for e in range(16):
        seg = rows[offs[e]:offs[e + 1]]
        assert np.all(exps[offs[e]:offs[e + 1]] == e)
        assert np.all(np.diff(seg) > 0)                      # token order inside an expert
    for t in range(64):
        picked = exps[rows == t]
        others = np.setdiff1d(np.arange(16), picked)
        assert logits[t, picked].min() >= logits[t, others].max()
    # ties go to the lower expert index
    tie = np.zeros((1, 8), np.float32)
    _, e_tie, _ = routing.topk_route(tie, 3)
    assert sorted(e_tie.tolist()) == [0, 1, 2]


def test_synth_routing_matches_oracle_routing():
    lg = synth.router_logits(256, 32, seed=9)
    r1, e1, o1 = synth.route_topk(lg, 8)
    r2, e2, o2 = routing.topk_route(lg.numpy(), 8)
    assert np.array_equal(r1.numpy(), r2) and np.array_equal(e1.numpy(), e2)
    assert np.array_equal(o1.numpy().astype(np.int64), o2)


def test_grouped_gemm_rowwise_against_dequantised_expert_weights():
    E, T, K, N, k = 6, 20, 256, 130, 2
    lg = synth.router_logits(T, E, seed=5).numpy()
    rows, exps, offs = routing.topk_route(lg, k)
    # make expert 3 empty to cover zero-token experts
    lg[:, 3] = -100.0
    rows, exps, offs = routing.topk_route(lg, k)
    assert offs[4] == offs[3]
    x = synth.to_numpy(synth.activations(T, K, seed=6))
    Aq, sa = quant.quant_act_group(x[rows])
    Wq = np.empty((E, N, K), np.int8)
    sw = np.empty((E, 2, 2), np.float32)
    Wf = []
    for e in range(E):
        we = synth.to_numpy(synth.weights(N, K, seed=50 + e))
        Wq[e], sw[e] = quant.quant_weight_block(we)
        Wf.append(_deq_rows(Wq[e], sw[e][np.arange(N) // 128]))
    y64, y32 = gemm.gemm_block_grouped(Aq, sa, Wq, sw, offs)
    A_deq = _deq_rows(Aq, sa)
    for i in range(T * k):
        ref = A_deq[i] @ Wf[exps[i]].T
        assert np.allclose(y64[i], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert gemm.normwise_rel_err(y32, y64) < 1e-5
    # quantise-then-gather equals gather-then-quantise (the quantiser is row-local)
    Aq_all, sa_all = quant.quant_act_group(x)
    assert np.array_equal(Aq_all[rows], Aq) and np.array_equal(sa_all[rows], sa)


def test_w8a16_y32_within_fixed_order_fp32_bound():
    """y32 is a fixed-order fp32 evaluation: 128 sequential sums inside each
    group and KB sequential sums across groups.  Against the exact rational
    value each output lies within (128 + KB + 2) 2^-24 of the sum of the
    absolute terms (a dropped group, a wrong scale index or fp16 rounding of
    the partials would break it)."""
    M, K, N = 2, 384, 3
    x = synth.activations(M, K, seed=31, dtype=__import__("torch").float16).numpy()
    w = synth.weights(N, K, seed=32, dtype=__import__("torch").float16).numpy()
    Wq, s = quant.quant_act_group(w)
    _, y32 = gemm.gemm_w8a16_group(x, Wq, s)
    KB = K // 128
    for m in range(M):
        for n in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for g in range(KB):
                terms = [Fraction(float(x[m, k])) * int(Wq[n, k]) for k in range(g * 128, g * 128 + 128)]
                exact += Fraction(float(s[n, g])) * sum(terms)
                mag += abs(Fraction(float(s[n, g]))) * sum(abs(t) for t in terms)
            assert abs(Fraction(float(y32[m, n])) - exact) <= (128 + KB + 2) * Fraction(1, 2 ** 24) * mag


def test_w8a16_y32_group_partials_are_not_rounded_to_fp16():
    """A group whose fp32 partial is not representable in fp16 (2049 = 2^11 + 1
    is exact in fp32 but not in fp16) keeps its value: with unit scale and
    x = 1 everywhere, Y = sum of the codes exactly."""
    K = 256
    x = np.ones((1, K), np.float16)
    Wq = np.zeros((1, K), np.int8)
    Wq[0, :17] = 121            # 17 * 121 = 2057 in group 0 (odd, > 2048)
    Wq[0, 128:130] = (-1, 3)    # 2 in group 1
    s = np.ones((1, 2), np.float32)
    y64, y32 = gemm.gemm_w8a16_group(x, Wq, s)
    assert y64[0, 0] == 2059.0 and y32[0, 0] == np.float32(2059.0)


def test_normwise_rel_err_hand_worked():
    """The comparison of every float parity check: max|y - ref| / max|ref| over
    the whole tensor (reading R12), worked by hand."""
    ne = gemm.normwise_rel_err
    # denominator is max|ref| = 4, not max|y| = 3, and not a mean
    assert ne(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 4.0])) == 0.25
    # a negative entry dominates: max|ref| = 8 (max(ref) = 1 would give 2)
    assert ne(np.array([-8.0, 3.0]), np.array([-8.0, 1.0])) == 0.25
    # one outlier error on a small entry is measured against the largest
    # entry (elementwise relative error would be 1.0 here)
    assert ne(np.array([100.0, 1.0, 1.0, 2.0]), np.array([100.0, 1.0, 1.0, 1.0])) == 0.01
    # the worst element decides (a mean of the errors would give 0.0125)
    assert ne(np.array([10.0, 10.0, 10.0, 10.5]), np.array([10.0, 10.0, 10.0, 10.0])) == 0.05
    # over the whole 2-D tensor, not per row: the row max is 2, the tensor max 4
    y = np.array([[2.0, 0.0], [4.0, 1.0]])
    r = np.array([[1.0, 0.0], [4.0, 1.0]])
    assert ne(y, r) == 0.25
    # zero reference: the absolute error; empty tensors compare equal
    assert ne(np.array([0.0, -3.0, 1.0]), np.zeros(3)) == 3.0
    assert ne(np.zeros(0), np.zeros(0)) == 0.0
    # symmetric in the sign of the difference, exact on equal inputs
    assert ne(np.array([1.0, -5.0]), np.array([1.0, -4.0])) == ne(np.array([1.0, -3.0]), np.array([1.0, -4.0]))
    assert ne(r, r) == 0.0
