"""CPU check of the candidate margin of the fused prefill top-k.

The candidate pass of dsa_prefill_topk sums the 16 heads' ReLU logits on the
bf16 matrix cores: the weights w_h and the ReLU logits R_h are each rounded
to bf16 (round to nearest even), multiplied exactly and summed in fp32.  The
kernel adds 0.01 * sum_h |w~_h| R~_h to its candidate test, claiming that the
rounding moves the weighted sum by at most 2^-7 (1 - 2^-8)^-2 of that sum
(2^-8 unit roundoff for each operand, plus fp32 sums).  This test checks that
claim with the rounding emulated (torch's bf16 conversion is round to
nearest even), on random inputs and on inputs placed at rounding midpoints
with cancelling weights, where the bound is nearly reached.
"""
import numpy as np
import torch

KERNEL_FACTOR = 0.01                        # the kernel's margin factor
CLAIM = 2.0 ** -7 / (1 - 2.0 ** -8) ** 2    # the rounding bound it covers


def bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def rounded_sum(w: np.ndarray, lg: np.ndarray):
    """(the weighted ReLU sum with w and R rounded to bf16 and summed in fp32
    in three orders, its exact value, sum_h |w~_h| R~_h)"""
    r = np.maximum(lg.astype(np.float32), np.float32(0)).astype(np.float64)
    wt, rt = bf16(w), bf16(r)
    prods = (wt * rt).astype(np.float32)     # bf16 x bf16 products are exact in fp32
    sums = []
    for order in (slice(None), slice(None, None, -1), np.argsort(np.abs(prods), axis=-1)):
        p = prods[..., order] if not isinstance(order, np.ndarray) else np.take_along_axis(prods, order, -1)
        acc = np.zeros(p.shape[:-1], np.float32)
        for h in range(p.shape[-1]):
            acc = (acc + p[..., h]).astype(np.float32)
        sums.append(acc.astype(np.float64))
    exact = (w.astype(np.float64) * r).sum(-1)
    bound_sum = (np.abs(wt) * rt).sum(-1)
    return np.stack(sums), exact, bound_sum


def test_random_inputs_stay_inside_the_claim():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((20000, 16)).astype(np.float32)
    lg = (rng.standard_normal((20000, 16)) * 30).astype(np.float32)
    sums, exact, a = rounded_sum(w, lg)
    err = np.abs(sums - exact).max(0)
    assert np.all(err <= CLAIM * a + 1e-30)
    assert CLAIM * 1.25 <= KERNEL_FACTOR


def test_midpoint_inputs_with_cancelling_weights_nearly_reach_it():
    # weights and logits just off bf16 rounding midpoints, chosen so that
    # every term's two rounding errors push the sum the same way, with
    # weights of alternating sign so that the weighted sum itself cancels
    rng = np.random.default_rng(1)
    n = 4000
    pos = np.arange(16) % 2 == 0
    half = 2.0 ** -8                                                   # half a bf16 step in [1, 2)
    off = np.where(pos, 1 - 2.0 ** -12, 1 + 2.0 ** -12)               # below / above the midpoint
    bw = 1.0 + rng.integers(0, 127, size=(n, 16)) / 128.0             # bf16 grid points in [1, 2)
    br = 1.0 + rng.integers(0, 127, size=(n, 16)) / 128.0
    # w > 0 rounds down, w < 0 rounds away from zero; R under a positive
    # weight rounds down, under a negative one up: every term moves down
    w = (np.where(pos, 1.0, -1.0) * (bw + half * off)).astype(np.float32)
    lg = (8 * (br + half * off)).astype(np.float32)
    sums, exact, a = rounded_sum(w, lg)
    ratio = (np.abs(sums - exact) / a).max(0)
    assert np.all(ratio <= CLAIM)
    assert ratio.max() >= 0.5 * CLAIM, f"adversarial case too weak: {ratio.max():.3e}"


def test_zero_and_negative_logits_contribute_nothing():
    w = np.full((1, 16), 3.0, np.float32)
    lg = np.array([[-1.0, -0.0, 0.0] + [-5.0] * 13], np.float32)
    sums, exact, a = rounded_sum(w, lg)
    assert np.all(sums == 0.0) and exact[0] == 0.0 and a[0] == 0.0
