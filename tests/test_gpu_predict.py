"""The budget predictor on the GPU (chunk totals, then the final pass with the
class dots on the int8 matrix cores, an in-workgroup scan and the first
argmax) against the oracle's predictor on every position of every pair, at
seeded random shapes: lengths below one wave's 64 positions and above 64
chunks of 256 (the offsets' second loop), every head dimension, class counts
1 .. 32, keys per class 1 .. 4, caps 1 .. 128 and key, query and weight
magnitudes up to the declared bounds.  Predictor of the ALHR README,
"Inference stage"; caps in "Results and Variables"."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def predictor_case(i):
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([16, 32, 64, 128, 256]))
    T = int(rng.choice([2, 8, 32, 64, 128, 512, 4096, 32768]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    nc = int(rng.integers(1, 33))
    kpc = int(rng.integers(1, 5))
    cap = int(rng.integers(1, 129))
    # magnitudes inside the declared bounds the library checks (node sums,
    # scores and predictor logits within int32)
    wmax = int(rng.choice([1, 4, 127]))
    kmax = int(rng.choice([1, 8, 127]))
    qmax = int(rng.choice([8, 127]))

    def fits(k, q):
        return (k * T < 2 ** 31 and q * k * d * T // 2 < 2 ** 31
                and wmax * d * (q + k * T) < 2 ** 31)
    while not fits(kmax, qmax) and kmax > 1:
        kmax //= 2
    while not fits(kmax, qmax):
        qmax //= 2
    return rng, dict(B=B, H=H, T=T, d=d, nc=nc, kpc=kpc, cap=cap, wmax=wmax, kmax=kmax, qmax=qmax)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("i", range(12))
def test_predictor_random_shapes_every_position(torch_dev, i):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    rng, c = predictor_case(i)
    B, H, T, d = c["B"], c["H"], c["T"], c["d"]
    Q = rng.integers(-c["qmax"], c["qmax"] + 1, size=(B, H, T, d)).astype(np.int8)
    K = rng.integers(-c["kmax"], c["kmax"] + 1, size=(B, H, T, d)).astype(np.int8)
    W = rng.integers(-c["wmax"], c["wmax"] + 1, size=(c["nc"], 2 * d)).astype(np.int8)
    cfg = alhr.Config(batch=B, heads=H, T=T, d=d, n_classes=c["nc"], keys_per_class=c["kpc"],
                      max_budget=c["cap"], kmax=c["kmax"], qmax=c["qmax"], wmax=c["wmax"])
    print("predictor case", i, c, flush=True)
    q, k, w = (torch.from_numpy(x).to(dev) for x in (Q, K, W))
    bud = alhr.alhr_predict_budget(cfg, q, k, w)
    _, bud2 = alhr.alhr_prepare(cfg, q, k, w)
    torch.cuda.synchronize()
    assert torch.equal(bud, bud2)
    got = bud.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = oracle.pair_budgets(Q[b, h], K[b, h], W, keys_per_class=c["kpc"],
                                      max_budget=c["cap"])
            np.testing.assert_array_equal(got[b, h], ref, err_msg="pair (%d, %d)" % (b, h))
