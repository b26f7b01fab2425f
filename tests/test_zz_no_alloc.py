"""bt_gemm_grouped_static, the grouped product for callers that cannot
allocate: through the C ABI, its outputs equal bt_gemm_grouped's bit for bit
(and the oracle's) on plans of every kind, on calls in a row that share the
library's static scratch array, the second with a smaller input."""
import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bt = pytest.importorskip("gemm_i2_bit_amd")

NTHREADS = 16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bt.lib()
    oracle.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def make_case(specs, m, seed):
    """Problems (host inputs, GPU inputs and two output sets) of one plan."""
    rng = np.random.default_rng(seed)
    host, probs_a, probs_b = [], [], []
    for n, k in specs:
        t = wl.trits(rng, (n, k), wl.DECODE_2B)
        x = wl.x_normal_outliers(rng, (m, k))
        s_w = np.float32(rng.uniform(0.01, 0.05))
        packed = bt.bt_pack_i2s(dev(t))
        x_q, s_a = bt.bt_quant_act(dev(x))
        for lst in (probs_a, probs_b):
            lst.append(dict(packed=packed, s_w=s_w, n=n, k=k, x_q=x_q,
                            s_a=s_a,
                            y=torch.full((m, n), float("nan"),
                                         device="cuda:0"),
                            acc=torch.full((m, n), 0x7EADBEEF,
                                           dtype=torch.int32,
                                           device="cuda:0")))
        host.append((t, x, s_w))
    return host, probs_a, probs_b


def check(host, probs_a, probs_b, label):
    plan_a = bt.bt_grouped_plan(probs_a)
    plan_b = bt.bt_grouped_plan(probs_b)
    bt.bt_gemm_grouped(plan_a)
    bt.bt_gemm_grouped_static(plan_b)
    torch.cuda.synchronize()
    for i, ((t, x, s_w), pa, pb) in enumerate(zip(host, probs_a, probs_b)):
        assert torch.equal(pa["acc"], pb["acc"]), (label, i)
        assert torch.equal(pa["y"], pb["y"]), (label, i)
        p, _ = oracle.pack_i2s(t)
        q, s_a = oracle.quant_act(x)
        acc_r, y_r = oracle.gemm(p, s_w, t.shape[0], t.shape[1], q, s_a,
                                 nthreads=NTHREADS)
        acc = pb["acc"].cpu().numpy()
        assert np.array_equal(acc, acc_r), (label, i)
        y = pb["y"].cpu().numpy().astype(np.float64)
        nz = acc_r != 0
        assert (y[~nz] == 0).all()
        assert (np.abs(y[nz] - y_r[nz]) / np.abs(y_r[nz])).max() <= 1e-6


def test_static_scratch_matches_grouped():
    # 1. a plan that fills every CU at m = 1: row blocks of 1024 chunks cut
    #    among many waves (atomic hand-offs through the scratch slots)
    big = make_case([(640, 65536), (4096, 256), (300, 2560)], 1, 120)
    check(*big, "full grid m=1")
    # 2. a smaller plan right after it (the slots it uses were left zero)
    small = make_case([(512, 256), (64, 64), (70, 192), (130, 320)], 1, 121)
    check(*small, "small m=1")
    # 3. a prefill-sized plan whose long reductions are split (partial-sum
    #    regions and arrival counters in the scratch array)
    split = make_case([(300, 2048), (200, 8384), (64, 64)], 130, 122)
    check(*split, "split ranges m=130")
    # 4. the first plan again, and m = 3 (three tokens per slot)
    check(*big, "full grid m=1 again")
    check(*make_case([(2560, 2560), (640, 6912)], 3, 123), "m=3")
    # 5. skinny matrix-core plans (m = 8 and 40; no scratch), then the
    #    split prefill plan again: its counters were left zero by the last
    #    launch that used them, and only they are cleared
    check(*make_case([(600, 16384), (2560, 2560), (640, 6912)], 8, 124),
          "matrix cores m=8")
    check(*make_case([(300, 4096), (640, 2560)], 40, 125), "matrix cores m=40")
    check(*split, "split ranges m=130 again")
