"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for packed bytes, int8 activations, their
scales and int32 accumulators; fp32 outputs within 1e-6 relative error of the
oracle's float64 rescale (exactly 0 where the accumulator is 0).

Inputs come from workloads.py (random numbers only).  Expected values come
only from the oracle."""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bt = pytest.importorskip("gemm_i2_bit_amd")

NTHREADS = min(16, os.cpu_count() or 1)
RTOL = 1e-6
GUARD_BYTES = 16  # guard on each side of every output (keeps alignment)


def guard_len(dtype):
    return GUARD_BYTES // torch.empty((), dtype=dtype).element_size()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bt.lib()
    oracle.lib()
    return torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def guarded(numel, dtype, fill):
    g = guard_len(dtype)
    buf = torch.full((numel + 2 * g,), fill, dtype=dtype, device="cuda:0")
    return buf, buf[g:g + numel]


def check_guards(buf, fill):
    host = buf.cpu()
    g = guard_len(buf.dtype)
    head, tail = host[:g], host[-g:]
    if buf.dtype == torch.float32:
        assert torch.isnan(head).all() and torch.isnan(tail).all(), \
            "write outside the output"
    else:
        assert (head == fill).all() and (tail == fill).all(), \
            "write outside the output"


def check_y(y_gpu, y_ref, acc_ref):
    y_gpu = np.asarray(y_gpu, np.float64)
    zero = acc_ref == 0
    assert (y_gpu[zero] == 0).all()
    nz = ~zero
    rel = np.abs(y_gpu[nz] - y_ref[nz]) / np.abs(y_ref[nz])
    assert rel.size == 0 or rel.max() <= RTOL, f"max rel err {rel.max()}"


def gpu_product(t, x, s_w, guards=True):
    """Pack, quantize and multiply on the GPU; return host arrays."""
    n, k = t.shape
    m = x.shape[0]
    packed = bt.bt_pack_i2s(dev(t))
    x_q, s_a = bt.bt_quant_act(dev(x))
    ybuf, y = guarded(m * n, torch.float32, float("nan"))
    abuf, acc = guarded(m * n, torch.int32, 0x7EADBEEF)
    bt.bt_gemm(packed, s_w, n, k, x_q, s_a, y=y.view(m, n), acc=acc.view(m, n))
    torch.cuda.synchronize()
    if guards:
        check_guards(ybuf, None)
        check_guards(abuf, 0x7EADBEEF)
    return (packed.cpu().numpy(), x_q.cpu().numpy(), s_a.cpu().numpy(),
            acc.view(m, n).cpu().numpy(), y.view(m, n).cpu().numpy())


def oracle_product(t, x, s_w, rows=None):
    p, bad = oracle.pack_i2s(t)
    assert bad == 0
    q, s_a = oracle.quant_act(x)
    acc, y = oracle.gemm(p, s_w, t.shape[0], t.shape[1], q, s_a,
                         nthreads=NTHREADS, rows=rows)
    return p, q, s_a, acc, y


# ----------------------------------------------------------------- packing
@pytest.mark.parametrize("n,k,dist", [
    (512, 256, wl.UNIFORM), (70, 64, wl.UNIFORM), (130, 192, wl.DECODE_2B),
    (2560, 2560, wl.DECODE_2B), (100, 6912, wl.SKEWED_8B), (1, 64, wl.UNIFORM)])
def test_pack_matches_oracle(n, k, dist):
    t = wl.trits(np.random.default_rng([100, n, k]), (n, k), dist)
    p_ref, _ = oracle.pack_i2s(t)
    p_gpu = bt.bt_pack_i2s(dev(t)).cpu().numpy()
    np.testing.assert_array_equal(p_gpu, p_ref)


def test_pack_counts_invalid():
    t = np.zeros((70, 128), np.int8)
    t[3, 5], t[69, 127], t[10, 64] = 2, -2, 100
    n_bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    bt.bt_pack_i2s(dev(t), n_invalid=n_bad)
    assert int(n_bad.item()) == 3


# ------------------------------------------------------------ quantization
def quant_cases():
    rng = np.random.default_rng(101)
    ties = np.zeros((1, 64), np.float32)
    ties[0, :7] = [127, 2.5, -3.5, 0.5, -0.5, 1.5, -2.5]
    zero_tiny = np.zeros((2, 128), np.float32)
    zero_tiny[1, 7] = 1e-30
    return [
        ("single", wl.single_gemv()[2]),
        ("outliers", wl.x_normal_outliers(rng, (1, 2560))),
        ("batch8", wl.x_normal(rng, (8, 2560))),
        ("student_t", wl.x_student_t(rng, (3, 6912))),
        ("small", wl.x_normal(rng, (5, 64)) * np.float32(1e3)),
        ("long", wl.x_normal(rng, (2, 14336))),
        ("ties", ties),
        ("zero_tiny", zero_tiny),
        ("quarter_steps", np.round(wl.x_normal(rng, (4, 256)) * 4) / 4),
        ("held_in_registers", wl.x_normal_outliers(rng, (2, 8192))),
        ("read_twice", wl.x_normal_outliers(rng, (2, 8256))),
        ("read_twice_longest", wl.x_normal_outliers(rng, (1, 65536))),
    ]


@pytest.mark.parametrize("name,x", quant_cases(), ids=lambda v: v if isinstance(v, str) else "")
def test_quant_matches_oracle(name, x):
    x = np.ascontiguousarray(x, np.float32)
    q_ref, s_ref = oracle.quant_act(x)
    q_gpu, s_gpu = bt.bt_quant_act(dev(x))
    np.testing.assert_array_equal(q_gpu.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s_gpu.cpu().numpy().view(np.uint32),
                                  s_ref.view(np.uint32))


def check_quant_many(xs):
    xs = [np.ascontiguousarray(x, np.float32) for x in xs]
    qbufs = [guarded(x.size, torch.int8, 0x5A) for x in xs]
    sbufs = [guarded(x.shape[0], torch.float32, float("nan")) for x in xs]
    x_qs = [q.view(x.shape) for (_, q), x in zip(qbufs, xs)]
    s_as = [s for _, s in sbufs]
    bt.bt_quant_act_many([dev(x) for x in xs], x_qs, s_as)
    torch.cuda.synchronize()
    for x, q, s, (qb, _), (sb, _) in zip(xs, x_qs, s_as, qbufs, sbufs):
        q_ref, s_ref = oracle.quant_act(x)
        np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
        np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32),
                                      s_ref.view(np.uint32))
        check_guards(qb, 0x5A)
        check_guards(sb, None)


def test_quant_many_matches_oracle():
    """Every quantization case in one launch (rows of different lengths,
    both the register-held and the two-read paths)."""
    check_quant_many([x for _, x in quant_cases()])


def test_quant_many_limits():
    rng = np.random.default_rng(102)
    check_quant_many([wl.x_normal(rng, (1, 2560))])
    check_quant_many([wl.x_normal(rng, (m, 64 * (m + 1)))
                      for m in range(1, bt.BT_MAX_QUANT_JOBS + 1)])


# ------------------------------------------------------------- the product
def test_pipeline_worked_example():
    t = np.zeros((2, 64), np.int8)
    t[0, :4] = [1, 0, -1, 1]
    t[1, :4] = [-1, -1, 0, 1]
    x = np.zeros((1, 64), np.float32)
    x[0, :4] = [127, 2.5, -3.5, 0.5]
    _, q, s_a, acc, y = gpu_product(t, x, 0.5)
    assert q[0, :4].tolist() == [127, 2, -4, 0] and s_a[0] == 1.0
    assert acc[0].tolist() == [131, -129]
    assert y[0].tolist() == [65.5, -64.5]


def test_single_gemv_config():
    """M=1, K=256, N=512, seed 0, s_w = 0.02: every output."""
    t, s_w, x = wl.single_gemv()
    p, q, s_a, acc, y = gpu_product(t, x, s_w)
    p_r, q_r, s_r, acc_r, y_r = oracle_product(t, x, s_w)
    np.testing.assert_array_equal(p, p_r)
    np.testing.assert_array_equal(q, q_r)
    np.testing.assert_array_equal(s_a, s_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r, acc_r)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33,
                               63, 64, 65, 100, 257])
@pytest.mark.parametrize("n,k", [(200, 192), (64, 64), (130, 2560),
                                 (70, 6912)])
def test_gemm_matches_oracle(m, n, k):
    rng = np.random.default_rng([102, m, n, k])
    t = wl.trits(rng, (n, k), wl.DECODE_2B)
    x = wl.x_normal_outliers(rng, (m, k))
    s_w = wl.scale(rng, 0.01, 0.05)
    p, q, s_a, acc, y = gpu_product(t, x, s_w)
    p_r, q_r, s_r, acc_r, y_r = oracle_product(t, x, s_w)
    np.testing.assert_array_equal(q, q_r)
    np.testing.assert_array_equal(s_a, s_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r, acc_r)


def test_gemm_extremes():
    """All +1 against all 127 at the largest k: the int32 extreme; and all -1
    rows, zero rows and an all-zero token."""
    k, n, m = 65536, 66, 6
    t = np.zeros((n, k), np.int8)
    t[0] = 1
    t[1] = -1
    t[2:] = wl.trits(np.random.default_rng(103), (n - 2, k))
    t[5] = 0
    x = np.ones((m, k), np.float32)
    x[1] = -1
    x[2] = 0
    x[3:] = wl.x_normal(np.random.default_rng(104), (m - 3, k))
    for mm in (1, m):
        p, q, s_a, acc, y = gpu_product(t, x[:mm], 1.0)
        p_r, q_r, s_r, acc_r, y_r = oracle_product(t, x[:mm], 1.0)
        assert acc[0, 0] == 127 * k and acc[0, 1] == -127 * k
        np.testing.assert_array_equal(acc, acc_r)
        check_y(y, y_r, acc_r)


def test_gemv_entry_matches_gemm():
    rng = np.random.default_rng(105)
    t = wl.trits(rng, (300, 2560), wl.DECODE_2B)
    x = wl.x_normal_outliers(rng, (1, 2560))
    packed = bt.bt_pack_i2s(dev(t))
    x_q, s_a = bt.bt_quant_act(dev(x))
    y1, a1 = bt.bt_gemv(packed, 0.03, 300, 2560, x_q[0], s_a, want_acc=True)
    y2, a2 = bt.bt_gemm(packed, 0.03, 300, 2560, x_q, s_a, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(y1, y2)
    _, _, _, acc_r, y_r = oracle_product(t, x, np.float32(0.03))
    np.testing.assert_array_equal(a1.cpu().numpy(), acc_r)


@pytest.mark.parametrize("n,k", [(200, 192), (64, 64), (130, 2560),
                                 (70, 6912), (66, 65536)])
def test_gemv_lut_matches_oracle(n, k):
    """The lookup-table GEMV: the oracle's accumulators exactly (all +1, all
    -1 and zero rows against all-127 activations at the largest k), and the
    dot-product GEMV's outputs bit for bit."""
    rng = np.random.default_rng([112, n, k])
    t = wl.trits(rng, (n, k), wl.DECODE_2B)
    x = wl.x_normal_outliers(rng, (1, k))
    if k == 65536:
        t[0], t[1], t[2] = 1, -1, 0
        x[0] = 1.0
    s_w = wl.scale(rng, 0.01, 0.05)
    packed = bt.bt_pack_i2s(dev(t))
    x_q, s_a = bt.bt_quant_act(dev(x))
    y1, a1 = bt.bt_gemv_lut(packed, s_w, n, k, x_q[0], s_a, want_acc=True)
    y2, a2 = bt.bt_gemv(packed, s_w, n, k, x_q[0], s_a, want_acc=True)
    torch.cuda.synchronize()
    _, _, _, acc_r, y_r = oracle_product(t, x, s_w)
    np.testing.assert_array_equal(a1.cpu().numpy(), acc_r)
    check_y(y1.cpu().numpy(), y_r, acc_r)
    assert torch.equal(a1, a2) and torch.equal(y1, y2)
    if k == 65536:
        assert acc_r[0, 0] == 127 * k and acc_r[0, 1] == -127 * k
        assert acc_r[0, 2] == 0


# ------------------------------------------------------------ grouped calls
def grouped_case(work, layers):
    """Upload, pack and quantize `layers` layers of a workload; return the
    problem dicts and the host inputs per problem."""
    probs, host = [], []
    for p in work.problems():
        if p.layer >= layers:
            continue
        t, s_w = work.weights(p.layer, p.proj)
        x = work.activations(p.layer, p.proj)
        packed = bt.bt_pack_i2s(dev(t))
        x_q, s_a = bt.bt_quant_act(dev(x))
        y = torch.full((p.m, p.n), float("nan"), device="cuda:0")
        acc = torch.full((p.m, p.n), 0x7EADBEEF, dtype=torch.int32,
                         device="cuda:0")
        probs.append(dict(packed=packed, s_w=s_w, n=p.n, k=p.k, x_q=x_q,
                          s_a=s_a, y=y, acc=acc))
        host.append((t, x, s_w))
    return probs, host


@pytest.mark.parametrize("m,layers", [(1, 2), (3, 2), (8, 2), (16, 2),
                                      (32, 2), (40, 1), (64, 1), (130, 1)])
def test_grouped_layers_match_oracle(m, layers):
    work = wl.decode_2b(m=m, layers=layers)
    probs, host = grouped_case(work, layers)
    plan = bt.bt_grouped_plan(probs)
    refs = [oracle_product(t, x, s_w) for t, x, s_w in host]
    for _ in range(2):  # the plan is reusable; each launch writes everything
        for p in probs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(0x7EADBEEF)
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for prob, (_, q_r, s_r, acc_r, y_r) in zip(probs, refs):
            np.testing.assert_array_equal(prob["x_q"].cpu().numpy(), q_r)
            np.testing.assert_array_equal(prob["acc"].cpu().numpy(), acc_r)
            check_y(prob["y"].cpu().numpy(), y_r, acc_r)


@pytest.mark.parametrize("m,fused", [(1, False), (2, False), (4, False),
                                     (8, False), (32, False), (1, True)])
def test_decode_set_grouped_full_size(m, fused):
    """The whole 2B-shaped decode set (30 layers x 7 projections, 521 MB of
    packed weights) in one grouped launch, as the benchmark runs it, three
    times in a row; every output of every launch against the oracle.  M=1
    streams with dot products; M=2 and 4 (sets this large) and the batched
    decode sizes M=8 and 32 run on the matrix cores.  To
    keep the host side short, the 30 layers share layer 0's seven weight
    tensors (the launch still streams 521 MB); every (layer, projection) has
    its own activations.  fused: the launch quantizes the fp32 activations
    itself."""
    work = wl.decode_2b(m=m)
    shared = {}
    for p in work.problems():
        if p.layer == 0:
            t, s_w = work.weights(0, p.proj)
            shared[p.proj] = (t, s_w, bt.bt_pack_i2s(dev(t)),
                              oracle.pack_i2s(t)[0])
    probs, refs = [], []
    for p in work.problems():
        t, s_w, packed, packed_ref = shared[p.proj]
        x = work.activations(p.layer, p.proj)
        prob = dict(packed=packed, s_w=s_w, n=p.n, k=p.k,
                    y=torch.empty((m, p.n), device="cuda:0"),
                    acc=torch.empty((m, p.n), dtype=torch.int32,
                                    device="cuda:0"))
        if fused:
            prob["x"] = dev(x)
        else:
            prob["x_q"], prob["s_a"] = bt.bt_quant_act(dev(x))
        probs.append(prob)
        q_r, sa_r = oracle.quant_act(x)
        acc_r, y_r = oracle.gemm(packed_ref, s_w, p.n, p.k, q_r, sa_r,
                                 nthreads=NTHREADS)
        refs.append((acc_r, y_r))
    plan = (bt.bt_grouped_plan_f32(probs) if fused
            else bt.bt_grouped_plan(probs))
    for launch in range(3):
        for p in probs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(0x7EADBEEF)
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for i, (prob, (acc_r, y_r)) in enumerate(zip(probs, refs)):
            acc = prob["acc"].cpu().numpy()
            assert np.array_equal(acc, acc_r), f"launch {launch} problem {i}"
            check_y(prob["y"].cpu().numpy(), y_r, acc_r)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 32, 33, 64])
def test_grouped_small_problems(m):
    """Grouped calls with fewer 1 KiB chunks than waves (tiny shapes, ragged
    rows, k of one chunk): row blocks shared by many waves; each plan is
    launched twice to check that the scratch area is left clean."""
    specs = [(512, 256), (64, 64), (70, 192), (1, 64), (130, 320)]
    probs, host = [], []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([107, m, i])
        t = wl.trits(rng, (n, k), wl.DECODE_2B)
        x = wl.x_normal_outliers(rng, (m, k))
        s_w = wl.scale(rng, 0.01, 0.05)
        x_q, s_a = bt.bt_quant_act(dev(x))
        probs.append(dict(packed=bt.bt_pack_i2s(dev(t)), s_w=s_w, n=n, k=k,
                          x_q=x_q, s_a=s_a,
                          y=torch.full((m, n), float("nan"), device="cuda:0"),
                          acc=torch.full((m, n), 0x7EADBEEF, dtype=torch.int32,
                                         device="cuda:0")))
        host.append((t, x, s_w))
    for sub in (probs[:1], probs):
        plan = bt.bt_grouped_plan(sub)
        for _ in range(2):
            for p in sub:
                p["y"].fill_(float("nan"))
            bt.bt_gemm_grouped(plan)
            torch.cuda.synchronize()
            for prob, (t, x, s_w) in zip(sub, host):
                _, q_r, s_r, acc_r, y_r = oracle_product(t, x, s_w)
                np.testing.assert_array_equal(prob["acc"].cpu().numpy(), acc_r)
                check_y(prob["y"].cpu().numpy(), y_r, acc_r)


@pytest.mark.parametrize("m", [1, 4, 8, 130])
def test_grouped_extremes(m):
    """Grouped calls at the largest k (65536, the int32 extreme of all +1
    weights against all 127 activations), with all -1 and all-zero rows, an
    all-zero token and a second, one-chunk problem in the same plan: a row
    block of 1024 chunks is cut among many waves (m <= 4) or split into
    reduction ranges (prefill sizes)."""
    k, n = 65536, 70
    rng = np.random.default_rng([111, m])
    t = wl.trits(rng, (n, k), wl.DECODE_2B)
    t[0] = 1
    t[1] = -1
    t[2] = 0
    x = wl.x_normal(rng, (m, k))
    x[0] = 1.0
    if m > 1:
        x[1] = -1.0
    if m > 2:
        x[2] = 0.0
    t2 = wl.trits(rng, (64, 64))
    x2 = wl.x_normal(rng, (m, 64))
    cases = [(t, x, np.float32(1.0)), (t2, x2, np.float32(0.02))]
    probs = []
    for tt, xx, s_w in cases:
        x_q, s_a = bt.bt_quant_act(dev(xx))
        probs.append(dict(packed=bt.bt_pack_i2s(dev(tt)), s_w=s_w,
                          n=tt.shape[0], k=tt.shape[1], x_q=x_q, s_a=s_a,
                          y=torch.full((m, tt.shape[0]), float("nan"),
                                       device="cuda:0"),
                          acc=torch.full((m, tt.shape[0]), 0x7EADBEEF,
                                         dtype=torch.int32, device="cuda:0")))
    plan = bt.bt_grouped_plan(probs)
    for _ in range(2):
        for p in probs:
            p["y"].fill_(float("nan"))
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for prob, (tt, xx, s_w) in zip(probs, cases):
            _, _, _, acc_r, y_r = oracle_product(tt, xx, s_w)
            acc = prob["acc"].cpu().numpy()
            np.testing.assert_array_equal(acc, acc_r)
            check_y(prob["y"].cpu().numpy(), y_r, acc_r)
        acc = probs[0]["acc"].cpu().numpy()
        assert acc[0, 0] == 127 * k and acc[0, 1] == -127 * k
        assert (acc[:, 2] == 0).all()
        if m > 2:
            assert (acc[2] == 0).all()


@pytest.mark.parametrize("m", [1, 3])
def test_grouped_full_grid_cuts(m):
    """A plan large enough to fill every CU (more than 16 chunks per
    workgroup slot), so the streaming kernel runs its widest workgroups:
    row blocks of 1024 chunks (k = 65536) cut among a hundred waves and more
    (the atomic hand-off), next to blocks of 4 chunks (k = 256) shared by two
    neighbouring waves (combined inside the workgroup); three launches in a
    row, every output against the oracle."""
    rng = np.random.default_rng([112, m])
    cases = []
    for n, k in ((640, 65536), (4096, 256)):
        cases.append((wl.trits(rng, (n, k), wl.DECODE_2B),
                      wl.x_normal(rng, (m, k)),
                      np.float32(rng.uniform(0.01, 0.05))))
    probs = []
    for tt, xx, s_w in cases:
        x_q, s_a = bt.bt_quant_act(dev(xx))
        probs.append(dict(packed=bt.bt_pack_i2s(dev(tt)), s_w=s_w,
                          n=tt.shape[0], k=tt.shape[1], x_q=x_q, s_a=s_a,
                          y=torch.empty((m, tt.shape[0]), device="cuda:0"),
                          acc=torch.empty((m, tt.shape[0]), dtype=torch.int32,
                                          device="cuda:0")))
    refs = [oracle_product(tt, xx, s_w)[3:] for tt, xx, s_w in cases]
    plan = bt.bt_grouped_plan(probs)
    for launch in range(3):
        for p in probs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(0x7EADBEEF)
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for i, (prob, (acc_r, y_r)) in enumerate(zip(probs, refs)):
            acc = prob["acc"].cpu().numpy()
            assert np.array_equal(acc, acc_r), f"launch {launch} problem {i}"
            check_y(prob["y"].cpu().numpy(), y_r, acc_r)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_grouped_fused_quant(m):
    """Grouped calls that quantize their own fp32 activations: outputs equal
    to the oracle's (which quantizes with its own code) and bit-identical to
    the two-step path (bt_quant_act, then the grouped product); ragged and
    tiny shapes, one-chunk rows, the longest rows that fit (m k = 16384);
    each plan launched twice."""
    kmax = bt.BT_FUSED_MAX_MK // m // 64 * 64
    specs = [(512, 256), (64, 64), (70, 192), (1, 64), (130, 320),
             (300, 2560), (200, kmax)]
    probs, steps, refs = [], [], []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([109, m, i])
        t = wl.trits(rng, (n, k), wl.DECODE_2B)
        x = wl.x_normal_outliers(rng, (m, k))
        if i == 1:
            x[0] = 0  # an all-zero row: amax floor, q = 0
        s_w = wl.scale(rng, 0.01, 0.05)
        packed = bt.bt_pack_i2s(dev(t))
        probs.append(dict(packed=packed, s_w=s_w, n=n, k=k, x=dev(x),
                          y=torch.empty((m, n), device="cuda:0"),
                          acc=torch.empty((m, n), dtype=torch.int32,
                                          device="cuda:0")))
        x_q, s_a = bt.bt_quant_act(dev(x))
        steps.append(dict(packed=packed, s_w=s_w, n=n, k=k, x_q=x_q, s_a=s_a,
                          y=torch.empty((m, n), device="cuda:0"),
                          acc=torch.empty((m, n), dtype=torch.int32,
                                          device="cuda:0")))
        refs.append(oracle_product(t, x, s_w))
    plan = bt.bt_grouped_plan_f32(probs)
    plan2 = bt.bt_grouped_plan(steps)
    bt.bt_gemm_grouped(plan2)
    for _ in range(2):
        for p in probs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(0x7EADBEEF)
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for prob, two, (_, _, _, acc_r, y_r) in zip(probs, steps, refs):
            np.testing.assert_array_equal(prob["acc"].cpu().numpy(), acc_r)
            check_y(prob["y"].cpu().numpy(), y_r, acc_r)
            assert torch.equal(prob["y"], two["y"])
            assert torch.equal(prob["acc"], two["acc"])


@pytest.mark.parametrize("m", [70, 130])
@pytest.mark.parametrize("specs", [
    [(300, 2048), (200, 8384)],            # 131 chunks: 3 x 34 and 29
    [(300, 2048), (200, 8384), (64, 64)],  # plus one-chunk rows, which do
])                                         # not shorten the ranges
def test_grouped_split_ranges(m, specs):
    """Grouped prefill-sized calls whose long reductions are cut into ranges
    combined through the plan's scratch slots (odd chunk counts, partial row
    and token tiles); each plan is launched twice to check that the slots and
    counters are left clean."""
    probs, host = [], []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([108, m, i, len(specs)])
        t = wl.trits(rng, (n, k))
        x = wl.x_normal(rng, (m, k))
        s_w = wl.scale(rng, 0.01, 0.05)
        x_q, s_a = bt.bt_quant_act(dev(x))
        probs.append(dict(packed=bt.bt_pack_i2s(dev(t)), s_w=s_w, n=n, k=k,
                          x_q=x_q, s_a=s_a,
                          y=torch.full((m, n), float("nan"), device="cuda:0"),
                          acc=torch.full((m, n), 0x7EADBEEF, dtype=torch.int32,
                                         device="cuda:0")))
        host.append((t, x, s_w))
    plan = bt.bt_grouped_plan(probs)
    for _ in range(2):
        for p in probs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(0x7EADBEEF)
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for prob, (t, x, s_w) in zip(probs, host):
            _, q_r, s_r, acc_r, y_r = oracle_product(t, x, s_w)
            np.testing.assert_array_equal(prob["acc"].cpu().numpy(), acc_r)
            check_y(prob["y"].cpu().numpy(), y_r, acc_r)


def test_prefill_layer_sampled():
    """One 2B-shaped layer at M=512 (7 products): 24 sampled output rows per
    projection against the oracle, all 512 tokens."""
    work = wl.prefill_2b()
    for p in work.problems():
        t, s_w = work.weights(p.layer, p.proj)
        x = work.activations(p.layer, p.proj)
        _, q, s_a, acc, y = gpu_product(t, x, s_w)
        rng = np.random.default_rng([106, wl.PROJ_NAMES.index(p.proj)])
        starts = sorted(set(rng.integers(0, p.n - 8, size=3).tolist()))
        for r0 in starts:
            rows = (r0, r0 + 8)
            q_r, s_r = oracle.quant_act(x)
            pk, _ = oracle.pack_i2s(t[r0:r0 + 8])
            acc_r, y_r = oracle.gemm(pk, s_w, 8, p.k, q_r, s_r,
                                     nthreads=NTHREADS)
            np.testing.assert_array_equal(acc[:, r0:r0 + 8], acc_r)
            check_y(y[:, r0:r0 + 8], y_r, acc_r)


def shared_weight_set(work, sample=None, launches=2, seed=110):
    """The products of `work` in one grouped plan, the way the benchmark
    launches them, with every layer reusing layer 0's weight tensors (the
    launch still streams the whole set); each (layer, projection) has its
    own activations.  Every launch is checked against the oracle: every
    output, or, with sample = r, r sampled row groups of 8 per product (all
    tokens)."""
    m = work.m
    shared = {}
    for p in work.problems():
        if p.layer == 0:
            t, s_w = work.weights(0, p.proj)
            shared[p.proj] = (t, s_w, bt.bt_pack_i2s(dev(t)))
    probs, checks = [], []
    for i, p in enumerate(work.problems()):
        t, s_w, packed = shared[p.proj]
        x = work.activations(p.layer, p.proj)
        x_q, s_a = bt.bt_quant_act(dev(x))
        probs.append(dict(packed=packed, s_w=s_w, n=p.n, k=p.k, x_q=x_q,
                          s_a=s_a, y=torch.empty((m, p.n), device="cuda:0"),
                          acc=torch.empty((m, p.n), dtype=torch.int32,
                                          device="cuda:0")))
        q_r, sa_r = oracle.quant_act(x)
        if sample is None:
            spans = [(0, p.n)]
        else:
            rng = np.random.default_rng([seed, i])
            spans = [(r0, r0 + 8) for r0 in sorted(set(
                rng.integers(0, p.n - 8, size=sample).tolist()))]
        refs = []
        for r0, r1 in spans:
            pk = oracle.pack_i2s(t[r0:r1])[0]
            refs.append((r0, r1) + tuple(oracle.gemm(
                pk, s_w, r1 - r0, p.k, q_r, sa_r, nthreads=NTHREADS)))
        checks.append(refs)
    plan = bt.bt_grouped_plan(probs)
    for launch in range(launches):
        for p in probs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(0x7EADBEEF)
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for i, (prob, refs) in enumerate(zip(probs, checks)):
            acc = prob["acc"].cpu().numpy()
            y = prob["y"].cpu().numpy()
            for r0, r1, acc_r, y_r in refs:
                assert np.array_equal(acc[:, r0:r1], acc_r), \
                    f"launch {launch} product {i} rows {r0}..{r1}"
                check_y(y[:, r0:r1], y_r, acc_r)


@pytest.mark.parametrize("m", [1, 64])
def test_decode_8b_set_grouped_full_size(m):
    """The 8B-shaped set (32 layers x 7 projections, 1.74 GB of packed
    weights) in one grouped launch: every output at M=1, sampled rows at
    M=64."""
    shared_weight_set(wl.decode_8b(m), sample=None if m == 1 else 3)


def test_prefill_layer_grouped_sampled():
    """The M=512 layer's seven products in one grouped launch (split
    reductions for the long down projection), as the benchmark runs it."""
    shared_weight_set(wl.prefill_2b(512), sample=4)


# ------------------------------------------------------- layer-chained decode
def oracle_chain(work, layers):
    """The chained decode on the CPU: every phase quantizes its input (O3),
    multiplies (O4) and rescales in fp32 (O5), and the fp32 outputs feed the
    next phase as they would on the GPU."""
    x = wl.chain_input(work)
    outs = []
    for l in range(layers):
        ys = {}
        for src, dsts in wl.CHAIN_PHASES:
            xin = x if src == "x" else ys[src]
            q, s_a = oracle.quant_act(xin)
            for d in dsts:
                t, s_w = work.weights(l, d)
                p, bad = oracle.pack_i2s(t)
                assert bad == 0
                acc, _ = oracle.gemm(p, s_w, t.shape[0], t.shape[1], q, s_a,
                                     nthreads=NTHREADS)
                ys[d] = oracle.rescale_f32(acc, s_w, s_a)
        outs.append(ys)
        x = ys[wl.CHAIN_OUT]
    return outs


@pytest.mark.parametrize("fused", [False, True])
def test_chained_decode_matches_oracle(fused):
    """Two 2B-shaped layers chained phase by phase (two launches per phase,
    or one launch that quantizes its fp32 input): every output of every
    projection equals the oracle's bit for bit (each phase's fp32 output is
    the next phase's input), eagerly and on each replay of the token captured
    as a HIP graph, with eager launches between the replays."""
    import bench
    work = wl.decode_2b(1)
    cs = bench.ChainSet(work, torch, bt, layers=2, fused=fused)
    cs.step()
    torch.cuda.synchronize()
    ref = oracle_chain(work, 2)

    def check(label):
        for l in range(2):
            for proj in wl.PROJ_NAMES:
                got = cs.y[l][proj].cpu().numpy()
                assert np.array_equal(got, ref[l][proj]), (label, l, proj)

    check("eager")
    graph = cs.capture()
    for rep in range(3):
        for ys in cs.y:
            for t in ys.values():
                t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        cs.step()
        torch.cuda.synchronize()
        check(f"eager after replay {rep}")
