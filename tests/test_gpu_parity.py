"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for packed bytes, int8 activations, their
scales and int32 accumulators; fp32 outputs within 1e-6 relative error of the
oracle's float64 rescale (exactly 0 where the accumulator is 0).

Inputs come from workloads.py (random numbers only).  Expected values come
only from the oracle."""
import itertools
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


class Arena:
    """The outputs of one grouped plan carved from one device buffer per
    dtype, each output 16-byte aligned, with GAP guard elements before,
    between and after them (NaN for fp32, a sentinel for int32).  check()
    asserts that no guard element changed, so a store anywhere outside a
    problem's own outputs but inside the arena is caught."""
    GAP = 64  # elements (256 bytes)

    def __init__(self, sizes, dtype, fill):
        self.dtype, self.fill = dtype, fill
        offs, pos = [], self.GAP
        for s in sizes:
            offs.append(pos)
            pos += (s + 3) // 4 * 4 + self.GAP
        self.buf = torch.full((pos,), fill, dtype=dtype, device="cuda:0")
        self.views = [self.buf[o:o + s] for o, s in zip(offs, sizes)]
        mask = np.zeros(pos, bool)
        for o, s in zip(offs, sizes):
            mask[o:o + s] = True
        self.mask = mask

    def reset(self):
        for v in self.views:
            v.fill_(self.fill)

    def check(self):
        guards = self.buf.cpu().numpy()[~self.mask]
        if self.dtype == torch.float32:
            assert np.isnan(guards).all(), "write outside the outputs"
        else:
            assert (guards == self.fill).all(), "write outside the outputs"


class OutSet:
    """y and acc arenas for a list of (m, n) outputs."""

    def __init__(self, shapes):
        self.y = Arena([m * n for m, n in shapes], torch.float32,
                       float("nan"))
        self.acc = Arena([m * n for m, n in shapes], torch.int32, 0x7EADBEEF)
        self.shapes = shapes

    def out(self, i):
        m, n = self.shapes[i]
        return self.y.views[i].view(m, n), self.acc.views[i].view(m, n)

    def reset(self):
        self.y.reset()
        self.acc.reset()

    def check(self):
        self.y.check()
        self.acc.check()


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


# ------------------------------------------------------ RMSNorm + quantize
def near_scale_boundary(r64, k):
    """Rows whose RMSNorm scale (the oracle's double value) lies so close to
    a rounding boundary of fp32 that a double sum of squares taken in another
    order (within (k + 4) roundings of 2^-53) could round it to the other
    side.  Such a row may legitimately differ; every other row must match
    bit for bit."""
    r64 = np.asarray(r64, np.float64)
    r32 = r64.astype(np.float32)
    lo = np.nextafter(r32, np.float32(0)).astype(np.float64)
    hi = np.nextafter(r32, np.float32(np.inf)).astype(np.float64)
    mid_lo = (r32.astype(np.float64) + lo) / 2
    mid_hi = (r32.astype(np.float64) + hi) / 2
    d = np.minimum(np.abs(r64 - mid_lo), np.abs(r64 - mid_hi)) / r64
    return d < (k + 4) * 2.0 ** -53


def norm_cases():
    rng = np.random.default_rng(130)
    zero = np.zeros((2, 128), np.float32)
    zero[1, 5] = 3.0
    return [
        ("decode", wl.x_normal_outliers(rng, (3, 2560)), 1e-5),
        ("student_t", wl.x_student_t(rng, (5, 6912)), 1e-6),
        ("held", wl.x_normal(rng, (2, 2048)) * np.float32(40), 1e-5),
        ("held_plus_one", wl.x_normal(rng, (2, 2112)), 0.0),
        ("long_8b", wl.x_student_t(rng, (2, 14336)), 1e-5),
        ("longest", wl.x_normal_outliers(rng, (1, 65536)), 1e-5),
        ("one_chunk", wl.x_normal(rng, (7, 64)), 1e-5),
        ("zero_rows", zero, 1e-5),
    ]


@pytest.mark.parametrize("name,x,eps", norm_cases(),
                         ids=lambda v: v if isinstance(v, str) else "")
def test_rmsnorm_quant_matches_oracle(name, x, eps):
    """RMSNorm then quantization: the normalized rows, x_q and s_a equal the
    oracle's bit for bit (rows of every length class: held in registers,
    one float4 past them, re-read, the longest), except on rows whose scale
    sits on an fp32 rounding boundary (none expected)."""
    m, k = x.shape
    g = np.random.default_rng([131, k]).uniform(-1.5, 1.5, k).astype(
        np.float32)
    q_r, s_r, h_r, r64 = oracle.rmsnorm_quant(x, g, eps)
    qbuf, q = guarded(m * k, torch.int8, 0x5A)
    sbuf, s = guarded(m, torch.float32, float("nan"))
    hbuf, h = guarded(m * k, torch.float32, float("nan"))
    bt.bt_rmsnorm_quant(dev(x), dev(g), eps, x_q=q.view(m, k), s_a=s,
                        h=h.view(m, k))
    torch.cuda.synchronize()
    check_guards(qbuf, 0x5A)
    check_guards(sbuf, None)
    check_guards(hbuf, None)
    ok = ~near_scale_boundary(r64, k)
    assert ok.sum() >= m - 1
    np.testing.assert_array_equal(h.view(m, k).cpu().numpy()[ok], h_r[ok])
    np.testing.assert_array_equal(q.view(m, k).cpu().numpy()[ok], q_r[ok])
    np.testing.assert_array_equal(s.cpu().numpy()[ok].view(np.uint32),
                                  s_r[ok].view(np.uint32))


@pytest.mark.parametrize("m", [1, 2, 4])
def test_grouped_norm_plan(m):
    """Grouped plans that normalize, quantize and multiply in one launch:
    outputs equal to bt_rmsnorm_quant followed by the grouped product, bit
    for bit, and to the oracle (RMSNorm, quantization and product) on rows
    away from a scale rounding boundary; ragged shapes, the longest rows
    that fit; launched twice."""
    kmax = bt.BT_FUSED_MAX_MK // m // 64 * 64
    specs = [(512, 256), (64, 64), (70, 192), (300, 2560), (200, kmax)]
    outs = OutSet([(m, n) for n, _ in specs])
    outs2 = OutSet([(m, n) for n, _ in specs])
    probs, steps, refs, host = [], [], [], []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([132, m, i])
        t = wl.trits(rng, (n, k), wl.DECODE_2B)
        x = wl.x_normal_outliers(rng, (m, k))
        g = rng.uniform(0.5, 1.5, k).astype(np.float32)
        s_w = wl.scale(rng, 0.01, 0.05)
        packed = bt.bt_pack_i2s(dev(t))
        y, acc = outs.out(i)
        probs.append(dict(packed=packed, s_w=s_w, n=n, k=k, x=dev(x),
                          g=dev(g), eps=1e-5, y=y, acc=acc))
        x_q, s_a, _ = bt.bt_rmsnorm_quant(dev(x), dev(g), 1e-5)
        y2, acc2 = outs2.out(i)
        steps.append(dict(packed=packed, s_w=s_w, n=n, k=k, x_q=x_q, s_a=s_a,
                          y=y2, acc=acc2))
        q_r, s_r, _, r64 = oracle.rmsnorm_quant(x, g, 1e-5)
        p_r, _ = oracle.pack_i2s(t)
        acc_r, y_r = oracle.gemm(p_r, s_w, n, k, q_r, s_r, nthreads=NTHREADS)
        ok = ~near_scale_boundary(r64, k)
        refs.append((acc_r, y_r, ok))
    bt.bt_gemm_grouped(bt.bt_grouped_plan(steps))
    plan = bt.bt_grouped_plan_norm(probs)
    for _ in range(2):
        outs.reset()
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        outs.check()
        for prob, two, (acc_r, y_r, ok) in zip(probs, steps, refs):
            assert torch.equal(prob["y"], two["y"])
            assert torch.equal(prob["acc"], two["acc"])
            acc = prob["acc"].cpu().numpy()
            np.testing.assert_array_equal(acc[ok], acc_r[ok])
            check_y(prob["y"].cpu().numpy()[ok], y_r[ok], acc_r[ok])


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


@pytest.mark.parametrize("n,k", [(200, 192), (64, 64), (130, 2560),
                                 (70, 6912), (300, 4096), (66, 65536)])
def test_gemv_b3_matches_oracle(n, k):
    """The five-trits-per-byte format: packed bytes equal the oracle's
    packing bit for bit (and unpack to the trits), and the product equals
    the oracle's accumulators exactly and bt_gemv's outputs bit for bit;
    k that is not a multiple of 80 leaves a padded last piece; at the
    largest k, all +1, all -1 and zero rows against all-127 activations."""
    rng = np.random.default_rng([115, n, k])
    t = wl.trits(rng, (n, k), wl.DECODE_2B)
    x = wl.x_normal_outliers(rng, (1, k))
    if k == 65536:
        t[0], t[1], t[2] = 1, -1, 0
        x[0] = 1.0
    s_w = wl.scale(rng, 0.01, 0.05)
    n_bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    pbuf, packed = guarded(bt.bt_b3_packed_bytes(n, k), torch.uint8, 0xA5)
    bt.bt_pack_b3(dev(t), packed=packed, n_invalid=n_bad)
    p_ref, bad = oracle.pack_b3(t)
    assert bad == 0 and int(n_bad.item()) == 0
    np.testing.assert_array_equal(packed.cpu().numpy(), p_ref)
    check_guards(pbuf, 0xA5)
    back, bad = oracle.unpack_b3(packed.cpu().numpy(), n, k)
    assert bad == 0
    np.testing.assert_array_equal(back, t)
    x_q, s_a = bt.bt_quant_act(dev(x))
    ybuf, y = guarded(n, torch.float32, float("nan"))
    abuf, acc = guarded(n, torch.int32, 0x7EADBEEF)
    bt.bt_gemv_b3(packed, s_w, n, k, x_q[0], s_a, y=y.view(1, n),
                  acc=acc.view(1, n))
    y2, a2 = bt.bt_gemv(bt.bt_pack_i2s(dev(t)), s_w, n, k, x_q[0], s_a,
                        want_acc=True)
    torch.cuda.synchronize()
    check_guards(ybuf, None)
    check_guards(abuf, 0x7EADBEEF)
    _, _, _, acc_r, y_r = oracle_product(t, x, s_w)
    np.testing.assert_array_equal(acc.view(1, n).cpu().numpy(), acc_r)
    check_y(y.view(1, n).cpu().numpy(), y_r, acc_r)
    assert torch.equal(acc.view(1, n), a2) and torch.equal(y.view(1, n), y2)
    if k == 65536:
        assert acc_r[0, 0] == 127 * k and acc_r[0, 1] == -127 * k
        assert acc_r[0, 2] == 0


def test_pack_b3_counts_invalid():
    t = np.zeros((70, 128), np.int8)
    t[3, 5], t[69, 127], t[10, 64] = 2, -2, 100
    n_bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    packed = bt.bt_pack_b3(dev(t), n_invalid=n_bad)
    assert int(n_bad.item()) == 3
    back, _ = oracle.unpack_b3(packed.cpu().numpy(), 70, 128)
    assert back[3, 5] == 0 and back[69, 127] == 0 and back[10, 64] == 0


# ------------------------------------------------------------ grouped calls
def launch_and_check(plan, probs, outs, refs, launches=2, label=""):
    """Launch `plan` `launches` times; before each launch every output is
    reset to its guard fill; after it every output must match its reference
    (acc_r, y_r) and every guard element of the arenas must be untouched.
    refs[i] is a list of (r0, r1, acc_r, y_r) row spans of problem i."""
    for launch in range(launches):
        outs.reset()
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        for i, (prob, spans) in enumerate(zip(probs, refs)):
            acc = prob["acc"].cpu().numpy()
            y = prob["y"].cpu().numpy()
            for r0, r1, acc_r, y_r in spans:
                got = acc[:, r0:r1]
                if not np.array_equal(got, acc_r):
                    bad = np.argwhere(got != acc_r)
                    detail = [(int(t), r0 + int(c), int(acc_r[t, c]),
                               int(got[t, c])) for t, c in bad[:8]]
                    raise AssertionError(
                        f"{label} launch {launch} problem {i} rows {r0}..{r1}:"
                        f" {len(bad)} of {got.size} accumulators differ"
                        f" (token, row, expected, got): {detail}; unwritten"
                        f" (guard fill) {int((got == 0x7EADBEEF).sum())}")
                check_y(y[:, r0:r1], y_r, acc_r)
        outs.check()


def grouped_problems(cases, m, fused=False):
    """cases: list of (t, x, s_w) host inputs.  Packs, quantizes (unless
    fused) and returns (problem dicts, OutSet, whole-output references)."""
    outs = OutSet([(m, t.shape[0]) for t, _, _ in cases])
    probs, refs = [], []
    for i, (t, x, s_w) in enumerate(cases):
        y, acc = outs.out(i)
        prob = dict(packed=bt.bt_pack_i2s(dev(t)), s_w=s_w, n=t.shape[0],
                    k=t.shape[1], y=y, acc=acc)
        if fused:
            prob["x"] = dev(x)
        else:
            prob["x_q"], prob["s_a"] = bt.bt_quant_act(dev(x))
        probs.append(prob)
        _, _, _, acc_r, y_r = oracle_product(t, x, s_w)
        refs.append([(0, t.shape[0], acc_r, y_r)])
    return probs, outs, refs


def grouped_plan(probs, fused=False):
    return (bt.bt_grouped_plan_f32(probs) if fused
            else bt.bt_grouped_plan(probs))


# Plan header fields (int64 at byte 16 on) and the start-table entry layout.
HDR = ["units", "desc_off", "chunk_off", "unit_off", "sacc_off", "scnt_off",
       "bytes", "total_chunks", "blocks", "fused", "start_off", "start_waves"]
START_BYTES = 128


def plan_header(host):
    vals = host[16:16 + 8 * len(HDR)].view(np.int64)
    return dict(zip(HDR, (int(v) for v in vals)))


def without_start_table(plan):
    """The same plan with its header's start-table wave count set to 0: the
    launch then finds every wave's range and first problem by itself."""
    host = plan.host.copy()
    host[16 + 8 * HDR.index("start_waves"):][:8].view(np.int64)[0] = 0
    return bt.GroupedPlan(host, plan.dev, plan._tensors)


def expected_waves(total_chunks):
    """Waves of a streaming launch on this GPU: workgroups of 4 waves, at
    most 2 per CU, and at least 16 chunks per workgroup; no more waves than
    chunks."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = min(cus * 2, (total_chunks + 15) // 16)
    return min(4 * wgs, total_chunks)


@pytest.mark.parametrize("m,layers", [(1, 2), (3, 2), (8, 2), (16, 2),
                                      (32, 2), (40, 1), (64, 1), (130, 1)])
def test_grouped_layers_match_oracle(m, layers):
    work = wl.decode_2b(m=m, layers=layers)
    cases = []
    for p in work.problems():
        t, s_w = work.weights(p.layer, p.proj)
        cases.append((t, work.activations(p.layer, p.proj), s_w))
    probs, outs, refs = grouped_problems(cases, m)
    for prob, (t, x, _) in zip(probs, cases):
        q_r, _ = oracle.quant_act(x)
        np.testing.assert_array_equal(prob["x_q"].cpu().numpy(), q_r)
    # the plan is reusable; each launch writes everything
    launch_and_check(bt.bt_grouped_plan(probs), probs, outs, refs)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 32, 33, 64])
def test_grouped_small_problems(m):
    """Grouped calls with fewer 1 KiB chunks than waves (tiny shapes, ragged
    rows, k of one chunk): row blocks shared by many waves; each plan is
    launched twice to check that the scratch area is left clean."""
    specs = [(512, 256), (64, 64), (70, 192), (1, 64), (130, 320)]
    cases = []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([107, m, i])
        cases.append((wl.trits(rng, (n, k), wl.DECODE_2B),
                      wl.x_normal_outliers(rng, (m, k)),
                      wl.scale(rng, 0.01, 0.05)))
    probs, outs, refs = grouped_problems(cases, m)
    for cnt in (1, len(probs)):
        launch_and_check(bt.bt_grouped_plan(probs[:cnt]), probs[:cnt], outs,
                         refs[:cnt])


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
    cases = [(t, x, np.float32(1.0)),
             (wl.trits(rng, (64, 64)), wl.x_normal(rng, (m, 64)),
              np.float32(0.02))]
    probs, outs, refs = grouped_problems(cases, m)
    launch_and_check(bt.bt_grouped_plan(probs), probs, outs, refs)
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
    cases = [(wl.trits(rng, (n, k), wl.DECODE_2B), wl.x_normal(rng, (m, k)),
              np.float32(rng.uniform(0.01, 0.05)))
             for n, k in ((640, 65536), (4096, 256))]
    probs, outs, refs = grouped_problems(cases, m)
    plan = bt.bt_grouped_plan(probs)
    assert plan_header(plan.host)["start_waves"] > 0
    launch_and_check(plan, probs, outs, refs, launches=3)
    # the same plan with the waves finding their starts themselves
    launch_and_check(without_start_table(plan), probs, outs, refs,
                     launches=2, label="search")


@pytest.mark.parametrize("m,fused", [(1, False), (2, False), (1, True),
                                     (3, True)])
def test_grouped_many_problems(m, fused):
    """Plans of 300 small problems, each with its own weights and
    activations (ragged rows, k from one to twelve chunks), large enough to
    fill every CU: waves whose range starts past problem 255 look their
    problem up beyond the first 256 descriptors.  Three launches in a row,
    every output and every guard element checked."""
    rng = np.random.default_rng([113, m, int(fused)])
    cases = []
    for i in range(300):
        n = int(rng.integers(1, 7)) * 64 + int(rng.integers(0, 64))
        k = 64 * int(rng.integers(1, 15))
        cases.append((wl.trits(rng, (n, k), wl.DECODE_2B),
                      wl.x_normal_outliers(rng, (m, k)),
                      np.float32(rng.uniform(0.01, 0.05))))
    probs, outs, refs = grouped_problems(cases, m, fused)
    chunks = sum((t.shape[0] + 63) // 64 * t.shape[1] // 64
                 for t, _, _ in cases)
    assert chunks >= 512 * 16, "the plan must fill every CU"
    plan = grouped_plan(probs, fused)
    check_start_table(plan, probs, fused)
    launch_and_check(plan, probs, outs, refs, launches=3)
    launch_and_check(without_start_table(plan), probs, outs, refs,
                     launches=2, label="search")


def expected_shares(W, fused):
    """Shares of the waves of a streaming launch on this GPU (1000 = one
    equal share): equal, except on a grid of 8 waves per CU, where the
    younger wave of each SIMD takes less (waves 4-7 of each 8-wave
    workgroup 0.87 of a share for unfused plans, the upper half of the
    grid's 4-wave workgroups 0.9 for fused plans) and, on a GPU of 8 XCDs
    (the 256-CU gfx950 parts), the workgroups of the odd XCDs 0.9."""
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    full = W == 8 * cus
    eight_xcds = cus == 256 and props.gcnArchName.startswith("gfx950")
    wpw = 4 if fused else 8
    wt = [1000] * W
    if full:
        for w in range(W):
            if fused and w >= W // 2:
                wt[w] = wt[w] * 9 // 10
            if not fused and w % 8 >= 4:
                wt[w] = wt[w] * 87 // 100
            if eight_xcds and (w // wpw) % 2 == 1:
                wt[w] = wt[w] * 9 // 10
    return wt, full


def cost_bounds(sizes, q, T, wt):
    """Range ends placed by cost (plans that quantize their own
    activations): a chunk costs 10 and a segment of problem p costs q[p];
    wave w's range ends where the running cost first reaches C x (shares up
    to w) / (all shares), moving on to the next problem only if at least
    half of its quantization fits; C is the least total cost for which the
    last wave's cost does not exceed its share."""
    W = len(wt)
    ends = list(itertools.accumulate(sizes))
    cw = [0] + list(itertools.accumulate(wt))

    def place(C):
        b = [0]
        pos = A = p = 0
        for w in range(W - 1):
            target = C * cw[w + 1] // cw[W]
            if pos < T:
                while p + 1 < len(sizes) and ends[p] <= pos:
                    p += 1
                A += q[p]
                while True:
                    left = ends[p] - pos
                    if A + 10 * left <= target and p + 1 < len(sizes):
                        A += 10 * left
                        pos = ends[p]
                        p += 1
                        if 2 * A + q[p] > 2 * target:
                            break
                        A += q[p]
                    else:
                        step = max(0, min(left, (target - A + 5) // 10))
                        A += 10 * step
                        pos += step
                        break
            b.append(pos)
        b.append(T)
        last = 0
        if pos < T:
            while p + 1 < len(sizes) and ends[p] <= pos:
                p += 1
            last = sum(q[p:]) + 10 * (T - pos)
        return b, last - C * (cw[W] - cw[W - 1]) // cw[W]

    lo, hi = 0, 10 * T + W * max(q) + 10
    while lo < hi:
        mid = (lo + hi) // 2
        if place(mid)[1] > 0:
            lo = mid + 1
        else:
            hi = mid
    return np.array(place(hi)[0], np.int64)


def expected_bounds(T, W, fused, probs):
    """Range ends of the waves: by share, or by cost for fused plans on a
    grid of 8 waves per CU."""
    wt, full = expected_shares(W, fused)
    if fused and full:
        sizes = [(p["n"] + 63) // 64 * (p["k"] // 64) for p in probs]
        m = probs[0]["x"].shape[0] if probs[0]["x"].dim() == 2 else 1
        q = [4 * m * (p["k"] // 64) for p in probs]
        return cost_bounds(sizes, q, T, wt)
    c = np.concatenate([[0], np.cumsum(np.array(wt, np.int64))])
    return c * T // c[-1]


def check_start_table(plan, probs, fused):
    """The plan's start table against the waves' ranges and first problems
    computed here: wave w streams chunks [b[w], b[w + 1]) (expected_bounds),
    and its first chunk lies in the last problem whose first chunk is not
    past it."""
    h = plan_header(plan.host)
    T = h["total_chunks"]
    W = expected_waves(T)
    assert h["start_waves"] == W
    assert h["start_off"] % 256 == 0
    assert h["unit_off"] >= h["start_off"] + W * START_BYTES
    sizes = [(p["n"] + 63) // 64 * (p["k"] // 64) for p in probs]
    assert sum(sizes) == T
    first = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    b = expected_bounds(T, W, fused, probs)
    assert b[0] == 0 and b[-1] == T and (np.diff(b) >= 0).all()
    tab = plan.host[h["start_off"]:h["start_off"] + W * START_BYTES]
    tab = tab.reshape(W, START_BYTES)
    q = tab.view(np.int64)   # 16 int64 per entry
    d = tab.view(np.int32)   # 32 int32 per entry
    for w in range(W):
        lo, hi = b[w], b[w + 1]
        p = min(int(np.searchsorted(first, lo, side="right")) - 1,
                len(probs) - 1)
        prob = probs[p]
        x = prob["x"] if fused else prob["x_q"]
        assert q[w, 0] == prob["packed"].data_ptr(), w
        assert q[w, 1] == x.data_ptr(), w
        assert q[w, 2] == first[p] and (q[w, 3], q[w, 4]) == (lo, hi), w
        assert d[w, 10] == p and d[w, 11] == prob["k"] // 64, w
        assert d[w, 12] == (prob["n"] + 63) // 64, w
        assert q[w, 7] == (0 if w == 0 else b[w - 1]), w
        assert q[w, 8] == (T if w == W - 1 else b[w + 2]), w


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
    cases = []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([109, m, i])
        t = wl.trits(rng, (n, k), wl.DECODE_2B)
        x = wl.x_normal_outliers(rng, (m, k))
        if i == 1:
            x[0] = 0  # an all-zero row: amax floor, q = 0
        cases.append((t, x, wl.scale(rng, 0.01, 0.05)))
    probs, outs, refs = grouped_problems(cases, m, fused=True)
    steps, souts, _ = grouped_problems(cases, m, fused=False)
    bt.bt_gemm_grouped(bt.bt_grouped_plan(steps))
    launch_and_check(bt.bt_grouped_plan_f32(probs), probs, outs, refs)
    for prob, two in zip(probs, steps):
        assert torch.equal(prob["y"], two["y"])
        assert torch.equal(prob["acc"], two["acc"])
    souts.check()


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
    cases = []
    for i, (n, k) in enumerate(specs):
        rng = np.random.default_rng([108, m, i, len(specs)])
        cases.append((wl.trits(rng, (n, k)), wl.x_normal(rng, (m, k)),
                      wl.scale(rng, 0.01, 0.05)))
    probs, outs, refs = grouped_problems(cases, m)
    launch_and_check(bt.bt_grouped_plan(probs), probs, outs, refs)


# ------------------------------------------------- full-size weight sets
class WeightSet:
    """Every (layer, projection) tensor of a workload packed on the GPU and
    by the oracle, each from its own seeded generator (distinct weights per
    layer, as the benchmark uploads them), or, with shared=True, every layer
    reusing layer 0's seven tensors (the launch still streams the whole
    set)."""

    def __init__(self, work, shared=False):
        from concurrent.futures import ThreadPoolExecutor
        self.work = work
        self.gpu, self.ref, self.s_w = {}, {}, {}
        keys = sorted({(0 if shared else p.layer, p.proj)
                       for p in work.problems()})

        def make(key):  # host side: trits and the oracle's packing
            t, s_w = work.weights(*key)
            return t, s_w, oracle.pack_i2s(t)[0]

        with ThreadPoolExecutor(NTHREADS) as ex:
            for i in range(0, len(keys), 32):
                batch = keys[i:i + 32]
                for key, (t, s_w, ref) in zip(batch, ex.map(make, batch)):
                    self.gpu[key] = bt.bt_pack_i2s(dev(t))
                    self.ref[key] = ref
                    self.s_w[key] = s_w
                    del t
        self.shared = shared

    def key(self, p):
        return (0 if self.shared else p.layer, p.proj)


def run_weight_set(ws, work, fused=False, full_layers=None, sample=3,
                   launches=3, seed=110):
    """All products of `work` (the workload of ws's weights at some M, with
    its own activations) in one grouped launch, as the benchmark launches
    them.  Products of the layers in full_layers (None: every layer) are
    checked on every output; the others on `sample` random groups of 8 rows
    (all tokens)."""
    assert work.seed == ws.work.seed and work.shapes == ws.work.shapes
    m = work.m
    plist = work.problems()
    outs = OutSet([(m, p.n) for p in plist])
    probs, refs = [], []
    for i, p in enumerate(plist):
        key = ws.key(p)
        x = work.activations(p.layer, p.proj)
        y, acc = outs.out(i)
        prob = dict(packed=ws.gpu[key], s_w=ws.s_w[key], n=p.n, k=p.k, y=y,
                    acc=acc)
        if fused:
            prob["x"] = dev(x)
        else:
            prob["x_q"], prob["s_a"] = bt.bt_quant_act(dev(x))
        probs.append(prob)
        q_r, sa_r = oracle.quant_act(x)
        if full_layers is None or p.layer in full_layers:
            acc_r, y_r = oracle.gemm(ws.ref[key], ws.s_w[key], p.n, p.k, q_r,
                                     sa_r, nthreads=NTHREADS)
            refs.append([(0, p.n, acc_r, y_r)])
            continue
        rng = np.random.default_rng([seed, i])
        spans = []
        for r0 in sorted(set(rng.integers(0, p.n - 8, size=sample).tolist())):
            # rows r0..r0+7 of the packed tensor: the oracle reads whole row
            # blocks, so multiply the enclosing block and cut the rows out
            b0 = r0 // 64 * 64
            b1 = min(p.n, (r0 + 8 + 63) // 64 * 64)
            blk = ws.ref[key][b0 * p.k // 4:(b1 + 63) // 64 * 64 * p.k // 4]
            acc_r, y_r = oracle.gemm(blk, ws.s_w[key], b1 - b0, p.k, q_r,
                                     sa_r, nthreads=NTHREADS)
            spans.append((r0, r0 + 8, acc_r[:, r0 - b0:r0 - b0 + 8],
                          y_r[:, r0 - b0:r0 - b0 + 8]))
        refs.append(spans)
    plan = grouped_plan(probs, fused)
    launch_and_check(plan, probs, outs, refs, launches=launches,
                     label=f"{work.name}")


@pytest.fixture(scope="module")
def decode_2b_distinct():
    """The 2B-shaped decode set (30 layers x 7 projections, 521 MB packed),
    every tensor distinct."""
    return WeightSet(wl.decode_2b(1))


@pytest.mark.parametrize("m,fused", [(1, False), (1, True), (2, False),
                                     (2, True), (4, False), (8, False),
                                     (16, False), (32, False)])
def test_decode_set_distinct_full_size(decode_2b_distinct, m, fused):
    """The whole 2B-shaped decode set with distinct weights per layer in one
    grouped launch, as the benchmark runs it, three times in a row; every
    output of every launch against the oracle.  M=1 streams with dot
    products (fused: the launch quantizes the fp32 activations itself, with
    range ends placed by cost, also at M=2); M=2 and 4 (sets this large) and
    the batched decode sizes M=8, 16 and 32 run on the matrix cores."""
    run_weight_set(decode_2b_distinct, wl.decode_2b(m), fused)


@pytest.mark.parametrize("m,fused", [(1, False), (1, True), (64, False)])
def test_decode_8b_set_grouped_full_size(m, fused):
    """The 8B-shaped set (32 layers x 7 projections, 1.74 GB of packed
    weights, every layer reusing layer 0's tensors) in one grouped launch:
    every output at M=1 (also with the launch quantizing its fp32
    activations); at M=64 every output of layer 0 and sampled rows of the
    other layers."""
    ws = WeightSet(wl.decode_8b(m), shared=True)
    run_weight_set(ws, wl.decode_8b(m), fused,
                   full_layers=None if m == 1 else {0}, launches=2)


@pytest.mark.parametrize("which,m", [("8b", 64), ("2b", 64), ("2b", 48),
                                     ("2b", 32)])
def test_skinny_launches_repeat(decode_2b_distinct, which, m):
    """The matrix-core decode plans launched 40 times in a row: every launch
    writes the same bits as the first to every output.  The tiles count
    their outstanding loads to know when a ring slot has arrived; a load
    the count misses races with the reads of the slot, and a race shows up
    as launches that differ.  Covers token tiles of 32 and 64 (48: a ragged
    tile), reductions of 20, 32, 54 and 112 stages (54: the ring's last pass
    is partial) and split reductions."""
    if which == "8b":
        ws = WeightSet(wl.decode_8b(m), shared=True)
        work = wl.decode_8b(m)
    else:
        ws, work = decode_2b_distinct, wl.decode_2b(m)
    plist = work.problems()
    outs = OutSet([(m, p.n) for p in plist])
    probs = []
    for i, p in enumerate(plist):
        key = ws.key(p)
        y, acc = outs.out(i)
        x_q, s_a = bt.bt_quant_act(dev(work.activations(p.layer, p.proj)))
        probs.append(dict(packed=ws.gpu[key], s_w=ws.s_w[key], n=p.n, k=p.k,
                          x_q=x_q, s_a=s_a, y=y, acc=acc))
    plan = bt.bt_grouped_plan(probs)
    bt.bt_gemm_grouped(plan)
    torch.cuda.synchronize()
    first_acc = outs.acc.buf.clone()
    first_y = outs.y.buf.view(torch.int32).clone()
    assert not bool((first_acc[torch.from_numpy(outs.acc.mask).cuda()]
                     == 0x7EADBEEF).any()), "an output was not written"
    for launch in range(1, 40):
        outs.reset()
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        same_acc = torch.equal(outs.acc.buf, first_acc)
        same_y = torch.equal(outs.y.buf.view(torch.int32), first_y)
        if not (same_acc and same_y):
            base = outs.acc.buf.data_ptr()
            where = []
            for i, v in enumerate(outs.acc.views):
                o = (v.data_ptr() - base) // 4
                bad = int((v != first_acc[o:o + v.numel()]).sum())
                if bad:
                    where.append((i, bad))
            raise AssertionError(
                f"{work.name} launch {launch} differs from launch 0 (acc "
                f"equal {same_acc}, y equal {same_y}); (problem, elements): "
                f"{where[:8]}")
    outs.check()


@pytest.fixture(scope="module")
def prefill_layer():
    """The M=512 prefill layer: host inputs and the oracle's outputs of all
    seven products (every output)."""
    work = wl.prefill_2b(512)
    out = []
    for p in work.problems():
        t, s_w = work.weights(p.layer, p.proj)
        x = work.activations(p.layer, p.proj)
        out.append((t, x, s_w) + oracle_product(t, x, s_w))
    return out


def test_prefill_layer_single(prefill_layer):
    """One 2B-shaped layer at M=512, each product through bt_gemm: every
    output of all seven products against the oracle."""
    for t, x, s_w, p_r, q_r, s_r, acc_r, y_r in prefill_layer:
        p, q, s_a, acc, y = gpu_product(t, x, s_w)
        np.testing.assert_array_equal(p, p_r)
        np.testing.assert_array_equal(q, q_r)
        np.testing.assert_array_equal(s_a, s_r)
        np.testing.assert_array_equal(acc, acc_r)
        check_y(y, y_r, acc_r)


def test_prefill_layer_grouped(prefill_layer):
    """The M=512 layer's seven products in one grouped launch, as the
    benchmark runs it (split reductions for the long down projection):
    every output of three launches in a row, guards around every output."""
    cases = [(t, x, s_w) for t, x, s_w, *_ in prefill_layer]
    outs = OutSet([(512, t.shape[0]) for t, _, _ in cases])
    probs, refs = [], []
    for i, (t, x, s_w, p_r, q_r, s_r, acc_r, y_r) in enumerate(prefill_layer):
        y, acc = outs.out(i)
        x_q, s_a = bt.bt_quant_act(dev(x))
        probs.append(dict(packed=bt.bt_pack_i2s(dev(t)), s_w=s_w,
                          n=t.shape[0], k=t.shape[1], x_q=x_q, s_a=s_a, y=y,
                          acc=acc))
        refs.append([(0, t.shape[0], acc_r, y_r)])
    plan = bt.bt_grouped_plan(probs)
    check_prefill_order(plan)
    launch_and_check(plan, probs, outs, refs, launches=3)


def test_grouped_plan_xcd_shares_same_outputs():
    """A full-grid streaming plan with the caller's per-XCD shares
    (bt_grouped_plan_xcd): the waves' ranges follow the shares (each XCD's
    chunks in proportion), and the outputs are bit-identical to the default
    plan's."""
    work = wl.decode_2b(1)
    probs = []
    rng = np.random.default_rng(116)
    for pr in work.problems()[:4 * 7]:  # four layers, 69 MB of weights
        n, k = pr.n, pr.k
        t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
        packed = bt.bt_pack_i2s(dev(t))
        xq = dev(rng.integers(-127, 128, size=(1, k), dtype=np.int8))
        sa = dev(np.array([0.01], np.float32))
        y = torch.empty((1, n), dtype=torch.float32, device="cuda:0")
        probs.append(dict(packed=packed, s_w=0.02, n=n, k=k, x_q=xq,
                          s_a=sa, y=y))
    base = bt.bt_grouped_plan(probs)
    shares = [1100, 800, 1000, 950, 1000, 900, 1200, 850]
    tuned = bt.bt_grouped_plan(probs, xcd_shares=shares)
    h = plan_header(tuned.host)
    W = h["start_waves"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert W == 8 * cus
    tab = tuned.host[h["start_off"]:h["start_off"] + W * 128].reshape(W, 128)
    lo, hi = tab.view(np.int64)[:, 3], tab.view(np.int64)[:, 4]
    xcd = (np.arange(W) // 8) % 8
    per = np.array([(hi - lo)[xcd == x].sum() for x in range(8)], np.float64)
    want = np.array(shares, np.float64)
    np.testing.assert_allclose(per / per.sum(), want / want.sum(), rtol=0.01)
    ys = []
    for plan in (base, tuned, base, tuned):
        for p in probs:
            p["y"].fill_(float("nan"))
        bt.bt_gemm_grouped(plan)
        torch.cuda.synchronize()
        ys.append(torch.cat([p["y"].flatten() for p in probs]).clone())
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int32), ys[0].view(torch.int32))
    assert not torch.isnan(ys[0]).any()


def check_prefill_order(plan):
    """A prefill plan with more units than CUs but at most two per CU puts
    the ranges of split reductions at the end of the first round (the units
    [cus - ranges, cus)), every other unit in the plain order around them,
    and lists every unit once."""
    host = plan.host
    h = plan_header(host)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    U = h["units"]
    units = host[h["unit_off"]:h["unit_off"] + 8 * U].view(np.int32)
    units = units.reshape(U, 2)
    count = int(host[4:8].view(np.int32)[0])
    desc = host[h["desc_off"]:h["desc_off"] + 128 * count].reshape(count, 128)
    nsplit = desc[:, 80:84].copy().view(np.int32)[:, 0]
    is_range = nsplit[units[:, 0]] > 1
    n = int(is_range.sum())
    assert cus < U <= 2 * cus and 0 < n <= cus
    assert is_range[cus - n:cus].all() and not is_range[:cus - n].any()
    assert not is_range[cus:].any()
    assert len({(int(p), int(q)) for p, q in units}) == U


# ------------------------------------------------------ read-ceiling probe
def test_read_probe_reads_every_word_once():
    """The read-ceiling probe: the XOR of the per-wave results equals the XOR
    of every 32-bit word of the buffer (each word read exactly once), for a
    buffer whose length does not divide evenly among the waves."""
    rng = np.random.default_rng(114)
    words = rng.integers(0, 1 << 32, size=(3 * 1024 * 1024 + 37 * 256),
                         dtype=np.uint32)
    buf = dev(words.view(np.uint8))
    for wpc in (4, 8):
        for groups in (1, 2, 3, 4):
            sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
            bt.bt_read_probe(buf, sink, wpc, groups)
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
            assert got == np.bitwise_xor.reduce(words), (wpc, groups)


def test_mix_probe_reads_and_writes_every_word_once():
    """The mixed read/write probe: reads every word of its buffer once (XOR
    of the per-wave results) and writes every 1 KiB piece of its output
    once with the piece's index, for shares that do not divide evenly among
    the waves, including no writes and as many bytes written as read, in
    bursts of 1 to 64 pieces."""
    rng = np.random.default_rng(115)
    words = rng.integers(0, 1 << 32, size=(3 * 1024 * 1024 + 37 * 256),
                         dtype=np.uint32)
    buf = dev(words.view(np.uint8))
    nbytes = words.size * 4
    for frac in (0.0, 0.16, 1.0):
        pieces = int(nbytes * frac) // 1024
        for wpc, groups, burst in ((4, 2, 1), (8, 4, 1), (8, 1, 8),
                                   (4, 3, 64)):
            print(f"mix probe: {pieces} pieces, {wpc} waves/CU, {groups} "
                  f"groups, bursts of {burst}", flush=True)
            out = torch.full((pieces * 256 + 256,), -1, dtype=torch.int32,
                             device="cuda:0")
            sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
            bt.bt_mix_probe(buf, out[:pieces * 256].view(torch.uint8), sink,
                            wpc, groups, burst)
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
            assert got == np.bitwise_xor.reduce(words), (frac, wpc, groups)
            o = out.cpu().numpy()
            want = np.repeat(np.arange(pieces, dtype=np.int32), 256)
            np.testing.assert_array_equal(o[:pieces * 256], want)
            assert (o[pieces * 256:] == -1).all()  # guard past the end


# ------------------------------------------------------- layer-chained decode
def oracle_chain(work, layers, norm=False):
    """The chained decode on the CPU: every phase quantizes its input (O3;
    with norm, after the RMSNorm), multiplies (O4) and rescales in fp32
    (O5), and the fp32 outputs feed the next phase as they would on the
    GPU.  Returns the outputs and whether any phase's RMSNorm scale sat on
    an fp32 rounding boundary (then the chain may legitimately differ)."""
    x = wl.chain_input(work)
    outs = []
    boundary = False
    for l in range(layers):
        ys = {}
        for ph, (src, dsts) in enumerate(wl.CHAIN_PHASES):
            xin = x if src == "x" else ys[src]
            if norm:
                q, s_a, _, r64 = oracle.rmsnorm_quant(
                    xin, wl.norm_gain(work, l, ph), wl.NORM_EPS)
                boundary |= bool(near_scale_boundary(r64, xin.shape[1]).any())
            else:
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
    return outs, boundary


@pytest.mark.parametrize("fused,norm,persistent", [
    (False, False, False), (True, False, False), (False, True, False),
    (True, True, False), (True, False, True), (True, True, True)])
def test_chained_decode_matches_oracle(fused, norm, persistent):
    """Two 2B-shaped layers chained phase by phase (two launches per phase,
    or one launch that quantizes its fp32 input; with norm, RMSNorm before
    every quantization): every output of every projection equals the
    oracle's bit for bit (each phase's fp32 output is the next phase's
    input), eagerly and on each replay of the token captured as a HIP graph,
    with eager launches between the replays.  persistent: every phase of
    the token in one cooperative launch with grid barriers between phases;
    its status word must report a complete launch each time."""
    import bench
    work = wl.decode_2b(1)
    cs = bench.ChainSet(work, torch, bt, layers=2, fused=fused, norm=norm,
                        persistent=persistent)
    cs.step()
    torch.cuda.synchronize()
    if persistent:
        assert bt.bt_chain_status(cs.chain) == 0
    ref, boundary = oracle_chain(work, 2, norm)
    assert not boundary, "an RMSNorm scale sits on a rounding boundary"

    def check(label):
        for l in range(2):
            for proj in wl.PROJ_NAMES:
                got = cs.y[l][proj].cpu().numpy()
                assert np.array_equal(got, ref[l][proj]), (label, l, proj)

    check("eager")
    # the persistent launch is one cooperative launch per token: it is
    # repeated eagerly instead of from a graph
    graph = None if persistent else cs.capture()
    for rep in range(3):
        for ys in cs.y:
            for t in ys.values():
                t.fill_(float("nan"))
        if graph is None:
            cs.step()
        else:
            graph.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        if persistent:
            assert bt.bt_chain_status(cs.chain) == 0
        cs.step()
        torch.cuda.synchronize()
        check(f"eager after replay {rep}")
