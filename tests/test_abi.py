"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call.  CPU only: every call below fails
an argument check first, so no kernel is launched and no pointer is used.

Fake device pointers (small aligned integers) are only ever passed together
with at least one argument that the host check rejects."""
import ctypes
import os
import re

import numpy as np
import pytest

import gemm_i2_bit_amd as bt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bt.h")

P = 0x10000  # a 16-byte aligned fake address; never dereferenced here


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bt_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bt.LIB_PATH):
        import importlib
        build = importlib.import_module("gemm_i2_bit_amd.build")
        build.build()
    return bt.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"bt_pack_i2s", "bt_quant_act", "bt_quant_act_many", "bt_gemv",
            "bt_gemm",
            "bt_gemm_grouped", "bt_grouped_plan"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_timing_build_exports(L):
    """The timing build (per-wave timestamps) exports what bt.h declares
    and the two calls of bt_timing.h; the product library has neither of
    the latter."""
    path = os.path.join(os.path.dirname(bt.LIB_PATH), "libbt_timing.so")
    assert os.path.exists(path), "libbt_timing.so is built with libbt.so"
    T = ctypes.CDLL(path)
    timing = declared_functions(os.path.join(ROOT, "include", "bt_timing.h"))
    assert timing == ["bt_probe_timestamps", "bt_wave_timestamps"]
    for name in declared_functions() + timing:
        assert hasattr(T, name), name
    for name in timing:
        assert not hasattr(L, name), name
        fn = getattr(T, name)
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int32
        assert fn(None, None) == bt.BT_E_NULL  # checked before any HIP call


def test_status_strings(L):
    for code in range(-6, 1):
        assert len(bt.bt_status_str(code)) > 0
    assert bt.bt_status_str(-99) == "unknown status"


def test_packed_bytes(L):
    assert L.bt_packed_bytes(512, 256) == 512 * 256 // 4
    assert L.bt_packed_bytes(1, 64) == 64 * 16          # padded to 64 rows
    assert L.bt_packed_bytes(70, 2560) == 128 * 640
    assert L.bt_packed_bytes(2560, 6912) == 2560 * 6912 // 4
    for n, k in [(0, 64), (1, 0), (1, 32), (1, 100), (1, 65536 + 64),
                 (-5, 64), (1 << 29, 64)]:
        assert L.bt_packed_bytes(n, k) == bt.BT_E_SHAPE


def test_gemm_argument_errors(L):
    g = L.bt_gemm
    ok = dict(packed=P, s_w=0.5, n=64, k=64, m=1, x_q=P, s_a=P, y=P, acc=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(a["packed"], a["s_w"], a["n"], a["k"], a["m"], a["x_q"],
                 a["s_a"], a["y"], a["acc"], None)

    assert call(packed=None, k=0) == bt.BT_E_NULL
    assert call(x_q=None, k=0) == bt.BT_E_NULL
    assert call(s_a=None, k=0) == bt.BT_E_NULL
    assert call(y=None, k=0) == bt.BT_E_NULL
    for bad in [dict(k=32), dict(k=100), dict(k=0), dict(k=65600),
                dict(n=0), dict(m=0), dict(m=1 << 25), dict(n=1 << 29)]:
        assert call(**bad) == bt.BT_E_SHAPE, bad
    for bad in [dict(packed=P + 4), dict(x_q=P + 8), dict(y=P + 4),
                dict(s_a=P + 2), dict(acc=P + 4)]:
        assert call(k=64, s_w=float("nan"), **bad) == bt.BT_E_ALIGN, bad
    for bad in [float("nan"), float("inf"), -1.0]:
        assert call(s_w=bad, acc=P + 4) in (bt.BT_E_ALIGN,)  # align first
        assert call(s_w=bad, n=0) == bt.BT_E_SHAPE
    # the scale check itself, with everything else valid except alignment of
    # nothing: use a NULL y so no HIP call can follow
    assert call(s_w=-1.0, y=None) == bt.BT_E_NULL


def test_scale_check_precedes_hip(L):
    # all pointers valid-looking, shapes valid, scale invalid -> BT_E_ARG,
    # returned before the device is queried (no HIP call, no launch)
    for bad in [float("nan"), float("inf"), -0.5]:
        assert L.bt_gemm(P, bad, 64, 64, 1, P, P, P, None, None) == bt.BT_E_ARG
        assert L.bt_gemv(P, bad, 64, 64, P, P, P, None, None) == bt.BT_E_ARG


def test_pack_and_quant_argument_errors(L):
    assert L.bt_pack_i2s(None, 64, 64, P, None, None) == bt.BT_E_NULL
    assert L.bt_pack_i2s(P, 64, 64, None, None, None) == bt.BT_E_NULL
    assert L.bt_pack_i2s(P, 64, 63, P, None, None) == bt.BT_E_SHAPE
    assert L.bt_pack_i2s(P, 0, 64, P, None, None) == bt.BT_E_SHAPE
    assert L.bt_pack_i2s(P + 1, 64, 64, P, None, None) == bt.BT_E_ALIGN
    assert L.bt_pack_i2s(P, 64, 64, P + 8, None, None) == bt.BT_E_ALIGN
    assert L.bt_pack_i2s(P, 64, 64, P, P + 2, None) == bt.BT_E_ALIGN
    assert L.bt_quant_act(None, 1, 64, P, P, None) == bt.BT_E_NULL
    assert L.bt_quant_act(P, 1, 64, None, P, None) == bt.BT_E_NULL
    assert L.bt_quant_act(P, 1, 64, P, None, None) == bt.BT_E_NULL
    assert L.bt_quant_act(P, 0, 64, P, P, None) == bt.BT_E_SHAPE
    assert L.bt_quant_act(P, 1, 96, P, P, None) == bt.BT_E_SHAPE
    assert L.bt_quant_act(P + 4, 1, 64, P, P, None) == bt.BT_E_ALIGN
    assert L.bt_quant_act(P, 1, 64, P + 4, P, None) == bt.BT_E_ALIGN
    assert L.bt_quant_act(P, 1, 64, P, P + 1, None) == bt.BT_E_ALIGN


def quant_jobs(specs):
    arr = (bt.bt_quant_job * max(len(specs), 1))()
    for j, (m, k) in enumerate(specs):
        base = P * (j + 1) * 16
        arr[j] = bt.bt_quant_job(base, base + P, base + 2 * P, m, k)
    return arr


def test_quant_many_argument_errors(L):
    ok = quant_jobs([(1, 64), (3, 128)])
    assert L.bt_quant_act_many(None, 1, None) == bt.BT_E_NULL
    assert L.bt_quant_act_many(ok, 0, None) == bt.BT_E_ARG
    many = quant_jobs([(1, 64)] * (bt.BT_MAX_QUANT_JOBS + 1))
    assert L.bt_quant_act_many(many, bt.BT_MAX_QUANT_JOBS + 1,
                               None) == bt.BT_E_ARG
    for field, code in (("x", bt.BT_E_NULL), ("x_q", bt.BT_E_NULL),
                        ("s_a", bt.BT_E_NULL)):
        arr = quant_jobs([(1, 64), (3, 128)])
        setattr(arr[1], field, None)
        assert L.bt_quant_act_many(arr, 2, None) == code, field
    for j, (m, k) in enumerate([(0, 64), (1, 96), (1, 0)]):
        arr = quant_jobs([(1, 64), (m, k)])
        assert L.bt_quant_act_many(arr, 2, None) == bt.BT_E_SHAPE, (m, k)
    big = quant_jobs([(bt.BT_MAX_M, 64), (1, 64)])
    assert L.bt_quant_act_many(big, 2, None) == bt.BT_E_SHAPE
    for field, delta in (("x", 4), ("x_q", 4), ("s_a", 1)):
        arr = quant_jobs([(1, 64), (3, 128)])
        setattr(arr[0], field, getattr(arr[0], field) + delta)
        assert L.bt_quant_act_many(arr, 2, None) == bt.BT_E_ALIGN, field


# ------------------------------------------------------------ grouped plans
def problems(specs):
    arr = (bt.bt_problem * len(specs))()
    for i, (n, k, m) in enumerate(specs):
        base = P * (i + 1) * 16
        arr[i] = bt.bt_problem(base, base + P, base + 2 * P, base + 3 * P,
                               None, 0.25, n, k, m)
    return arr


HDR_FIELDS = ["units", "desc_off", "chunk_off", "unit_off", "sacc_off",
              "scnt_off", "bytes", "total_chunks", "blocks", "fused",
              "start_off", "start_waves"]
DESC_BYTES = 128


def parse_plan(img):
    magic, count, m, kind = np.frombuffer(img[:16].tobytes(), dtype=np.int32)
    vals = np.frombuffer(img[16:16 + 8 * len(HDR_FIELDS)].tobytes(),
                         dtype=np.int64)
    p = dict(zip(HDR_FIELDS, (int(v) for v in vals)))
    p.update(magic=int(magic) & 0xFFFFFFFF, count=int(count), m=int(m),
             kind=int(kind))
    u0 = p["unit_off"]
    p["unit"] = np.frombuffer(img[u0:u0 + 8 * p["units"]].tobytes(),
                              dtype=np.int32).reshape(-1, 2)
    c0 = p["chunk_off"]
    p["chunk0"] = np.frombuffer(img[c0:c0 + 8 * p["count"]].tobytes(),
                                dtype=np.int64)
    return p


def desc(img, p, i):
    base = p["desc_off"] + DESC_BYTES * i
    raw = img[base:base + DESC_BYTES]
    ptrs = raw[:40].view(np.int64)
    s_w = raw[40:44].view(np.float32)[0]
    n, k, m, nblk, ntt = raw[44:64].view(np.int32)
    chunk0 = raw[64:72].view(np.int64)[0]
    blk0, kc, nsplit, split_len, slot0, region0 = raw[72:96].view(np.int32)
    xf = raw[96:104].view(np.int64)[0]
    return dict(ptrs=ptrs, s_w=s_w, n=n, k=k, m=m, nblk=nblk, ntt=ntt,
                chunk0=chunk0, blk0=blk0, kc=kc, nsplit=nsplit,
                split_len=split_len, slot0=slot0, region0=region0, xf=xf)


def test_grouped_plan_layout_stream(L):
    specs = [(2560, 2560, 1), (640, 2560, 1), (2560, 6912, 1), (100, 64, 1)]
    arr = problems(specs)
    nbytes = L.bt_grouped_plan_bytes(arr, len(specs))
    nblk = [(n + 63) // 64 for n, _, _ in specs]
    kc = [k // 64 for _, k, _ in specs]
    img = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(arr, len(specs), img.ctypes.data, nbytes) == 0
    p = parse_plan(img)
    assert p["magic"] == 0x31475442 and p["count"] == 4 and p["m"] == 1
    assert p["kind"] == 0 and p["units"] == 0
    assert p["blocks"] == sum(nblk)
    assert p["total_chunks"] == sum(b * c for b, c in zip(nblk, kc))
    assert p["desc_off"] == 256 and nbytes == p["bytes"]
    for off in ("desc_off", "chunk_off", "start_off", "unit_off", "sacc_off",
                "scnt_off", "bytes"):
        assert p[off] % 256 == 0
    # the start table (one 128-byte entry per wave of a launch on the
    # current device; none without a device) sits between the first-chunk
    # offsets and the units
    assert p["start_off"] >= p["chunk_off"] + 8 * p["count"]
    assert 0 <= p["start_waves"] <= p["total_chunks"]
    assert p["unit_off"] >= p["start_off"] + 128 * p["start_waves"]
    # scratch: one 64-bit slot (chunk count, partial total) per row of every
    # row block and token
    assert p["scnt_off"] - p["sacc_off"] >= sum(nblk) * 64 * 8
    assert p["bytes"] >= p["scnt_off"]
    assert not img[p["sacc_off"]:].any()
    # problems keep their order; chunk and block offsets are prefix sums
    prefix_c = np.cumsum([0] + [b * c for b, c in zip(nblk, kc)])[:-1]
    prefix_b = np.cumsum([0] + nblk)[:-1]
    assert p["chunk0"].tolist() == prefix_c.tolist()
    for i, (n, k, m) in enumerate(specs):
        d = desc(img, p, i)
        assert d["ptrs"][0] == P * (i + 1) * 16
        assert (d["n"], d["k"], d["m"]) == (n, k, m)
        assert (d["nblk"], d["kc"]) == (nblk[i], kc[i])
        assert d["chunk0"] == prefix_c[i] and d["blk0"] == prefix_b[i]
        assert d["s_w"] == np.float32(0.25)


def tile_rows(m):
    """Weight rows per matrix-core workgroup tile: 512 for the 64-token
    tiles (m = 33..64), else 256."""
    return 512 if 32 < m <= 64 else 256


def test_grouped_plan_layout_mfma(L):
    specs = [(640, 2560, 40), (96, 6912, 40)]
    arr = problems(specs)
    nbytes = L.bt_grouped_plan_bytes(arr, 2)
    img = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(arr, 2, img.ctypes.data, nbytes) == 0
    p = parse_plan(img)
    # one 64-token tile; its workgroups cover 512 rows (two 64-row blocks
    # per wave): 640 rows in 2 tiles, 96 rows in 1
    assert p["kind"] == 1 and p["units"] == 2 + 1
    # largest reduction length first
    assert p["unit"][0].tolist() == [1, 0]
    assert p["unit"][1:].tolist() == [[0, 0], [0, 1]]
    assert p["scnt_off"] == p["sacc_off"]  # no scratch for this kind
    assert p["start_waves"] == 0  # the tiles need no start table


@pytest.mark.parametrize("m", [8, 32, 64])
def test_grouped_plan_xcd_order(L, m):
    """Skinny matrix-core plans of the 2B-shaped decode set (30 layers x 7
    projections): whole problems per XCD (workgroup i runs on XCD i mod 8),
    longest reductions first within each XCD, every unit once, padding
    (problem -1) only after an XCD's last unit, and the XCDs' work within a
    few percent of each other."""
    shapes = [(2560, 2560), (640, 2560), (640, 2560), (2560, 2560),
              (6912, 2560), (6912, 2560), (2560, 6912)]
    specs = [(n, k, m) for _ in range(30) for n, k in shapes]
    arr = problems(specs)
    nbytes = L.bt_grouped_plan_bytes(arr, len(specs))
    img = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(arr, len(specs), img.ctypes.data, nbytes) == 0
    p = parse_plan(img)
    assert p["kind"] == 1 and p["units"] % 8 == 0
    u = p["unit"]
    rows = tile_rows(m)
    tiles = [(n + rows - 1) // rows for n, _, _ in specs]
    real = [tuple(x) for x in u.tolist() if x[0] >= 0]
    assert sorted(real) == sorted((i, t) for i, n in enumerate(tiles)
                                  for t in range(n))
    work = [0] * 8
    for x in range(8):
        col = u[x::8]
        live = col[:, 0] >= 0
        nlive = int(live.sum())
        assert live[:nlive].all() and not live[nlive:].any()
        ks = [specs[i][1] for i in col[:nlive, 0]]
        assert ks == sorted(ks, reverse=True)
        work[x] = sum(k // 64 for k in ks)
    owner = {}
    for pos, (prob, _) in enumerate(u.tolist()):
        if prob >= 0:
            assert owner.setdefault(prob, pos % 8) == pos % 8
    assert max(work) <= 1.05 * min(work)


def test_grouped_plan_layout_prefill(L):
    # m >= 65: 256-row x 128-token tiles; the k=6912 problem's reduction is
    # cut into 3 ranges of 36 chunks (about the 40 chunks of k=2560, even)
    specs = [(2560, 2560, 512), (640, 2560, 512), (2560, 6912, 512)]
    arr = problems(specs)
    nbytes = L.bt_grouped_plan_bytes(arr, 3)
    img = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(arr, 3, img.ctypes.data, nbytes) == 0
    p = parse_plan(img)
    tiles = [(n + 255) // 256 * 4 for n, _, _ in specs]
    splits = [1, 1, 3]
    assert p["kind"] == 2
    assert p["units"] == sum(t * s for t, s in zip(tiles, splits))
    # longest range first: the 40-chunk problems, then the 36-chunk ranges
    u = p["unit"]
    assert u[:tiles[0], 0].tolist() == [0] * tiles[0]
    assert u[:tiles[0], 1].tolist() == list(range(tiles[0]))
    assert u[tiles[0]:tiles[0] + tiles[1], 0].tolist() == [1] * tiles[1]
    rest = u[tiles[0] + tiles[1]:]
    assert rest[:, 0].tolist() == [2] * (tiles[2] * 3)
    assert rest[:, 1].tolist() == list(range(tiles[2] * 3))
    for i, want in enumerate([(1, 40, -1, -1), (1, 40, -1, -1),
                              (3, 36, 0, 0)]):
        d = desc(img, p, i)
        assert (d["nsplit"], d["split_len"], d["slot0"], d["region0"]) == want
    # per (64-row block, token tile) of the split problem: one region of
    # 64 rows x 128 tokens of int32 per range, and one counter
    slots = 40 * 4
    assert p["scnt_off"] - p["sacc_off"] >= slots * 3 * 64 * 128 * 4
    assert p["bytes"] - p["scnt_off"] >= slots * 4
    assert not img[p["sacc_off"]:].any()  # the scratch area starts at zero


def test_grouped_plan_errors(L):
    arr = problems([(64, 64, 1), (64, 64, 2)])
    assert L.bt_grouped_plan_bytes(arr, 2) == bt.BT_E_SHAPE  # mixed m
    assert L.bt_grouped_plan_bytes(arr, 0) == bt.BT_E_ARG
    assert L.bt_grouped_plan_bytes(None, 1) == bt.BT_E_NULL
    bad = problems([(64, 96, 1)])
    assert L.bt_grouped_plan_bytes(bad, 1) == bt.BT_E_SHAPE
    good = problems([(64, 64, 1)])
    nbytes = L.bt_grouped_plan_bytes(good, 1)
    img = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(good, 1, img.ctypes.data, nbytes - 1) == bt.BT_E_ARG
    assert L.bt_grouped_plan(good, 1, None, nbytes) == bt.BT_E_NULL
    # a launch with a corrupted host image is refused before any HIP call
    assert L.bt_grouped_plan(good, 1, img.ctypes.data, nbytes) == 0
    broken = img.copy()
    broken[0] ^= 0xFF
    assert L.bt_gemm_grouped(P, broken.ctypes.data, None) == bt.BT_E_ARG
    broken = img.copy()
    broken[8:12] = np.frombuffer(np.int32(7).tobytes(), np.uint8)  # m = 7
    assert L.bt_gemm_grouped(P, broken.ctypes.data, None) == bt.BT_E_ARG
    broken = img.copy()
    broken[24:32] = np.frombuffer(np.int64(64).tobytes(), np.uint8)  # desc
    assert L.bt_gemm_grouped(P, broken.ctypes.data, None) == bt.BT_E_ARG
    assert L.bt_gemm_grouped(None, img.ctypes.data, None) == bt.BT_E_NULL
    assert L.bt_gemm_grouped(P + 16, img.ctypes.data, None) == bt.BT_E_ALIGN


def test_grouped_plan_xcd_errors_and_default(L):
    good = problems([(2560, 2560, 1), (640, 2560, 1)])
    nbytes = L.bt_grouped_plan_bytes(good, 2)
    img = np.zeros(nbytes, np.uint8)
    g = L.bt_grouped_plan_xcd
    sh = np.full(8, 1000, np.int32)
    assert g(good, 2, None, 8, img.ctypes.data, nbytes) == bt.BT_E_NULL
    for n in (0, -1, 33):
        assert g(good, 2, sh.ctypes.data, n, img.ctypes.data,
                 nbytes) == bt.BT_E_ARG, n
    for bad in (499, 2001, 0, -1000):
        b = sh.copy()
        b[5] = bad
        assert g(good, 2, b.ctypes.data, 8, img.ctypes.data,
                 nbytes) == bt.BT_E_ARG, bad
    assert g(good, 2, sh.ctypes.data, 8, img.ctypes.data,
             nbytes - 1) == bt.BT_E_ARG
    # with no device (no full grid) the shares are ignored: the image is
    # bt_grouped_plan's, byte for byte
    assert g(good, 2, sh.ctypes.data, 8, img.ctypes.data, nbytes) == 0
    ref = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(good, 2, ref.ctypes.data, nbytes) == 0
    assert np.array_equal(img, ref)


def test_binding_rejects_host_tensors(L):
    torch = pytest.importorskip("torch")
    t = torch.zeros((64, 64), dtype=torch.int8)
    with pytest.raises(TypeError):
        bt.bt_pack_i2s(t, packed=torch.zeros(1024, dtype=torch.uint8))


# ------------------------------------------------- fused-quantization plans
def problems_f32(specs):
    arr = (bt.bt_problem_f32 * len(specs))()
    for i, (n, k, m) in enumerate(specs):
        base = P * (i + 1) * 16
        arr[i] = bt.bt_problem_f32(base, base + P, base + 2 * P, None, 0.25,
                                   n, k, m)
    return arr


def test_grouped_plan_f32_layout(L):
    specs = [(2560, 2560, 1), (2560, 6912, 1), (100, 64, 1)]
    arr = problems_f32(specs)
    nbytes = L.bt_grouped_plan_f32_bytes(arr, len(specs))
    assert nbytes > 0
    img = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan_f32(arr, len(specs), img.ctypes.data,
                                 nbytes) == 0
    p = parse_plan(img)
    assert p["kind"] == 0 and p["fused"] == 1 and p["units"] == 0
    for i in range(len(specs)):
        d = desc(img, p, i)
        base = P * (i + 1) * 16
        # w, xq, sa, y, acc: the int8 activations and scales are not used
        assert d["ptrs"].tolist() == [base, 0, 0, base + 2 * P, 0]
        assert d["xf"] == base + P
    # the same problems through the int8 entry give an unfused plan
    img2 = np.zeros(L.bt_grouped_plan_bytes(problems(specs), 3), np.uint8)
    assert L.bt_grouped_plan(problems(specs), 3, img2.ctypes.data,
                             img2.size) == 0
    p2 = parse_plan(img2)
    assert p2["fused"] == 0 and desc(img2, p2, 0)["xf"] == 0


def test_grouped_plan_f32_errors(L):
    img = np.zeros(1 << 20, np.uint8)
    assert L.bt_grouped_plan_f32_bytes(None, 1) == bt.BT_E_NULL
    assert L.bt_grouped_plan_f32_bytes(problems_f32([(64, 64, 1)]),
                                       0) == bt.BT_E_ARG
    for spec in [(64, 64, 5), (64, 64, 0), (64, 2 * 8192 + 64, 1),
                 (64, 8192, 3), (64, 96, 1)]:
        assert L.bt_grouped_plan_f32_bytes(problems_f32([spec]),
                                           1) == bt.BT_E_SHAPE, spec
    assert L.bt_grouped_plan_f32_bytes(problems_f32([(64, 16384, 1)]), 1) > 0
    assert L.bt_grouped_plan_f32_bytes(problems_f32([(64, 4096, 4)]), 1) > 0
    arr = problems_f32([(64, 64, 1), (64, 64, 1)])
    arr[1].x = None
    assert L.bt_grouped_plan_f32(arr, 2, img.ctypes.data,
                                 img.size) == bt.BT_E_NULL
    arr = problems_f32([(64, 64, 1), (64, 64, 1)])
    arr[1].x = arr[1].x + 4
    assert L.bt_grouped_plan_f32(arr, 2, img.ctypes.data,
                                 img.size) == bt.BT_E_ALIGN
    arr = problems_f32([(64, 64, 1), (64, 64, 2)])
    assert L.bt_grouped_plan_f32(arr, 2, img.ctypes.data,
                                 img.size) == bt.BT_E_SHAPE
    arr = problems_f32([(64, 64, 1)])
    assert L.bt_grouped_plan_f32(arr, 1, None, img.size) == bt.BT_E_NULL
    assert L.bt_grouped_plan_f32(arr, 1, img.ctypes.data, 16) == bt.BT_E_ARG


def test_grouped_plan_kind_by_m_and_size(L):
    """m = 1 streams; m = 2 streams below 131072 chunks and m = 3, 4 below
    32768, larger plans use the matrix cores; fused plans always stream."""
    def kind(specs, f32=False):
        arr = (problems_f32 if f32 else problems)(specs)
        nb = (L.bt_grouped_plan_f32_bytes if f32
              else L.bt_grouped_plan_bytes)(arr, len(specs))
        assert nb > 0
        img = np.zeros(nb, np.uint8)
        build = L.bt_grouped_plan_f32 if f32 else L.bt_grouped_plan
        assert build(arr, len(specs), img.ctypes.data, nb) == 0
        p = parse_plan(img)
        return p["kind"], p["total_chunks"], p["fused"]

    big = [(8192, 16384)] * 2         # 2 x 128 x 256 = 65536 chunks
    edge = [(4096, 8192)]             # 64 x 128 = 8192 chunks
    for m in (1, 2):
        assert kind([(n, k, m) for n, k in big])[0] == 0
    assert kind([(n, k, 1) for n, k in big * 2])[0] == 0
    assert kind([(n, k, 2) for n, k in big * 2]) == (1, 131072, 0)
    for m in (3, 4):
        assert kind([(n, k, m) for n, k in big]) == (1, 65536, 0)
        assert kind([(n, k, m) for n, k in edge])[0] == 0
        assert kind([(n, k, m) for n, k in edge * 4]) == (1, 32768, 0)
        assert kind([(n, k, m) for n, k in edge * 3])[0] == 0
        # fused: rows of at most 16384 / m inputs, always the streaming kind
        k = 16384 // m // 64 * 64
        assert kind([(65536, k, m)], f32=True) == (0, 1024 * (k // 64), 1)
    assert kind([(64, 64, 5)])[0] == 1


def test_read_probe_argument_errors(L):
    g = L.bt_read_probe
    assert g(None, 1024, P, 4096, 8, 2, None) == bt.BT_E_NULL
    assert g(P, 1024, None, 4096, 8, 2, None) == bt.BT_E_NULL
    for nbytes in (0, 512, 1000, 1024 + 16):
        assert g(P, nbytes, P, 4096, 8, 2, None) == bt.BT_E_SHAPE, nbytes
    assert g(P + 8, 1024, P, 4096, 8, 2, None) == bt.BT_E_ALIGN
    assert g(P, 1024, P + 2, 4096, 8, 2, None) == bt.BT_E_ALIGN
    for wpc in (0, 1, 2, 3, 5, 16):
        assert g(P, 1024, P, 4096, wpc, 2, None) == bt.BT_E_ARG, wpc
    for groups in (0, 5, -1):
        assert g(P, 1024, P, 4096, 4, groups, None) == bt.BT_E_ARG, groups


def test_mix_probe_argument_errors(L):
    g = L.bt_mix_probe
    assert g(None, 1024, P, 1024, 1, P, 4096, 8, 2, None) == bt.BT_E_NULL
    assert g(P, 1024, None, 1024, 1, P, 4096, 8, 2, None) == bt.BT_E_NULL
    assert g(P, 1024, P, 1024, 1, None, 4096, 8, 2, None) == bt.BT_E_NULL
    # no output pointer is needed for no writes (checks pass up to the device)
    assert g(P, 1024, None, 0, 1, P, 4096, 0, 2, None) == bt.BT_E_ARG
    for nbytes, obytes in [(0, 0), (512, 0), (1024 + 16, 1024), (1024, 512),
                           (1024, -1024), (1024, 2048)]:
        assert g(P, nbytes, P, obytes, 1, P, 4096, 8, 2,
                 None) == bt.BT_E_SHAPE, (nbytes, obytes)
    assert g(P + 8, 1024, P, 1024, 1, P, 4096, 8, 2, None) == bt.BT_E_ALIGN
    assert g(P, 1024, P + 8, 1024, 1, P, 4096, 8, 2, None) == bt.BT_E_ALIGN
    assert g(P, 1024, P, 1024, 1, P + 2, 4096, 8, 2, None) == bt.BT_E_ALIGN
    for wpc in (0, 3, 16):
        assert g(P, 1024, P, 0, 1, P, 4096, wpc, 2, None) == bt.BT_E_ARG, wpc
    for groups in (0, 5):
        assert g(P, 1024, P, 0, 1, P, 4096, 4, groups, None) == bt.BT_E_ARG
    for burst in (0, -1, 65):
        assert g(P, 1024, P, 0, burst, P, 4096, 4, 2, None) == bt.BT_E_ARG


def test_b3_sizes_and_argument_errors(L):
    assert L.bt_b3_packed_bytes(64, 80 * 4) == 64 * 4 * 16
    assert L.bt_b3_packed_bytes(70, 64) == 128 * 16      # 64 inputs -> 80
    assert L.bt_b3_packed_bytes(2560, 6912) == 2560 * 87 * 16
    for n, k in [(0, 64), (1, 32), (1, 100), (1, 65536 + 64)]:
        assert L.bt_b3_packed_bytes(n, k) == bt.BT_E_SHAPE
    assert L.bt_pack_b3(None, 64, 64, P, None, None) == bt.BT_E_NULL
    assert L.bt_pack_b3(P, 64, 100, P, None, None) == bt.BT_E_SHAPE
    assert L.bt_pack_b3(P, 64, 64, P + 8, None, None) == bt.BT_E_ALIGN
    g = L.bt_gemv_b3
    assert g(None, 0.5, 64, 64, P, P, P, None, None) == bt.BT_E_NULL
    assert g(P, 0.5, 64, 100, P, P, P, None, None) == bt.BT_E_SHAPE
    assert g(P + 4, 0.5, 64, 64, P, P, P, None, None) == bt.BT_E_ALIGN
    assert g(P, -1.0, 64, 64, P, P, P, None, None) == bt.BT_E_ARG
    assert g(P, float("nan"), 64, 64, P, P, P, None, None) == bt.BT_E_ARG


def test_grouped_static_rejects_large_scratch(L):
    """A plan whose scratch area exceeds the static array is refused before
    any HIP call (fake device pointers, never dereferenced)."""
    assert L.bt_gemm_grouped_static(None, P, None) == bt.BT_E_NULL
    n = (bt.BT_STATIC_SCRATCH_BYTES // 512 + 1) * 64   # m = 1: 512 B/block
    probs = (bt.bt_problem * 1)()
    probs[0] = bt.bt_problem(P, P, P, P, None, 0.5, n, 64, 1)
    nbytes = L.bt_grouped_plan_bytes(probs, 1)
    assert nbytes > bt.BT_STATIC_SCRATCH_BYTES
    host = np.zeros(nbytes, np.uint8)
    assert L.bt_grouped_plan(probs, 1, host.ctypes.data, nbytes) == bt.BT_OK
    assert L.bt_gemm_grouped_static(P, host.ctypes.data, None) == \
        bt.BT_E_SHAPE
    assert L.bt_gemm_grouped_static(P + 16, host.ctypes.data, None) == \
        bt.BT_E_ALIGN


def test_rmsnorm_quant_and_norm_plan_errors(L):
    g = L.bt_rmsnorm_quant
    assert g(None, P, 1, 64, 1e-5, P, P, None, None) == bt.BT_E_NULL
    assert g(P, None, 1, 64, 1e-5, P, P, None, None) == bt.BT_E_NULL
    assert g(P, P, 1, 100, 1e-5, P, P, None, None) == bt.BT_E_SHAPE
    assert g(P, P, 0, 64, 1e-5, P, P, None, None) == bt.BT_E_SHAPE
    assert g(P, P + 4, 1, 64, 1e-5, P, P, None, None) == bt.BT_E_ALIGN
    assert g(P, P, 1, 64, 1e-5, P, P, P + 4, None) == bt.BT_E_ALIGN
    for eps in (-1.0, float("nan"), float("inf")):
        assert g(P, P, 1, 64, eps, P, P, None, None) == bt.BT_E_ARG
    probs = (bt.bt_problem_norm * 1)()
    probs[0] = bt.bt_problem_norm(P, P, P, P, None, 0.5, 1e-5, 64, 64, 1)
    n = L.bt_grouped_plan_norm_bytes(probs, 1)
    assert n > 0
    img = np.zeros(n, np.uint8)
    assert L.bt_grouped_plan_norm(probs, 1, img.ctypes.data, n) == bt.BT_OK
    p = parse_plan(img)
    assert p["fused"] == 1
    d = img[p["desc_off"]:p["desc_off"] + DESC_BYTES]
    assert np.frombuffer(d[104:112].tobytes(), np.uint64)[0] == P   # gain
    assert np.frombuffer(d[112:116].tobytes(), np.float32)[0] == \
        np.float32(1e-5)
    for bad, code in [((P, P, None, P, None, 0.5, 1e-5, 64, 64, 1),
                       bt.BT_E_NULL),
                      ((P, P, P + 4, P, None, 0.5, 1e-5, 64, 64, 1),
                       bt.BT_E_ALIGN),
                      ((P, P, P, P, None, 0.5, -1.0, 64, 64, 1), bt.BT_E_ARG),
                      ((P, P, P, P, None, 0.5, 1e-5, 64, 64, 5),
                       bt.BT_E_SHAPE)]:
        probs[0] = bt.bt_problem_norm(*bad)
        assert L.bt_grouped_plan_norm_bytes(probs, 1) == code, bad
