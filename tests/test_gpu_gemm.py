"""GPU parity of the MX-scaled GEMM (dense and grouped along M) with the
oracle's fp64 definition.  Operands are MX casts made by the ORACLE from
seeded bf16 data (or seeded random codes and scales); the scales go to the
GEMM in the blocked layouts, rearranged by the oracle's layout functions.
The pipeline tests instead feed the GEMM what the library's own casts write
and compare with the oracle's cast followed by the oracle's GEMM.

Tolerance, from the arithmetic: the block-scaled MFMA sums the 64 products
of a K step with less than binary32 precision -- an in-bounds probe on
MI355X measured at most 3.4e-4 of the step's largest product and 1.7e-4 of
the sum of the step's |products| -- and the steps accumulate in binary32.
So |C - C_exact| <= 2^-10 * sum_k |A(m,k) B(n,k)| (about 6x the measured
worst case), plus half a bf16 ulp of |C| when C is stored as bf16."""
import numpy as np
import pytest
import torch

import fp8_precision_quantization_amd as mx
from fp8_precision_quantization_amd import workloads
from tests.gpu_util import device, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu

REL_SUM = 2.0 ** -10


def _codes_scales(rows, k, seed, lo=118, hi=136):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s = rng.integers(lo, hi, size=(rows, k // 32), dtype=np.uint8)
    return q, s


def _cast_operand(oracle_mod, rows, k, seed):
    return oracle_mod.cast_dim0(workloads.heavy_tailed_rows(rows, k, seed=seed))


def _blocked(oracle_mod, s, dev):
    """(R, K/32) or (G, R, K/32) scales -> blocked bytes on the device."""
    return to_dev_u8(oracle_mod.to_blocked(s), dev)


def _blocked_m_groups(oracle_mod, s, ends, dev):
    return to_dev_u8(oracle_mod.to_blocked_grouped(s, np.asarray(ends, np.int32), 0)[0], dev)


def _check(got, want, absum, bf16, what):
    got = got.float().cpu().numpy().astype(np.float64)
    tol = REL_SUM * absum + (np.abs(want) * 2.0 ** -8 if bf16 else 0.0) + 1e-30
    err = np.abs(got - want)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), bad.size, float((err / tol).max()))
    return float((err / (absum + 1e-300)).max())


@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (256, 384, 128), (200, 136, 96), (1, 1, 32),
                                   (300, 260, 5120), (64, 1000, 2080)])
@pytest.mark.parametrize("bf16", [False, True])
def test_gemm_random_operands(oracle_mod, m, n, k, bf16):
    dev = device()
    qa, sa = _codes_scales(m, k, m + k)
    qb, sb = _codes_scales(n, k, n + 2 * k)
    want, absum = oracle_mod.mx_gemm(qa, sa, qb, sb)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), _blocked(oracle_mod, sa, dev), to_dev_u8(qb, dev),
                           _blocked(oracle_mod, sb, dev), out_dtype=torch.bfloat16 if bf16 else torch.float32)
    _check(got, want, absum, bf16, "gemm %dx%dx%d" % (m, n, k))


def test_gemm_of_casts(oracle_mod):
    """Operands as the dim0 cast makes them from bf16 data (heavy-tailed rows:
    scales over many binades, zero and denormal-free)."""
    dev = device()
    qa, sa = _cast_operand(oracle_mod, 384, 1024, 3)
    qb, sb = _cast_operand(oracle_mod, 256, 1024, 4)
    want, absum = oracle_mod.mx_gemm(qa, sa, qb, sb)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), _blocked(oracle_mod, sa, dev), to_dev_u8(qb, dev),
                           _blocked(oracle_mod, sb, dev), out_dtype=torch.float32)
    worst = _check(got, want, absum, False, "gemm of casts")
    assert worst < 2.0 ** -11


def test_gemm_zero_k_and_empty():
    dev = device()
    z = torch.empty((0,), dtype=torch.uint8, device=dev)
    c = torch.full((4, 3), 7.0, device=dev)
    mx.mx_gemm_mxfp8(z.view(4, 0), z.view(4, 0), z.view(3, 0), z.view(3, 0), out_dtype=torch.float32, out=c)
    torch.cuda.synchronize(dev)
    assert torch.all(c == 0)
    e = mx.mx_gemm_mxfp8(z.view(0, 0), z.view(0, 0), z.view(3, 0), z.view(3, 0))
    assert tuple(e.shape) == (0, 3)


GROUP_CASES = [("one", 500, [500]), ("four", 1000, [100, 100, 613, 1000]), ("ragged", 777, [1, 130, 700, 777]),
               ("malformed", 600, [300, 200, 900, 600]), ("short", 600, [128, 300]),
               ("many", 2000, [29 * i for i in range(1, 70)] + [2000]),   # 70 groups, some spanning 2 tiles
               ("tall", 1800, [40, 1700, 1800])]                            # a group of 7 tile rows (one band)


@pytest.mark.parametrize("name,m,ends", GROUP_CASES, ids=[c[0] for c in GROUP_CASES])
def test_grouped_gemm(oracle_mod, name, m, ends):
    dev = device()
    n, k, g = 192, 256, len(ends)
    qa, sa = _codes_scales(m, k, 7)
    qb = np.stack([_codes_scales(n, k, 20 + i)[0] for i in range(g)])
    sb = np.stack([_codes_scales(n, k, 20 + i)[1] for i in range(g)])
    want, absum = oracle_mod.mx_gemm_grouped(qa, sa, qb, sb, np.asarray(ends, np.int32))
    out = torch.full((m, n), 12345.0, device=dev)
    mx.mx_grouped_gemm_mxfp8(to_dev_u8(qa, dev), _blocked_m_groups(oracle_mod, sa, ends, dev), to_dev_u8(qb, dev),
                             _blocked(oracle_mod, sb, dev), torch.tensor(ends, dtype=torch.int32, device=dev),
                             out_dtype=torch.float32, out=out)
    torch.cuda.synchronize(dev)
    rows = ~np.isnan(want[:, 0])
    _check(out[torch.from_numpy(rows).to(dev)], want[rows], absum[rows], False, "grouped " + name)
    # rows past the last (clamped) end are left as they were
    assert torch.all(out[torch.from_numpy(~rows).to(dev)] == 12345.0)


def test_gemm_full_size_sampled(oracle_mod):
    """The benchmark's dense shape, M = 16640, N = 8192, K = 5120, in its launch
    configuration; 24 sampled rows compared against the oracle in full."""
    dev = device()
    m, n, k = 16640, 8192, 5120
    qa, sa = _codes_scales(m, k, 101)
    qb, sb = _codes_scales(n, k, 102)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), _blocked(oracle_mod, sa, dev), to_dev_u8(qb, dev),
                           _blocked(oracle_mod, sb, dev))
    rows = np.sort(np.random.default_rng(5).choice(m, 24, replace=False))
    want, absum = oracle_mod.mx_gemm(qa[rows], sa[rows], qb, sb)
    _check(got[torch.from_numpy(rows).to(dev)], want, absum, True, "16640x8192x5120 sampled")


def test_grouped_gemm_full_size_sampled(oracle_mod):
    """The benchmark's grouped shape: M = 16640 MoE rows in 4 groups, N = 8192,
    K = 5120, per-group weights; 24 sampled rows compared in full."""
    dev = device()
    m, n, k = 16640, 8192, 5120
    _, ends = workloads.moe_activations()
    g = len(ends)
    qa, sa = _codes_scales(m, k, 101)
    ops = [_codes_scales(n, k, 200 + i) for i in range(g)]
    qb = np.stack([o[0] for o in ops])
    sb = np.stack([o[1] for o in ops])
    got = mx.mx_grouped_gemm_mxfp8(to_dev_u8(qa, dev), _blocked_m_groups(oracle_mod, sa, ends, dev),
                                   to_dev_u8(qb, dev), _blocked(oracle_mod, sb, dev),
                                   torch.from_numpy(ends).to(dev))
    rows = np.sort(np.random.default_rng(6).choice(m, 24, replace=False))
    grp = np.searchsorted(ends, rows, side="right")
    for gi in np.unique(grp):
        r = rows[grp == gi]
        want, absum = oracle_mod.mx_gemm(qa[r], sa[r], qb[gi], sb[gi])
        _check(got[torch.from_numpy(r).to(dev)], want, absum, True, "grouped 16640x8192x5120 group %d" % gi)


def test_pipeline_cast_then_gemm(oracle_mod):
    """The library's fused cast (blocked row scales) feeding the GEMM, against
    the oracle's cast followed by the oracle's GEMM.  M = 320 and N = 224 end
    inside a tile; K = 1056 ends a block of 32 into a 128-deep stage."""
    dev = device()
    xa = workloads.heavy_tailed_rows(320, 1056, seed=11)
    xb = workloads.heavy_tailed_rows(224, 1056, seed=12)
    qa, sa, _, _ = mx.mx_cast_dim0_dim1_blocked(to_dev_bf16(xa, dev), dim1=False, raw=True)
    qb, sb, _, _ = mx.mx_cast_dim0_dim1_blocked(to_dev_bf16(xb, dev), dim1=False, raw=True)
    got = mx.mx_gemm_mxfp8(qa, sa, qb, sb, out_dtype=torch.float32)
    oqa, osa = oracle_mod.cast_dim0(xa)
    oqb, osb = oracle_mod.cast_dim0(xb)
    want, absum = oracle_mod.mx_gemm(oqa, osa, oqb, osb)
    _check(got, want, absum, False, "cast -> gemm")


def test_pipeline_grouped_cast_then_gemm(oracle_mod):
    """MoE path: the M-grouped cast of the activations and the blocked casts
    of the per-group weights feeding the grouped GEMM, against the oracle."""
    dev = device()
    ends = np.array([100, 100, 420, 640], np.int32)
    x = workloads.heavy_tailed_rows(640, 512, seed=13)
    ws = [workloads.heavy_tailed_rows(192, 512, seed=20 + i) for i in range(len(ends))]
    offs = torch.from_numpy(ends).to(dev)
    q0, s0g, _, _, _ = mx.mx_cast_dim0_dim1_mgrouped(to_dev_bf16(x, dev), offs, dim1=False, raw=True)
    casts = [mx.mx_cast_dim0_dim1_blocked(to_dev_bf16(w, dev), dim1=False, raw=True) for w in ws]
    qb = torch.stack([c[0] for c in casts])
    sb = torch.cat([c[1].reshape(-1) for c in casts])
    got = mx.mx_grouped_gemm_mxfp8(q0, s0g, qb, sb, offs, out_dtype=torch.float32)
    oq, os_ = oracle_mod.cast_dim0(x)
    wc = [oracle_mod.cast_dim0(w) for w in ws]
    want, absum = oracle_mod.mx_gemm_grouped(oq, os_, np.stack([c[0] for c in wc]), np.stack([c[1] for c in wc]),
                                             ends)
    _check(got, want, absum, False, "grouped cast -> gemm")


@pytest.mark.parametrize("bf16", [False, True])
def test_gemm_nan_code_and_scale_propagate(oracle_mod, bf16):
    """A NaN e4m3 code (0x7F) in row 5 of A and a NaN e8m0 scale (0xFF) on
    block 3 of row 7 of B: row 5 and column 7 of C are NaN, nothing else."""
    dev = device()
    m, n, k = 96, 80, 256
    qa, sa = _codes_scales(m, k, 5)
    qb, sb = _codes_scales(n, k, 6)
    qa[5, 70] = 0x7F
    sb[7, 3] = 0xFF
    want, absum = oracle_mod.mx_gemm(qa, sa, qb, sb)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), _blocked(oracle_mod, sa, dev), to_dev_u8(qb, dev),
                           _blocked(oracle_mod, sb, dev), out_dtype=torch.bfloat16 if bf16 else torch.float32)
    g = got.float().cpu().numpy()
    nan_want = np.zeros((m, n), bool)
    nan_want[5, :] = True
    nan_want[:, 7] = True
    assert np.array_equal(np.isnan(want), nan_want)        # the oracle's own reading
    assert np.array_equal(np.isnan(g), nan_want)
    fin = ~nan_want
    _check(got.float()[torch.from_numpy(fin).to(dev)], want[fin], absum[fin], bf16, "finite part")


def _kgroup_ref(oracle_mod, qa, sa, qb, sb, ends, k):
    """Per group, the oracle's GEMM over the group's 32-blocks [lo // 32,
    hi // 32) of the clamped ends; an empty group gives zeros."""
    out = []
    lo = 0
    for e in ends:
        hi = min(max(int(e), lo), k)
        klo, khi = lo // 32, hi // 32
        if khi > klo:
            out.append(oracle_mod.mx_gemm(qa[:, 32 * klo:32 * khi], sa[:, klo:khi],
                                          qb[:, 32 * klo:32 * khi], sb[:, klo:khi]))
        else:
            z = np.zeros((qa.shape[0], qb.shape[0]))
            out.append((z, z))
        lo = hi
    return out


KGROUP_CASES = [("one", 512, [512]), ("four", 1024, [128, 128, 640, 1024]),
                ("not_128", 800, [96, 300, 800]),            # 300 -> 9 whole blocks; a K tail per group
                ("malformed", 640, [300, 200, 900, 640]), ("short", 640, [128, 320]),
                ("negative", 384, [-40, 100, 384]),
                ("ties", 1024, [256, 512, 768, 1024]),                # equal K lengths: kept in index order
                ("many", 4224, [60 * i for i in range(1, 70)] + [4224])]   # 70 groups: past the ordered count


@pytest.mark.parametrize("name,k,ends", KGROUP_CASES, ids=[c[0] for c in KGROUP_CASES])
def test_kgrouped_gemm(oracle_mod, name, k, ends):
    dev = device()
    m, n = 200, 136
    qa, sa = _codes_scales(m, k, 31)
    qb, sb = _codes_scales(n, k, 32)
    e = np.asarray(ends, np.int32)
    sab = to_dev_u8(oracle_mod.to_blocked_grouped(sa, e // 32, 1)[0], dev)
    sbb = to_dev_u8(oracle_mod.to_blocked_grouped(sb, e // 32, 1)[0], dev)
    out = torch.full((len(ends), m, n), 12345.0, device=dev)
    mx.mx_kgrouped_gemm_mxfp8(to_dev_u8(qa, dev), sab, to_dev_u8(qb, dev), sbb, torch.from_numpy(e).to(dev),
                              out_dtype=torch.float32, out=out)
    for gi, (want, absum) in enumerate(_kgroup_ref(oracle_mod, qa, sa, qb, sb, ends, k)):
        _check(out[gi], want, absum, False, "%s group %d" % (name, gi))


def test_pipeline_weight_gradient(oracle_mod):
    """MoE weight gradient: the grouped-blocked casts of the token-major X
    (T, K) and dY (T, N) feed the K-grouped GEMM dW_g = dY_g^T X_g, against
    the oracle's dim1 casts and per-group GEMMs."""
    dev = device()
    ends = np.array([128, 128, 448, 640], np.int32)
    x = workloads.heavy_tailed_rows(640, 256, seed=51)
    dy = workloads.heavy_tailed_rows(640, 192, seed=52)
    offs = torch.from_numpy(ends).to(dev)
    _, _, _, qx, sx, _ = mx.mx_cast_dim0_dim1_grouped_blocked(to_dev_bf16(x, dev), offs, raw=True)
    _, _, _, qdy, sdy, _ = mx.mx_cast_dim0_dim1_grouped_blocked(to_dev_bf16(dy, dev), offs, raw=True)
    got = mx.mx_kgrouped_gemm_mxfp8(qdy, sdy, qx, sx, offs, out_dtype=torch.float32)
    oqx, osx = oracle_mod.cast_dim1(x)
    oqdy, osdy = oracle_mod.cast_dim1(dy)
    for gi, (want, absum) in enumerate(_kgroup_ref(oracle_mod, oqdy, osdy, oqx, osx, ends, 640)):
        _check(got[gi], want, absum, False, "weight gradient group %d" % gi)


def test_kgrouped_gemm_long_groups(oracle_mod):
    """The MoE token split (16640 tokens, 4 groups) as K, bf16 out."""
    dev = device()
    _, ends = workloads.moe_activations()
    k = 16640
    m, n = 256, 320
    qa, sa = _codes_scales(m, k, 61)
    qb, sb = _codes_scales(n, k, 62)
    sab = to_dev_u8(oracle_mod.to_blocked_grouped(sa, ends // 32, 1)[0], dev)
    sbb = to_dev_u8(oracle_mod.to_blocked_grouped(sb, ends // 32, 1)[0], dev)
    got = mx.mx_kgrouped_gemm_mxfp8(to_dev_u8(qa, dev), sab, to_dev_u8(qb, dev), sbb, torch.from_numpy(ends).to(dev))
    for gi, (want, absum) in enumerate(_kgroup_ref(oracle_mod, qa, sa, qb, sb, ends, k)):
        _check(got[gi], want, absum, True, "long group %d" % gi)
