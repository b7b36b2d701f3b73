"""Selection / compaction on the GPU against the oracle: bit-exact index
sets, masks, counts and frequencies (integer work)."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from gpu_common import banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]


def run_select(keys_np, key_type, r_lo, r_hi, nonzero_only=False, include=None, want_freq=False):
    rows, n = keys_np.shape
    keys = dev(keys_np)
    ld_idx = n if include is not None else max(1, min(r_hi - r_lo, n))
    idx = torch.full((rows, ld_idx), -1, dtype=torch.int32, device="cuda")
    mask = torch.zeros(rows, n, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(rows, dtype=torch.int32, device="cuda")
    freq = torch.zeros(n, dtype=torch.int32, device="cuda") if want_freq else None
    inc = dev(include.astype(np.uint8)) if include is not None else None
    B.sparse_ffn_select(keys, key_type, r_lo, r_hi, nonzero_only=nonzero_only, include_mask=inc,
                        mask_out=mask, idx_out=idx, count_out=cnt, freq=freq)
    torch.cuda.synchronize()
    return host(idx), host(mask), host(cnt), (host_u32(freq) if want_freq else None)


def oracle_keys(keys_np, key_type):
    if key_type == B.KEY_ABS_F32:
        return oracle.key_abs(keys_np)
    if key_type == B.KEY_F32:
        return oracle.key_signed(keys_np)
    return keys_np.astype(np.uint32)


def check(keys_np, key_type, r_lo, r_hi, nonzero_only=False, include=None, want_freq=False):
    idx, mask, cnt, freq = run_select(keys_np, key_type, r_lo, r_hi, nonzero_only, include,
                                      want_freq)
    expect_freq = np.zeros(keys_np.shape[1], dtype=np.uint32)
    for r in range(keys_np.shape[0]):
        exp = oracle.rank_range(oracle_keys(keys_np[r], key_type), r_lo, r_hi, nonzero_only, include)
        assert cnt[r] == exp.size, (r, cnt[r], exp.size)
        assert np.array_equal(idx[r, :cnt[r]], exp), r
        m = np.zeros(keys_np.shape[1], dtype=np.uint8)
        m[exp] = 1
        assert np.array_equal(mask[r], m), r
        expect_freq[exp] += 1
    if want_freq:
        assert np.array_equal(freq, expect_freq)


@pytest.mark.parametrize("n", [1, 7, 64, 1000, 1024, 4097, 8192, 14336, 17408, 20480, 23001, 32768])
def test_topk_float_magnitude(n):
    banner(f"select float n={n}")
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((2, n)) * np.exp(rng.standard_normal((2, n)))).astype(np.float32)
    x[1, : n // 3] = x[1, n // 3: 2 * (n // 3)]          # many exact ties (also across signs)
    x[1, ::5] = -x[1, ::5]
    for lo, hi in [(0, max(1, n // 2)), (0, n), (n // 7, n // 3 + 1), (0, n + 5), (n, n)]:
        check(x, B.KEY_ABS_F32, min(lo, hi), hi)


def test_special_values_and_zero_runs():
    banner("select special values")
    x = np.zeros((1, 300), dtype=np.float32)
    x[0, 10] = np.nan
    x[0, 20] = -np.inf
    x[0, 30] = np.inf
    x[0, 40:60] = -0.0
    x[0, 100:200] = 1.5
    for lo, hi in [(0, 3), (0, 50), (2, 150), (0, 300)]:
        check(x, B.KEY_ABS_F32, lo, hi)
    check(x, B.KEY_ABS_F32, 0, 300, nonzero_only=True)
    check(x, B.KEY_ABS_F32, 5, 300, nonzero_only=True)


def test_all_equal_keys():
    banner("select all-equal keys")
    keys = np.full((3, 5000), 7, dtype=np.uint32)
    check(keys, B.KEY_U32, 0, 2500)
    check(keys, B.KEY_U32, 1234, 4321)


def test_counts_with_heavy_ties_union_and_freq():
    banner("select counts + union + freq")
    rng = np.random.default_rng(5)
    n = 8192
    counts = rng.binomial(256, 0.3, size=(1, n)).astype(np.uint32)
    include = rng.random(n) < 0.2
    check(counts, B.KEY_U32, 0, 1638, include=include)
    keys = rng.integers(0, 50, size=(256, n)).astype(np.uint32)
    check(keys, B.KEY_U32, 0, 2457, want_freq=True)


def test_signed_router_keys():
    banner("select signed keys")
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((4096, 8)).astype(np.float32)
    logits[::7, 3] = logits[::7, 5]
    check(logits, B.KEY_F32, 0, 2)


def test_nonzero_only_clusters():
    banner("select nonzero clusters")
    rng = np.random.default_rng(7)
    kappa = np.where(rng.random((1, 448)) < 0.2, rng.integers(1, 1 << 30, size=(1, 448)), 0)
    check(kappa.astype(np.uint32), B.KEY_U32, 0, 448, nonzero_only=True)
    check(np.zeros((1, 448), np.uint32), B.KEY_U32, 0, 448, nonzero_only=True)


def test_cluster_keys():
    """cluster > 1: an entry is a block of contiguous values keyed by its
    largest |value| (the oracle forms the cluster keys, then ranks them)."""
    banner("select cluster keys")
    rng = np.random.default_rng(8)
    for n_c, c in [(448, 32), (1000, 3), (4096, 4), (4000, 2), (7, 5), (1, 64)]:
        r = np.where(rng.random((2, n_c * c)) < 0.1, rng.standard_normal((2, n_c * c)), 0.0)
        r = r.astype(np.float32)
        if n_c >= 10:
            r[1, : c * 5] = r[1, c * 5: c * 10]         # tied clusters
        keys = dev(r)
        idx = torch.full((2, n_c), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int32, device="cuda")
        mask = torch.zeros(2, n_c, dtype=torch.uint8, device="cuda")
        for nz, lo, hi in [(True, 0, n_c), (False, 0, n_c // 3), (True, 2, n_c // 5 + 2)]:
            B.sparse_ffn_select(keys, B.KEY_ABS_F32, lo, hi, cluster=c, nonzero_only=nz,
                                idx_out=idx, count_out=cnt, mask_out=mask)
            torch.cuda.synchronize()
            gi, gc, gm = host(idx), host(cnt), host(mask)
            for row in range(2):
                ck = oracle.cluster_max_key(oracle.key_abs(r[row]), c)
                exp = oracle.rank_range(ck, lo, hi, nz, None)
                assert gc[row] == exp.size, (n_c, c, row)
                assert np.array_equal(gi[row, :gc[row]], exp), (n_c, c, row)
                m = np.zeros(n_c, np.uint8)
                m[exp] = 1
                assert np.array_equal(gm[row], m)
                if nz and lo == 0:
                    assert np.array_equal(exp, oracle.active_clusters(r[row], c))


@pytest.mark.parametrize("n,k_top,k_mid", [(6144, 1536, 3072), (17408, 4352, 8704),
                                           (100, 0, 30), (100, 30, 0), (5000, 5000, 10)])
def test_two_lists(n, k_top, k_mid):
    """One call yields the ranks [0, k_top) and [k_top, k_top + k_mid) as two
    ascending lists (the two SpAx tiers)."""
    banner(f"select two lists n={n}")
    rng = np.random.default_rng(n + k_top)
    x = (rng.standard_normal((3, n)) * np.exp(rng.standard_normal((3, n)))).astype(np.float32)
    x[2, : n // 2] = np.round(x[2, : n // 2])              # heavy ties
    keys = dev(x)
    mid = torch.full((3, max(1, k_mid)), -1, dtype=torch.int32, device="cuda")
    top = torch.full((3, max(1, k_top)), -1, dtype=torch.int32, device="cuda")
    cm = torch.zeros(3, dtype=torch.int32, device="cuda")
    ct = torch.zeros(3, dtype=torch.int32, device="cuda")
    B.sparse_ffn_select(keys, B.KEY_ABS_F32, k_top, k_top + k_mid, idx_out=mid, count_out=cm,
                        idx_top_out=top, count_top_out=ct)
    torch.cuda.synchronize()
    gm, gt, gcm, gct = host(mid), host(top), host(cm), host(ct)
    for row in range(3):
        k = oracle.key_abs(x[row])
        exp_top = oracle.rank_range(k, 0, k_top, False, None)
        exp_mid = oracle.rank_range(k, k_top, k_top + k_mid, False, None)
        assert gct[row] == exp_top.size and np.array_equal(gt[row, :gct[row]], exp_top), row
        assert gcm[row] == exp_mid.size and np.array_equal(gm[row, :gcm[row]], exp_mid), row


@pytest.mark.parametrize("n", [1, 7, 1000, 4096, 14336, 20480])
def test_weight_aware_scale(n):
    """key_scale: entries ranked by the magnitude of the fp32 product x_j *
    s_j (WiSparse saliency), as two tier lists; bit-exact with the oracle."""
    banner(f"select weight-aware n={n}")
    rng = np.random.default_rng(1000 + n)
    x = (rng.standard_normal((3, n)) * np.exp(rng.standard_normal((3, n)))).astype(np.float32)
    s = np.exp(rng.standard_normal(n) * 0.5).astype(np.float32)
    x[1, : n // 2] = np.round(x[1, : n // 2])               # ties in x ...
    s[: n // 4] = 1.0                                      # ... and in the products
    s[n // 4: n // 4 + n // 10] = 0.0                      # zero-norm channels
    x[2, ::3] = -x[2, ::3]
    x[2, 1::7] *= np.float32(1e-30)                        # products down to subnormals
    k_top, k_mid = (15 * n) // 100, (35 * n) // 100
    mid = torch.full((3, max(1, k_mid)), -1, dtype=torch.int32, device="cuda")
    top = torch.full((3, max(1, k_top)), -1, dtype=torch.int32, device="cuda")
    cm = torch.zeros(3, dtype=torch.int32, device="cuda")
    ct = torch.zeros(3, dtype=torch.int32, device="cuda")
    mask = torch.zeros(3, n, dtype=torch.uint8, device="cuda")
    B.sparse_ffn_select(dev(x), B.KEY_ABS_F32, k_top, k_top + k_mid, idx_out=mid, count_out=cm,
                        idx_top_out=top, count_top_out=ct, mask_out=mask, key_scale=dev(s))
    torch.cuda.synchronize()
    gm, gt, gcm, gct, gmask = host(mid), host(top), host(cm), host(ct), host(mask)
    for row in range(3):
        exp_top, exp_mid = oracle.weighted_tier_sets(x[row], s, k_top, k_mid)
        assert gct[row] == exp_top.size and np.array_equal(gt[row, :gct[row]], exp_top), row
        assert gcm[row] == exp_mid.size and np.array_equal(gm[row, :gcm[row]], exp_mid), row
        m = np.zeros(n, np.uint8)
        m[exp_mid] = 1
        assert np.array_equal(gmask[row], m), row
    # unit scales reproduce the plain |x| ranking
    k = max(1, n // 2)
    idx = torch.full((3, k), -1, dtype=torch.int32, device="cuda")
    B.sparse_ffn_select(dev(x), B.KEY_ABS_F32, 0, k, idx_out=idx, count_out=cm,
                        key_scale=dev(np.ones(n, np.float32)))
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cm)
    for row in range(3):
        exp = oracle.rank_range(oracle.key_abs(x[row]), 0, k)
        assert gc[row] == exp.size and np.array_equal(gi[row, :gc[row]], exp), row
