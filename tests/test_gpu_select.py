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
    """Rows whose eligible keys are all equal (every key on one histogram bin
    in every pass): index order alone decides, for every row length class,
    for all-zero float rows, with zeros left out by nonzero_only, with an
    exclusion mask and with the two-list split."""
    banner("select all-equal keys")
    keys = np.full((3, 5000), 7, dtype=np.uint32)
    check(keys, B.KEY_U32, 0, 2500)
    check(keys, B.KEY_U32, 1234, 4321)
    for n in (1, 300, 4096, 14336, 28000, 32768):
        z = np.zeros((2, n), dtype=np.float32)
        z[1] = -0.0
        for lo, hi in ((0, max(1, n // 3)), (n // 5, n // 2 + 1), (0, n)):
            check(z, B.KEY_ABS_F32, lo, hi)
        v = np.full((1, n), np.float32(-2.5))
        check(v, B.KEY_F32, 0, max(1, n // 4))
    rng = np.random.default_rng(8)
    n = 6000
    sparse = np.where(rng.random((2, n)) < 0.3, 9, 0).astype(np.uint32)   # equal nonzero keys
    check(sparse, B.KEY_U32, 0, 700, nonzero_only=True)
    check(sparse, B.KEY_U32, 100, 5000, nonzero_only=True)
    # excluded entries hold other keys; the eligible ones are all equal
    keys = np.full(n, 5, dtype=np.uint32)
    ex = rng.random(n) < 0.4
    keys[ex] = rng.integers(0, 50, int(ex.sum()))
    md = dev(ex.astype(np.uint8))
    idx = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.sparse_ffn_select(dev(keys), B.KEY_U32, 0, 1000, exclude_mask=md, idx_out=idx, count_out=cnt)
    torch.cuda.synchronize()
    elig = np.flatnonzero(~ex)
    c = int(host(cnt)[0])
    assert c == 1000 and np.array_equal(host(idx)[:c], elig[:1000])
    # the two-list split on an all-equal row
    eq = dev(np.full((1, n), np.float32(0.25)))
    mid = torch.full((1, 3000), -1, dtype=torch.int32, device="cuda")
    top = torch.full((1, 1000), -1, dtype=torch.int32, device="cuda")
    cm = torch.zeros(1, dtype=torch.int32, device="cuda")
    ct = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.sparse_ffn_select(eq, B.KEY_ABS_F32, 1000, 4000, idx_out=mid, count_out=cm, idx_top_out=top,
                        count_top_out=ct)
    torch.cuda.synchronize()
    assert int(host(ct)[0]) == 1000 and np.array_equal(host(top)[0], np.arange(1000))
    assert int(host(cm)[0]) == 3000 and np.array_equal(host(mid)[0], np.arange(1000, 4000))


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


@pytest.mark.parametrize("n_c,c", [(4096, 3), (4096, 7), (1000, 2047), (4096, 2000), (4096, 4095)])
def test_cluster_keys_large(n_c, c):
    """Large clusters whose size is not a power of two: every cluster's two
    largest values sit on its first and last entry (distinct per cluster),
    so a value credited to a neighbouring cluster changes the keys and the
    ranking."""
    banner(f"select cluster keys n={n_c} cluster={c}")
    rng = np.random.default_rng(n_c + c)
    r = (rng.random((2, n_c * c), dtype=np.float32) * 0.5).astype(np.float32)
    first = np.arange(n_c) * c
    r[0, first] = 1.0 + rng.permutation(n_c).astype(np.float32)
    r[0, first + c - 1] = -(1.0 + n_c + rng.permutation(n_c).astype(np.float32))
    r[1, first + c - 1] = 2.0 + rng.permutation(n_c).astype(np.float32)
    r[1, first[: n_c // 2]] = 1e6                      # tied clusters
    keys = dev(r)
    idx = torch.full((2, n_c), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int32, device="cuda")
    for lo, hi in [(0, n_c // 3), (n_c // 5, n_c // 2 + 1)]:
        B.sparse_ffn_select(keys, B.KEY_ABS_F32, lo, hi, cluster=c, idx_out=idx, count_out=cnt)
        torch.cuda.synchronize()
        gi, gc = host(idx), host(cnt)
        for row in range(2):
            ck = oracle.cluster_max_key(oracle.key_abs(r[row]), c)
            exp = oracle.rank_range(ck, lo, hi)
            assert gc[row] == exp.size, (n_c, c, row)
            assert np.array_equal(gi[row, :gc[row]], exp), (n_c, c, row, lo, hi)


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


@pytest.mark.parametrize("n,k_set,k_add", [(8192, 2457, 3277), (5734, 2457, 819), (7, 2, 3),
                                           (1000, 0, 400), (1000, 300, 0), (1000, 300, 900),
                                           (20000, 6000, 5000)])
def test_exclude_mask_fill(n, k_set, k_add):
    """include = exclude = a set S and ranks [0, k): S plus the k best-ranked
    entries outside S (SelectInfer's secondary neurons / fill to phi),
    bit-exact with the oracle's add-until-reached walk."""
    banner(f"select exclude n={n} set={k_set} add={k_add}")
    rng = np.random.default_rng(n + k_set + k_add)
    for key_type in (B.KEY_ABS_F32, B.KEY_U32):
        if key_type == B.KEY_ABS_F32:
            keys = (rng.standard_normal(n) * np.exp(rng.standard_normal(n))).astype(np.float32)
            keys[: n // 3] = np.round(keys[: n // 3])                  # ties, zeros
            okeys = oracle.key_abs(keys)
        else:
            keys = rng.integers(0, 40, n).astype(np.uint32)            # frequency-like counts
            okeys = keys
        S = np.sort(rng.choice(n, size=k_set, replace=False)).astype(np.int32)
        m = np.zeros(n, np.uint8)
        m[S] = 1
        md = dev(m)
        idx = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
        mask = torch.zeros(n, dtype=torch.uint8, device="cuda")
        B.sparse_ffn_select(dev(keys), key_type, 0, k_add, include_mask=md, exclude_mask=md,
                            idx_out=idx, count_out=cnt, mask_out=mask)
        torch.cuda.synchronize()
        exp = oracle.fill_to_phi(S, okeys, k_set + k_add)
        c = int(host(cnt)[0])
        assert c == exp.size and np.array_equal(host(idx)[:c], exp), key_type
        mm = np.zeros(n, np.uint8)
        mm[exp] = 1
        assert np.array_equal(host(mask), mm)
        # exclusion alone: ranks among the entries outside S
        B.sparse_ffn_select(dev(keys), key_type, 0, k_add, exclude_mask=md, idx_out=idx,
                            count_out=cnt)
        torch.cuda.synchronize()
        ok = okeys.copy()
        elig = np.setdiff1d(np.arange(n), S)
        order = elig[oracle.rank_order(ok[elig])][:k_add]
        c = int(host(cnt)[0])
        assert c == order.size and np.array_equal(host(idx)[:c], np.sort(order))


@pytest.mark.parametrize("n_src,k", [(1, 1), (8192, 5734), (5734, 2457), (100, 0), (300, 257)])
def test_gather(n_src, k):
    banner(f"gather n_src={n_src} k={k}")
    rng = np.random.default_rng(n_src + k)
    src = rng.standard_normal(n_src).astype(np.float32)
    idx = rng.integers(0, n_src, max(k, 1)).astype(np.int32)
    dst = torch.full((max(k, 1) + 3,), 7.0, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gather(dev(src), dev(idx[:k]) if k else dev(idx), dst, k_max=k)
    torch.cuda.synchronize()
    got = host(dst)
    assert np.array_equal(got[:k].view(np.uint32), src[idx[:k]].view(np.uint32))
    assert np.all(got[k:] == 7.0)
    # device count below k_max: only the first count entries are written
    c = k // 2
    dst.fill_(7.0)
    B.sparse_ffn_gather(dev(src), dev(idx), dst, count=dev(np.array([c], np.int32)),
                        k_max=max(k, 1))
    torch.cuda.synchronize()
    got = host(dst)
    assert np.array_equal(got[:c].view(np.uint32), src[idx[:c]].view(np.uint32))
    assert np.all(got[c:] == 7.0)


def test_clear_keys():
    """clear_keys: the selection is unchanged and the rows' keys read as zero
    afterwards (a frequency count consumed and reset in one pass); entries
    past n in a wider row are untouched."""
    banner("select clear_keys")
    rng = np.random.default_rng(44)
    rows, n, ld = 3, 5000, 5008
    counts = rng.integers(0, 17, size=(rows, ld)).astype(np.uint32)
    keys = dev(counts)
    idx = torch.full((rows, n), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(rows, dtype=torch.int32, device="cuda")
    B.sparse_ffn_select(keys[:, :n], B.KEY_U32, 0, n, nonzero_only=True, idx_out=idx,
                        count_out=cnt, clear_keys=True)
    torch.cuda.synchronize()
    after = host_u32(keys)
    assert not after[:, :n].any() and np.array_equal(after[:, n:], counts[:, n:])
    gi, gc = host(idx), host(cnt)
    for r in range(rows):
        exp = oracle.rank_range(counts[r, :n], 0, n, True, None)
        assert gc[r] == exp.size and np.array_equal(gi[r, :gc[r]], exp), r
