"""Pins for the CPU oracle: checks against things other than the oracle itself.

* fp16 conversions against numpy over every half bit pattern;
* paged attention against float64 dense attention written with numpy matrix
  products, and against torch's scaled_dot_product_attention (float64, CPU),
  both on the sequence gathered from the pool by numpy indexing;
* closed forms: one token returns v_0, constant values return the constant,
  q = 0 or scale = 0 returns the mean of v, two tokens give the logistic
  weights, a dominating key returns its value even when exp(score) would
  overflow fp32, and a per-group constant V reveals the query-head to KV-head
  mapping;
* bit-exact invariances that follow from paging moving bytes and not
  numbers [PagedAttention, intro; "Sharing is the part that pays twice"]:
  physical block relabelling, free-list history, batch position, block size,
  and the contiguous special case;
* kv_append against a numpy scatter of the whole pool;
* FP8 (E4M3) pools: decoding of all 256 codes against torch's float8_e4m3fn
  and the format's closed-form values, encoding against torch's cast inside
  the finite range (ties included) and saturation outside it, the
  quantization error bound, the quantizing append against a numpy scatter of
  torch-quantized values, and the FP8 attention against the fp16 oracle on
  pools whose dequantized values are exact in fp16 and against float64
  dense attention otherwise.
"""

import numpy as np
import pytest

import workloads as wl


def f64_dense(q, k, v, scale):
    """softmax(scale * q k^T) v in float64 for one row: q [Hq][D], k/v [L][Hkv][D]."""
    Hq, D = q.shape
    L, Hkv, _ = k.shape
    nrep = Hq // Hkv
    out = np.zeros((Hq, D))
    if L == 0:
        return out
    for h in range(Hq):
        g = h // nrep
        s = scale * (k[:, g, :].astype(np.float64) @ q[h].astype(np.float64))
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ v[:, g, :].astype(np.float64)
    return out


def close(a, ref, atol=1e-5, rtol=1e-5):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(a - ref) <= atol + rtol * np.abs(ref)))


def run_oracle(oracle, w, layer=0, ld=None):
    ld = ld or w.layer(layer)
    return oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale)


# ---------------------------------------------------------------------------
# conversions
# ---------------------------------------------------------------------------


def test_half_to_float_all_patterns(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_float(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_rne(oracle):
    rng = np.random.default_rng(0)
    # every half value, every midpoint between neighbours, and random floats
    # across the whole half range including subnormals and overflow
    h = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1)]).astype(np.float32)
    rand = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-9, 5, 200000)).astype(np.float32)
    special = np.array([0.0, -0.0, 65504, 65519.99, 65520, 70000, np.inf, -np.inf, 2**-24, 2**-25,
                        2**-25 * 1.0001, 2**-14, -(2**-14) * 0.75], np.float32)
    x = np.concatenate([near, -near, rand, special])
    got = oracle.float_to_half(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    nanbits = oracle.float_to_half(np.array([np.nan], np.float32))
    assert np.isnan(nanbits.view(np.float16)[0])


# ---------------------------------------------------------------------------
# attention against dense references
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["tiny", "mixed_small", "bs16_small", "mha"])
def test_paged_matches_float64_dense(oracle, name):
    if name == "tiny":
        w = wl.tiny()
    elif name == "mixed_small":
        w = wl.make_workload("ms", 6, 12, 2, 128, 64, 64, [1, 63, 64, 65, 300, 700], seed=11, events=40)
    elif name == "bs16_small":
        w = wl.make_workload("b16", 5, 12, 2, 128, 16, 128, [17, 2, 160, 31, 250], seed=12, events=60)
    else:
        w = wl.make_workload("mha", 3, 4, 4, 64, 16, 64, [9, 40, 100], seed=13, events=10)
    ld = w.layer(0)
    got, got16 = run_oracle(oracle, w, ld=ld)
    for b in range(w.B):
        k, v = wl.read_row(ld.k_pool, ld.v_pool, w.tables[b], int(w.seq_lens[b]), w.bs)
        ref = f64_dense(ld.q[b], k, v, w.scale)
        assert close(got[b], ref), (name, b, np.abs(got[b] - ref).max())
        assert np.array_equal(got16[b], got[b].astype(np.float16))


def test_paged_matches_torch_sdpa(oracle):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    w = wl.make_workload("sdpa", 4, 12, 2, 128, 64, 64, [5, 64, 129, 500], seed=21, events=30)
    ld = w.layer(0)
    got, _ = run_oracle(oracle, w, ld=ld)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        k, v = wl.read_row(ld.k_pool, ld.v_pool, w.tables[b], L, w.bs)
        qt = torch.from_numpy(ld.q[b].astype(np.float64))[:, None, :]            # [Hq][1][D]
        kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).contiguous()  # [Hkv][L][D]
        vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).contiguous()
        rep = w.Hq // w.Hkv
        kt = kt.repeat_interleave(rep, dim=0)
        vt = vt.repeat_interleave(rep, dim=0)
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=w.scale)[:, 0, :].numpy()
        assert close(got[b], ref), (b, np.abs(got[b] - ref).max())


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------


def _one_row(oracle, q, k_log, v_log, bs, scale, N=None, seed=0):
    """Run the oracle for one row whose logical K/V are given ([L][Hkv][D])."""
    L, Hkv, D = k_log.shape
    Hq = q.shape[0]
    nb = max(1, wl.blocks_for(L, bs))
    N = N or nb + 3
    rng = np.random.default_rng(seed)
    table = np.full((1, nb), -1, np.int32)
    table[0, : wl.blocks_for(L, bs)] = rng.permutation(N)[: wl.blocks_for(L, bs)]
    kp = wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))
    vp = wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))
    wl.write_row(kp, vp, table[0], k_log, v_log, bs)
    return oracle.paged_decode_attn(q[None], kp, vp, table, np.array([L], np.int32), bs, scale)


def test_single_token_returns_v0(oracle):
    rng = np.random.default_rng(1)
    q = wl.normal_f16(rng, (12, 128))
    k = wl.normal_f16(rng, (1, 2, 128))
    v = wl.normal_f16(rng, (1, 2, 128))
    o, o16 = _one_row(oracle, q, k, v, 64, 0.088)
    expect = np.repeat(v[0].astype(np.float32), 6, axis=0)
    assert np.array_equal(o[0], expect)
    assert np.array_equal(o16[0].view(np.uint16), np.repeat(v[0], 6, axis=0).view(np.uint16))


def test_constant_values_return_constant(oracle):
    rng = np.random.default_rng(2)
    L = 333
    q = wl.normal_f16(rng, (12, 128))
    k = wl.normal_f16(rng, (L, 2, 128))
    c = wl.normal_f16(rng, (1, 2, 128))
    v = np.repeat(c, L, axis=0)
    o, _ = _one_row(oracle, q, k, v, 16, 0.088)
    assert close(o[0], np.repeat(c[0].astype(np.float64), 6, axis=0), atol=1e-6, rtol=1e-5)


@pytest.mark.parametrize("mode", ["q_zero", "scale_zero"])
def test_uniform_weights_give_mean(oracle, mode):
    rng = np.random.default_rng(3)
    L = 200
    q = wl.normal_f16(rng, (12, 128))
    scale = 0.088
    if mode == "q_zero":
        q[:] = 0
    else:
        scale = 0.0
    k = wl.normal_f16(rng, (L, 2, 128))
    v = wl.normal_f16(rng, (L, 2, 128))
    o, _ = _one_row(oracle, q, k, v, 64, scale)
    mean = v.astype(np.float64).mean(axis=0)  # [Hkv][D]
    assert close(o[0], np.repeat(mean, 6, axis=0), atol=1e-6, rtol=1e-5)


def test_two_tokens_logistic(oracle):
    rng = np.random.default_rng(4)
    q = wl.normal_f16(rng, (2, 64))
    k = wl.normal_f16(rng, (2, 1, 64))
    v = wl.normal_f16(rng, (2, 1, 64))
    scale = 0.125
    o, _ = _one_row(oracle, q, k, v, 16, scale)
    for h in range(2):
        s0 = scale * float(q[h].astype(np.float64) @ k[0, 0].astype(np.float64))
        s1 = scale * float(q[h].astype(np.float64) @ k[1, 0].astype(np.float64))
        w0 = 1.0 / (1.0 + np.exp(s1 - s0))
        ref = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
        assert close(o[0, h], ref, atol=1e-6, rtol=1e-5)


def test_dominant_key_without_overflow(oracle):
    # Scores near 1e3: exp(score) overflows fp32, exp(score - max) does not.
    rng = np.random.default_rng(5)
    L, D = 50, 64
    k = wl.normal_f16(rng, (L, 1, D)) * np.float16(0.1)
    v = wl.normal_f16(rng, (L, 1, D))
    j = 37
    k[j, 0] = np.float16(1.0)
    q = np.full((1, D), 8.0, np.float16)
    scale = 2.0  # score_j = 2 * 8 * 64 = 1024; others are far below
    o, _ = _one_row(oracle, q, k, v, 16, scale)
    assert np.all(np.isfinite(o))
    assert close(o[0, 0], v[j, 0].astype(np.float64), atol=1e-6, rtol=0)


def test_all_scores_very_negative(oracle):
    # Every score near -1e3: exp(score) underflows to zero in fp32, while the
    # max-shifted weights stay a proper softmax.
    rng = np.random.default_rng(8)
    L, D = 40, 64
    k = (np.abs(wl.normal_f16(rng, (L, 1, D))) + np.float16(1.0)).astype(np.float16)
    v = wl.normal_f16(rng, (L, 1, D))
    q = np.full((1, D), -8.0, np.float16)
    o, _ = _one_row(oracle, q, k, v, 16, 1.0)
    ref = f64_dense(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and close(o[0], ref, atol=1e-5, rtol=1e-4)


def test_query_head_to_kv_head_mapping(oracle):
    # V of KV head g is the constant g + 1: query heads 0..5 read head 0,
    # 6..11 read head 1 (contiguous groups).
    rng = np.random.default_rng(6)
    L = 70
    q = wl.normal_f16(rng, (12, 128))
    k = wl.normal_f16(rng, (L, 2, 128))
    v = np.empty((L, 2, 128), np.float16)
    v[:, 0, :] = 1.0
    v[:, 1, :] = 2.0
    o, _ = _one_row(oracle, q, k, v, 16, 0.088)
    assert close(o[0, :6], np.ones((6, 128)), atol=1e-6, rtol=1e-6)
    assert close(o[0, 6:], 2 * np.ones((6, 128)), atol=1e-6, rtol=1e-6)


def test_zero_length_row_gives_zeros(oracle):
    w = wl.make_workload("z", 3, 12, 2, 128, 64, 16, [0, 5, 0], seed=7)
    o, o16 = run_oracle(oracle, w)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(o16[0].view(np.uint16) == 0)


# ---------------------------------------------------------------------------
# bit-exact invariances
# ---------------------------------------------------------------------------


def test_block_relabelling_invariance(oracle):
    w = wl.make_workload("perm", 5, 12, 2, 128, 64, 48, [3, 64, 100, 640, 1000], seed=31, events=20)
    ld = w.layer(0)
    base, _ = run_oracle(oracle, w, ld=ld)
    pi = np.random.default_rng(99).permutation(w.N)
    kp = np.empty_like(ld.k_pool)
    vp = np.empty_like(ld.v_pool)
    kp[pi] = ld.k_pool
    vp[pi] = ld.v_pool
    t = np.where(w.tables >= 0, pi[np.maximum(w.tables, 0)], -1).astype(np.int32)
    got, _ = oracle.paged_decode_attn(ld.q, kp, vp, t, w.seq_lens, w.bs, w.scale)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


def _logical(oracle, w, ld):
    out = []
    for b in range(w.B):
        out.append(wl.read_row(ld.k_pool, ld.v_pool, w.tables[b], int(w.seq_lens[b]), w.bs))
    return out


def _repack(rows, q, bs, N, seed, events):
    """Write the same logical rows into a pool built from another history."""
    lens = np.array([r[0].shape[0] for r in rows], np.int32)
    rng = np.random.default_rng(seed)
    pool = wl.BlockPool(N, rng.permutation(N))
    wl.churn(pool, events, rng)
    W = max(1, max(wl.blocks_for(L, bs) for L in lens))
    tables = wl.build_tables(pool, lens, bs, W)
    Hkv, D = rows[0][0].shape[1], rows[0][0].shape[2]
    kp = wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))
    vp = wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))
    for b, (k, v) in enumerate(rows):
        wl.write_row(kp, vp, tables[b], k, v, bs)
    return kp, vp, tables, lens


@pytest.mark.parametrize("bs2", [16, 64, 1024])
def test_history_and_block_size_invariance(oracle, bs2):
    w = wl.make_workload("hist", 4, 12, 2, 128, 64, 64, [1, 65, 333, 1000], seed=41, events=30)
    ld = w.layer(0)
    base, _ = run_oracle(oracle, w, ld=ld)
    rows = _logical(oracle, w, ld)
    N = 256 if bs2 < 1024 else 12
    kp, vp, t, lens = _repack(rows, ld.q, bs2, N, seed=77, events=150 if bs2 < 1024 else 4)
    assert oracle.validate(t, lens, bs2, N) == 0
    got, _ = oracle.paged_decode_attn(ld.q, kp, vp, t, lens, bs2, w.scale)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


def test_batch_position_and_dense_special_case(oracle):
    w = wl.make_workload("pos", 4, 12, 2, 128, 16, 128, [10, 200, 77, 300], seed=51, events=25)
    ld = w.layer(0)
    base, _ = run_oracle(oracle, w, ld=ld)
    rows = _logical(oracle, w, ld)
    order = [2, 0, 3, 1]
    kp, vp, t, lens = _repack([rows[i] for i in order], ld.q[order], 16, 128, seed=5, events=9)
    got, _ = oracle.paged_decode_attn(np.ascontiguousarray(ld.q[order]), kp, vp, t, lens, 16, w.scale)
    assert np.array_equal(got.view(np.uint32), base[order].view(np.uint32))
    for b in range(w.B):
        k, v = rows[b]
        dense = oracle.dense_attn(ld.q[b], k, v, w.scale)
        assert np.array_equal(dense.view(np.uint32), base[b].view(np.uint32))


def test_rows_sharing_blocks_agree(oracle):
    w = wl.full_step(layers=1, N=2048)
    ld = w.layer(0)
    sh = np.flatnonzero(w.sharers)
    assert len(sh) == 16
    assert all(np.array_equal(w.tables[b, :10], w.shared_blocks) for b in sh)
    # Give two sharers the same length, table and query: identical outputs.
    a, b2 = int(sh[0]), int(sh[1])
    lens = w.seq_lens.copy()
    tables = w.tables.copy()
    q = ld.q.copy()
    lens[b2] = lens[a]
    tables[b2] = tables[a]
    q[b2] = q[a]
    o, _ = oracle.paged_decode_attn(q, ld.k_pool, ld.v_pool, tables, lens, w.bs, w.scale)
    assert np.array_equal(o[a].view(np.uint32), o[b2].view(np.uint32))


# ---------------------------------------------------------------------------
# kv_append and gather
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("cfg", ["tiny", "high_occupancy_small"])
def test_kv_append_matches_numpy_scatter(oracle, cfg):
    if cfg == "tiny":
        w = wl.tiny()
    else:
        w = wl.make_workload("ho", 20, 12, 2, 128, 16, 512, np.arange(1, 41, 2), seed=61, events=100, W=8)
    ld = w.layer(0)
    assert oracle.validate(w.tables, w.seq_lens, w.bs, w.N) == 0
    kp, vp = ld.k_pool.copy(), ld.v_pool.copy()
    rc = oracle.kv_append(ld.k_new, ld.v_new, kp, vp, w.tables, w.seq_lens, w.bs)
    assert rc == 0
    ek, ev = ld.k_pool.copy(), ld.v_pool.copy()
    for b in range(w.B):
        pos = int(w.seq_lens[b]) - 1
        blk = w.tables[b, pos // w.bs]
        slot = pos % w.bs
        ek[blk, :, :, slot, :] = ld.k_new[b].reshape(w.Hkv, w.D // 8, 8)
        ev[blk, :, :, slot] = ld.v_new[b]
    assert np.array_equal(kp.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(vp.view(np.uint16), ev.view(np.uint16))


def test_kv_append_then_attention_sees_new_token(oracle):
    # After the append, position L-1 of each row holds k_new / v_new.
    w = wl.tiny()
    ld = w.layer(0)
    kp, vp = ld.k_pool.copy(), ld.v_pool.copy()
    oracle.kv_append(ld.k_new, ld.v_new, kp, vp, w.tables, w.seq_lens, w.bs)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        k, v = wl.read_row(kp, vp, w.tables[b], L, w.bs)
        assert np.array_equal(k[L - 1].view(np.uint16), ld.k_new[b].view(np.uint16))
        assert np.array_equal(v[L - 1].view(np.uint16), ld.v_new[b].view(np.uint16))


@pytest.mark.parametrize("shape", [(2, 128, 64), (1, 64, 16)])
def test_kv_copy_blocks_matches_numpy(oracle, shape):
    # Copy-on-write clones whole blocks: block dst[i] becomes block src[i]
    # (K and V, every head and slot) and no other byte moves. Pinned against
    # numpy's fancy-index assignment on disjoint pairs.
    Hkv, D, bs = shape
    N = 40
    rng = np.random.default_rng(81)
    kp = wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))
    vp = wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))
    perm = rng.permutation(N)
    src, dst = perm[:9].astype(np.int32), perm[9:18].astype(np.int32)
    k2, v2 = kp.copy(), vp.copy()
    assert oracle.kv_copy_blocks(k2, v2, src, dst) == 0
    ek, ev = kp.copy(), vp.copy()
    ek[dst] = kp[src]
    ev[dst] = vp[src]
    assert np.array_equal(k2.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(v2.view(np.uint16), ev.view(np.uint16))
    # a pair naming a block outside the pool is skipped and reported
    k3, v3 = kp.copy(), vp.copy()
    assert oracle.kv_copy_blocks(k3, v3, np.array([N, 1], np.int32), np.array([2, 3], np.int32)) == -2
    ek, ev = kp.copy(), vp.copy()
    ek[3], ev[3] = kp[1], vp[1]
    assert np.array_equal(k3.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(v3.view(np.uint16), ev.view(np.uint16))


def test_kv_scatter_prefill_drops_the_left_padding(oracle):
    # A left-padded prefill group's K/V: row b's prompt occupies the last P_b
    # of the S positions. After the scatter, reading row b back through its
    # table gives exactly those P_b positions, in order (numpy slicing and the
    # workloads' own block reader, not the oracle), and no other slot moved.
    rng = np.random.default_rng(83)
    B, Hkv, D, bs, S = 5, 2, 64, 16, 70
    lens = [70, 1, 16, 33, 0]
    N = sum(wl.blocks_for(L, bs) for L in lens) + 6
    w = wl.make_workload("pf", B, 4, Hkv, D, bs, N, lens, seed=84, events=12)
    ld = w.layer(0)
    k_src = wl.normal_f16(rng, (B, Hkv, S, D))
    v_src = wl.normal_f16(rng, (B, Hkv, S, D))
    kp, vp = ld.k_pool.copy(), ld.v_pool.copy()
    assert oracle.kv_scatter_prefill(k_src, v_src, kp, vp, w.tables, w.seq_lens, bs) == 0
    touched = np.zeros((N, bs), bool)
    for b, P in enumerate(lens):
        k, v = wl.read_row(kp, vp, w.tables[b], P, bs)  # [P][Hkv][D]
        assert np.array_equal(k.view(np.uint16), k_src[b, :, S - P:, :].transpose(1, 0, 2).view(np.uint16))
        assert np.array_equal(v.view(np.uint16), v_src[b, :, S - P:, :].transpose(1, 0, 2).view(np.uint16))
        for t in range(P):
            touched[w.tables[b, t // bs], t % bs] = True
    kd = np.broadcast_to(~touched[:, None, None, :, None], kp.shape)
    vd = np.broadcast_to(~touched[:, None, None, :], vp.shape)
    assert np.array_equal(kp.view(np.uint16)[kd], ld.k_pool.view(np.uint16)[kd])
    assert np.array_equal(vp.view(np.uint16)[vd], ld.v_pool.view(np.uint16)[vd])
    # a prompt wider than the group is refused
    bad = np.array(lens, np.int32)
    bad[1] = S + 1
    assert oracle.kv_scatter_prefill(k_src, v_src, ld.k_pool.copy(), ld.v_pool.copy(), w.tables, bad, bs) == -2


def test_gather_matches_numpy(oracle):
    w = wl.make_workload("g", 5, 12, 2, 128, 16, 128, [0, 1, 16, 17, 300], seed=71, events=40)
    ld = w.layer(0)
    ko, vo = oracle.gather_kv(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.Hkv, w.D)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        k, v = wl.read_row(ld.k_pool, ld.v_pool, w.tables[b], L, w.bs)
        assert np.array_equal(ko[b, :, :L].view(np.uint16), k.transpose(1, 0, 2).view(np.uint16))
        assert np.array_equal(vo[b, :, :L].view(np.uint16), v.transpose(1, 0, 2).view(np.uint16))
        assert np.all(ko[b, :, L:].view(np.uint16) == 0)


def test_validate_flags(oracle):
    w = wl.tiny()
    t = w.tables.copy()
    assert oracle.validate(t, w.seq_lens, w.bs, w.N) == 0
    bad = t.copy()
    bad[3, 0] = w.N
    assert oracle.validate(bad, w.seq_lens, w.bs, w.N) & 1
    lens = w.seq_lens.copy()
    lens[0] = w.W * w.bs + 1
    assert oracle.validate(t, lens, w.bs, w.N) & 2
    dup = t.copy()
    lens2 = w.seq_lens.copy()
    dup[1, 0] = dup[0, 0]
    lens2[1] = lens2[0]  # both append into slot 4 of the same block
    f = oracle.validate(dup, lens2, w.bs, w.N)
    assert f & 4 and f & 8
    assert oracle.validate(dup, lens2, w.bs, w.N, check_append=False) & 12 == 0
    twice = t.copy()
    twice[3, 1] = twice[3, 0]
    assert oracle.validate(twice, w.seq_lens, w.bs, w.N) & 16


# ---------------------------------------------------------------------------
# FP8 (E4M3) pools
# ---------------------------------------------------------------------------


def torch_fp8_decode(codes):
    import torch

    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def torch_fp8_encode(x):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_fp8_to_float_all_codes(oracle):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_to_float(codes)
    ref = torch_fp8_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # signed zeros included
    # closed forms of the format: bias 7, 3 mantissa bits, subnormals below 2^-6
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x39] == 1.125 and got[0x40] == 2.0 and got[0x30] == 0.5
    finite = got[:0x7F]
    assert np.all(np.diff(finite) > 0)  # magnitudes increase with the code


def test_float_to_fp8_matches_torch_in_range(oracle):
    rng = np.random.default_rng(80)
    mag = np.exp2(rng.uniform(-12, np.log2(447.9), size=20000)).astype(np.float32)
    x = np.where(rng.integers(0, 2, size=mag.size) == 1, -mag, mag).astype(np.float32)
    vals = oracle.fp8_to_float(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact ties between neighbouring codes
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11])])
    assert np.all(np.abs(x) < 448)
    got = oracle.float_to_fp8(x)
    ref = torch_fp8_encode(x)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]
    finite = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    assert np.array_equal(oracle.float_to_fp8(oracle.fp8_to_float(finite)), finite)
    # ties go to the even mantissa: 1.0625 -> 1.0 (0x38), 1.1875 -> 1.25 (0x3A)
    assert list(oracle.float_to_fp8(np.float32([1.0625, 1.1875]))) == [0x38, 0x3A]


def test_float_to_fp8_saturates(oracle):
    x = np.float32([448.0, 460.0, 464.0, 500.0, 1e6, np.inf, -500.0, -np.inf, np.nan])
    assert list(oracle.float_to_fp8(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]


def test_fp8_quantization_error_bound(oracle):
    # code value c of x / s: |c*s - x| <= 2^-4 |x| (half a step of a 3-bit
    # mantissa) in the normal range, <= 2^-10 s (half the subnormal step)
    # below it, plus the fp32 rounding of the quotient
    rng = np.random.default_rng(81)
    for s in (1.0, 0.0371, 2.5, 2.0 ** -6):
        x = (rng.standard_normal(50000) * rng.choice([1e-3, 0.1, 1.0, 50.0], size=50000)).astype(np.float16)
        x = x[np.abs(x.astype(np.float64)) <= 448 * s]
        c = oracle.quantize_fp8(x, s)
        back = oracle.fp8_to_float(c).astype(np.float64) * s
        xv = x.astype(np.float64)
        err = np.abs(back - xv)
        assert np.all(err <= 2.0 ** -4 * np.abs(xv) + 2.0 ** -10 * s + 2.0 ** -22 * np.abs(xv)), err.max()
        assert np.array_equal(c, torch_fp8_encode(x.astype(np.float32) / np.float32(s)))


def fp8_pool_case(seed, B=5, Hq=4, Hkv=2, D=32, bs=16, lens=(1, 15, 16, 40, 77)):
    rng = np.random.default_rng(seed)
    N = sum(wl.blocks_for(L, bs) for L in lens) + 4
    w = wl.make_workload("fp8", B, Hq, Hkv, D, bs, N, list(lens), seed=seed, events=10)
    q = wl.normal_f16(rng, (B, Hq, D))
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs))
    return w, q, kp, vp


def test_kv_append_fp8_matches_numpy(oracle):
    w, q, kp, vp = fp8_pool_case(82)
    rng = np.random.default_rng(83)
    kn = (wl.normal_f16(rng, (w.B, w.Hkv, w.D)).astype(np.float32) * 3).astype(np.float16)
    vn = wl.normal_f16(rng, (w.B, w.Hkv, w.D))
    ks, vs = 0.0371, 0.5
    ek, ev = kp.copy(), vp.copy()
    for b in range(w.B):
        pos = int(w.seq_lens[b]) - 1
        blk = int(w.tables[b, pos // w.bs])
        for g in range(w.Hkv):
            kc = torch_fp8_encode(kn[b, g].astype(np.float32) / np.float32(ks))
            vc = torch_fp8_encode(vn[b, g].astype(np.float32) / np.float32(vs))
            for d in range(w.D):
                ek[blk, g, d // 16, pos % w.bs, d % 16] = kc[d]
                ev[blk, g, d, pos % w.bs] = vc[d]
    assert oracle.kv_append_fp8(kn, vn, kp, vp, w.tables, w.seq_lens, w.bs, ks, vs) == 0
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)


def fp8_logical(oracle, w, kp, vp, ks, vs):
    """Each row's logical [L][Hkv][D] float64 K and V from an FP8 pool (numpy reads, torch decoding)."""
    ks_, vs_ = [], []
    for b in range(w.B):
        k, v = wl.read_row(kp, vp, w.tables[b], int(w.seq_lens[b]), w.bs)
        ks_.append(torch_fp8_decode(k).astype(np.float64) * np.float32(ks))
        vs_.append(torch_fp8_decode(v).astype(np.float64) * np.float32(vs))
    return ks_, vs_


def test_fp8_attention_equals_fp16_oracle_on_exact_pools(oracle):
    # with power-of-two scales every dequantized value is exact in fp16, so
    # the fp8 attention must equal the fp16 oracle on the converted pools bit
    # for bit
    w, q, kp, vp = fp8_pool_case(84)
    ks, vs = 0.25, 2.0
    k16 = np.empty(wl.k_pool_shape(w.N, w.Hkv, w.D, w.bs), np.float16)
    v16 = (torch_fp8_decode(vp) * vs).astype(np.float16)
    kl = (torch_fp8_decode(kp) * ks)  # [N][Hkv][D/16][bs][16]
    kl = kl.transpose(0, 1, 3, 2, 4).reshape(w.N, w.Hkv, w.bs, w.D)  # [N][Hkv][bs][D]
    k16[:] = kl.reshape(w.N, w.Hkv, w.bs, w.D // 8, 8).transpose(0, 1, 3, 2, 4).astype(np.float16)
    assert np.array_equal(k16.astype(np.float32), kl.reshape(w.N, w.Hkv, w.bs, w.D // 8, 8).transpose(0, 1, 3, 2, 4))
    ref, _ = oracle.paged_decode_attn(q, k16, v16, w.tables, w.seq_lens, w.bs, w.scale)
    got, _ = oracle.paged_decode_attn_fp8(q, kp, vp, w.tables, w.seq_lens, w.bs, w.scale, ks, vs)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fp8_attention_matches_float64_dense(oracle):
    w, q, kp, vp = fp8_pool_case(85, lens=(3, 64, 100, 17, 250))
    ks, vs = 0.0371, 0.113
    got, _ = oracle.paged_decode_attn_fp8(q, kp, vp, w.tables, w.seq_lens, w.bs, w.scale, ks, vs)
    kl, vl = fp8_logical(oracle, w, kp, vp, ks, vs)
    for b in range(w.B):
        ref = f64_dense(q[b], kl[b], vl[b], w.scale)
        assert close(got[b], ref, atol=2e-6, rtol=1e-4), b


def test_kv_copy_blocks_fp8_matches_numpy(oracle):
    rng = np.random.default_rng(86)
    N, Hkv, D, bs = 24, 2, 32, 16
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs))
    perm = rng.permutation(N)
    src, dst = perm[:6].astype(np.int32), perm[6:12].astype(np.int32)
    ek, ev = kp.copy(), vp.copy()
    ek[dst] = kp[src]
    ev[dst] = vp[src]
    assert oracle.kv_copy_blocks_fp8(kp, vp, src, dst) == 0
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)
    bad = np.int32([N, 3]), np.int32([1, -1])
    assert oracle.kv_copy_blocks_fp8(kp, vp, *bad) == -2
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)  # both pairs skipped


def test_kv_scatter_prefill_fp8_reads_back_quantized(oracle):
    # every prompt token, read back through its row's table from the E4M3
    # pools, is the torch-quantized value of the group's unpadded position;
    # nothing else in the pools moves
    rng = np.random.default_rng(87)
    B, Hkv, D, bs = 4, 2, 32, 16
    prompts = [5, 16, 0, 37]
    S = max(prompts)
    N = sum(wl.blocks_for(P, bs) for P in prompts) + 3
    w = wl.make_workload("pf8", B, 4, Hkv, D, bs, N, prompts, seed=88, events=5)
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs))
    k_src = wl.normal_f16(rng, (B, Hkv, S, D))
    v_src = wl.normal_f16(rng, (B, Hkv, S, D))
    ks, vs = 0.05, 0.3
    k0, v0 = kp.copy(), vp.copy()
    assert oracle.kv_scatter_prefill_fp8(k_src, v_src, kp, vp, w.tables, w.seq_lens, bs, ks, vs) == 0
    live = wl.live_slot_mask(w.tables, w.seq_lens, bs, N)
    for b, P in enumerate(prompts):
        if P == 0:
            continue
        k, v = wl.read_row(kp, vp, w.tables[b], P, bs)  # [P][Hkv][D] codes
        ek = torch_fp8_encode(k_src[b, :, S - P:, :].transpose(1, 0, 2).astype(np.float32) / np.float32(ks))
        ev = torch_fp8_encode(v_src[b, :, S - P:, :].transpose(1, 0, 2).astype(np.float32) / np.float32(vs))
        assert np.array_equal(k, ek) and np.array_equal(v, ev), b
    kd = np.broadcast_to(~live[:, None, None, :, None], kp.shape)
    vd = np.broadcast_to(~live[:, None, None, :], vp.shape)
    assert np.array_equal(kp[kd], k0[kd]) and np.array_equal(vp[vd], v0[vd])

