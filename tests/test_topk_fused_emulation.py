"""Host emulation of the top-k selection fused into the single-launch decode
kernel (csrc/decode.hip), with every lane, LDS and workspace index checked.

Every streaming wave of the grid (4 per workgroup, NV v-blocks of 16 rows
each) leaves the largest key of its rows in the workspace, tkw[wave], and its
logits in memory.  The last workgroup (256 threads) then
  1. loads the wave keys, thread t keys t, t + 256, ... (Q of them);
  2. in each of its 4 waves takes the K-th largest of the 64 threads' maxima
     by ranking each against the other 63; the largest of the four is the
     bound B;
  3. gathers the wave keys at or above B into an LDS array of capacity
     4 K Q and ranks them: the K largest name the source waves, the K-th of
     them is T (0 with fewer than K nonzero wave keys);
  4. reads the logits of the source waves, rows gws NV 16 + i (i < NV 16),
     thread t items t, t + 256, ... < SI 256, and gathers the keys at or
     above T into an LDS array of capacity K NV 16;
  5. ranks those: the K largest in order.
Ranking n keys: with n <= 64 lane c of each wave compares key c with the
keys j = wave mod 4 and the four partial ranks are added; with n <= 256
each thread ranks one key against all n; beyond that K rounds of a 64-lane
maximum below the previous winner.
Both arrays keep 8 slots past their capacity, which the ranking's eight-key
reads may touch.  The emulation asserts that neither array overflows its capacity (step 3: at
most K threads per wave hold a maximum at or above that wave's bound, each
with at most Q keys; step 4: at most K source waves of NV 16 rows) and that
the result equals the oracle's top-k of the same logits (larger value first,
equal values by lower index).
"""
import numpy as np
import pytest

from oracle.select import top_k

WAVES, LANES, NT, VB = 4, 64, 256, 16
KMAX = 16
SPARE = 8        # slots past each LDS array's capacity


def orderable(y):
    b = np.asarray(y, dtype=np.float32).astype(np.float32) + np.float32(0.0)
    u = b.view(np.uint32).astype(np.uint64)
    return np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)


def keys_of(y, rows):
    return (orderable(y) << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - rows.astype(np.uint64))


def select_k(s, n, K):
    """The K largest of s[0, n) (unique nonzero keys), zeros past n."""
    out = np.zeros(K, dtype=np.uint64)
    if n <= LANES:
        # lane c of wave w ranks key c against keys j = w mod 4 (j < n, read
        # through a clamped index); the partial ranks add up in 64 counters
        s_rank = np.zeros(LANES, dtype=np.int64)
        for w in range(WAVES):
            for lane in range(LANES):
                if lane < n:
                    c = s[lane]
                    part = 0
                    for j0 in range(0, 64, 16):
                        if j0 >= n:
                            break
                        for i in range(4):
                            j = j0 + 4 * i + w
                            q = s[j if j < n else n - 1]
                            part += int(j < n and q > c)
                    s_rank[lane] += part
        for t in range(NT):
            if t < n:
                assert t < LANES
                if s_rank[t] < K:
                    out[s_rank[t]] = s[t]
        return out
    if n <= NT:
        for t in range(NT):
            if t < n:
                c = s[t]
                rank = 0
                for j in range(0, n, 8):              # eight keys read per step
                    assert j + 7 < s.size             # the spare slots past n are readable
                    rank += sum(int(j + i < n and s[j + i] > c) for i in range(8))
                if rank < K:
                    out[rank] = c
    else:
        win = None
        for r in range(K):
            best = np.uint64(0)
            for lane in range(LANES):
                for q in range(lane, n, LANES):
                    k = s[q]
                    if (win is None or k < win) and k > best:
                        best = k
            out[r] = best
            win = best
    return out


def resolve(y, tkw, NV, K, QMAX=12):
    """tkw: the wave keys of one hidden state (4 nwg of them); y: its logits."""
    V = y.size
    nw = tkw.size
    Q = (nw // WAVES + 63) // 64
    assert 1 <= Q <= QMAX
    cap1, cap2 = WAVES * K * Q, K * NV * VB
    si = (KMAX * NV * VB + NT - 1) // NT
    # 1.
    kk = np.zeros((NT, QMAX), dtype=np.uint64)
    for t in range(NT):
        for i in range(QMAX):
            g = t + NT * i
            if i < Q and g < nw:
                kk[t, i] = tkw[g]
    tmax = kk.max(axis=1)
    # 2.
    bnd = np.zeros(WAVES, dtype=np.uint64)
    for w in range(WAVES):
        sl = tmax[w * LANES:(w + 1) * LANES]
        for lane in range(LANES):
            rank = int(np.sum(sl > sl[lane]))
            if sl[lane] != 0 and rank == K - 1:
                bnd[w] = sl[lane]
    B = bnd.max()
    # 3.
    s_wk = np.zeros(cap1 + SPARE, dtype=np.uint64)
    n1 = 0
    for t in range(NT):
        for i in range(QMAX):
            if kk[t, i] != 0 and kk[t, i] >= B:
                assert n1 < cap1, f"wave-key overflow: {n1} >= {cap1}"
                s_wk[n1] = kk[t, i]
                n1 += 1
    win = select_k(s_wk, n1, K)
    T = win[K - 1]
    # 4.
    s_cand = np.zeros(cap2 + SPARE, dtype=np.uint64)
    n2 = 0
    for t in range(NT):
        for i in range(si):
            it = t + NT * i
            src = it // (NV * VB)
            wk = win[src] if src < K else np.uint64(0)
            row = V
            if wk != 0:
                gws = (0xFFFFFFFF - int(wk & np.uint64(0xFFFFFFFF))) // VB // NV
                row = gws * NV * VB + (it - src * NV * VB)
            if row < V:
                key = keys_of(y[row:row + 1], np.array([row]))[0]
                if key >= T:
                    assert n2 < cap2, f"candidate overflow: {n2} >= {cap2}"
                    s_cand[n2] = key
                    n2 += 1
    return select_k(s_cand, n2, K), n1, n2


def run_head(y, NV, K):
    """y: the logits of one hidden state.  Emulates the grid: 4 waves x NV
    v-blocks of 16 rows per workgroup, each wave's largest key."""
    V = y.size
    nvb = (V + VB - 1) // VB
    nwg = (nvb + WAVES * NV - 1) // (WAVES * NV)
    tkw = np.zeros(nwg * WAVES, dtype=np.uint64)
    allkeys = keys_of(y, np.arange(V))
    for gw in range(nwg * WAVES):
        r0, r1 = gw * NV * VB, min((gw + 1) * NV * VB, V)
        tkw[gw] = allkeys[r0:r1].max() if r0 < V else 0
    return resolve(y, tkw, NV, K)


def decode_keys(keys):
    hi = (keys >> np.uint64(32)).astype(np.uint64)
    bits = np.where(hi & 0x80000000, hi & 0x7FFFFFFF, (~hi) & 0xFFFFFFFF).astype(np.uint32)
    idx = (np.uint64(0xFFFFFFFF) - (keys & np.uint64(0xFFFFFFFF))).astype(np.int64)
    return bits.view(np.float32), idx


def check(y, NV, K):
    keys, n1, n2 = run_head(y, NV, K)
    vals, idx = decode_keys(keys)
    rv, ri = top_k(y[None, :].astype(np.float64), K)
    assert np.array_equal(idx, ri[0]), f"indices {idx} vs {ri[0]}"
    assert np.array_equal(vals.astype(np.float64), rv[0]) or np.array_equal(vals + 0, rv[0] + 0)
    return n1, n2


@pytest.mark.parametrize("V,NV,K", [(1, 5, 1), (16, 5, 16), (17, 5, 3), (320, 5, 16), (321, 5, 16),
                                    (3001, 5, 16), (3001, 4, 7), (20000, 5, 16), (40000, 4, 16)])
def test_random_logits(V, NV, K):
    rng = np.random.default_rng(V + NV * 7 + K)
    y = rng.standard_normal(V).astype(np.float32)
    check(y, NV, K)


@pytest.mark.parametrize("kind", ["all_equal", "few_values", "sorted_up", "sorted_down", "neg_inf", "top_in_one_wg",
                                  "zeros_signed", "one_thread_holds_the_top"])
def test_adversarial_logits(kind):
    V, NV, K = 12000, 5, 16
    rng = np.random.default_rng(3)
    if kind == "all_equal":
        y = np.full(V, 1.5, np.float32)
    elif kind == "few_values":
        y = rng.integers(0, 3, V).astype(np.float32)
    elif kind == "sorted_up":
        y = np.arange(V, dtype=np.float32)
    elif kind == "sorted_down":
        y = -np.arange(V, dtype=np.float32)
    elif kind == "neg_inf":
        y = np.full(V, -np.inf, np.float32)
        y[rng.integers(0, V, 5)] = 1.0
    elif kind == "top_in_one_wg":
        y = rng.standard_normal(V).astype(np.float32)
        y[640:640 + 320] += 100.0          # one workgroup's rows hold every top key
    elif kind == "zeros_signed":
        y = np.where(rng.random(V) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    else:
        # the waves 0, 256, 512, ... hold the largest keys: one thread of the
        # last workgroup loads all of them
        V = 151936
        y = rng.standard_normal(V).astype(np.float32)
        for w in range(0, V // (NV * 16), 256):
            y[w * NV * 16 + 7] = 50.0 + w
    n1, n2 = check(y, NV, K)
    if kind == "all_equal":
        assert n2 > 256                    # the K-round branch of the final selection


def test_wave_key_ranking_beyond_one_per_thread():
    """More than 256 wave keys at or above the bound: the K-round branch of
    step 3.  Threads 0..K-1 of each wave of the last workgroup hold every
    large wave key (waves t + 256 i), thread t's all above thread t - 1's, so
    each wave's bound is thread 0's maximum and the keys of threads 1..K-1
    all reach it."""
    NV, K = 5, 16
    V = 768 * 4 * NV * 16                  # 3072 waves, 12 per thread
    rng = np.random.default_rng(5)
    y = rng.standard_normal(V).astype(np.float32)
    for w in range(4):
        for t in range(K):
            for i in range(12):
                g = w * 64 + t + 256 * i
                y[g * NV * 16 + 3] = 10.0 + 0.01 * t + 0.0001 * i
    n1, n2 = check(y, NV, K)
    assert n1 > 256


def test_candidates_are_few_at_the_qwen_shape():
    """At V = 151936 with NV = 5 (1900 waves, 8 wave keys per thread) random
    logits leave a handful of wave keys and candidate rows."""
    rng = np.random.default_rng(9)
    V, NV, K = 151936, 5, 16
    y = (rng.standard_normal(V) * 3).astype(np.float32)
    n1, n2 = check(y, NV, K)
    assert n1 < 64 and n2 < 64
