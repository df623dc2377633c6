"""The C boundary without a GPU: the library loads, exports every declared symbol,
its host arithmetic matches the oracle, and bad arguments are refused before any
device work (all calls here pass NULL device pointers)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import cod as ocod
from token_drafting_amd import build, peagle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "peagle.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(peagle.lib_path()):
        build.build()
    return peagle.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(peagle_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
        assert name in peagle.SIGNATURES, name


def test_version_and_status_strings(lib):
    assert lib.peagle_version() >= 100
    for code in (0, -1, -2, -3, -4):
        assert lib.peagle_status_string(code).decode() != "unknown status"


@pytest.mark.parametrize("n,K,r,r_min", [(256, 4, 0.7, 0.2), (4096, 4, 0.7, 0.2), (32768, 4, 0.7, 0.2),
                                         (16384, 8, 0.7, 0.2), (10, 3, 0.5, 0.0), (4, 3, 0.1, 0.0),
                                         (1, 8, 0.7, 0.2), (100, 64, 0.95, 0.01), (7, 5, 1.0, 1.0)])
def test_cod_counts_match_oracle(lib, n, K, r, r_min):
    m, T = peagle.cod_counts(n, K, r, r_min)
    want = ocod.retained_counts(n, K, r, r_min)
    assert m == want and T == sum(want)


def test_cod_counts_random_against_oracle(lib):
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 200000))
        K = int(rng.integers(1, 12))
        r = float(rng.uniform(0.05, 1.0))
        r_min = float(rng.uniform(0.0, 1.0))
        m, _ = peagle.cod_counts(n, K, r, r_min)
        assert m == ocod.retained_counts(n, K, r, r_min), (n, K, r, r_min)


def _code(fn, *args):
    return getattr(peagle.lib(), fn)(*args)


def test_cod_argument_errors(lib):
    T = C.c_int64()
    for bad in [(0, 4, 0.7, 0.2), (10, 0, 0.7, 0.2), (10, 65, 0.7, 0.2), (10, 4, 0.0, 0.2),
                (10, 4, 1.5, 0.2), (10, 4, 0.7, -0.1), (10, 4, 0.7, 1.1), (10, 4, float("nan"), 0.2)]:
        assert _code("peagle_cod_counts", *bad, None, C.byref(T)) == peagle.ERR_ARG
    # valid counts, NULL device pointers -> refused
    assert _code("peagle_cod_select", 10, 4, 0.7, 0.2, 1, None, 1, None, None, None, None, None, 0,
                 None) == peagle.ERR_ARG
    assert _code("peagle_cod_select", 10, 4, 0.7, 0.2, 1, None, 0, None, None, None, None, None, 0,
                 None) == peagle.ERR_ARG
    # a workspace below peagle_cod_workspace_bytes is refused before any launch (the
    # pointers are never dereferenced on this path)
    fake = C.c_void_p(1 << 20)
    need = peagle.cod_workspace_bytes(5000, 4)
    assert need >= 64 * 8 + 5 * 4 * 4 and need % 256 == 0
    assert _code("peagle_cod_select", 5000, 4, 0.7, 0.2, 1, fake, 1, fake, fake, fake, fake, fake,
                 need - 1, None) == peagle.ERR_WORKSPACE
    assert _code("peagle_cod_select", 5000, 4, 0.7, 0.2, 1, fake, 1, fake, fake, fake, fake,
                 C.c_void_p((1 << 20) + 16), need, None) == peagle.ERR_ARG   # misaligned
    assert peagle.cod_workspace_bytes(0, 4) == 0 and peagle.cod_workspace_bytes(10, 65) == 0
    # the allocation-free variant refuses sizes past its static scratch on the host
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "peagle.h")).read()
    m = re.search(r"#define PEAGLE_COD_NOALLOC_SCRATCH_BYTES \(\(size_t\)1 << (\d+)\)", hdr)
    assert m and (1 << int(m.group(1))) == peagle.COD_NOALLOC_SCRATCH_BYTES
    big = 1 << 24
    assert peagle.cod_workspace_bytes(big, 64) > peagle.COD_NOALLOC_SCRATCH_BYTES
    assert _code("peagle_cod_select_noalloc", big, 64, 0.7, 0.2, 1, fake, 1, fake, fake, fake,
                 fake, None) == peagle.ERR_WORKSPACE
    assert _code("peagle_cod_select_noalloc", 10, 4, 0.7, 0.2, 1, None, 1, None, None, None,
                 None, None) == peagle.ERR_ARG


def test_fuse_argument_errors(lib):
    args = dict(n=8, K=2, T=12, aux_dim=16, vocab=10, ptd=9, H=8)

    def call(**kw):
        a = {**args, **kw}
        return _code("peagle_fuse_inputs", a["n"], a["K"], a["T"], None, None, a["aux_dim"], None,
                     None, None, None, a["vocab"], a["ptd"], a["H"], None, None, None)
    assert call() == peagle.ERR_ARG                 # valid shapes, NULL pointers
    assert call(ptd=10) == peagle.ERR_ARG           # ptd_token_id out of range
    assert call(ptd=-1) == peagle.ERR_ARG
    assert call(T=7) == peagle.ERR_ARG              # T < n
    assert call(T=17) == peagle.ERR_ARG             # T > K n
    assert call(aux_dim=12) == peagle.ERR_ARG       # not a multiple of 8
    assert call(H=12) == peagle.ERR_ARG


def test_attention_argument_errors(lib):
    base = dict(n=64, K=4, T=150, S=1, Hq=4, Hkv=1, D=64, scale=0.125, max_pos=66, ws=1 << 30)

    def call(**kw):
        a = {**base, **kw}
        return _code("peagle_draft_attn_fwd", a["n"], a["K"], a["T"], None, None, None, None, a["S"],
                     None, None, None, a["Hq"], a["Hkv"], a["D"], a["scale"], None, None,
                     a["max_pos"], None, None, None, a["ws"], None)
    assert call() == peagle.ERR_ARG                    # NULL pointers
    assert call(D=96) == peagle.ERR_UNSUPPORTED
    assert call(D=32) == peagle.ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=2) == peagle.ERR_UNSUPPORTED   # group of 3 does not divide 256
    assert call(Hq=1 << 19, Hkv=1 << 19) == peagle.ERR_WORKSPACE     # Hkv D = 2^25: shape taken
    assert call(Hq=1 << 20, Hkv=1 << 20) == peagle.ERR_UNSUPPORTED   # 2^26: past the tile limit
    assert call(Hq=1 << 19, Hkv=1 << 19, D=128) == peagle.ERR_UNSUPPORTED
    assert call(Hq=5, Hkv=2) == peagle.ERR_ARG
    assert call(max_pos=65) == peagle.ERR_ARG          # below n + K - 2
    assert call(ws=1024) == peagle.ERR_WORKSPACE
    assert call(scale=0.0) == peagle.ERR_ARG
    assert call(T=63) == peagle.ERR_ARG
    assert call(S=0) == peagle.ERR_ARG
    for fn in ("peagle_draft_attn_prepare", "peagle_draft_attn_core"):
        assert _code(fn, 64, 4, 150, None, None, None, None, 1, None, None, None, 4, 1, 96, 0.125,
                     None, None, 66, None, None, None, 1 << 30, None) == peagle.ERR_UNSUPPORTED


def test_rope_and_accept_argument_errors(lib):
    assert _code("peagle_rope_table", 63, 1e4, 10, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_rope_table", 64, -1.0, 10, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_rope_table", 64, 1e4, -1, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_rope_table", 64, 1e4, 10, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_accept_prefix", 4, 0, 100, None, None, None, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_accept_prefix", 4, 65, 100, None, None, None, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_accept_prefix", 4, 8, 0, None, None, None, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_accept_prefix", 4, 8, 100, None, None, None, None, None, None) == peagle.ERR_ARG
    assert _code("peagle_accept_prefix_d2t", 4, 8, 100, 200, None, None, None, None, None, None,
                 None) == peagle.ERR_ARG
    assert _code("peagle_accept_prefix_d2t", 4, 8, 0, 200, None, None, None, None, None, None,
                 None) == peagle.ERR_ARG
    # sampling verification: null pointers, K beyond 64, empty vocabulary, tau <= 0 or NaN
    fake = 1 << 20  # never dereferenced: every call below fails its host checks
    for args in ((4, 8, 100, None, None, None, None, None, 1.0, None, None),
                 (4, 65, 100, fake, fake, fake, fake, fake, 1.0, fake, fake),
                 (4, 8, 0, fake, fake, fake, fake, fake, 1.0, fake, fake),
                 (4, 8, 100, fake, fake, fake, fake, fake, 0.0, fake, fake),
                 (4, 8, 100, fake, fake, fake, fake, fake, -1.0, fake, fake),
                 (4, 8, 100, fake, fake, fake, fake, fake, float("nan"), fake, fake),
                 (-1, 8, 100, fake, fake, fake, fake, fake, 1.0, fake, fake)):
        assert _code("peagle_accept_sampled", *args, None) == peagle.ERR_ARG, args
    assert _code("peagle_accept_sampled", 0, 8, 100, None, None, None, None, None, 1.0, None,
                 None, None) == peagle.OK


def test_workspace_bytes(lib):
    # enough chunks for the whole chip: no key-range split, size grows with T
    a = peagle.attn_workspace_bytes(32768, 83001, 4, 1, 256)
    b = peagle.attn_workspace_bytes(32768, 90000, 4, 1, 256)
    assert 0 < a < b
    assert a % 256 == 0
    # 163 chunks: split in up to 4 segments, so three fp32 partial outputs of [T, Hq, D]
    c = peagle.attn_workspace_bytes(4096, 10375, 4, 1, 256)
    assert c % 256 == 0 and c >= 3 * 10375 * 4 * 256 * 4
    assert peagle.attn_workspace_bytes(0, 10, 4, 1, 64) == 0


def test_decode_argument_errors(lib):
    base = dict(B=3, K=4, total=100, max_ctx=60, vtb=1 << 30, Hq=4, Hkv=1, D=64, scale=0.125,
                max_pos=63, ws=1 << 30)

    def call(**kw):
        a = {**base, **kw}
        return _code("peagle_draft_decode_attn", a["B"], a["K"], None, a["total"], a["max_ctx"],
                     None, None, a["vtb"], None, None, None, a["Hq"], a["Hkv"], a["D"], a["scale"],
                     None, None, a["max_pos"], None, None, None, a["ws"], None)
    assert call() == peagle.ERR_ARG                       # NULL pointers
    assert call(D=96) == peagle.ERR_UNSUPPORTED
    assert call(K=33) == peagle.ERR_UNSUPPORTED
    assert call(K=0) == peagle.ERR_ARG
    assert call(B=0) == peagle.ERR_ARG
    assert call(B=65536) == peagle.ERR_ARG
    assert call(Hq=5, Hkv=2) == peagle.ERR_ARG
    assert call(max_ctx=101) == peagle.ERR_ARG            # above total_ctx
    assert call(max_pos=62) == peagle.ERR_ARG             # below max_ctx + K - 1
    assert call(scale=float("inf")) == peagle.ERR_ARG
    assert _code("peagle_decode_pack_v", 3, None, 100, 60, None, 1, 64, None, 1 << 30,
                 None) == peagle.ERR_ARG
    assert _code("peagle_decode_pack_v", 3, None, 100, 60, None, 1, 96, None, 1 << 30,
                 None) == peagle.ERR_UNSUPPORTED


def test_decode_sizes(lib):
    # V tiles: floor(total / 32) + B + 1 tiles of D x 32 bf16 per kv head
    assert peagle.decode_v_tiles_bytes(1000, 3, 2, 128) == (1000 // 32 + 3 + 1) * 2 * 128 * 32 * 2
    assert peagle.decode_v_tiles_bytes(0, 1, 1, 64) == 2 * 64 * 32 * 2
    assert peagle.decode_v_tiles_bytes(-1, 1, 1, 64) == 0
    a = peagle.decode_workspace_bytes(8, 4, 4, 1, 256, 8 * 32768, 32768)
    b = peagle.decode_workspace_bytes(64, 4, 4, 1, 256, 64 * 32768, 32768)
    assert 0 < a < b and a % 256 == 0
    assert peagle.decode_workspace_bytes(8, 33, 4, 1, 256, 1000, 100) == 0
    assert peagle.decode_workspace_bytes(8, 4, 4, 1, 256, 99, 100) == 0    # total < max


def test_decode_tile_bases_never_overlap():
    """Request b's V tiles start at floor(cu[b] / 32) + b: for any split of a cache into
    requests the ranges [start, start + ceil(L_b / 32)) are disjoint and below
    floor(total / 32) + B + 1 (host arithmetic of the layout, no GPU)."""
    rng = np.random.default_rng(5)
    for _ in range(2000):
        B = int(rng.integers(1, 12))
        lens = rng.integers(0, 200, B)
        cu = np.concatenate([[0], np.cumsum(lens)])
        total = int(cu[-1])
        ntiles = total // 32 + B + 1
        prev_end = 0
        for b in range(B):
            start = cu[b] // 32 + b
            end = start + (lens[b] + 31) // 32
            assert start >= prev_end and end <= ntiles
            if lens[b]:
                prev_end = end


def test_decode_range_split_covers_each_request_once():
    """The decode attention's work split, as host arithmetic (no GPU): request b takes
    max(1, ceil(L_b / 32)) slots from rstart[b]; range r of P takes slots [r len,
    (r + 1) len) with len = ceil(S / P), starting at the request that holds slot r len;
    each (range, request) pair it meets writes partial slot r + b. Checked: every slot of
    every request is taken by exactly one range, partial slots are unique and below
    P + B, and a request's partials are exactly slots r + b for r = s_b / len ..
    (e_b - 1) / len, the list the merge reads."""
    rng = np.random.default_rng(11)
    for trial in range(1500):
        B = int(rng.integers(1, 300))
        lens = rng.integers(0, int(rng.choice([2, 40, 1000, 40000])), B)
        if trial % 9 == 0:
            lens[:] = 0
        nt = np.maximum(1, (lens + 31) // 32)
        rstart = np.concatenate([[0], np.cumsum(nt)]).astype(np.int64)
        S = int(rstart[-1])
        assert S <= int(lens.sum()) // 32 + B          # the bound the workspace is sized by
        P = int(rng.integers(1, 1100))
        ln = (S + P - 1) // P
        rfirst = {}
        for b in range(B):                              # each request writes its ranges
            for r in range((int(rstart[b]) + ln - 1) // ln, (int(rstart[b + 1]) + ln - 1) // ln):
                assert r not in rfirst
                rfirst[r] = b
        taken = {b: [] for b in range(B)}
        slots = set()
        for r in range(P):
            t0 = r * ln
            if t0 >= S:
                continue
            t1 = min(t0 + ln, S)
            b = rfirst[r]
            while b < B and rstart[b] < t1:
                j0, j1 = max(t0, rstart[b]) - rstart[b], min(t1, rstart[b + 1]) - rstart[b]
                assert j0 < j1
                slot = r + b
                assert slot not in slots and slot < P + B
                slots.add(slot)
                taken[b].append((j0, j1, slot))
                b += 1
        for b in range(B):
            segs = sorted(taken[b])
            assert [j for s in segs for j in s[:2]][0] == 0
            assert all(segs[i][1] == segs[i + 1][0] for i in range(len(segs) - 1))
            assert segs[-1][1] == nt[b]
            r0, r1 = int(rstart[b]) // ln, (int(rstart[b + 1]) - 1) // ln
            assert sorted(s[2] for s in segs) == [r + b for r in range(r0, r1 + 1)]


def test_layer1_argument_errors(lib):
    base = dict(n=64, K=4, T=150, H=640, eps=1e-6, Hq=4, Hkv=1, D=256, ws=1 << 30)

    def call(**kw):
        a = {**base, **kw}
        return _code("peagle_layer1_qkv", a["n"], a["K"], a["T"], None, None, a["H"], None, None,
                     a["eps"], None, a["Hq"], a["Hkv"], a["D"], None, None, None, None, a["ws"],
                     None)
    assert call() == peagle.ERR_ARG                        # NULL pointers
    assert call(H=48) == peagle.ERR_UNSUPPORTED            # not a multiple of 32
    assert call(D=12) == peagle.ERR_UNSUPPORTED
    assert call(T=63) == peagle.ERR_ARG
    assert call(T=257) == peagle.ERR_ARG                   # T > K n
    assert call(Hq=5, Hkv=2) == peagle.ERR_ARG
    assert call(eps=0.0) == peagle.ERR_ARG
    # rows 0 .. n of [emb, hidden] normalised, bf16: (n + 1) x 2H x 2 bytes, 256-aligned
    assert peagle.layer1_qkv_workspace_bytes(64, 150, 640) == ((65 * 1280 * 2 + 255) // 256) * 256
    assert peagle.layer1_qkv_workspace_bytes(64, 64, 640) == 64 * 1280 * 2
    assert peagle.layer1_qkv_workspace_bytes(0, 10, 640) == 0


def test_attn_bwd_argument_errors(lib):
    """Host checks of peagle_draft_attn_bwd; fake aligned addresses are never dereferenced
    because every call below fails before anything is enqueued."""
    f = 1 << 20
    n, K, T, Hq, Hkv, D = 256, 4, 648, 4, 1, 64
    need = peagle.lib().peagle_draft_attn_bwd_workspace_bytes(n, T, Hq, Hkv, D)
    fwd = peagle.attn_workspace_bytes(n, T, Hq, Hkv, D)
    assert need > fwd > 0
    assert peagle.lib().peagle_draft_attn_bwd_workspace_bytes(n, T, 3, 2, D) == 0

    def call(D=D, lse=f, dout=f, dq=f, ws_bytes=need, scale=0.125):
        return _code("peagle_draft_attn_bwd", n, K, T, f, f, f, f, 1, f, f, f, Hq, Hkv, D, scale,
                     f, f, n + K, f, lse, dout, dq, f, f, f, ws_bytes, None)
    assert call(D=96) == peagle.ERR_UNSUPPORTED
    assert call(lse=None) == peagle.ERR_ARG
    assert call(dout=None) == peagle.ERR_ARG
    assert call(dq=f + 4) == peagle.ERR_ARG          # misaligned
    assert call(scale=0.0) == peagle.ERR_ARG
    assert call(ws_bytes=fwd) == peagle.ERR_WORKSPACE


def test_decode_loop_argument_errors(lib):
    """Host checks of the grow-in-place decode entries (fake aligned addresses, never
    dereferenced: every call fails before anything is enqueued)."""
    f = 1 << 20
    B, Hkv, D, total, maxc = 4, 1, 64, 400, 120
    big = 1 << 30
    # append: lens_out must differ from lens_in; n_add within [0, max_new]; capacity bounds
    def app(lens_in=f, lens_out=f + 256, n_add=1, max_new=5, max_pos=maxc, D=D, vt_bytes=big):
        return _code("peagle_decode_append", B, f, lens_in, f, n_add, max_new, f, f, Hkv, D, f, f,
                     max_pos, total, maxc, f, f, vt_bytes, lens_out, None)
    assert app(lens_out=f) == peagle.ERR_ARG
    assert app(n_add=6) == peagle.ERR_ARG
    assert app(n_add=-1) == peagle.ERR_ARG
    assert app(max_new=0) == peagle.ERR_ARG
    assert app(max_pos=maxc - 2) == peagle.ERR_ARG
    assert app(D=96) == peagle.ERR_UNSUPPORTED
    assert app(vt_bytes=16) == peagle.ERR_WORKSPACE
    # decode attention over lengths: lens required
    assert _code("peagle_draft_decode_attn_lens", B, 4, f, None, total, maxc, f, f, big, f, f, f,
                 4, Hkv, D, 0.125, f, f, maxc + 3, f, f, f, big, None) == peagle.ERR_ARG
    assert _code("peagle_decode_pack_v_lens", B, f, None, total, maxc, f, Hkv, D, f, big,
                 None) == peagle.ERR_ARG
