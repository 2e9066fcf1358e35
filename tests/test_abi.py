"""C-ABI checks that need no GPU: the library loads, exports every symbol
the header declares, validates host-checkable arguments without launching,
and its host helpers agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "graft.h")


@pytest.fixture(scope="module")
def native():
    from draft_tree_verification_parent_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        from draft_tree_verification_parent_amd import build
        build.build()
    return _native


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(graft_[a-z_]+)\s*\(", src)))


def test_header_declares_the_round(native):
    names = declared_functions()
    for n in ("graft_build_tree", "graft_tree_attention", "graft_lmhead_topk", "graft_accept",
              "graft_table_update_retrieve"):
        assert n in names


def test_library_exports_every_declared_symbol(native):
    lib = ctypes.CDLL(native.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in native.SIGNATURES, f"{n} missing from the Python binding"


def test_template_helper_matches_oracle(native):
    from draft_tree_verification_parent_amd import api
    from oracle.template import template
    for R in range(0, 65, 3):
        for k in (1, 2, 8, 10, 16):
            for dmax in (1, 3, 8):
                try:
                    tp, tr, _ = template(R, k, dmax)
                except ValueError:
                    with pytest.raises(native.GraftError):
                        api.graft_make_template(R, k, dmax)
                    continue
                gp, gr = api.graft_make_template(R, k, dmax)
                assert gp.tolist() == tp and gr.tolist() == tr


def test_stage_budgets(native):
    from draft_tree_verification_parent_amd import api
    # Graft page, section 2: 8/52, 24/36, 40/20 of 60 slots; no prune -> no retrieval
    assert api.graft_stage_budget(0) == (8, 52)
    assert api.graft_stage_budget(1) == (24, 36)
    assert api.graft_stage_budget(5) == (40, 20)
    assert api.graft_stage_budget(-1) == (60, 0)
    with pytest.raises(native.GraftError):
        api.graft_stage_budget(3)


def test_host_argument_validation_launches_nothing(native):
    L = native.lib()
    E, U = native.GRAFT_EINVAL, native.GRAFT_EUNSUPPORTED
    # lm-head / top-k
    assert L.graft_lmhead_topk(4, 256, 100, 17, 1, 1, 0, 1, 1, None, 1, 1 << 20, None) == E
    assert L.graft_lmhead_topk(4, 100, 100, 4, 1, 1, 0, 1, 1, None, 1, 1 << 20, None) == E
    assert L.graft_lmhead_topk(4, 256, 100, 0, 1, 1, 0, None, None, None, None, 0, None) == E
    assert L.graft_lmhead_topk(4, 256, 100, 4, None, None, 0, None, 1, None, 1, 1 << 20, None) == E
    assert L.graft_lmhead_topk(4, 256, 100, 200, None, None, 0, 1, 1, None, 1, 1 << 20, None) == E
    assert L.graft_lmhead_topk(0, 256, 100, 4, None, None, 0, 1, 1, None, None, 0, None) == 0
    # unknown weight layout; packed weights need H % 128 == 0
    assert L.graft_lmhead_topk(4, 256, 100, 4, 1, 1, 7, None, 1, None, 1, 1 << 20, None) == E
    assert L.graft_lmhead_topk(4, 192, 100, 4, 1, 1, 1, None, 1, None, 1, 1 << 20, None) == E
    assert L.graft_lmhead_topk(17000, 256, 100, 4, 1, 1, 1, None, 1, None, 1, 1 << 30, None) == E
    # vocabularies past 2^30 - 1 ids (the sort keys hold an id in 30 bits)
    assert L.graft_lmhead_topk(4, 0, 1 << 30, 4, None, None, 0, 1, 1, None, 1, 1 << 40, None) == E
    assert L.graft_lmhead_pack(100, 192, 1, 1, None) == E
    assert L.graft_lmhead_pack(100, 256, None, 1, None) == E
    # attention
    args = [1, 1, 1, 1, 1 << 20, 1, 100, 1, 10, 1, 1, 1, None, None, 0, None, None]
    assert L.graft_tree_attention(1, 8, 2, 96, 0.1, *args) == U
    assert L.graft_tree_attention(1, 8, 3, 128, 0.1, *args) == E
    assert L.graft_tree_attention(0, 8, 2, 128, 0.1, *args) == 0
    assert L.graft_tree_attention(8193, 8, 2, 128, 0.1, *args) == E  # above GRAFT_ATTN_MAX_BATCH
    assert b"B=8193" in L.graft_last_error()
    big = args[:6] + [1 << 30] + args[7:]  # 2^24 chunks per unit: 2^31 over 64 requests x 2 KV heads
    assert L.graft_tree_attention(64, 8, 2, 128, 0.1, *big) == E
    assert b"key chunks" in L.graft_last_error()
    # build tree
    bt = [1] * 24
    assert L.graft_build_tree(1, 7, *bt[:4], 10, *bt[:6], 100, 8, 0.0, *bt[:11]) == E
    assert L.graft_build_tree(1, 0, *bt[:4], 5000, *bt[:6], 100, 8, 0.0, *bt[:11]) == E
    assert L.graft_build_tree(0, 0, *bt[:4], 10, *bt[:6], 100, 8, 0.0, *bt[:11]) == 0
    # retrieval anchor
    assert L.graft_prune_anchor(1, *bt[:4], 0, *bt[:5], None, None) == E          # max_cand 0
    assert L.graft_prune_anchor(1, *bt[:4], 3000, *bt[:5], None, None) == E       # above GRAFT_MAX_CAND
    assert L.graft_prune_anchor(1, *bt[:4], 10, 1, None, 1, 1, None, None) == E   # NULL stage
    assert L.graft_prune_anchor(0, *bt[:4], 10, *bt[:5], None, None) == 0
    # table
    assert L.graft_table_update_retrieve(1, 100, 17, 0, None, None, 0, None, None, 0, None, None,
                                         None, None, 0, None, None, None) == E
    assert L.graft_table_update_retrieve(1, 100, 8, 1, 1, 1, 5000, 1, 1, 0, None, None, None,
                                         None, 0, None, None, None) == E
    assert L.graft_table_update_retrieve(1, 100, 8, 0, None, None, 0, None, None, 0, None, None,
                                         None, None, 0, None, None, None) == 0
    # batches above GRAFT_MAX_BATCH requests are rejected before any launch
    assert L.graft_table_update_retrieve(1, 100, 8, 1025, 1, 1, 10, 1, 1, 0, None, None, None,
                                         None, 0, None, None, None) == E
    assert L.graft_table_update_retrieve(1, 100, 8, 0, None, None, 0, None, None, 1025, 1, 1, 1,
                                         1, 10, 1, None, None) == E
    # accept
    assert L.graft_accept(1, 1, 1, 1, 1, 1, 0, 1, 1, 1, None, None) == E
    assert L.graft_accept(0, None, None, None, None, None, 8, None, None, None, None, None) == 0
    assert b"k=" in L.graft_last_error()


def test_workspace_sizes(native):
    L = native.lib()
    # packed weights: whole 128-row tiles, rows past V padded
    assert L.graft_lmhead_pack_bytes(100, 256) == 128 * 256 * 2
    assert L.graft_lmhead_pack_bytes(128256, 4096) == 128256 * 4096 * 2
    assert L.graft_lmhead_pack_bytes(129, 128) == 256 * 128 * 2
    assert L.graft_lmhead_pack_bytes(100, 192) == 0
    # one key list per (row, persistent workgroup) fits in the advertised workspace
    assert L.graft_lmhead_topk_workspace_bytes(60, 1000, 8) >= 60 * 256 * 8 * 8
    assert L.graft_lmhead_topk_workspace_bytes(60, 128256, 8) > 0
    assert L.graft_lmhead_topk_workspace_bytes(0, 128256, 8) == 0

    # the fused packed path keeps one k-key list per (row, vocabulary stream):
    # up to 64 rows one 64-row m tile, above that 128-row tiles; T m tiles
    # share the 256 persistent workgroups as 32 // T groups per XCD (T <= 32)
    # or 256 // T streams
    def streams(T):
        return (32 // T) * 8 if T <= 32 else 256 // T

    for M in (1, 60, 64, 65, 128, 129, 960, 2112):
        for k in (1, 8, 16):
            T = -(-M // 64) if M <= 64 else -(-M // 128)
            assert L.graft_lmhead_topk_workspace_bytes(M, 151936, k) >= M * streams(T) * k * 8, (M, k)
            # sampling: 64-row m tiles at every M, k keys plus one draw key per list
            T64 = -(-M // 64)
            assert L.graft_lmhead_sample_workspace_bytes(M, 151936, k) == M * streams(T64) * (k + 1) * 8, (M, k)
    # tree attention: two partial slots per workgroup (rows of one row group
    # by d + 2 floats) and B + 1 chunk offsets.  One row block of 16 rows per
    # wave while that keeps <= 2 row groups and < 256 units, else the fewest
    # groups; workgroups: a multiple of the units while there are <= 128 of
    # them (each taking >= 8 chunks), else one per eight chunks of the
    # largest batch the bounds allow, at most 256
    def attn_ws(B, Hq, Hkv, d, max_ctx, max_n):
        rows = max_n * (Hq // Hkv)
        rb = -(-rows // 16)
        rg1 = -(-rows // 128)
        rbw = 1 if (rg1 <= 2 and B * Hkv * rg1 < 256) else (1 if rb <= 8 else 2 if rb <= 16 else 3)
        per_wg = 128 * rbw
        groups = -(-rows // per_wg)
        nch = -(-(max_ctx + max_n) // 64)
        units = B * Hkv * groups
        if 2 * units <= 256:
            nwg = units * max(1, min(256 // units, nch // 8))
        else:
            nwg = -(-(units * nch) // 8)
        nwg = max(1, min(256, nwg))
        return 2 * nwg * min(rb * 16, per_wg) * (d + 2) * 4 + (B + 1) * 4

    for shape in ((1, 4, 2, 64, 100, 15), (1, 32, 8, 128, 32768, 63), (16, 32, 8, 128, 16384, 60),
                  (3, 64, 8, 128, 7000, 64), (41, 4, 2, 64, 3000, 64), (1, 4, 2, 64, 0, 1)):
        assert L.graft_tree_attention_workspace_bytes(*shape) == attn_ws(*shape), shape
    # worked by hand: 30 rows, 2 units of 2 chunks, one workgroup each
    assert attn_ws(1, 4, 2, 64, 100, 15) == 2 * 2 * 32 * 66 * 4 + 8
    # one request at 4K context, 240 rows: 2 row groups of 128 x 8 KV heads
    # = 16 units of 65 chunks, 8 workgroups each
    assert attn_ws(1, 32, 8, 128, 4096, 60) == 2 * 128 * 128 * 130 * 4 + 8
    assert L.graft_tree_attention_workspace_bytes(0, 32, 8, 128, 4096, 60) == 0


def test_kv_compact_host_validation_launches_nothing(native):
    L = native.lib()
    E, U = native.GRAFT_EINVAL, native.GRAFT_EUNSUPPORTED
    p = 1  # never dereferenced: every call below fails before a launch
    args = lambda B=1, Hkv=8, d=128, nl=1, ls=0, hs=128 * 100, ctx=2, nxt=3: (  # noqa: E731
        B, Hkv, d, nl, p, p, ls, p, hs, ctx, p, p, p, p, nxt, p, None, None)
    assert L.graft_kv_compact(*args(B=0)) == 0                  # nothing to do
    assert L.graft_kv_compact(*args(d=96)) == U                 # head dim not built
    assert L.graft_kv_compact(*args(hs=100)) == E               # stride not a multiple of d
    assert L.graft_kv_compact(*args(hs=0)) == E
    assert L.graft_kv_compact(*args(nl=0)) == E
    assert L.graft_kv_compact(*args(nl=2, ls=0)) == E           # layers without a layer stride
    assert L.graft_kv_compact(*args(Hkv=0)) == E
    assert L.graft_kv_compact(*args(B=-1)) == E
    assert L.graft_kv_compact(*args(nxt=2)) == E                # ctx_next aliases ctx_len
    a = list(args())
    a[14] = None                                                 # ctx_next NULL
    assert L.graft_kv_compact(*a) == E


def test_sampling_host_validation_launches_nothing(native):
    L = native.lib()
    E = native.GRAFT_EINVAL
    p = 1
    ok_ws = 1 << 30
    # graft_lmhead_topk_sample(M, H, V, k, T, hidden, w, gumbel, ids, vals, sample, ws, ws_bytes, stream)
    assert L.graft_lmhead_topk_sample(4, 256, 100, 4, 0.0, p, p, p, p, p, p, p, ok_ws, None) == E   # T = 0
    assert L.graft_lmhead_topk_sample(4, 256, 100, 4, float("nan"), p, p, p, p, p, p, p, ok_ws, None) == E
    assert L.graft_lmhead_topk_sample(4, 256, 100, 4, float("inf"), p, p, p, p, p, p, p, ok_ws, None) == E
    assert L.graft_lmhead_topk_sample(4, 200, 100, 4, 1.0, p, p, p, p, p, p, p, ok_ws, None) == E   # H % 128
    assert L.graft_lmhead_topk_sample(4, 256, 100, 0, 1.0, p, p, p, p, p, p, p, ok_ws, None) == E   # k = 0
    assert L.graft_lmhead_topk_sample(4, 256, 100, 17, 1.0, p, p, p, p, p, p, p, ok_ws, None) == E
    assert L.graft_lmhead_topk_sample(4, 256, 100, 4, 1.0, p, p, None, p, p, p, p, ok_ws, None) == E  # no noise
    assert L.graft_lmhead_topk_sample(4, 256, 100, 4, 1.0, p, p, p, p, p, p, p, 8, None) == E  # workspace
    assert L.graft_lmhead_topk_sample(0, 256, 100, 4, 1.0, None, None, None, None, None, None, None, 0, None) == 0
    assert L.graft_lmhead_sample_workspace_bytes(60, 1000, 8) > L.graft_lmhead_topk_workspace_bytes(60, 1000, 8) - 1
    assert L.graft_lmhead_sample_workspace_bytes(60, 1000, 0) == 0
    # graft_sample_rows(M, V, T, logits, gumbel, sample, stream)
    assert L.graft_sample_rows(4, 100, -1.0, p, p, p, None) == E
    assert L.graft_sample_rows(4, 0, 1.0, p, p, p, None) == E
    assert L.graft_sample_rows(4, 100, 1.0, p, None, p, None) == E
    assert L.graft_sample_rows(0, 100, 1.0, None, None, None, None) == 0
    # graft_accept_sampled(B, n, row_off, parent, token, sample, len, path, bonus, err, stream)
    assert L.graft_accept_sampled(-1, p, p, p, p, p, p, p, p, None, None) == E
    assert L.graft_accept_sampled(2, p, p, p, p, None, p, p, p, None, None) == E
    assert L.graft_accept_sampled(0, None, None, None, None, None, None, None, None, None, None) == 0


def test_tail_host_validation_launches_nothing(native):
    L = native.lib()
    E = native.GRAFT_EINVAL
    p = 1
    assert L.graft_tail_cut(4, 0, p, p, p, 0.5, p, p, None) == E      # empty block
    assert L.graft_tail_cut(4, 64, p, p, p, 0.5, p, p, None) == E     # tree of 65 nodes
    assert L.graft_tail_cut(4, 16, p, p, None, 0.5, p, p, None) == E
    assert L.graft_tail_cut(0, 16, None, None, None, 0.5, None, None, None) == 0
    # build_tree accepts the tail mode (and still rejects unknown ones)
    args = [p, p, p, p, 17, p, None, None, None, None, None, 1000, 8, 0.5, p, p, p, p, p, p, p, p, p, None, None]
    assert L.graft_build_tree(0, 2, *args) == 0
    assert L.graft_build_tree(1, 3, *args) == E


def test_treegraft_host_helper_and_validation(native):
    from oracle import treegraft as OTG
    L = native.lib()
    E = native.GRAFT_EINVAL
    for D, W, m in [(5, 10, 10), (3, 4, 7), (0, 1, 1), (6, 64, 2)]:
        for mask in (0, 1, 0b10101, (1 << D) - 1):
            assert L.graft_treegraft_node_count(D, W, m, mask) == OTG.node_count(D, W, m, mask)
    assert L.graft_treegraft_node_count(5, 65, 10, 0) == -1       # W > 64
    assert L.graft_treegraft_node_count(5, 64, 64, 0) == -1       # more than 2048 nodes
    p = 1
    assert L.graft_treegraft_build(2, 5, 0, 10, p, p, p, p, p, p, p, p, p, None, None) == E
    assert L.graft_treegraft_build(2, 5, 10, 10, p, p, None, p, p, p, p, p, p, None, None) == E
    assert L.graft_treegraft_build(0, 5, 10, 10, None, None, None, None, None, None, None, None, None, None, None) == 0


def test_misaligned_arrays_are_rejected_before_any_launch(native):
    """Arrays the kernels move 16 bytes at a time must be 16-byte aligned,
    K/V strides multiples of 8 elements: otherwise GRAFT_EINVAL, nothing
    launched (the addresses below are never dereferenced)."""
    L = native.lib()
    E = native.GRAFT_EINVAL
    A, X = 1 << 20, (1 << 20) + 8  # aligned / 8 bytes off
    ws = 1 << 40
    # lm-head: hidden, w, logits
    for h, w, lg in ((X, A, A), (A, X, A), (A, A, X)):
        assert L.graft_lmhead_topk(4, 256, 100, 4, h, w, 0, lg, A, A, A, ws, None) == E
        assert b"16-byte aligned" in L.graft_last_error()
    assert L.graft_lmhead_pack(100, 256, X, A, None) == E
    assert L.graft_lmhead_pack(100, 256, A, X, None) == E
    for h, w, g in ((X, A, A), (A, X, A), (A, A, X)):
        assert L.graft_lmhead_topk_sample(4, 256, 100, 4, 1.0, h, w, g, A, A, A, A, ws, None) == E
    # tree attention: q, kcache, vcache, out, the workspace, and the head stride
    def att(q=A, k=A, v=A, out=A, wsp=A, stride=4096 * 128):
        return L.graft_tree_attention(1, 8, 2, 128, 0.1, q, k, v, A, stride, A, 4000, A, 60, A, A, out, None,
                                      wsp, ws, A, None)
    assert L.graft_tree_attention_workspace_bytes(1, 8, 2, 128, 4000, 60) > 0
    for kw in ({"q": X}, {"k": X}, {"v": X}, {"out": X}, {"wsp": X}, {"stride": 4096 * 128 + 4}):
        assert att(**kw) == E, kw
    # KV compaction: caches and the layer stride
    def kvc(k=A, v=A, layers=1, layer_stride=0):
        return L.graft_kv_compact(1, 8, 128, layers, k, v, layer_stride, A, 4096 * 128, A, A, A, A, A, A + 64,
                                  A + 128, A, None)
    assert kvc(k=X) == E
    assert kvc(v=X) == E
    assert kvc(layers=2, layer_stride=8 * 4096 * 128 + 4) == E


# ----------------------------------------------------------------------------- table checkpoint files

def _fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit, from its published definition (offset basis, prime)."""
    h = 0xCBF29CE484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def write_table_file(path, table, magic=b"GRAFTTB1", V=None, k=None, checksum=None, extra=b""):
    """An independent writer of the table file format (header: magic, V, k,
    FNV-1a of the payload; then int32 rows, little-endian)."""
    t = np.ascontiguousarray(table, dtype="<i4")
    payload = t.tobytes()
    V = t.shape[0] if V is None else V
    k = t.shape[1] if k is None else k
    cs = _fnv1a64(payload) if checksum is None else checksum
    with open(path, "wb") as f:
        f.write(magic + int(V).to_bytes(8, "little") + int(k).to_bytes(8, "little") + int(cs).to_bytes(8, "little"))
        f.write(payload + extra)


def test_fnv1a64_matches_published_vectors():
    # test vectors of the FNV-1a 64-bit definition
    assert _fnv1a64(b"") == 0xCBF29CE484222325
    assert _fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert _fnv1a64(b"foobar") == 0x85944171F73967E8


def test_table_load_rejects_bad_files_before_any_copy(native, tmp_path):
    """Every check of a table file runs on the host before the device copy:
    the device pointer given here is never dereferenced."""
    L = native.lib()
    E, EIO = native.GRAFT_EINVAL, native.GRAFT_EIO
    fake = 1 << 20
    V, k = 50, 4
    t = np.random.default_rng(3).integers(0, V, (V, k)).astype(np.int32)
    p = str(tmp_path / "t.bin").encode()
    assert L.graft_table_load(str(tmp_path / "missing.bin").encode(), V, k, fake, None) == EIO
    write_table_file(p, t, magic=b"NOTTABLE")
    assert L.graft_table_load(p, V, k, fake, None) == E and b"not a table file" in L.graft_last_error()
    write_table_file(p, t)
    assert L.graft_table_load(p, V + 1, k, fake, None) == E and b"50 x 4" in L.graft_last_error()
    assert L.graft_table_load(p, V, k + 1, fake, None) == E
    write_table_file(p, t, extra=b"\0")
    assert L.graft_table_load(p, V, k, fake, None) == E and b"payload bytes" in L.graft_last_error()
    write_table_file(p, t[:-1], V=V)
    assert L.graft_table_load(p, V, k, fake, None) == E
    write_table_file(p, t, checksum=_fnv1a64(t.tobytes()) ^ 1)
    assert L.graft_table_load(p, V, k, fake, None) == E and b"checksum" in L.graft_last_error()
    bad = t.copy()
    bad[7, 2] = V  # a token id out of range, with a valid checksum
    write_table_file(p, bad)
    assert L.graft_table_load(p, V, k, fake, None) == E and b"entry 30" in L.graft_last_error()
    # arguments
    assert L.graft_table_load(None, V, k, fake, None) == E
    assert L.graft_table_load(p, V, 0, fake, None) == E
    assert L.graft_table_load(p, V, 17, fake, None) == E
    assert L.graft_table_load(p, V, k, None, None) == E
    assert L.graft_table_save(p, 0, k, fake, None) == E
    assert L.graft_table_save(None, V, k, fake, None) == E
