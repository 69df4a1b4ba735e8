"""CPU-only checks of the C ABI: the library loads, exports what include/nsa.h
declares, and rejects every invalid call on the host before any launch.

No call here reaches a kernel launch: each either fails validation or has an
empty problem (batch 0, fewer tokens than a block), which returns before
touching the GPU.
"""

import ctypes

import pytest

from long_context_sparse_fwd_amd import nsa

OK, INV, UNS, WS = (nsa.NSA_OK, nsa.NSA_ERR_INVALID_ARGUMENT, nsa.NSA_ERR_UNSUPPORTED,
                    nsa.NSA_ERR_WORKSPACE_TOO_SMALL)
FAKE = 1 << 20  # an aligned non-null address; never dereferenced by these calls


@pytest.fixture(scope="module")
def L():
    return nsa.lib()


def test_library_exports_every_declared_function(L):
    names = nsa.header_functions()
    assert {"nsa_fwd_prefill", "nsa_fwd_decode", "nsa_compress_kv", "nsa_prefill_workspace_bytes",
            "nsa_decode_workspace_bytes", "nsa_status_string", "nsa_last_error", "nsa_version",
            "nsa_fwd_prefill_timed", "nsa_fwd_decode_timed", "nsa_fwd_prefill_chunk", "nsa_fwd_prefill_varlen",
            "nsa_bwd_prefill", "nsa_bwd_prefill_timed", "nsa_bwd_prefill_workspace_bytes",
            "nsa_fwd_prefill_save", "nsa_bwd_prefill_saved", "nsa_bwd_prefill_saved_timed"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.nsa_version() >= 100


def test_status_strings(L):
    for code, name in [(0, "NSA_OK"), (1, "NSA_ERR_INVALID_ARGUMENT"), (2, "NSA_ERR_UNSUPPORTED"),
                       (3, "NSA_ERR_WORKSPACE_TOO_SMALL"), (4, "NSA_ERR_HIP")]:
        assert L.nsa_status_string(code).decode() == name


def pdesc(B=1, Lq=65536, Hq=64, G=4, D=128, dt=nsa.NSA_BF16, odt=nsa.NSA_BF16):
    d = nsa.PrefillDesc()
    d.batch, d.seqlen, d.n_q_heads, d.n_kv_heads, d.head_dim = B, Lq, Hq, G, D
    d.in_dtype, d.out_dtype = dt, odt
    d.q_stride[:] = (Lq * Hq * D, Hq * D, D)
    d.k_stride[:] = (Lq * G * D, G * D, D)
    d.v_stride[:] = (Lq * G * D, G * D, D)
    d.g_stride[:] = (Lq * Hq * 3, Hq * 3, 3)
    d.o_stride[:] = (Lq * Hq * D, Hq * D, D)
    return d


def ddesc(B=64, Lm=65536, Hq=64, G=4, D=128, nmax=None):
    d = nsa.DecodeDesc()
    d.batch, d.max_seqlen = B, Lm
    d.max_blocks = Lm // 64 if nmax is None else nmax
    d.n_q_heads, d.n_kv_heads, d.head_dim = Hq, G, D
    d.in_dtype = d.out_dtype = nsa.NSA_BF16
    d.q_stride[:] = (Hq * D, D)
    d.k_stride[:] = (G * Lm * D, Lm * D, D)
    d.v_stride[:] = (G * Lm * D, Lm * D, D)
    d.kc_stride[:] = (G * d.max_blocks * D, d.max_blocks * D, D)
    d.vc_stride[:] = (G * d.max_blocks * D, d.max_blocks * D, D)
    d.g_stride[:] = (Hq * 3, 3)
    d.o_stride[:] = (Hq * D, D)
    return d


def ws_prefill(L, d, p):
    n = ctypes.c_size_t(0)
    st = L.nsa_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def test_prefill_workspace_size_is_the_sum_of_its_parts(L):
    st, n = ws_prefill(L, pdesc(), nsa.make_params(16, 512))
    assert st == OK
    tiles = 2 * 4 * 1024 * 64 * 128 * 2          # K and V tiles
    ctiles = 3 * 4 * 16 * 64 * 128 * 2           # block-mean tiles (K high, K low, V)
    idx = 65536 * 4 * 16 * 4
    part = 65536 * 64 * 128 * 4                  # fp32 window + compressed rows (bf16 output)
    assert n == tiles + ctiles + idx + part
    d = pdesc()
    d.out_dtype = nsa.NSA_F32                    # an fp32 output holds that part itself
    st, n32 = ws_prefill(L, d, nsa.make_params(16, 512))
    assert st == OK and n32 == tiles + ctiles + idx


@pytest.mark.parametrize("mut,code", [
    (lambda d, p: setattr(d, "n_q_heads", 65), INV),          # not a multiple of G
    (lambda d, p: setattr(d, "n_kv_heads", 2), UNS),          # 32 heads per group
    (lambda d, p: setattr(d, "head_dim", 96), UNS),
    (lambda d, p: setattr(d, "head_dim", 0), INV),
    (lambda d, p: setattr(d, "batch", -1), INV),
    (lambda d, p: setattr(d, "in_dtype", 7), INV),
    (lambda d, p: setattr(d, "in_dtype", nsa.NSA_F32), UNS),  # f32 in, bf16 out
    (lambda d, p: d.q_stride.__setitem__(1, 8 * 1000 + 4), INV),
    (lambda d, p: d.k_stride.__setitem__(0, -8), INV),
    (lambda d, p: setattr(p, "compress_block_size", 128), UNS),     # above the selection block
    (lambda d, p: setattr(p, "select_block_size", 48), UNS),        # not a multiple of 32
    (lambda d, p: (setattr(p, "select_block_size", 128), setattr(p, "select_top_k", 33)), UNS),  # > 4096 tokens
    (lambda d, p: setattr(p, "select_block_size", 0), INV),
    (lambda d, p: setattr(p, "select_top_k", 0), INV),
    (lambda d, p: setattr(p, "select_top_k", 65), UNS),
    (lambda d, p: setattr(p, "sliding_window", 0), INV),
    (lambda d, p: setattr(p, "softmax_scale", float("nan")), INV),
])
def test_prefill_validation(L, mut, code):
    d, p = pdesc(), nsa.make_params(16, 512)
    mut(d, p)
    st, _ = ws_prefill(L, d, p)
    assert st == code, L.nsa_last_error()
    st = L.nsa_fwd_prefill(ctypes.byref(d), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                           FAKE, 1 << 40, None)
    assert st == code
    assert L.nsa_last_error().decode() != ""


@pytest.mark.parametrize("block,select_block,top_k", [(32, 64, 16), (64, 128, 16), (16, 32, 64), (64, 256, 16)])
def test_prefill_accepts_general_block_sizes(L, block, select_block, top_k):
    d, p = pdesc(Lq=4096), nsa.make_params(top_k, 512, block=block, select_block=select_block)
    st, n = ws_prefill(L, d, p)
    assert st == OK, L.nsa_last_error()
    # the compressed tiles follow the number of compressed blocks
    _, n64 = ws_prefill(L, d, nsa.make_params(top_k, 512))
    assert (n > n64) == (block < 64)


def test_general_entry_checks(L):
    d, p = pdesc(Lq=4096), nsa.make_params(16, 512, block=32, select_block=64)
    n = ctypes.c_size_t()
    ws = lambda g: L.nsa_prefill_general_workspace_bytes(ctypes.byref(d), ctypes.byref(p), g, ctypes.byref(n))
    assert ws(None) == OK
    plain = n.value
    g = nsa.NsaGeneral()
    g.compress_stride = 16
    assert ws(ctypes.byref(g)) == OK
    assert n.value > plain                       # twice the compressed blocks
    for bad in (0, 33):                          # stride outside [1, compress_block_size]
        g.compress_stride = bad
        assert ws(ctypes.byref(g)) == INV
    g.compress_stride = 32
    g.wk = FAKE                                   # an incomplete compressor
    assert ws(ctypes.byref(g)) == INV
    g.bk, g.wv, g.bv = FAKE, FAKE, FAKE
    assert ws(ctypes.byref(g)) == OK
    g.wv = FAKE + 8                               # misaligned
    assert ws(ctypes.byref(g)) == INV
    g.wv = FAKE
    g.gate_w = FAKE                               # gate layer without its bias
    assert ws(ctypes.byref(g)) == INV
    g.gate_b = FAKE
    assert ws(ctypes.byref(g)) == OK
    assert n.value == plain + 4096 * 64 * 3 * 4   # + the fp32 gates
    # with a gate layer the gates argument may be NULL; the workspace must cover the gates
    call = lambda gates, nb: L.nsa_fwd_prefill_general(ctypes.byref(d), ctypes.byref(p), ctypes.byref(g), FAKE,
                                                       FAKE, FAKE, gates, FAKE, None, 0, FAKE, nb, None)
    assert call(None, n.value - 1) == WS
    g.gate_w = g.gate_b = None
    assert call(None, n.value) == INV             # no gate layer: gates are required
    # the selected branch is kept for the backward only in the plain geometry
    assert L.nsa_fwd_prefill_save(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 5), None, 0, FAKE, FAKE, FAKE,
                                  n.value, None) == UNS


def test_general_decode_entry_checks(L):
    # blocks of 32 with stride 16 over a 4096-token cache: 255 compressed blocks
    d, p = ddesc(B=2, Lm=4096, nmax=255), nsa.make_params(16, 512, block=32, select_block=64)
    n = ctypes.c_size_t()
    ws = lambda g: L.nsa_decode_general_workspace_bytes(ctypes.byref(d), ctypes.byref(p), g, ctypes.byref(n))
    g = nsa.NsaGeneral()
    g.compress_stride = 16
    assert ws(ctypes.byref(g)) == OK
    plain = n.value
    d.max_blocks = 254                            # fewer cache rows than compressed blocks
    assert ws(ctypes.byref(g)) == INV
    d.max_blocks = 255
    for bad in (0, 33):                           # stride outside [1, compress_block_size]
        g.compress_stride = bad
        assert ws(ctypes.byref(g)) == INV
    g.compress_stride = 16
    g.gate_w = FAKE                               # gate layer without its bias
    assert ws(ctypes.byref(g)) == INV
    g.gate_b = FAKE
    assert ws(ctypes.byref(g)) == OK
    assert n.value == plain + 2 * 64 * 3 * 4       # + the fp32 gates of 2 sequences x 64 heads
    # with a gate layer the gates argument may be NULL; the workspace must cover the gates
    call = lambda gates, nb: L.nsa_fwd_decode_general(ctypes.byref(d), ctypes.byref(p), ctypes.byref(g), FAKE,
                                                      FAKE, FAKE, FAKE, FAKE, FAKE, gates, FAKE, None, 0, FAKE,
                                                      nb, None)
    assert call(None, n.value - 1) == WS
    g.gate_w = g.gate_b = None
    assert call(None, n.value) == INV             # no gate layer: gates are required
    # the plain decode still needs blocks and selection blocks of 64
    assert L.nsa_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == UNS
    # selection blocks below the compressed blocks, or top_k * select_block above 4096
    for bad in (nsa.make_params(16, 512, block=64, select_block=32), nsa.make_params(64, 512, block=32,
                                                                                      select_block=128)):
        assert L.nsa_decode_general_workspace_bytes(ctypes.byref(d), ctypes.byref(bad), None,
                                                    ctypes.byref(n)) == UNS


def test_prefill_score_rows_move_to_the_workspace_past_what_lds_holds(L):
    # The compressed kernel keeps 8 waves x 2 tokens of block-score rows (NcT * 64
    # floats each) in LDS next to its 64 KiB staging while that fits: up to 24
    # chunks of 64 blocks (98304 tokens). One token more, and the rows of every
    # query row ([B][G][L + 2][NcT * 64] floats) go to the workspace.
    p = nsa.make_params(16, 512)
    st0, below = ws_prefill(L, pdesc(Lq=98304), p)
    st1, above = ws_prefill(L, pdesc(Lq=98368), p)
    assert st0 == OK and st1 == OK
    rows = 4 * (98368 + 2) * 25 * 64 * 4
    assert 0 <= above - below - rows < 16 << 20   # the rest grows by 64 tokens' worth


def test_prefill_pointer_and_workspace_checks(L):
    d, p = pdesc(Lq=4096), nsa.make_params(16, 512)
    _, need = ws_prefill(L, d, p)
    call = lambda q=FAKE, out=FAKE, idx=None, mode=0, ws=FAKE, nb=need: L.nsa_fwd_prefill(
        ctypes.byref(d), ctypes.byref(p), q, FAKE, FAKE, FAKE, out, idx, mode, ws, nb, None)
    assert call(q=None) == INV
    assert call(q=FAKE + 2) == INV            # misaligned
    assert call(out=None) == INV
    assert call(ws=None) == INV
    assert call(mode=1) == INV                # inject without idx
    assert call(mode=5) == INV
    assert call(idx=FAKE + 2) == INV
    assert call(nb=need - 1) == WS
    assert "workspace" in L.nsa_last_error().decode()


def test_prefill_empty_problem_is_ok_without_launch(L):
    p = nsa.make_params(16, 512)
    for d in (pdesc(B=0), pdesc(Lq=0)):
        assert L.nsa_fwd_prefill(ctypes.byref(d), ctypes.byref(p), None, None, None, None, None, None,
                                 0, None, 0, None) == OK


def test_prefill_chunk_offset_checks(L):
    """The chunked prefill rejects a query offset outside [0, seqlen] before
    anything else, and an empty chunk (offset == seqlen) returns without a
    launch."""
    d, p = pdesc(Lq=4096), nsa.make_params(16, 512)
    _, need = ws_prefill(L, d, p)
    call = lambda off, q=FAKE: L.nsa_fwd_prefill_chunk(ctypes.byref(d), ctypes.byref(p), off, q, FAKE, FAKE,
                                                      FAKE, FAKE, None, 0, FAKE, need, None)
    assert call(-1) == INV
    assert "q_offset" in L.nsa_last_error().decode()
    assert call(4097) == INV
    assert call(4096, q=None) == OK           # no query rows: nothing is read
    assert call(1000, q=None) == INV          # rows to compute, but no q
    bad = pdesc(Lq=4096, D=96)
    assert L.nsa_fwd_prefill_chunk(ctypes.byref(bad), ctypes.byref(p), 10, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   0, FAKE, need, None) == UNS


def test_prefill_varlen_checks(L):
    """The varlen prefill needs seq_lens and a row count in [0, seqlen]; with
    zero query rows it returns without a launch."""
    d, p = pdesc(Lq=4096), nsa.make_params(16, 512)
    _, need = ws_prefill(L, d, p)
    call = lambda lens, rows, q=FAKE: L.nsa_fwd_prefill_varlen(
        ctypes.byref(d), ctypes.byref(p), lens, None, rows, q, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, need, None)
    assert call(None, 100) == INV
    assert "seq_lens" in L.nsa_last_error().decode()
    assert call(FAKE, -1) == INV
    assert call(FAKE, 4097) == INV
    assert call(FAKE, 0, q=None) == OK      # no query rows: nothing is read
    assert call(FAKE + 2, 100) == INV       # misaligned lengths
    assert call(FAKE, 100, q=None) == INV


def test_timed_variants_need_events(L):
    d, p = pdesc(Lq=256), nsa.make_params(4, 64)
    assert L.nsa_fwd_prefill_timed(ctypes.byref(d), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None, 0, FAKE, 1 << 40, None, None) == INV
    ev = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    assert L.nsa_fwd_prefill_timed(ctypes.byref(d), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None, 0, FAKE, 1 << 40, None, ev) == INV
    dd = ddesc(B=2, Lm=512)
    assert L.nsa_fwd_decode_timed(ctypes.byref(dd), ctypes.byref(p), *([FAKE] * 8), None, 0, FAKE,
                                  1 << 40, None, None) == INV


def test_backward_workspace_size_is_the_sum_of_its_parts(L):
    d, p = pdesc(), nsa.make_params(16, 512)
    n = ctypes.c_size_t(0)
    assert L.nsa_bwd_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    T, B, G, Hq, D, Nb, Nc = 65536, 1, 4, 64, 128, 1024, 1024
    tiles = 4 * B * G * Nb * 64 * D * 2          # K, K^T, V, V^T layouts
    means = 2 * B * Nc * G * D * 2               # block means of K and V
    ctiles = 4 * B * G * 16 * 64 * D * 2         # their four tile layouts
    heads = 2 * B * T * G * D * 16 * 2 + B * T * Hq * D * 2   # head-minor q, dout; dout copy
    stat = B * T * Hq * 3 * 8
    dmeans = 2 * B * Nc * G * D * 4
    lists = 3 * B * G * (Nb + 1) * 4 + B * G * T * 16 * 4
    assert abs(n.value - (tiles + means + ctiles + heads + stat + dmeans + lists)) <= 21 * 256


def test_backward_validation_and_empty_problem(L):
    d, p = pdesc(Lq=4096), nsa.make_params(16, 512)
    n = ctypes.c_size_t(0)
    assert L.nsa_bwd_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    need = n.value

    def call(q=FAKE, dout=FAKE, idx=FAKE, dq=FAKE, ws=FAKE, nb=need, desc=d, params=p):
        return L.nsa_bwd_prefill(ctypes.byref(desc), ctypes.byref(params), q, FAKE, FAKE, FAKE, dout, idx, dq,
                                 FAKE, FAKE, FAKE, ws, nb, None)
    assert call(q=None) == INV
    assert call(dout=None) == INV
    assert call(idx=None) == INV
    assert "idx" in L.nsa_last_error().decode()
    assert call(idx=FAKE + 2) == INV
    assert call(dq=FAKE + 4) == INV            # dq needs 16-byte alignment
    assert call(ws=None) == INV
    assert call(nb=need - 1) == WS
    assert call(desc=pdesc(Lq=4096, D=96)) == UNS
    assert call(params=nsa.make_params(16, 512, block=32)) == UNS
    assert call(params=nsa.make_params(16, 512, select_block=128)) == UNS
    for empty in (pdesc(B=0), pdesc(Lq=0)):
        assert L.nsa_bwd_prefill(ctypes.byref(empty), ctypes.byref(p), None, None, None, None, None, None, None,
                                 None, None, None, None, 0, None) == OK
    # the saved variants need both kept arrays
    # (q, k, v, gates, dout, idx), o_slc, lse_slc, (dq, dk, dv, dgates), workspace
    assert L.nsa_bwd_prefill_saved(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 6), None, FAKE, *([FAKE] * 4),
                                   FAKE, need, None) == INV
    assert "o_slc" in L.nsa_last_error().decode()
    assert L.nsa_bwd_prefill_saved(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 6), FAKE + 4, FAKE, *([FAKE] * 4),
                                   FAKE, need, None) == INV
    assert L.nsa_bwd_prefill_saved(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 6), FAKE, None, *([FAKE] * 4),
                                   FAKE, need, None) == INV
    assert "lse_slc" in L.nsa_last_error().decode()
    st, fneed = ws_prefill(L, d, p)
    assert L.nsa_fwd_prefill_save(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 5), None, 0, FAKE, None, FAKE,
                                  fneed, None) == INV
    assert "lse_slc" in L.nsa_last_error().decode()
    ev = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    assert L.nsa_bwd_prefill_timed(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 11), need, None, ev) == INV


def test_decode_workspace_and_validation(L):
    p = nsa.make_params(16, 512)
    n = ctypes.c_size_t()
    d = ddesc()
    assert L.nsa_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    # the compressed logits of 1024 blocks fit in LDS: only the selection
    assert n.value == 64 * 4 * 16 * 4
    f32 = ddesc()
    f32.in_dtype = f32.out_dtype = nsa.NSA_F32
    assert L.nsa_decode_workspace_bytes(ctypes.byref(f32), ctypes.byref(p), ctypes.byref(n)) == OK
    # fp32 staging leaves no room for them: the logits go to the workspace
    assert n.value == 64 * 4 * 16 * 1024 * 4 + 64 * 4 * 16 * 4
    bad = ddesc(nmax=1000)                       # block cache shorter than Lmax/64
    assert L.nsa_decode_workspace_bytes(ctypes.byref(bad), ctypes.byref(p), ctypes.byref(n)) == INV
    bad = ddesc()
    bad.max_seqlen = 0
    assert L.nsa_decode_workspace_bytes(ctypes.byref(bad), ctypes.byref(p), ctypes.byref(n)) == INV
    call = lambda d, ptrs, nb=n.value: L.nsa_fwd_decode(ctypes.byref(d), ctypes.byref(p), *ptrs, None, 0,
                                                       FAKE, nb, None)
    good = [FAKE] * 8
    for i in range(8):
        ptrs = list(good)
        ptrs[i] = None
        assert call(d, ptrs) == INV, i
    assert call(d, good, nb=10) == WS
    assert call(ddesc(B=0), [None] * 8) == OK
    # decode needs blocks of 64
    for pb in (nsa.make_params(16, 512, block=32), nsa.make_params(16, 512, select_block=128)):
        assert L.nsa_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(pb), ctypes.byref(n)) == UNS


def test_compress_validation(L):
    s = (ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 128)
    f = lambda B=1, G=4, T=128, D=128, dt=1, bs=64, k=FAKE: L.nsa_compress_kv(
        B, G, T, D, dt, bs, k, s, FAKE, s, FAKE, s, FAKE, s, None)
    assert f(bs=32) == UNS
    assert f(bs=0) == INV
    assert f(G=0) == INV
    assert f(dt=9) == INV
    assert f(k=None) == INV
    assert f(T=63) == OK          # no complete block: nothing to do
    assert f(B=0) == OK


def test_noalloc_decode_rejects_work_beyond_its_scratch(L):
    # bf16 caches of 262144 tokens: the compressed logits of 64 x 4 (sequence,
    # group) pairs need 64 MiB of scratch, more than the 40 MiB the
    # allocation-free decode holds; the call fails before any HIP call.
    # 131072 tokens (32 MiB + the selection) fit.
    p = nsa.make_params(16, 512)
    n = ctypes.c_size_t()
    d = ddesc(Lm=131072)
    assert L.nsa_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    assert (32 << 20) < n.value <= (40 << 20)
    d = ddesc(Lm=262144)
    assert L.nsa_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    assert n.value > 40 << 20
    st = L.nsa_fwd_decode_noalloc(ctypes.byref(d), ctypes.byref(p), *([FAKE] * 8), None, 0, None)
    assert st == WS
    assert "scratch" in L.nsa_last_error().decode()
    # an empty batch needs no scratch and no device
    assert L.nsa_fwd_decode_noalloc(ctypes.byref(ddesc(B=0)), ctypes.byref(p), *([None] * 9), 0, None) == OK
