"""C-ABI checks that need no GPU: the library loads, exports every symbol
declared in include/gqa_attn.h, and its host-side validation returns the
documented codes. No compute entry point is called here."""
import ctypes
import os
import re

import pytest

import grouped_query_attention_flash_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

A16 = 0x10000  # a fake, 16-byte aligned, never dereferenced address


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", src)))


def test_header_declarations_match_binding_list():
    assert declared_functions() == sorted(gqa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = gqa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def check_fwd(q=A16, k=A16, v=A16, o=A16, lse=None, qs=None, ks=None,
              B=1, K=1, G=4, T=64, S=64, H=128, causal=1):
    P = ctypes.c_void_p
    return gqa.load_library().attn_check_fwd(P(q), P(k), P(v), P(o), P(lse), P(qs), P(ks),
                                             B, K, G, T, S, H, causal)


def check_bwd(ws=A16, wsb=None, B=1, K=1, G=4, T=64, S=64, H=128, dq=A16, lse=A16, qs=None, ks=None, o=A16):
    P = ctypes.c_void_p
    if wsb is None:
        wsb = gqa.attn_bwd_workspace_bytes(B, K, G, T, S, H)
    return gqa.load_library().attn_check_bwd(P(A16), P(A16), P(A16), P(o), P(lse), P(A16), P(dq), P(A16),
                                             P(A16), P(qs), P(ks), B, K, G, T, S, H, 1, P(ws), wsb)


def test_check_fwd_codes():
    assert check_fwd() == gqa.GQA_ATTN_OK
    assert check_fwd(lse=A16, qs=A16, ks=A16) == gqa.GQA_ATTN_OK
    assert check_fwd(q=None) == gqa.GQA_ATTN_ERR_NULL
    assert check_fwd(o=None) == gqa.GQA_ATTN_ERR_NULL
    for bad in (dict(B=0), dict(K=0), dict(G=0), dict(T=0), dict(S=-1)):
        assert check_fwd(**bad) == gqa.GQA_ATTN_ERR_SHAPE, bad
    assert check_fwd(G=1 << 12, T=1 << 20) == gqa.GQA_ATTN_ERR_SHAPE  # slice >= 2^31 elements
    # each (b, kv head) slice is addressed in bytes by a signed 32-bit offset
    assert check_fwd(G=1, T=(1 << 23) - 1, S=64) == gqa.GQA_ATTN_OK      # q slice just under 2^30 elements
    assert check_fwd(G=1, T=1 << 23, S=64) == gqa.GQA_ATTN_ERR_SHAPE     # q slice 2^30 elements
    assert check_fwd(G=1, T=64, S=1 << 23) == gqa.GQA_ATTN_ERR_SHAPE     # k slice 2^30 elements
    # query rows rounded up to whole 32-row waves must stay below 2^31 (grid sizes)
    assert check_fwd(B=(1 << 26) - 1, G=1, T=1) == gqa.GQA_ATTN_OK        # (2^26 - 1) * 32 rows
    assert check_fwd(B=1 << 26, G=1, T=1) == gqa.GQA_ATTN_ERR_SHAPE       # 2^31 rows
    for h in (0, 32, 96, 129, 512):
        assert check_fwd(H=h) == gqa.GQA_ATTN_ERR_HEADDIM, h
    for h in (64, 128, 256):
        assert check_fwd(H=h) == gqa.GQA_ATTN_OK
    assert check_fwd(qs=A16) == gqa.GQA_ATTN_ERR_SEGMENTS
    assert check_fwd(ks=A16) == gqa.GQA_ATTN_ERR_SEGMENTS
    assert check_fwd(q=A16 + 8) == gqa.GQA_ATTN_ERR_ALIGN
    assert check_fwd(v=A16 + 2) == gqa.GQA_ATTN_ERR_ALIGN
    assert check_fwd(qs=A16 + 2, ks=A16) == gqa.GQA_ATTN_ERR_ALIGN
    assert check_fwd(qs=A16 + 4, ks=A16 + 4) == gqa.GQA_ATTN_OK
    # ragged sizes are accepted
    assert check_fwd(T=77, S=1031) == gqa.GQA_ATTN_OK


def test_check_bwd_codes_and_workspace():
    # D and lse * log2(e): one fp32 per query row each, each rounded up to 256 bytes
    assert gqa.attn_bwd_workspace_bytes(1, 8, 4, 8192, 8192, 128) == 2 * 4 * 8 * 4 * 8192
    assert gqa.attn_bwd_workspace_bytes(1, 1, 1, 3, 3, 128) == 512
    assert gqa.attn_bwd_workspace_bytes(0, 1, 1, 3, 3, 128) == 0
    assert check_bwd() == gqa.GQA_ATTN_OK
    assert check_bwd(lse=None) == gqa.GQA_ATTN_ERR_NULL
    assert check_bwd(dq=None) == gqa.GQA_ATTN_ERR_NULL
    assert check_bwd(ws=None) == gqa.GQA_ATTN_ERR_WORKSPACE
    assert check_bwd(wsb=16) == gqa.GQA_ATTN_ERR_WORKSPACE
    assert check_bwd(ws=A16 + 4) == gqa.GQA_ATTN_ERR_ALIGN
    assert check_bwd(H=96) == gqa.GQA_ATTN_ERR_HEADDIM
    assert check_bwd(o=None) == gqa.GQA_ATTN_OK          # o is not read by the backward
    assert check_bwd(o=A16 + 2) == gqa.GQA_ATTN_ERR_ALIGN
    assert check_bwd(qs=A16) == gqa.GQA_ATTN_ERR_SEGMENTS


def check_fwd_ws(ws=A16, wsb=None, B=1, K=2, G=4, T=1, S=4096, H=128, causal=0):
    P = ctypes.c_void_p
    if wsb is None:
        wsb = gqa.attn_fwd_workspace_bytes(B, K, G, T, S, H)
    return gqa.load_library().attn_check_fwd_ws(P(A16), P(A16), P(A16), P(A16), P(A16), None, None,
                                                B, K, G, T, S, H, causal, P(ws), wsb)


def test_split_plan_and_workspace_size():
    # the headline training shape fills the GPU: no split, no workspace
    assert gqa.attn_fwd_split_count(1, 8, 4, 8192, 8192, 128) == 1
    assert gqa.attn_fwd_workspace_bytes(1, 8, 4, 8192, 8192, 128) == 0
    # decoding shapes split the key range; the workspace holds every split's
    # fp32 output rows and lse, rounded up to 256 bytes
    for (B, K, G, T, S, H) in [(1, 2, 4, 1, 4096, 128), (16, 8, 4, 1, 32768, 128), (1, 1, 8, 1, 1030, 64),
                               (1, 1, 4, 5, 2500, 256)]:
        n = gqa.attn_fwd_split_count(B, K, G, T, S, H)
        assert n > 1, (B, K, G, T, S, H)
        rows = B * K * G * T
        want = 4 * n * rows * (H + 1)
        assert gqa.attn_fwd_workspace_bytes(B, K, G, T, S, H) == (want + 255) // 256 * 256
    # too few key tiles to split, and invalid sizes
    assert gqa.attn_fwd_split_count(1, 1, 4, 1, 100, 128) == 1
    assert gqa.attn_fwd_split_count(0, 1, 4, 1, 100, 128) == 0
    assert gqa.attn_fwd_workspace_bytes(1, 1, 4, 1, 100, 96) == 0


def test_check_fwd_ws_codes():
    assert check_fwd_ws() == gqa.GQA_ATTN_OK
    assert check_fwd_ws(ws=None) == gqa.GQA_ATTN_ERR_WORKSPACE
    need = gqa.attn_fwd_workspace_bytes(1, 2, 4, 1, 4096, 128)
    assert check_fwd_ws(wsb=need - 1) == gqa.GQA_ATTN_ERR_WORKSPACE
    assert check_fwd_ws(ws=A16 + 8) == gqa.GQA_ATTN_ERR_ALIGN
    # a shape that does not split needs no workspace
    assert check_fwd_ws(ws=None, wsb=0, T=8192, S=8192, K=8) == gqa.GQA_ATTN_OK
    # the forward's own checks come first
    assert check_fwd_ws(H=96) == gqa.GQA_ATTN_ERR_HEADDIM
    assert check_fwd_ws(B=0) == gqa.GQA_ATTN_ERR_SHAPE


def test_check_local_window_codes():
    P = ctypes.c_void_p
    lib = gqa.load_library()
    args = (P(A16), P(A16), P(A16), P(A16), P(A16), None, None, 1, 1, 4, 64, 64, 128, 1)
    for wl, wr, want in [(-1, -1, gqa.GQA_ATTN_OK), (0, 0, gqa.GQA_ATTN_OK), (31, -1, gqa.GQA_ATTN_OK),
                         (2 ** 31 - 1, 2 ** 31 - 1, gqa.GQA_ATTN_OK),
                         (-2, 0, gqa.GQA_ATTN_ERR_MASK), (0, -5, gqa.GQA_ATTN_ERR_MASK)]:
        assert lib.attn_check_fwd_local(*args, wl, wr, None, 0) == want, (wl, wr)
    wsb = gqa.attn_bwd_workspace_bytes(1, 1, 4, 64, 64, 128)
    bargs = (P(A16),) * 9 + (None, None, 1, 1, 4, 64, 64, 128, 1)
    assert lib.attn_check_bwd_local(*bargs, 5, -1, P(A16), wsb) == gqa.GQA_ATTN_OK
    assert lib.attn_check_bwd_local(*bargs, -3, -1, P(A16), wsb) == gqa.GQA_ATTN_ERR_MASK
    assert lib.attn_check_bwd_local(*bargs, 5, -1, None, wsb) == gqa.GQA_ATTN_ERR_WORKSPACE


def test_check_mask_codes():
    """causal modes 0..2, window sides >= -1 and prefix >= 0 are accepted by
    every entry point; anything else is ERR_MASK, reported before any launch."""
    P = ctypes.c_void_p
    lib = gqa.load_library()
    fargs = (P(A16), P(A16), P(A16), P(A16), P(A16), None, None, 1, 1, 4, 64, 128, 128)
    for causal, wl, wr, pfx, want in [
            (0, -1, -1, 0, gqa.GQA_ATTN_OK), (1, -1, -1, 0, gqa.GQA_ATTN_OK), (2, -1, -1, 0, gqa.GQA_ATTN_OK),
            (2, 10, 3, 7, gqa.GQA_ATTN_OK), (1, -1, -1, 1 << 30, gqa.GQA_ATTN_OK),
            (3, -1, -1, 0, gqa.GQA_ATTN_ERR_MASK), (-1, -1, -1, 0, gqa.GQA_ATTN_ERR_MASK),
            (1, -1, -1, -1, gqa.GQA_ATTN_ERR_MASK), (1, -2, -1, 0, gqa.GQA_ATTN_ERR_MASK),
            (0, -1, -7, 0, gqa.GQA_ATTN_ERR_MASK)]:
        assert lib.attn_check_fwd_mask(*fargs, causal, wl, wr, pfx, None, 0) == want, (causal, wl, wr, pfx)
    # the plain entry points take the causal mode too
    assert check_fwd(causal=2) == gqa.GQA_ATTN_OK
    assert check_fwd(causal=3) == gqa.GQA_ATTN_ERR_MASK
    wsb = gqa.attn_bwd_workspace_bytes(1, 1, 4, 64, 128, 128)
    bargs = (P(A16),) * 9 + (None, None, 1, 1, 4, 64, 128, 128)
    assert lib.attn_check_bwd(*bargs, 2, P(A16), wsb) == gqa.GQA_ATTN_OK
    assert lib.attn_check_bwd(*bargs, 5, P(A16), wsb) == gqa.GQA_ATTN_ERR_MASK
    assert lib.attn_check_bwd_mask(*bargs, 2, 4, -1, 16, P(A16), wsb) == gqa.GQA_ATTN_OK
    assert lib.attn_check_bwd_mask(*bargs, 1, -1, -1, -3, P(A16), wsb) == gqa.GQA_ATTN_ERR_MASK
    # shape errors still come first
    assert lib.attn_check_bwd_mask(*(bargs[:11] + (0,) + bargs[12:]), 9, -1, -1, 0, P(A16), wsb) == \
        gqa.GQA_ATTN_ERR_SHAPE


def test_check_head_mask_codes():
    """The per-head mask calls check the table pointer (NULL -> ERR_NULL, not
    4-byte aligned -> ERR_ALIGN) after the checks of attn_fwd / attn_bwd; its
    contents live on the device and every value is a valid mask."""
    P = ctypes.c_void_p
    lib = gqa.load_library()
    fargs = (P(A16), P(A16), P(A16), P(A16), P(A16), None, None, 1, 2, 4, 64, 128, 128)
    assert lib.attn_check_fwd_head_masks(*fargs, 1, P(A16)) == gqa.GQA_ATTN_OK
    assert lib.attn_check_fwd_head_masks(*fargs, 2, P(A16 + 4)) == gqa.GQA_ATTN_OK
    assert lib.attn_check_fwd_head_masks(*fargs, 1, None) == gqa.GQA_ATTN_ERR_NULL
    assert lib.attn_check_fwd_head_masks(*fargs, 1, P(A16 + 2)) == gqa.GQA_ATTN_ERR_ALIGN
    assert lib.attn_check_fwd_head_masks(*fargs, 3, P(A16)) == gqa.GQA_ATTN_ERR_MASK
    assert lib.attn_check_fwd_head_masks(*(fargs[:12] + (96,)), 1, P(A16)) == gqa.GQA_ATTN_ERR_HEADDIM
    wsb = gqa.attn_bwd_workspace_bytes(1, 2, 4, 64, 128, 128)
    bargs = (P(A16),) * 9 + (None, None, 1, 2, 4, 64, 128, 128)
    assert lib.attn_check_bwd_head_masks(*bargs, 2, P(A16), P(A16), wsb) == gqa.GQA_ATTN_OK
    assert lib.attn_check_bwd_head_masks(*bargs, 2, None, P(A16), wsb) == gqa.GQA_ATTN_ERR_NULL
    assert lib.attn_check_bwd_head_masks(*bargs, 2, P(A16), P(A16), wsb - 1) == gqa.GQA_ATTN_ERR_WORKSPACE


def test_causal_mode_mapping():
    assert gqa.causal_mode(False) == 0 and gqa.causal_mode(True) == 1
    assert gqa.causal_mode("top_left") == 1 and gqa.causal_mode("end") == 2 and gqa.causal_mode(2) == 2
    with pytest.raises(ValueError):
        gqa.causal_mode(3)
    with pytest.raises(ValueError):
        gqa.causal_mode("bottom")


def test_strerror_and_hip_error():
    for code in range(0, 9):
        s = gqa.attn_strerror(code)
        assert s and s != "unknown error code"
    assert gqa.attn_strerror(99) == "unknown error code"
    assert gqa.attn_last_hip_error() == 0


def test_python_binding_rejects_before_calling():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, k)  # CPU tensors are refused; nothing is launched


def _json_choice(table, key, H, G, T, S, causal, segments, window_col):
    """The first row of the committed tuning JSON that matches (the same
    first-match rule the library compiles in)."""
    def hit(row, name, have):
        return row.get(name, -1) in (-1, have)
    for r in table[key]:
        if not hit(r, "H", H):
            continue
        if key == "load_placement" and not (hit(r, "causal", causal) and hit(r, "segments", segments)
                                             and hit(r, "window", window_col) and hit(r, "g8", int(G % 8 == 0))):
            continue
        if not (r.get("t_min", 0) <= T <= r.get("t_max", 2 ** 31 - 1)
                and r.get("s_min", 0) <= S <= r.get("s_max", 2 ** 31 - 1)):
            continue
        return r[key]
    raise AssertionError("no catch-all row")


def test_tuning_table_matches_the_committed_json():
    """attn_fwd_tuning returns, for every shape class, the first matching row of
    tuning/mi355x.json: the runtime selection reads the committed sweep table."""
    import json
    table = json.load(open(os.path.join(ROOT, "grouped_query_attention_flash_amd", "tuning", "mi355x.json")))
    shapes = [
        # B, K, G, T, S, H, causal, window, prefix, segments, window column (0 none, 1 causal left, 2 other)
        (1, 8, 4, 8192, 8192, 128, 1, None, 0, False, 0),
        (2, 8, 4, 4096, 4096, 128, 1, None, 0, False, 0),
        (4, 8, 4, 2048, 2048, 128, 1, None, 0, True, 0),
        (1, 2, 8, 32768, 32768, 256, 1, None, 0, False, 0),
        (1, 1, 4, 256, 256, 128, 0, None, 0, False, 0),
        (1, 8, 4, 8192, 8192, 64, 1, None, 0, False, 0),
        (1, 8, 4, 8192, 8192, 128, 1, (1023, -1), 0, False, 1),
        (1, 8, 4, 8192, 8192, 64, 1, (1023, -1), 0, False, 1),
        (1, 8, 4, 4096, 4096, 128, 1, None, 100, False, 2),
        (16, 8, 4, 1, 32768, 128, 0, None, 0, False, 0),
        (1, 8, 4, 512, 8192, 128, 2, None, 0, False, 0),
    ]
    for B, K, G, T, S, H, causal, win, pfx, seg, wcol in shapes:
        lp, st = gqa.attn_fwd_tuning(B, K, G, T, S, H, causal=causal, window=win, prefix=pfx, segments=seg)
        assert lp == _json_choice(table, "load_placement", H, G, T, S, int(causal != 0), int(seg), wcol), (T, S, H)
        assert st == _json_choice(table, "split_target", H, G, T, S, causal, seg, wcol), (T, S, H)
        # the workspace of the table's split target is the plain call's
        assert gqa.attn_fwd_tuned_workspace_bytes(B, K, G, T, S, H, -1) == gqa.attn_fwd_workspace_bytes(B, K, G, T, S, H)
    # a split target of 0 never splits; invalid arguments are refused
    assert gqa.attn_fwd_tuned_workspace_bytes(16, 8, 4, 1, 32768, 128, 0) == 0
    assert gqa.attn_fwd_tuned_workspace_bytes(16, 8, 4, 1, 32768, 128, -7) == 0
    with pytest.raises(ValueError):
        gqa.attn_fwd_tuning(1, 1, 4, 64, 64, 96)
    with pytest.raises(ValueError):
        gqa.attn_fwd_tuning(1, 1, 4, 64, 64, 128, causal=3)


def test_generated_table_is_current():
    """csrc/tuning_table.inc is what gen_table.py writes from the JSON."""
    from grouped_query_attention_flash_amd.tuning import gen_table
    import json
    table = json.load(open(gen_table.JSON_PATH))
    gen_table.check(table)
    assert open(gen_table.INC_PATH).read() == gen_table.render(table)
