"""The C ABI on the CPU: libpa.so loads, exports every entry point that
include/pa.h declares, and rejects bad host arguments before any HIP call
(no GPU needed, no kernel launched)."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_page_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("pa.h", "pa_blocks.h", "pa_sample.h")]

OK, INVALID, UNSUPPORTED, WS_SMALL, HIPERR = 0, 1, 2, 3, 4
F32, BF16 = pa.PA_F32, pa.PA_BF16


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points_the_binding_knows():
    names = declared_functions()
    assert "pa_rope_and_cache_write" in names and "pa_paged_attention_varlen" in names
    assert set(names) == set(pa.SIGNATURES), set(names) ^ set(pa.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = pa.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else():
    # the dynamic symbol table lists only the pa_* API as defined functions
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", pa.lib_path], capture_output=True,
                         text=True, check=True).stdout
    funcs = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {f for f in funcs if f.startswith("pa_")} == set(declared_functions())
    assert not [f for f in funcs if f.startswith("_ZN2pa")], "internal C++ symbols leaked"


def test_status_strings_and_version():
    assert pa.pa_abi_version() == 7
    for code in range(5):
        assert pa.pa_status_string(code).startswith("PA_")
    assert "UNKNOWN" in pa.pa_status_string(99)


FAKE = ctypes.c_void_p(0x10000)      # an aligned non-null pointer; never dereferenced here


def attn(**kw):
    args = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, bt=FAKE, seq_lens=FAKE, qsl=FAKE,
                out=ctypes.c_void_p(0x900000000), S=4, T=4, Hq=8, Hkv=2, D=128, P=256,
                num_pages=64, max_blocks=16, max_query_len=1, max_seq_len=256, scale=0.1,
                split=0, dtype=BF16, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    a = args
    return pa.lib().pa_paged_attention_varlen(
        a["q"], a["k_pool"], a["v_pool"], a["bt"], a["seq_lens"], a["qsl"], a["out"], a["S"],
        a["T"], a["Hq"], a["Hkv"], a["D"], a["P"], a["num_pages"], a["max_blocks"],
        a["max_query_len"], a["max_seq_len"], a["scale"], a["split"], a["dtype"], a["ws"],
        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(S=-1), INVALID),
    (dict(S=2 ** 30), INVALID),                    # the plan marks rows with bit 30
    (dict(T=-1), INVALID),
    (dict(Hkv=0), INVALID),
    (dict(num_pages=0), INVALID),
    (dict(max_blocks=0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(dtype=7), INVALID),
    (dict(split=8), INVALID),
    (dict(split=100), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(D=16), UNSUPPORTED),                # bf16 needs D in {64, 128}
    (dict(P=24), UNSUPPORTED),
    (dict(P=48), UNSUPPORTED),                # pages must be a power of two
    (dict(P=8), UNSUPPORTED),
    (dict(Hq=32, Hkv=2), UNSUPPORTED),        # group 16
    (dict(q=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(out=None), INVALID),
    (dict(q=ctypes.c_void_p(0x10008)), INVALID),   # not 16-byte aligned
    (dict(out=FAKE), INVALID),                     # out aliases q
    (dict(max_seq_len=4096), WS_SMALL),            # needs split-KV scratch
    (dict(num_pages=2 ** 30, P=256), INVALID),     # slot index would overflow int32
])
def test_attention_rejects_bad_host_arguments(kw, code):
    assert attn(**kw) == code


def test_attention_empty_tick_is_ok_without_touching_memory():
    assert attn(T=0) == OK
    assert attn(S=0, T=0) == OK


def _plan_bytes(S, cap_dec, cap_pf, Hq):
    # header 32, one 32-int line per prefill queue cursor (Hq) and one for the counter
    # of claimed decode chunks; R = S + S // 2 + 1 rows of the decode row list (the
    # decode rows and at most one group row per two of them): the rows 4 * R, and
    # partitions, first partial slot, first key and first partition index per row
    # 4 * R; chunk starts cap_dec, then (16-byte aligned) prefill entries 4 * cap_pf,
    # their sequence shapes 4 * cap_pf and cut items 4 * cap_pf (ints), padded to 256 bytes
    R = S + S // 2 + 1
    pf = -(-(32 * (2 + Hq) + 8 * R + cap_dec) // 4) * 4
    return -(-(pf + 12 * cap_pf) * 4 // 256) * 256


def _auto_slots(S, Hq, max_seq_len, P, max_parts, dec_grid=256):
    """Partial slots with automatic partitions (bf16): at most max_parts per
    row, and at most rows + chunks plus 4 per row for the members of grouped
    rows (a shared prefix read once), the chunks of the decode key axis
    numbering at most the decode waves per KV head (dec_grid * 4 waves over at
    least Hq / 8 KV heads; without a GPU the library assumes 256 compute units)
    or the axis over the largest partition (63 pages, at most 65536 keys)."""
    waves = -(-(dec_grid * 4 * 8) // Hq)
    split_max = min(63 * P, 65536) // 16 * 16
    by_cap = -(-(S * (-(-max_seq_len // 16) * 16)) // split_max)
    chunks = max(waves, by_cap)
    return min(S * max_parts, chunks), min(S * max_parts, S + chunks + 4 * S)


def test_workspace_size_query():
    lib = pa.lib()
    ws = lib.pa_paged_attention_workspace_size
    # automatic split: decode rows share one key axis cut into chunks of at least 256
    # keys (P = 256), so a row of n keys has at most ceil(n / 256) + 1 partials
    cap, slots = _auto_slots(64, 32, 256, 256, 2)
    assert ws(64, 64, 32, 128, 1, 256, 256, 0, BF16) == (
        _plan_bytes(64, cap, 0, 32) + slots * 32 * 130 * 4)
    cap, slots = _auto_slots(64, 32, 4096, 256, 17)
    assert (cap, slots) == (256, 576)
    n = ws(64, 64, 32, 128, 1, 4096, 256, 0, BF16)
    assert n == _plan_bytes(64, cap, 0, 32) + slots * 32 * 130 * 4
    # long rows: 36 rows of up to 32768 keys with Hq = 32 (at most 256 waves per KV head)
    cap, slots = _auto_slots(36, 32, 32768, 256, 129)
    assert (cap, slots) == (256, 436)
    assert ws(36, 36, 32, 128, 1, 32768, 256, 0, BF16) == (
        _plan_bytes(36, cap, 0, 32) + slots * 32 * 130 * 4)
    # an explicit split of 1024 keys: partitions aligned to the row start, 4 partials
    assert ws(64, 64, 32, 128, 1, 4096, 256, 1024, BF16) == (
        _plan_bytes(64, 64 * 4, 0, 32) + 64 * 4 * 32 * 130 * 4)
    # a partition spans at most 64 pages: with P = 16 an explicit 4096 is capped at 63 * 16
    assert ws(4, 4, 4, 16, 1, 4096, 16, 4096, F32) == (
        _plan_bytes(4, 4 * 5, 0, 4) + -(-(4 * 5 * 4 * 18 * 4) // 256) * 256)  # padded to 256
    # prefill rows: a row tile holds at least 16 tokens (128 rows, group <= 8), so at
    # most min(S * ceil(Lmax / 16), T / 16 + S) row tiles are planned; with automatic
    # partitions long items may be cut into pieces: 512 partial slots of 128 rows
    # (D + 2 floats each), one more entry per slot at most
    pf_bytes = -(-(512 * 128 * 130 * 4) // 256) * 256
    cap, slots = _auto_slots(51, 32, 4096, 256, 17)
    assert ws(51, 2096, 32, 128, 1024, 4096, 256, 0, BF16) == (
        _plan_bytes(51, cap, min(51 * 64, 2096 // 16 + 51) + 512, 32)
        + slots * 32 * 130 * 4 + pf_bytes)
    # a fixed split never cuts prefill items
    assert ws(51, 2096, 32, 128, 1024, 4096, 256, 1024, BF16) == (
        _plan_bytes(51, 51 * 4, min(51 * 64, 2096 // 16 + 51), 32) + 51 * 4 * 32 * 130 * 4)
    # fp32 with prefill rows takes the per-token path (512-key partitions): one row per
    # token, no plan
    assert ws(4, 40, 4, 16, 20, 1024, 16, 0, F32) == 40 * 2 * 4 * 18 * 4
    assert ws(-1, 4, 4, 16, 1, 64, 16, 0, F32) == 0


def cache_write(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, pos=FAKE, slots=FAKE, cs=FAKE, kp=FAKE, vp=FAKE, T=4,
                Hq=8, Hkv=2, D=128, P=16, num_pages=8, max_pos=64, dtype=BF16, stream=None)
    args.update(kw)
    a = args
    return pa.lib().pa_rope_and_cache_write(a["q"], a["k"], a["v"], a["pos"], a["slots"], a["cs"],
                                            a["kp"], a["vp"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                            a["P"], a["num_pages"], a["max_pos"], a["dtype"],
                                            a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(Hkv=0), INVALID),
    (dict(dtype=3), INVALID),
    (dict(k=None), INVALID),
    (dict(v=None), INVALID),
    (dict(slots=None), INVALID),
    (dict(kp=None), INVALID),
    (dict(max_pos=0), INVALID),
    (dict(Hq=0), INVALID),                       # q given but no query heads
    (dict(D=40), UNSUPPORTED),
    (dict(D=2064), UNSUPPORTED),                 # past 2048
    (dict(k=ctypes.c_void_p(0x10004)), INVALID),
])
def test_cache_write_rejects_bad_host_arguments(kw, code):
    assert cache_write(**kw) == code


def test_cache_write_empty_is_ok():
    assert cache_write(T=0) == OK


def test_other_entry_points_reject_bad_arguments():
    lib = pa.lib()
    assert lib.pa_rope_cos_sin_table(None, 16, 64, 1e4, None) == INVALID
    assert lib.pa_rope_cos_sin_table(FAKE, 0, 64, 1e4, None) == INVALID
    assert lib.pa_rope_cos_sin_table(FAKE, 16, 63, 1e4, None) == INVALID
    assert lib.pa_rope_cos_sin_table(FAKE, 16, 64, -1.0, None) == INVALID
    assert lib.pa_compute_slot_mapping(FAKE, FAKE, FAKE, FAKE, 2, 4, 0, 16, 8, None) == INVALID
    assert lib.pa_compute_slot_mapping(None, FAKE, FAKE, FAKE, 2, 4, 4, 16, 8, None) == INVALID
    assert lib.pa_compute_slot_mapping(None, None, None, None, 0, 0, 4, 16, 8, None) == OK
    assert lib.pa_profile_start(0) == INVALID
    assert lib.pa_profile_get(0, None, 0, None) == INVALID
    assert lib.pa_profile_reset() == OK


def tick(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, pos=FAKE, bt=FAKE, seq_lens=FAKE, qsl=FAKE, cs=FAKE,
                kp=FAKE, vp=FAKE, out=ctypes.c_void_p(0x900000000), slots=FAKE, S=4, T=4, Hq=8,
                Hkv=2, D=128, P=256, num_pages=64, max_blocks=16, max_query_len=1,
                max_seq_len=256, max_pos=4096, scale=0.1, split=0, dtype=BF16, ws=None,
                ws_bytes=0, stream=None)
    args.update(kw)
    a = args
    return pa.lib().pa_tick_forward(
        a["q"], a["k"], a["v"], a["pos"], a["bt"], a["seq_lens"], a["qsl"], a["cs"], a["kp"],
        a["vp"], a["out"], a["slots"], a["S"], a["T"], a["Hq"], a["Hkv"], a["D"], a["P"],
        a["num_pages"], a["max_blocks"], a["max_query_len"], a["max_seq_len"], a["max_pos"],
        a["scale"], a["split"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),                     # the tick needs query rows
    (dict(slots=None), INVALID),                 # slot mapping's checks
    (dict(max_blocks=0), INVALID),
    (dict(D=40), UNSUPPORTED),                   # the cache write's checks
    (dict(max_pos=0), INVALID),
    (dict(k=ctypes.c_void_p(0x10004)), INVALID),
    (dict(Hq=7), INVALID),                       # the attention call's checks
    (dict(P=24), UNSUPPORTED),
    (dict(split=20), INVALID),
    (dict(max_query_len=64, max_seq_len=4096), WS_SMALL),
])
def test_tick_forward_rejects_bad_host_arguments(kw, code):
    # every check of the three calls runs before anything is enqueued, so no
    # pointer here is dereferenced and no GPU is needed
    assert tick(**kw) == code


def test_tick_forward_empty_tick_is_ok_without_touching_memory():
    assert tick(T=0) == OK


def test_sample_tokens_rejects_bad_scalars_before_any_launch():
    lib = pa.lib()
    p = ctypes.c_void_p(256)  # never dereferenced: every call below fails its host checks
    ws = lib.pa_sample_workspace_size(4, 10)
    assert ws > 0 and lib.pa_sample_workspace_size(0, 10) == 0
    assert lib.pa_sample_workspace_size(4, 0) == 0 and lib.pa_sample_workspace_size(4, (1 << 21) + 1) == 0
    assert lib.pa_sample_workspace_size(4, 151936) > 20 * ws
    f = lambda *a: lib.pa_sample_tokens(*a)
    assert f(p, 10, -1, 10, p, p, p, p, p, p, ws, None) == INVALID       # rows < 0
    assert f(p, 10, 1, 0, p, p, p, p, p, p, ws, None) == INVALID         # vocab < 1
    assert f(p, 5, 1, 10, p, p, p, p, p, p, ws, None) == INVALID         # row_stride < vocab
    assert f(p, 1 << 22, 1, (1 << 21) + 1, p, p, p, p, p, p, ws, None) == UNSUPPORTED
    assert f(None, 10, 1, 10, p, p, p, p, p, p, ws, None) == INVALID     # NULL logits
    assert f(p, 10, 1, 10, p, p, p, p, None, p, ws, None) == INVALID     # NULL out
    assert f(p, 10, 1, 10, p, p, p, p, p, None, ws, None) == INVALID     # NULL workspace
    assert f(p, 10, 1, 10, p, p, p, p, p, ctypes.c_void_p(264), ws, None) == INVALID  # misaligned
    assert f(p, 10, 4, 10, p, p, p, p, p, p, ws - 1, None) == WS_SMALL
    assert f(None, 10, 0, 10, None, None, None, None, None, None, 0, None) == OK  # no rows


def test_validation_switch_keeps_host_checks_first():
    # with validation on, bad host scalars are still rejected before any copy
    # of device metadata (no GPU needed), and an empty tick enqueues nothing
    assert pa.pa_validation_message() == ""
    pa.pa_set_validation(True)
    try:
        assert attn(Hq=6, Hkv=4) == INVALID
        assert attn(max_seq_len=4096) == WS_SMALL
        assert tick(q=None) == INVALID
        assert attn(T=0) == OK and tick(T=0) == OK
        assert cache_write(T=0) == OK
        assert pa.pa_validation_message() == ""
    finally:
        pa.pa_set_validation(False)


def tick_noalloc(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, pos=FAKE, bt=FAKE, seq_lens=FAKE, qsl=FAKE, cs=FAKE,
                kp=FAKE, vp=FAKE, out=ctypes.c_void_p(0x900000000), slots=FAKE, S=4, T=4, Hq=8,
                Hkv=2, D=128, P=256, num_pages=64, max_blocks=16, max_query_len=1,
                max_seq_len=256, max_pos=4096, scale=0.1, split=0, dtype=BF16, stream=None)
    args.update(kw)
    a = args
    return pa.lib().pa_tick_forward_noalloc(
        a["q"], a["k"], a["v"], a["pos"], a["bt"], a["seq_lens"], a["qsl"], a["cs"], a["kp"],
        a["vp"], a["out"], a["slots"], a["S"], a["T"], a["Hq"], a["Hkv"], a["D"], a["P"],
        a["num_pages"], a["max_blocks"], a["max_query_len"], a["max_seq_len"], a["max_pos"],
        a["scale"], a["split"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(Hq=7), INVALID),
    (dict(P=24), UNSUPPORTED),
    (dict(split=20), INVALID),
    # a fixed 16-key split over 4096-key rows: 64 x 256 partials of 32 heads, about
    # 272 MB of scratch, past the library's fixed 64 MiB
    (dict(S=64, T=64, Hq=32, Hkv=8, max_seq_len=4096, split=16), WS_SMALL),
])
def test_noalloc_tick_checks_everything_before_any_hip_call(kw, code):
    assert tick_noalloc(**kw) == code
    if code == WS_SMALL:
        msg = pa.pa_validation_message()
        assert "needs" in msg and str(64 << 20) in msg, msg


def test_noalloc_empty_tick_is_ok_without_touching_memory():
    assert tick_noalloc(T=0) == OK
