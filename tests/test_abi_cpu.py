"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function ``include/locks.h`` declares, sizes records and workspaces, and
rejects bad arguments with the documented status before enqueuing anything.

Every call below that reaches a compute entry point is invalid, so it returns
from host validation and never launches a kernel (the fake device addresses
are never dereferenced)."""

import ctypes
import json
import os
import re
import subprocess

import pytest

from long_context_sparse_page_amd import locks as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "locks.h")
FAKE = 0x10000  # never dereferenced: every call using it fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lk_[a-z_]+)\s*\(", text)))


def test_header_and_library_agree():
    names = declared_functions()
    assert set(names) == set(L.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (lk_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = L.library()
    for n in names:
        assert getattr(lib, n) is not None


def cfg(**kw):
    base = dict(head_dim=128, page_size=64, rank=8, num_q_heads=32, num_kv_heads=8, token_budget=2048,
                kv_dtype=L.LK_BF16, scale=128 ** -0.5)
    base.update(kw)
    return L.make_config(**base)


def test_record_bytes_and_budget():
    assert L.lk_summary_record_bytes(cfg()) == 3328            # (128 + 8*128 + 64*8) * 2
    assert L.lk_summary_record_bytes(cfg(rank=4)) == 1792
    assert L.lk_summary_record_bytes(cfg(rank=16)) == 6400
    assert L.lk_summary_record_bytes(cfg(kv_dtype=L.LK_F32)) == 6656
    # int4 basis + int8 coefficients and centroid + fp16 scales, padded to 16 bytes:
    # 128 + 8*64 + 64*8 codes and 2*(64 + 8 + 1) scale bytes = 1298 -> 1312
    i4 = dict(summary_format=L.LK_SUMMARY_I4)
    assert L.lk_summary_record_bytes(cfg(**i4)) == 1312
    assert L.lk_summary_record_bytes(cfg(rank=4, **i4)) == 784      # 128 + 256 + 256 + 138 = 778
    assert L.lk_summary_record_bytes(cfg(rank=16, **i4)) == 2352    # 128 + 1024 + 1024 + 162 = 2338
    assert L.lk_summary_record_bytes(cfg(summary_format=5)) == 0
    assert L.lk_page_budget(cfg()) == 32
    assert L.lk_page_budget(cfg(token_budget=2049)) == 33
    assert L.lk_page_budget(cfg(token_budget=256)) == 4


def test_q4_record_packing():
    """The int4/int8 record the tests write and read is the one include/locks.h
    documents: int8 centroid, then each basis row in 32-bit words of 8 dims with
    dim 8 g + 2 j in nibble j and dim 8 g + 2 j + 1 in nibble j + 4 (two's
    complement), int8 coefficients, fp16 scales; packing round-trips."""
    import numpy as np
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    import reference as ref
    from oracle import locks_oracle as lo
    rng = np.random.default_rng(7)
    n, r, d, B = 3, 8, 128, 16
    qs = lo.QuantSummary(centroid_q=rng.integers(-127, 128, (n, d)), centroid_s=rng.uniform(0.5, 2, n),
                         basis_q=rng.integers(-7, 8, (n, r, d)), basis_s=rng.uniform(0.5, 2, (n, r)),
                         coeffs_q=rng.integers(-127, 128, (n, B, r)), coeffs_s=rng.uniform(0.5, 2, (n, B)),
                         eigvals=np.zeros((n, B)), r_eff=np.full(n, r))
    qs.centroid_s, qs.basis_s, qs.coeffs_s = (lo.fp16_round(x) for x in (qs.centroid_s, qs.basis_s, qs.coeffs_s))
    buf = ref.pack_q4_records(qs)
    assert buf.shape == (n, L.lk_summary_record_bytes(cfg(page_size=16, summary_format=L.LK_SUMMARY_I4)))
    o = ref.q4_offsets(d, B, r)
    assert (buf[:, :d].view(np.int8) == qs.centroid_q).all()
    w = buf[:, o["basis"]:o["coef"]].reshape(n, r, d // 8, 4).astype(np.uint32)
    word = w[..., 0] | (w[..., 1] << 8) | (w[..., 2] << 16) | (w[..., 3] << 24)
    dims = qs.basis_q.reshape(n, r, d // 8, 8)
    for j in range(4):
        assert (((word >> (4 * j)) & 0xF) == (dims[..., 2 * j] & 0xF)).all()
        assert (((word >> (16 + 4 * j)) & 0xF) == (dims[..., 2 * j + 1] & 0xF)).all()
    u = ref.unpack_q4_records(buf, d, B, r)
    for a, b in [(u.centroid_q, qs.centroid_q), (u.basis_q, qs.basis_q), (u.coeffs_q, qs.coeffs_q),
                 (u.centroid_s, qs.centroid_s), (u.basis_s, qs.basis_s), (u.coeffs_s, qs.coeffs_s)]:
        assert (a == b).all()
    text = open(HEADER).read()
    assert "dim 8g+2j in nibble j" in text and "8g+2j+1 in nibble j+4" in text


def test_page16_record_bytes_match_table_d10(golden_dir):
    """Quantized records at B = 16 hold Table D.10's logical payload (Locks App.
    D, "State accounting") plus the fp16 scales (B + r + 1 of them), padded to
    16 bytes; the shipped r8i4 record is about a tenth of the page's bf16 KV."""
    g = json.load(open(os.path.join(golden_dir, "table_d10_bytes.json")))
    for row in g["rows"]:
        if row["basis_bits"] != 4 or row["rank"] == 2:
            continue
        r = row["rank"]
        got = L.lk_summary_record_bytes(cfg(page_size=16, rank=r, summary_format=L.LK_SUMMARY_I4))
        assert got == (row["bytes"] + 2 * (16 + r + 1) + 15) // 16 * 16
    r8 = L.lk_summary_record_bytes(cfg(page_size=16, rank=8, summary_format=L.LK_SUMMARY_I4))
    assert r8 == 832 and abs((768 + 2 * 25) / g["kv_bytes"] - 0.10) < 0.001
    assert L.lk_summary_record_bytes(cfg(page_size=16)) == (128 + 8 * 128 + 16 * 8) * 2


def test_page16_is_accepted_by_every_entry_point():
    """16-token pages run the whole path: argument errors still come first at
    every entry point, a workspace is sized for them (its attention splits
    cover two pages per 32-token unit), and other page sizes are refused."""
    c16 = cfg(page_size=16)
    expect(L.LK_ERR_INVALID_ARG, L.lk_build_page_summary, c16, fake_cache(), None, 3, None, None, 0, 0)
    L.lk_build_page_summary(c16, fake_cache(), None, 0, None, None, 0, 0)
    ws16 = L.lk_workspace_size(c16, 2, 64)
    expect(L.LK_ERR_WORKSPACE, L.lk_score_select, c16, fake_cache(max_pages_per_seq=64), 2, FAKE, None, None,
           FAKE, FAKE, 0x100000, ws16 - 1, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_decode_step, c16, fake_cache(), 2, FAKE, None, FAKE, FAKE, None, None,
           None, 0x100000, 1 << 30, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_sparse_decode_attn, c16, fake_cache(), 2, FAKE, None, FAKE, FAKE, None,
           0x100000, 1 << 30, 0)
    for bad in (32, 8, 128):
        expect(L.LK_ERR_UNSUPPORTED, L.lk_build_page_summary, cfg(page_size=bad), fake_cache(), FAKE, 3, None,
               None, 0, 0)
        expect(L.LK_ERR_UNSUPPORTED, L.lk_workspace_size, cfg(page_size=bad), 1, 16)


def test_workspace_size_scales():
    a = L.lk_workspace_size(cfg(), 4, 2049)
    b = L.lk_workspace_size(cfg(), 8, 2049)
    assert 0 < a < b
    assert a % 256 == 0
    # holds at least the page scores (fp32, batch x Hq x pages) and the selections
    assert a >= 4 * 32 * 2049 * 4 + 4 * 8 * 32 * 4


@pytest.mark.parametrize("kw,pages", [
    (dict(), 2049), (dict(), 16400), (dict(token_budget=4096), 20000),
    (dict(num_q_heads=8, num_kv_heads=8), 9000), (dict(num_q_heads=64, num_kv_heads=8), 12000),
    (dict(summary_format=1), 16400), (dict(token_budget=128), 16400),
])
def test_workspace_for_a_batch_serves_every_smaller_batch(kw, pages):
    """A workspace sized for `batch` sequences serves calls with fewer: the
    size never shrinks as the batch grows, whichever selection path a batch
    size takes (wide tables with few (sequence, KV head) pairs are selected in
    chunks, which need candidate lists in the workspace)."""
    c = cfg(**kw)
    sizes = [L.lk_workspace_size(c, b, pages) for b in range(1, 40)]
    assert all(x <= y for x, y in zip(sizes, sizes[1:])), sizes
    assert all(x % 256 == 0 for x in sizes)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), L.LK_ERR_UNSUPPORTED),
    (dict(page_size=32), L.LK_ERR_UNSUPPORTED),
    (dict(rank=3), L.LK_ERR_UNSUPPORTED),
    (dict(rank=0), L.LK_ERR_INVALID_ARG),
    (dict(num_q_heads=30), L.LK_ERR_INVALID_ARG),
    (dict(num_q_heads=24), L.LK_ERR_UNSUPPORTED),      # G = 3
    (dict(token_budget=64), L.LK_ERR_INVALID_ARG),     # k = 1 < 2
    (dict(token_budget=64 * 2000), L.LK_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), L.LK_ERR_INVALID_ARG),
    (dict(scale=float("nan")), L.LK_ERR_INVALID_ARG),
    (dict(summary_format=2), L.LK_ERR_INVALID_ARG),
    (dict(summary_format=1, kv_dtype=0), L.LK_ERR_UNSUPPORTED),  # int4/int8 records need bf16 queries
    (dict(summary_format=1, rank=2), L.LK_ERR_UNSUPPORTED),
])
def test_config_rejected(kw, status):
    with pytest.raises(L.LocksError) as e:
        L.lk_workspace_size(cfg(**kw), 1, 16)
    assert e.value.status == status
    assert L.lk_last_error() != ""


def test_sizes_rejected_and_error_cleared():
    for batch, pages, st in [(0, 16, L.LK_ERR_INVALID_ARG), (1, 0, L.LK_ERR_INVALID_ARG),
                             (1, 30000, L.LK_ERR_UNSUPPORTED)]:
        with pytest.raises(L.LocksError) as e:
            L.lk_workspace_size(cfg(), batch, pages)
        assert e.value.status == st
    L.lk_workspace_size(cfg(), 1, 16)
    assert L.lk_last_error() == ""


def fake_cache(**kw):
    base = dict(k_pool=FAKE, v_pool=FAKE, summary_pool=FAKE, block_table=FAKE, seq_lens=FAKE,
                max_pages_per_seq=16, num_phys_pages=16)
    base.update(kw)
    return L.lk_cache(**base)


def expect(status, fn, *args):
    with pytest.raises(L.LocksError) as e:
        fn(*args)
    assert e.value.status == status, L.lk_last_error()


def test_entry_points_reject_bad_arguments():
    c = cfg()
    ws_need = L.lk_workspace_size(c, 2, 16)
    ws = 0x100000  # 256-aligned fake address
    # null pointers
    expect(L.LK_ERR_INVALID_ARG, L.lk_score_select, c, fake_cache(), 2, None, None, None, FAKE, FAKE, ws, ws_need, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_score_select, c, fake_cache(summary_pool=None), 2, FAKE, None, None, FAKE,
           FAKE, ws, ws_need, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_sparse_decode_attn, c, fake_cache(k_pool=None), 2, FAKE, FAKE, FAKE, FAKE,
           None, ws, ws_need, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_dense_decode_attn, c, fake_cache(block_table=None), 2, FAKE, FAKE, None, ws,
           ws_need, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_decode_step, c, fake_cache(), 2, FAKE, None, FAKE, FAKE, None, None, None,
           ws, ws_need, 0)
    # sel_pages without sel_count
    expect(L.LK_ERR_INVALID_ARG, L.lk_decode_step, c, fake_cache(), 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
           ws, ws_need, 0)
    # batch, table sizes
    expect(L.LK_ERR_INVALID_ARG, L.lk_score_select, c, fake_cache(), 0, FAKE, None, None, FAKE, FAKE, ws, ws_need, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_score_select, c, fake_cache(num_phys_pages=0), 2, FAKE, None, None, FAKE,
           FAKE, ws, ws_need, 0)
    # workspace too small / missing / misaligned
    expect(L.LK_ERR_WORKSPACE, L.lk_score_select, c, fake_cache(), 2, FAKE, None, None, FAKE, FAKE, ws,
           ws_need - 1, 0)
    expect(L.LK_ERR_WORKSPACE, L.lk_sparse_decode_attn, c, fake_cache(), 2, FAKE, FAKE, FAKE, FAKE, None, None,
           ws_need, 0)
    expect(L.LK_ERR_WORKSPACE, L.lk_dense_decode_attn, c, fake_cache(), 2, FAKE, FAKE, None, ws + 4, ws_need, 0)
    expect(L.LK_ERR_WORKSPACE, L.lk_decode_step, c, fake_cache(), 2, FAKE, FAKE, FAKE, FAKE, None, None, None,
           ws, 16, 0)
    # the decode step without a workspace argument: same validation, and a step
    # whose workspace would exceed the static buffer is refused before any launch
    expect(L.LK_ERR_INVALID_ARG, L.lk_decode_step_noalloc, c, fake_cache(), 2, FAKE, None, FAKE, FAKE, None, None,
           None, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_decode_step_noalloc, c, fake_cache(), 0, FAKE, FAKE, FAKE, FAKE, None, None,
           None, 0)
    expect(L.LK_ERR_WORKSPACE, L.lk_decode_step_noalloc, c, fake_cache(max_pages_per_seq=20000), 256, FAKE, FAKE,
           FAKE, FAKE, None, None, None, 0)
    # unsupported config through a compute entry point
    expect(L.LK_ERR_UNSUPPORTED, L.lk_score_select, cfg(head_dim=96), fake_cache(), 2, FAKE, None, None, FAKE,
           FAKE, ws, ws_need, 0)
    # build: negative count, null ids
    expect(L.LK_ERR_INVALID_ARG, L.lk_build_page_summary, c, fake_cache(), FAKE, -1, None, None, 0, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_build_page_summary, c, fake_cache(), None, 3, None, None, 0, 0)
    expect(L.LK_ERR_INVALID_ARG, L.lk_build_page_summary, c, fake_cache(summary_pool=None), FAKE, 3, None, None, 0, 0)
    # null config / cache
    lib = L.library()
    assert lib.lk_workspace_size(None, 1, 1, ctypes.byref(ctypes.c_size_t())) == L.LK_ERR_INVALID_ARG
    assert lib.lk_score_select(ctypes.byref(c), None, 1, FAKE, None, None, FAKE, FAKE, ws, ws_need, 0) == \
        L.LK_ERR_INVALID_ARG


def test_build_with_no_pages_is_a_no_op():
    # n_pages == 0 is valid and enqueues nothing
    L.lk_build_page_summary(cfg(), fake_cache(), None, 0, None, None, 0, 0)


def test_status_strings():
    for st in range(5):
        assert L.lk_status_string(st)
    assert L.lk_status_string(99) == "unknown status"


def test_single_hip_runtime_in_process():
    """liblocks.so binds to the HIP runtime torch loaded (one libamdhip64 mapped),
    so torch's streams and allocations are valid in its calls."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
