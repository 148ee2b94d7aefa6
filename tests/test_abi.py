"""The C-ABI library loads, exports every declared symbol and rejects bad arguments on the host
(no GPU needed: every check below returns before any HIP call)."""
import ctypes
import os
import re

import pytest

import hybrid_compressed_sparse_amd as hcs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hcs.h")

needs_lib = pytest.mark.skipif(not os.path.exists(hcs.LIB_PATH), reason="libhcs.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hcs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ["hcs_compress_kv", "hcs_index_topk", "hcs_sparse_mla_decode", "hcs_sparse_mla_prefill_chunk"]:
        assert n in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hcs.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert hcs.lib().hcs_abi_version() == 1


def _paged(fmt=0, dim=512, base=16, pt=16, stride=4, pages=8):
    return hcs.Paged(base, pt, stride, pages, fmt, dim)


@needs_lib
def test_validation_errors_before_any_launch():
    L = hcs.lib()
    # attention: unsupported head dim
    st = L.hcs_sparse_mla_decode(16, _paged(), _paged(), None, 0, 16, 16, None, 4, 64, 256, 128, 4, 100,
                                 0.1, 16, None, None, 0, None)
    assert st == 2 and b"d must be" in L.hcs_last_error()
    # attention: negative window
    st = L.hcs_sparse_mla_decode(16, _paged(), _paged(), None, 0, 16, 16, None, 4, 64, 512, -1, 4, 100,
                                 0.1, 16, None, None, 0, None)
    assert st == 1
    # attention: fp8_ds needs dim 512
    st = L.hcs_sparse_mla_decode(16, _paged(1, 128), _paged(1, 128), None, 0, 16, 16, None, 4, 64, 128,
                                 16, 4, 100, 0.1, 16, None, None, 0, None)
    assert st == 2
    # attention: page table too narrow for the positions
    st = L.hcs_sparse_mla_decode(16, _paged(stride=1), _paged(), None, 0, 16, 16, None, 4, 64, 512, 128,
                                 4, 100, 0.1, 16, None, None, 0, None)
    assert st == 1 and b"pt_stride" in L.hcs_last_error()
    # attention: workspace too small when the row list is split
    need = L.hcs_sparse_mla_workspace_size(4, 64, 512, 128, 4, 0, 2000)
    assert need > 0
    # (the size covers the plans of every row format; a split plan of 4 queries needs far more
    # than 4 KiB whatever the format)
    st = L.hcs_sparse_mla_decode(16, _paged(stride=32), _paged(stride=32), None, 0, 16, 16, None, 4, 64, 512,
                                 128, 4, 2000,
                                 0.1, 16, None, 256, 4096, None)
    assert st == 3
    # indexer: top-k limits and formats
    st = L.hcs_index_topk(16, None, 16, _paged(0, 128), 16, 16, 4, 64, 128, 4, 5000, 1000, 16, None,
                          None, 0, None)
    assert st == 2
    st = L.hcs_index_topk(16, None, 16, _paged(2, 128), 16, 16, 4, 64, 128, 4, 64, 1000, 16, None,
                          None, 0, None)
    assert st == 2 and b"q_scale" in L.hcs_last_error()
    st = L.hcs_index_topk(16, None, 16, _paged(0, 128), 16, 16, 4, 64, 128, 4, 64, 1000, 16, None,
                          None, 0, None)
    assert st == 3
    # at most 4194304 visible entries per query (m = 1: max_pos + 1 entries)
    st = L.hcs_index_topk(16, None, 16, _paged(0, 128, stride=70000), 16, 16, 4, 64, 128, 1, 64, 4194304, 16,
                          None, None, 0, None)
    assert st == 2 and b"visible entries" in L.hcs_last_error()
    st = L.hcs_index_topk(16, None, 16, _paged(0, 128, stride=70000), 16, 16, 4, 64, 128, 1, 64, 4194303, 16,
                          None, None, 0, None)
    assert st == 3
    # compressor: bad dtype, coarse m, wrong cache dim
    assert L.hcs_compress_kv(16, 16, 7, 512, 16, 16, 2, 4, 512, 4, None, 16, _paged(), None, 0, None) == 1
    assert L.hcs_compress_kv(16, 16, 1, 512, 16, 16, 2, 4, 512, 2000, None, 16, _paged(), None, 0, None) == 2
    assert L.hcs_compress_kv(16, 16, 1, 512, 16, 16, 2, 4, 512, 4, None, 16, _paged(0, 128), None, 0,
                             None) == 1
    # empty calls are fine and launch nothing
    assert L.hcs_compress_kv(None, None, 1, 0, None, None, 0, 0, 512, 4, None, None, _paged(), None, 0,
                             None) == 0


@needs_lib
def test_insert_validation_errors_before_any_launch():
    L = hcs.lib()
    f = L.hcs_qnorm_rope_kv_insert
    # q, H, kv, kv_stride, tok_seq, tok_pos, N, d, q_norm, eps, cos, sin, d_rope, rows, swa, stream
    assert f(16, 64, 16, 512, 16, 16, 4, 256, 0, 0.0, None, None, 0, 0, _paged(), None) == 2
    assert f(16, 64, 16, 512, 16, 16, 4, 512, 0, 0.0, 16, None, 64, 100, _paged(), None) == 1
    assert f(16, 64, 16, 512, 16, 16, 4, 512, 0, 0.0, 16, 16, 63, 100, _paged(), None) == 1
    assert f(16, 64, 16, 512, 16, 16, 4, 512, 1, -1.0, None, None, 0, 0, _paged(), None) == 1
    assert f(16, 64, 16, 500, 16, 16, 4, 512, 0, 0.0, None, None, 0, 0, _paged(), None) == 1   # stride < d
    assert f(16, 64, 16, 512, 16, 16, 4, 512, 0, 0.0, None, None, 0, 0, _paged(0, 128), None) == 1
    assert f(16, 64, 16, 128, 16, 16, 4, 128, 0, 0.0, None, None, 0, 0, _paged(1, 128), None) == 2  # fp8_ds at d 128
    assert f(16, 64, 16, 512, None, 16, 4, 512, 0, 0.0, None, None, 0, 0, _paged(), None) == 1  # no tok_seq
    assert f(18, 64, None, 0, None, 16, 4, 512, 0, 0.0, None, None, 0, 0, _paged(), None) == 1  # q misaligned
    # nothing to do
    assert f(None, 0, None, 0, None, None, 4, 512, 0, 0.0, None, None, 0, 0, _paged(), None) == 0
    assert f(None, 64, None, 0, None, None, 0, 512, 0, 0.0, None, None, 0, 0, _paged(), None) == 0


@needs_lib
def test_indexer_prep_validation_errors_before_any_launch():
    L = hcs.lib()
    q = L.hcs_indexer_q_prep
    # q, w, tok_pos, N, H_I, d_I, w_scale, cos, sin, d_rope, rows, out_fmt, q_out, q_scale_out, w_out, stream
    assert q(16, 16, 16, 4, 64, 64, 1.0, None, None, 0, 0, 0, 16, None, 16, None) == 2          # d_I
    assert q(16, 16, 16, 4, 65, 128, 1.0, None, None, 0, 0, 0, 16, None, 16, None) == 2         # H_I
    assert q(16, 16, 16, 4, 64, 128, 1.0, None, None, 0, 0, 1, 16, 16, 16, None) == 1           # fp8_ds out
    assert q(16, 16, 16, 4, 64, 128, 1.0, None, None, 0, 0, 2, 16, None, 16, None) == 1         # no scales
    assert q(16, 16, 16, 4, 64, 128, 1.0, 16, 16, 63, 10, 0, 16, None, 16, None) == 1           # odd d_rope
    assert q(16, 16, 16, 0, 64, 128, 1.0, None, None, 0, 0, 0, None, None, None, None) == 0     # empty
    k = L.hcs_indexer_k_store
    # k, k_stride, ent_seq, ent_idx, n, d_I, m, norm_w, eps, cos, sin, d_rope, rows, keys, stream
    assert k(16, 128, 16, 16, 4, 128, 0, 16, 1e-6, None, None, 0, 0, _paged(2, 128), None) == 1   # m
    assert k(16, 120, 16, 16, 4, 128, 4, 16, 1e-6, None, None, 0, 0, _paged(2, 128), None) == 1   # stride
    assert k(16, 128, 16, 16, 4, 128, 4, None, 1e-6, None, None, 0, 0, _paged(2, 128), None) == 1  # weight
    assert k(16, 128, 16, 16, 4, 128, 4, 16, 1e-6, None, None, 0, 0, _paged(1, 512), None) == 1   # dim
    assert k(16, 128, 16, 16, 4, 128, 4, 16, 1e-6, None, None, 0, 0, _paged(3, 64), None) == 1    # fp8ix dim
    assert k(16, 128, 16, 16, 0, 128, 4, 16, 1e-6, None, None, 0, 0, _paged(3, 128), None) == 0   # empty


@needs_lib
def test_candidate_filtering_validation_errors_before_any_launch():
    L = hcs.lib()
    f = L.hcs_index_topk_cand
    # q, q_scale, w, keys, q_seq, q_pos, N, H_I, d_I, m, topk, max_pos, cb, n_cand, cand_in, cand_out,
    # out_idx, out_score, ws, ws_bytes, stream
    k0 = _paged(0, 128)
    assert f(16, None, 16, k0, 16, 16, 4, 64, 128, 4, 64, 1000, 64, 8, None, None, 16, None, 16, 1 << 20, None) == 1
    assert f(16, None, 16, k0, 16, 16, 4, 64, 128, 4, 64, 1000, 64, 8, 16, 16, 16, None, 16, 1 << 20, None) == 1
    assert f(16, None, 16, k0, 16, 16, 4, 64, 128, 4, 64, 1000, 0, 8, 16, None, 16, None, 16, 1 << 20, None) == 1
    assert f(16, None, 16, k0, 16, 16, 4, 64, 128, 4, 64, 1000, 64, 5000, 16, None, 16, None, 16, 1 << 20, None) == 2
    # a source whose queries may see more than 32768 blocks
    assert f(16, None, 16, k0, 16, 16, 4, 64, 128, 1, 64, 40000, 1, 8, None, 16, 16, None, 16, 1 << 30, None) == 2
    need = L.hcs_index_topk_cand_workspace_size(4, 1000, 4, 64, 64, 8)
    assert need > L.hcs_index_topk_workspace_size(4, 1000, 4, 64)
    assert f(16, None, 16, k0, 16, 16, 4, 64, 128, 4, 64, 1000, 64, 8, 16, None, 16, None, 256, need - 1, None) == 3


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(hcs, "_lib", None)
    monkeypatch.setattr(hcs, "LIB_PATH", "/nonexistent/libhcs.so")
    with pytest.raises(hcs.HcsError):
        hcs.lib()


@needs_lib
def test_device_errors_rejects_null_before_any_hip_call():
    L = hcs.lib()
    assert L.hcs_device_errors(None, 1) == 1 and b"null bits" in L.hcs_last_error()


@needs_lib
def test_noalloc_rejects_plans_beyond_its_scratch_before_any_launch():
    L = hcs.lib()
    # 64 queries over 18528 rows each split nine ways: ~38 MB of partials, above the 32 MiB scratch
    need = L.hcs_sparse_mla_workspace_size(64, 64, 512, 128, 4, 0, 4 * 18400)
    assert need > (32 << 20)
    st = L.hcs_sparse_mla_decode_noalloc(16, _paged(stride=400), _paged(stride=400), None, 0, 16, 16, None, 64,
                                         64, 512, 128, 4, 4 * 18400, 0.1, 16, None, None)
    assert st == 3 and b"static scratch" in L.hcs_last_error()
