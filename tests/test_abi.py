"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
host-side validation rejects bad calls before anything is enqueued (no GPU)."""
import ctypes as C
import os
import re

import pytest

from compressed_sparse_attention_compress_amd import csa2 as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = K.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) <= set(K.EXPORTS), set(names) - set(K.EXPORTS)
    assert K.version().startswith("csa2-mi355x")


def test_status_strings():
    L = K.lib()
    for s in range(9):
        assert L.csa2_status_string(s)


def test_runtime_slots_start_empty_and_reset():
    rt = K.Runtime()
    for s in range(4):
        info = rt.slot(s)
        assert info.filled == 0 and info.generation == 0
    rt.reset()
    with pytest.raises(K.CSA2Error) as e:
        rt.slot(7)
    assert e.value.name == "CSA2_ERR_INVALID_ARG"
    rt.close()


def test_reuse_before_full_is_slot_empty():
    rt = K.Runtime()
    cfg = K.layer_cfg(K.REUSE, K.CSA2_BF16, m=2, k=512, W=128, H_I=32, H=64)
    io = K.LayerIO(B=1, T=1, L_w=128, q_pos=0x1000, q=0x1000, swa_kv=0x1000, swa_pos0=0x1000, o=0x1000)
    st = K.lib().csa2_layer_forward(rt.handle, C.byref(cfg), C.byref(io), None)
    assert K.STATUS[st] == "CSA2_ERR_SLOT_EMPTY"
    assert b"compress_kv" in K.lib().csa2_last_error()
    cfg.mode = K.REINDEX
    st = K.lib().csa2_layer_forward(rt.handle, C.byref(cfg), C.byref(io), None)
    assert K.STATUS[st] == "CSA2_ERR_SLOT_EMPTY"


def test_score_reindex_without_index_slot():
    rt = K.Runtime()
    a = K.ScoreTopkArgs(dtype=1, B=1, T=1, H_I=32, N_cap=10, n_entries=10, m=1, k=4, q_idx=0x1000, w=0x1000,
                        q_pos=0x1000, topk=0x1000, workspace=0x1000, workspace_bytes=1 << 20)
    st = K.lib().csa2_score_topk(rt.handle, C.byref(a), None)
    assert K.STATUS[st] == "CSA2_ERR_SLOT_EMPTY"
    st = K.lib().csa2_score_topk(None, C.byref(a), None)
    assert K.STATUS[st] == "CSA2_ERR_INVALID_ARG"


@pytest.mark.parametrize("field,value,status", [
    ("m", 3, "CSA2_ERR_INVALID_ARG"),
    ("w_gate", 0x1000, "CSA2_ERR_INVALID_ARG"),    # m == 1 must not have a gate
    ("T", 7, "CSA2_ERR_SHAPE"),
    ("D", 100, "CSA2_ERR_SHAPE"),
    ("N_cap", 3, "CSA2_ERR_SHAPE"),
    ("dtype", 9, "CSA2_ERR_DTYPE"),
    ("x", None, "CSA2_ERR_INVALID_ARG"),
])
def test_compress_validation(field, value, status):
    a = K.CompressArgs(dtype=1, B=1, T=8, D=64, m=1, start_pos=0, N_cap=8, eps=1e-6, rope_base=1e4, x=0x1000,
                       w_kv=0x1000, w_gate=None, gamma=0x1000, latent_pre=0x1000, kv_cache=0x1000)
    if field == "T":
        a.m, a.w_gate = 2, 0x1000
    setattr(a, field, value)
    st = K.lib().csa2_compress(None, C.byref(a), None)
    assert K.STATUS[st] == status, K.lib().csa2_last_error()


def test_compress_gated_needs_gate():
    a = K.CompressArgs(dtype=1, B=1, T=8, D=64, m=2, start_pos=0, N_cap=8, eps=1e-6, rope_base=1e4, x=0x1000,
                       w_kv=0x1000, w_gate=None, gamma=0x1000, latent_pre=0x1000, kv_cache=0x1000)
    assert K.STATUS[K.lib().csa2_compress(None, C.byref(a), None)] == "CSA2_ERR_INVALID_ARG"


def test_score_workspace_too_small():
    a = K.ScoreTopkArgs(dtype=1, B=1, T=1, H_I=32, N_cap=4096, n_entries=4096, m=1, k=512, q_idx=0x1000,
                        w=0x1000, codes=0x1000, scales=0x1000, q_pos=0x1000, topk=0x1000, workspace=0x1000,
                        workspace_bytes=16)
    st = K.lib().csa2_score_topk(None, C.byref(a), None)
    assert K.STATUS[st] == "CSA2_ERR_WORKSPACE"
    n = C.c_size_t()
    assert K.lib().csa2_workspace_size(K.OP_SCORE_TOPK, C.cast(C.byref(a), C.c_void_p), None, C.byref(n)) == 0
    assert n.value > 512 * 8


@pytest.mark.parametrize("field,value,status", [
    ("m", 3, "CSA2_ERR_INVALID_ARG"), ("state", None, "CSA2_ERR_INVALID_ARG"),
    ("w_gate", None, "CSA2_ERR_INVALID_ARG"), ("D", 100, "CSA2_ERR_SHAPE"), ("dtype", 9, "CSA2_ERR_DTYPE"),
    ("workspace_bytes", 1024, "CSA2_ERR_WORKSPACE"), ("workspace", 0x1008, "CSA2_ERR_WORKSPACE"),
    ("pos", None, "CSA2_ERR_INVALID_ARG"), ("scale_fmt", 2, "CSA2_ERR_INVALID_ARG"),
    ("scale_fmt", -1, "CSA2_ERR_INVALID_ARG"),
])
def test_compress_step_validation(field, value, status):
    a = K.CompressStepArgs(dtype=1, B=4, D=256, m=2, N_cap=100, eps=1e-6, rope_base=1e4, x=0x1000, pos=0x1000,
                           w_kv=0x1000, w_gate=0x1000, gamma=0x1000, w_ik=0x1000, state=0x1000, kv_cache=0x1000,
                           ik_codes=0x1000, ik_scales=0x1000, workspace=0x1000, workspace_bytes=1 << 20)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_compress_step(None, C.byref(a), None)] == status
    n = C.c_size_t()
    a.workspace_bytes = 0
    assert K.lib().csa2_workspace_size(K.OP_COMPRESS_STEP, C.cast(C.byref(a), C.c_void_p), None, C.byref(n)) == 0
    assert n.value == a.B * 1024 * 4 * 4


def test_compress_step_with_runtime_checks_the_entry_count():
    # with a runtime the step republishes the caches with n_entries, which must fit
    # the cache; an invalid call leaves the slots untouched (nothing is enqueued)
    rt = K.Runtime()
    a = K.CompressStepArgs(dtype=1, B=4, D=256, m=2, N_cap=100, eps=1e-6, rope_base=1e4, x=0x1000, pos=0x1000,
                           w_kv=0x1000, w_gate=0x1000, gamma=0x1000, w_ik=0x1000, state=0x1000, kv_cache=0x1000,
                           ik_codes=0x1000, ik_scales=0x1000, workspace=0x1000, workspace_bytes=1 << 20,
                           n_entries=101)
    assert K.STATUS[K.lib().csa2_compress_step(rt.handle, C.byref(a), None)] == "CSA2_ERR_SHAPE"
    a.n_entries = -1
    assert K.STATUS[K.lib().csa2_compress_step(rt.handle, C.byref(a), None)] == "CSA2_ERR_SHAPE"
    assert rt.slot(K.SLOT_COMPRESS_KV).filled == 0 and rt.slot(K.SLOT_INDEX_K).filled == 0


def test_workspace_must_be_16_byte_aligned():
    a = K.ScoreTopkArgs(dtype=1, B=1, T=1, H_I=32, N_cap=4096, n_entries=4096, m=1, k=512, q_idx=0x1000,
                        w=0x1000, codes=0x1000, scales=0x1000, q_pos=0x1000, topk=0x1000, workspace=0x1008,
                        workspace_bytes=1 << 30)
    assert K.STATUS[K.lib().csa2_score_topk(None, C.byref(a), None)] == "CSA2_ERR_WORKSPACE"
    # a one-query attention call uses row-split partials, so it needs a workspace
    b = K.SparseAttnArgs(dtype=1, B=1, T=1, H=64, N_cap=100, k=512, L_w=128, W=128, q=0x1000, kv=0x1000,
                         topk=0x1000, swa_kv=0x1000, swa_pos0=0x1000, q_pos=0x1000, o=0x1000, workspace=0x1004,
                         workspace_bytes=1 << 30)
    assert K.STATUS[K.lib().csa2_sparse_attn(None, C.byref(b), None)] == "CSA2_ERR_WORKSPACE"


@pytest.mark.parametrize("field,value,status", [
    ("H_I", 33, "CSA2_ERR_SHAPE"), ("k", 0, "CSA2_ERR_SHAPE"), ("k", 2000, "CSA2_ERR_SHAPE"),
    ("n_entries", 5000, "CSA2_ERR_SHAPE"), ("hsi", 5, "CSA2_ERR_INVALID_ARG"),
    ("scale_fmt", 2, "CSA2_ERR_INVALID_ARG"),
])
def test_score_validation(field, value, status):
    a = K.ScoreTopkArgs(dtype=1, B=1, T=1, H_I=32, N_cap=4096, n_entries=4096, m=1, k=512, q_idx=0x1000,
                        w=0x1000, codes=0x1000, scales=0x1000, q_pos=0x1000, topk=0x1000, workspace=0x1000,
                        workspace_bytes=1 << 30)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_score_topk(None, C.byref(a), None)] == status


def test_hsi_use_needs_candidates():
    rt = K.Runtime()
    a = K.ScoreTopkArgs(dtype=1, B=1, T=1, H_I=32, N_cap=4096, n_entries=4096, m=1, k=512, hsi=K.HSI_USE,
                        hsi_s=64, hsi_nb=256, q_idx=0x1000, w=0x1000, codes=0x1000, scales=0x1000, q_pos=0x1000,
                        topk=0x1000, workspace=0x1000, workspace_bytes=1 << 30)
    assert K.STATUS[K.lib().csa2_score_topk(rt.handle, C.byref(a), None)] == "CSA2_ERR_SLOT_EMPTY"
    a.hsi_s = 48
    assert K.STATUS[K.lib().csa2_score_topk(rt.handle, C.byref(a), None)] == "CSA2_ERR_SHAPE"


@pytest.mark.parametrize("field,value,status", [
    ("H", 65, "CSA2_ERR_SHAPE"), ("W", 0, "CSA2_ERR_SHAPE"), ("k", 1100, "CSA2_ERR_SHAPE"),
    ("q", None, "CSA2_ERR_INVALID_ARG"), ("kv", None, "CSA2_ERR_INVALID_ARG"),
    # rows and queries are read, and outputs written, 16 bytes at a time
    ("q", 0x1008, "CSA2_ERR_INVALID_ARG"), ("o", 0x1004, "CSA2_ERR_INVALID_ARG"),
    ("kv", 0x1002, "CSA2_ERR_INVALID_ARG"), ("swa_kv", 0x1008, "CSA2_ERR_INVALID_ARG"),
])
def test_attn_validation(field, value, status):
    a = K.SparseAttnArgs(dtype=1, B=1, T=1, H=64, N_cap=100, k=512, L_w=128, W=128, q=0x1000, kv=0x1000,
                         topk=0x1000, swa_kv=0x1000, swa_pos0=0x1000, q_pos=0x1000, o=0x1000)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_sparse_attn(None, C.byref(a), None)] == status


def test_fp4_pack_zero_rows_is_noop():
    assert K.lib().csa2_fp4_pack(None, 0, None, None, None) == 0
    assert K.STATUS[K.lib().csa2_fp4_pack(None, 5, None, None, None)] == "CSA2_ERR_INVALID_ARG"


@pytest.mark.parametrize("field,value,status", [
    ("kv_fmt", 2, "CSA2_ERR_INVALID_ARG"), ("kv_scales", None, "CSA2_ERR_INVALID_ARG"),
    ("kv", 0x1008, "CSA2_ERR_INVALID_ARG"), ("kv_scales", 0x2002, "CSA2_ERR_INVALID_ARG"),
])
def test_attn_fp4_kv_validation(field, value, status):
    a = K.SparseAttnArgs(dtype=1, B=1, T=1, H=64, N_cap=100, k=512, L_w=128, W=128, q=0x1000, kv=0x1000,
                         topk=0x1000, swa_kv=0x1000, swa_pos0=0x1000, q_pos=0x1000, o=0x1000,
                         kv_fmt=K.KV_FP4, kv_scales=0x2000)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_sparse_attn(None, C.byref(a), None)] == status


def test_fp4_kv_workspace_sizes():
    # few-query bf16: split partials for selected-row and window splits (at least
    # one of each); many queries or float32: the dequantised cache
    def ws(dtype, B, T, fp4, N_cap=1000):
        a = K.SparseAttnArgs(dtype=dtype, B=B, T=T, H=64, k=512, W=128, N_cap=N_cap,
                             kv_fmt=K.KV_FP4 if fp4 else K.KV_DENSE)
        n = C.c_size_t()
        assert K.lib().csa2_workspace_size(K.OP_SPARSE_ATTN, C.cast(C.byref(a), C.c_void_p), None, C.byref(n)) == 0
        return n.value
    assert ws(1, 64, 1, True) == ws(1, 64, 1, False)          # 4 splits either way
    assert ws(1, 300, 1, False) == 0 and ws(1, 300, 1, True) == 300 * 2 * 64 * 1028 + 256
    assert ws(1, 1, 1024, True) == 1000 * 512 * 2 + 256 and ws(1, 1, 1024, False) == 0
    assert ws(0, 2, 8, True) == 2 * 1000 * 512 * 4 + 256


@pytest.mark.parametrize("field,value", [("kv_fmt", 3), ("kv_scales", None)])
def test_compress_fp4_kv_validation(field, value):
    a = K.CompressArgs(dtype=1, B=1, T=4, D=64, m=2, start_pos=0, N_cap=8, eps=1e-6, rope_base=1e4, x=0x1000,
                       w_kv=0x1000, w_gate=0x1000, gamma=0x1000, latent_pre=0x1000, kv_cache=0x1000,
                       kv_fmt=K.KV_FP4, kv_scales=0x1000)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_compress(None, C.byref(a), None)] == "CSA2_ERR_INVALID_ARG"


def test_kv_fp4_pack_zero_rows_is_noop():
    assert K.lib().csa2_kv_fp4_pack(None, 0, None, None, None) == 0
    assert K.STATUS[K.lib().csa2_kv_fp4_pack(None, 5, None, None, None)] == "CSA2_ERR_INVALID_ARG"
    assert K.STATUS[K.lib().csa2_kv_fp4_pack(0x1008, 5, 0x1000, 0x1000, None)] == "CSA2_ERR_INVALID_ARG"


def test_noalloc_score_refuses_oversized_calls_and_workspaces():
    # host checks come before any device call: 512 queries over 8192 entries need a
    # 16 MiB key matrix + 256 B, more than the fixed scratch holds
    a = K.ScoreTopkArgs(dtype=1, B=1, T=512, H_I=32, N_cap=8192, n_entries=8192, m=1, k=512, q_idx=0x1000,
                        w=0x1000, codes=0x1000, scales=0x1000, q_pos=0x1000, topk=0x1000)
    assert K.STATUS[K.lib().csa2_score_topk_noalloc(None, C.byref(a), None)] == "CSA2_ERR_WORKSPACE"
    assert b"scratch" in K.lib().csa2_last_error()
    a.T, a.workspace, a.workspace_bytes = 1, 0x1000, 1 << 20
    assert K.STATUS[K.lib().csa2_score_topk_noalloc(None, C.byref(a), None)] == "CSA2_ERR_INVALID_ARG"


@pytest.mark.parametrize("field,value,status", [
    ("swa_fmt", 2, "CSA2_ERR_INVALID_ARG"), ("W", 129, "CSA2_ERR_SHAPE"), ("swa_kv", 0x1008, "CSA2_ERR_INVALID_ARG"),
])
def test_attn_fp8_window_ring_validation(field, value, status):
    # a ring serves windows of at most L_w rows and is read 16 bytes at a time
    a = K.SparseAttnArgs(dtype=1, B=1, T=1, H=64, N_cap=100, k=512, L_w=128, W=128, q=0x1000, kv=0x1000,
                         topk=0x1000, swa_kv=0x1000, swa_pos0=0x1000, q_pos=0x1000, o=0x1000,
                         swa_fmt=K.SWA_FP8_RING)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_sparse_attn(None, C.byref(a), None)] == status


def test_fp8_window_ring_workspace_sizes():
    # the ring's dense rows (B * L_w * 512 elements) and B int32 follow the other
    # workspace contents at a 256-byte boundary, except where the decode kernel
    # reads the ring itself (bf16, two or more row splits per query: 64 queries)
    def ws(dtype, B, T, ring, L_w=200):
        a = K.SparseAttnArgs(dtype=dtype, B=B, T=T, H=64, k=512, W=128, N_cap=1000, L_w=L_w,
                             swa_fmt=K.SWA_FP8_RING if ring else K.SWA_DENSE)
        n = C.c_size_t()
        assert K.lib().csa2_workspace_size(K.OP_SPARSE_ATTN, C.cast(C.byref(a), C.c_void_p), None, C.byref(n)) == 0
        return n.value
    assert ws(1, 300, 1, False) == 0 and ws(1, 300, 1, True) == 300 * 200 * 512 * 2 + 300 * 4 + 256
    base = ws(1, 64, 1, False)
    assert base > 0 and ws(1, 64, 1, True) == base
    assert ws(0, 2, 8, True, L_w=64) == 2 * 64 * 512 * 4 + 8 + 256


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, "CSA2_ERR_DTYPE"), ("L_w", 0, "CSA2_ERR_SHAPE"), ("T", -1, "CSA2_ERR_SHAPE"),
    ("rows", None, "CSA2_ERR_INVALID_ARG"), ("pos", None, "CSA2_ERR_INVALID_ARG"),
    ("ring", None, "CSA2_ERR_INVALID_ARG"), ("rows", 0x1008, "CSA2_ERR_INVALID_ARG"),
    ("ring", 0x1004, "CSA2_ERR_INVALID_ARG"),
])
def test_swa_append_validation(field, value, status):
    a = K.SwaAppendArgs(dtype=1, B=2, T=1, L_w=128, rows=0x1000, pos=0x1000, ring=0x1000)
    setattr(a, field, value)
    assert K.STATUS[K.lib().csa2_swa_append(C.byref(a), None)] == status


def test_swa_append_empty_is_noop():
    a = K.SwaAppendArgs(dtype=1, B=0, T=1, L_w=128)
    assert K.lib().csa2_swa_append(C.byref(a), None) == 0
    a = K.SwaAppendArgs(dtype=0, B=3, T=0, L_w=128)
    assert K.lib().csa2_swa_append(C.byref(a), None) == 0


def test_score_dump_must_be_aligned():
    a = K.ScoreTopkArgs(dtype=1, B=1, T=1, H_I=32, N_cap=100, n_entries=100, m=1, k=8, q_idx=0x1000, w=0x1000,
                        codes=0x1000, scales=0x1000, q_pos=0x1000, topk=0x1000, workspace=0x1000,
                        workspace_bytes=1 << 30, scores=0x1002)
    assert K.STATUS[K.lib().csa2_score_topk(None, C.byref(a), None)] == "CSA2_ERR_INVALID_ARG"


@pytest.mark.parametrize("fmt,status", [(0, "CSA2_OK"), (1, "CSA2_OK"), (2, "CSA2_ERR_INVALID_ARG"),
                                        (-3, "CSA2_ERR_INVALID_ARG")])
def test_index_k_scale_format_validation(fmt, status):
    # N = 0 enqueues nothing, so a valid format returns OK without a GPU
    a = K.IndexKArgs(dtype=1, B=2, N=0, m=1, entry0=0, N_cap=10, rope_base=1e4, latent_pre=0x1000, w_ik=0x1000,
                     codes=0x1000, scales=0x1000, scale_fmt=fmt)
    assert K.STATUS[K.lib().csa2_index_k(None, C.byref(a), None)] == status


def test_layer_rejects_a_bad_scale_format_before_enqueueing():
    rt = K.Runtime()
    cfg = K.layer_cfg(K.FULL, K.CSA2_BF16, m=1, k=64, W=16, H_I=32, H=16, scale_fmt=7)
    io = K.LayerIO(B=1, T=16, D=256, N_cap=16, x=0x1000, w_kv=0x1000, gamma=0x1000, w_ik=0x1000,
                   latent_pre=0x1000, kv_cache=0x1000, ik_codes=0x1000, ik_scales=0x1000, q_idx=0x1000, w=0x1000,
                   topk=0x1000, q_pos=0x1000, q=0x1000, swa_kv=0x1000, L_w=16, swa_pos0=0x1000, o=0x1000,
                   workspace=0x1000, workspace_bytes=1 << 30)
    assert K.STATUS[K.lib().csa2_layer_forward(rt.handle, C.byref(cfg), C.byref(io), None)] == "CSA2_ERR_INVALID_ARG"
    assert rt.slot(K.SLOT_INDEX_K).filled == 0 and rt.slot(K.SLOT_COMPRESS_KV).filled == 0
