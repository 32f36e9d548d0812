"""Host-only checks of the C ABI: the libraries load, export every declared
symbol, and reject bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_dkv_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = {"mla.h": "libmla.so", "mla_inputs.h": "libmla_inputs.so"}


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def _lib(name):
    path = os.path.join(ROOT, "mla_latent_kv_dkv_amd", name)
    if not os.path.exists(path):
        pytest.fail(f"{name} not built (run python -m mla_latent_kv_dkv_amd.build)")
    return ctypes.CDLL(path)


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_every_declared_symbol_is_exported(header):
    lib = _lib(HEADERS[header])
    names = _declared(header)
    assert names, header
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_the_five_decode_calls_are_declared():
    assert {"mla_append_latent", "mla_absorb_q", "mla_decode_attention", "mla_merge_lse",
            "mla_absorb_out"} <= set(_declared("mla.h"))


def _dims(**kw):
    base = dict(hidden=64, n_heads=4, d_head=16, d_latent=32, d_rope=8, dtype="f32")
    base.update(kw)
    return M.make_dims(**base)


def test_status_strings_and_version():
    lib = M.load()
    assert lib.mla_abi_version() == M.MLA_ABI_VERSION
    for s in (0, -1, -2, -3, -4, -5):
        assert M.mla_status_string(s) != "unknown status"


def test_workspace_bytes():
    d = _dims()
    assert M.mla_workspace_bytes(d, 8) >= 8 * 4 * 16 * 4
    # full shape, bf16: the intermediate plus room for the fp32 K-split partials
    full = M.make_dims(5120, 128, 128, 512, 64, "bf16")
    assert M.mla_workspace_bytes(full, 64) >= 64 * 128 * 128 * 2 + 64 * 24576 * 4
    assert M.mla_append_workspace_bytes(full, 64) >= 64 * 576 * 4
    assert M.mla_append_workspace_bytes(full, 0) == 0
    assert M.mla_append_workspace_bytes(d, 64) <= 256        # fp32 dims use the vector path
    assert M.mla_workspace_bytes(_dims(dtype="bf16"), 8) >= 8 * 4 * 16 * 2
    assert M.mla_workspace_bytes(_dims(d_rope=7), 8) == 0
    assert M.mla_workspace_bytes(d, -1) == 0


P = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def test_invalid_dims_are_rejected_without_launch():
    lib = M.load()
    cases = [(_dims(d_rope=7), -2), (_dims(page_size=48), -3), (_dims(hidden=0), -2),
             (_dims(rope_base=0.0), -2)]
    bad_abi = _dims()
    bad_abi.abi_version = 99
    cases.append((bad_abi, -3))
    bad_dtype = _dims()
    bad_dtype.dtype = 7
    cases.append((bad_dtype, -3))
    yarn_bad = [_dims(yarn=(40.0, 0, 1.0, 32.0)), _dims(yarn=(40.0, 4096, 32.0, 32.0)),
                _dims(yarn=(40.0, 4096, -1.0, 32.0)), _dims(yarn=(float("nan"), 4096, 1.0, 32.0))]
    cases += [(d, -2) for d in yarn_bad]
    for d, want in cases:
        got = lib.mla_decode_attention(ctypes.byref(d), P, P, P, 1, P, 1, P, 1, 1, P, P, None)
        assert got == want, (d.d_rope, d.page_size, got)
        assert lib.mla_merge_lse(ctypes.byref(d), P, P, 1, 1, P, None, None) == want
    assert lib.mla_decode_attention(None, P, P, P, 1, P, 1, P, 1, 1, P, P, None) == -1


def test_argument_checks():
    lib = M.load()
    d = _dims()
    # null pointers
    assert lib.mla_decode_attention(ctypes.byref(d), None, P, P, 1, P, 1, P, 1, 1, P, P, None) == -1
    assert lib.mla_merge_lse(ctypes.byref(d), P, None, 1, 1, P, None, None) == -1
    assert lib.mla_absorb_out(ctypes.byref(d), P, P, None, 1, P, P, 1 << 20, None) == -1
    assert lib.mla_append_latent(ctypes.byref(d), P, P, None, P, P, 1, P, 1, 1, P, 1, None, 0,
                                 None) == -1
    # counts
    assert lib.mla_decode_attention(ctypes.byref(d), P, P, P, 1, P, 1, P, 1, 0, P, P, None) == -2
    assert lib.mla_decode_attention(ctypes.byref(d), P, P, P, 1, P, 1, P, 1, 5000, P, P, None) == -2
    assert lib.mla_decode_attention(ctypes.byref(d), P, P, P, 1, P, 1, P, -1, 1, P, P, None) == -2
    assert lib.mla_merge_lse(ctypes.byref(d), P, P, 1, 0, P, None, None) == -2
    assert lib.mla_append_latent(ctypes.byref(d), P, P, P, P, P, -3, P, 1, 1, P, 1, None, 0,
                                 None) == -2
    # workspace
    assert lib.mla_absorb_q(ctypes.byref(d), P, P, P, P, P, 4, P, P, None, 1 << 20, None) == -4
    assert lib.mla_absorb_q(ctypes.byref(d), P, P, P, P, P, 4, P, P, P, 16, None) == -4
    assert lib.mla_absorb_out(ctypes.byref(d), P, P, P, 4, P, P, 16, None) == -4
    misaligned = ctypes.c_void_p(0x1008)
    assert lib.mla_absorb_q(ctypes.byref(d), P, P, P, P, P, 4, P, P, misaligned, 1 << 20,
                            None) == -4
    assert lib.mla_absorb_out(ctypes.byref(d), P, P, P, 4, P, misaligned, 1 << 20, None) == -4
    # compressed query: rank, pointers, workspace
    lib.mla_absorb_q_cq.argtypes = [ctypes.POINTER(M.MlaDims), ctypes.c_int32] + \
        [ctypes.c_void_p] * 6 + [ctypes.c_int32] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t,
                                                                              ctypes.c_void_p]
    cq = ctypes.byref(d)
    assert lib.mla_absorb_q_cq(cq, 0, P, P, P, P, P, P, 4, P, P, P, 1 << 20, None) == -2
    assert lib.mla_absorb_q_cq(cq, 7, P, P, P, P, P, P, 4, P, P, P, 1 << 20, None) == -2
    assert lib.mla_absorb_q_cq(cq, 24, P, None, P, P, P, P, 4, P, P, P, 1 << 20, None) == -1
    assert lib.mla_absorb_q_cq(cq, 24, P, P, P, P, P, P, 4, P, P, P, 16, None) == -4
    assert lib.mla_absorb_q_cq(cq, 24, P, P, P, P, P, P, 4, P, P, misaligned, 1 << 20, None) == -4
    assert lib.mla_absorb_q_cq(cq, 24, None, None, None, None, None, None, 0, None, None, None,
                               0, None) == 0
    assert M.mla_workspace_bytes_cq(d, 24, 8) >= M.mla_workspace_bytes(d, 8) + 8 * 24 * 4
    assert M.mla_workspace_bytes_cq(d, 0, 8) == 0 and M.mla_workspace_bytes_cq(d, 5, 8) == 0
    # fused query + append: (dims, h, w_q, w_qr, w_uk, w_dkv, w_kr, pos, row_seq, batch,
    # table, n_seqs, max_pages, pool, num_pages, q_lat, q_pe, ws, ws_bytes, stream)
    qa = lib.mla_absorb_q_append
    big = 1 << 20
    assert qa(ctypes.byref(d), P, P, P, P, None, P, P, P, 4, P, 1, 1, P, 1, P, P, P, big, None) == -1
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, None, 4, P, 1, 1, P, 1, P, P, P, big, None) == -1
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, 4, P, 1, 1, None, 1, P, P, P, big, None) == -1
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, -2, P, 1, 1, P, 1, P, P, P, big, None) == -2
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, 4, P, 0, 1, P, 1, P, P, P, big, None) == -2
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, 4, P, 1, 0, P, 1, P, P, P, big, None) == -2
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 0, P, P, P, big, None) == -2
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 1, P, P, P, 16, None) == -4
    assert qa(ctypes.byref(d), P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 1, P, P, misaligned, big,
              None) == -4
    assert qa(ctypes.byref(d), None, None, None, None, None, None, None, None, 0, None, 0, 0, None,
              0, None, None, None, 0, None) == 0
    # empty batches are no-ops that never touch the pointers
    assert lib.mla_absorb_q(ctypes.byref(d), None, None, None, None, None, 0, None, None, None, 0,
                            None) == 0
    assert lib.mla_append_latent(ctypes.byref(d), None, None, None, None, None, 0, None, 0, 0, None,
                                 0, None, 0, None) == 0


def test_fp8_pool_sizes_and_argument_checks():
    lib = M.load()
    full = M.make_dims(5120, 128, 128, 512, 64, "bf16")
    # [512 e4m3 | 64 bf16] rows of 640 bytes, 64 of them, then 64 fp32 scales
    assert M.mla_fp8_page_bytes(full) == 64 * 640 + 64 * 4 == 41216
    assert M.mla_fp8_page_bytes(_dims(page_size=1)) == 32 + 16 + 4
    assert M.mla_fp8_page_bytes(_dims(d_latent=36)) == 0          # d_c must be a multiple of 8
    assert M.mla_fp8_page_bytes(_dims(d_rope=7)) == 0
    assert M.mla_append_workspace_bytes_fp8(full, 64) >= 64 * 576 * 4
    assert M.mla_append_workspace_bytes_fp8(full, 0) == 0
    d = ctypes.byref(_dims())
    d36 = ctypes.byref(_dims(d_latent=36))
    misaligned = ctypes.c_void_p(0x1008)
    # quantize_rows: (dims, rows, ld_rows, seq, pos, n, table, n_seqs, max_pages, pool, pages, stream)
    assert lib.mla_quantize_rows_fp8(d36, P, 44, P, P, 1, P, 1, 1, P, 1, None) == -3
    assert lib.mla_quantize_rows_fp8(d, P, 39, P, P, 1, P, 1, 1, P, 1, None) == -2   # ld < d_c + d_R
    assert lib.mla_quantize_rows_fp8(d, P, 42, P, P, 1, P, 1, 1, P, 1, None) == -2   # ld % 4
    assert lib.mla_quantize_rows_fp8(d, P, 40, P, P, -1, P, 1, 1, P, 1, None) == -2
    assert lib.mla_quantize_rows_fp8(d, None, 40, P, P, 1, P, 1, 1, P, 1, None) == -1
    assert lib.mla_quantize_rows_fp8(d, misaligned, 40, P, P, 1, P, 1, 1, P, 1, None) == -3
    assert lib.mla_quantize_rows_fp8(d, P, 40, P, P, 1, P, 1, 1, misaligned, 1, None) == -3
    assert lib.mla_quantize_rows_fp8(d, None, 40, None, None, 0, None, 0, 0, None, 0, None) == 0
    # append_fp8
    assert lib.mla_append_latent_fp8(d36, P, P, P, P, P, 1, P, 1, 1, P, 1, P, 1 << 20, None) == -3
    assert lib.mla_append_latent_fp8(d, P, P, None, P, P, 1, P, 1, 1, P, 1, P, 1 << 20, None) == -1
    assert lib.mla_append_latent_fp8(d, P, P, P, P, P, 4, P, 1, 1, P, 1, P, 64, None) == -4
    assert lib.mla_append_latent_fp8(d, P, P, P, P, P, 4, P, 1, 1, P, 1, misaligned, 1 << 20,
                                     None) == -4
    assert lib.mla_append_latent_fp8(d, P, P, P, P, P, 4, P, 1, 1, misaligned, 1, P, 1 << 20,
                                     None) == -3
    assert lib.mla_append_latent_fp8(d, None, None, None, None, None, 0, None, 0, 0, None, 0, None,
                                     0, None) == 0
    # fused query + FP8 append: (dims, h, w_q, w_qr, w_uk, w_dkv, w_kr, pos, row_seq, batch,
    # table, n_seqs, max_pages, pool, num_pages, q_lat, q_pe, ws, ws_bytes, stream)
    qa = lib.mla_absorb_q_append_fp8
    big = 1 << 20
    assert qa(d36, P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 1, P, P, P, big, None) == -3
    assert qa(d, P, P, P, P, None, P, P, P, 4, P, 1, 1, P, 1, P, P, P, big, None) == -1
    assert qa(d, P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 1, None, P, P, big, None) == -1
    assert qa(d, P, P, P, P, P, P, P, P, -1, P, 1, 1, P, 1, P, P, P, big, None) == -2
    assert qa(d, P, P, P, P, P, P, P, P, 4, P, 0, 1, P, 1, P, P, P, big, None) == -2
    assert qa(d, P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 1, P, P, P, 64, None) == -4
    assert qa(d, P, P, P, P, P, P, P, P, 4, P, 1, 1, P, 1, P, P, misaligned, big, None) == -4
    assert qa(d, P, P, P, P, P, P, P, P, 4, P, 1, 1, misaligned, 1, P, P, P, big, None) == -3
    assert qa(d, None, None, None, None, None, None, None, None, 0, None, 0, 0, None, 0, None,
              None, None, 0, None) == 0
    need = M.mla_absorb_q_append_fp8_workspace_bytes(full, 64)
    assert need >= M.mla_workspace_bytes(full, 64) + 64 * 576 * 4
    assert need >= M.mla_append_workspace_bytes_fp8(full, 64)
    assert M.mla_absorb_q_append_fp8_workspace_bytes(_dims(d_latent=36), 4) == 0
    # attention_fp8: the same checks as the plain call, plus the FP8 format's
    assert lib.mla_decode_attention_fp8(d36, P, P, P, 1, P, 1, P, 1, 1, P, P, None) == -3
    assert lib.mla_decode_attention_fp8(d, None, P, P, 1, P, 1, P, 1, 1, P, P, None) == -1
    assert lib.mla_decode_attention_fp8(d, P, P, P, 1, P, 1, P, 1, 0, P, P, None) == -2
    assert lib.mla_decode_attention_fp8(d, None, None, None, 1, None, 1, None, 0, 1, None, None,
                                        None) == 0


def test_prefill_attention_argument_checks():
    lib = M.load()
    d = ctypes.byref(_dims())
    # (dims, q_lat, q_pe, pool, pages, table, n_seqs, max_pages, q_seq, q_pos, n_q, S, o, lse, stream)
    assert lib.mla_prefill_attention(d, P, P, P, 1, P, 0, 1, P, P, 4, 1, P, P, None) == -2  # n_seqs
    assert lib.mla_prefill_attention(d, P, P, P, 1, P, 1, 1, None, P, 4, 1, P, P, None) == -1
    assert lib.mla_prefill_attention(d, P, P, P, 1, P, 1, 1, P, None, 4, 1, P, P, None) == -1
    assert lib.mla_prefill_attention(d, P, P, P, 1, P, 1, 1, P, P, 4, 0, P, P, None) == -2  # splits
    assert lib.mla_prefill_attention(d, P, P, P, 1, P, 1, 1, P, P, 70000, 1, P, P, None) == -2
    assert lib.mla_prefill_attention(d, None, None, None, 1, None, 1, 1, None, None, 0, 1, None,
                                     None, None) == 0
    d36 = ctypes.byref(_dims(d_latent=36))
    assert lib.mla_prefill_attention_fp8(d36, P, P, P, 1, P, 1, 1, P, P, 4, 1, P, P, None) == -3
    # the decode call still wants its lengths
    assert lib.mla_decode_attention(d, P, P, P, 1, P, 1, None, 1, 1, P, P, None) == -1


def test_device_fill_argument_checks():
    lib = _lib("libmla_inputs.so")
    lib.mla_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p]
    assert lib.mla_fill_normal(None, 0, 0, 1, 0, 1.0, None) == 0
    assert lib.mla_fill_normal(None, 5, 0, 1, 0, 1.0, None) == -1
    assert lib.mla_fill_normal(P, 5, 9, 1, 0, 1.0, None) == -3


def test_merge_absorb_out_argument_checks():
    lib = M.load()
    d = _dims(dtype="bf16")
    dp = ctypes.byref(d)
    misaligned = ctypes.c_void_p(0x1008)
    big = 1 << 24
    need = M.mla_merge_absorb_out_workspace_bytes(d, 8)
    # room for mla_absorb_out's scratch and one fp32 o_lat
    assert need >= M.mla_workspace_bytes(d, 8) + 8 * d.n_heads * d.d_latent * 4
    assert M.mla_merge_absorb_out_workspace_bytes(d, -1) == 0
    assert M.mla_merge_absorb_out_workspace_bytes(_dims(d_rope=7), 8) == 0
    # (dims, o_part, lse_part, batch, num_splits, plan, n_units, w_uv, w_o, u, lse, ws, bytes, stream)
    f = lib.mla_merge_absorb_out
    assert f(dp, P, P, -1, 2, None, 0, P, P, P, None, P, big, None) == -2
    assert f(dp, P, P, 8, 0, None, 0, P, P, P, None, P, big, None) == -2     # no splits
    assert f(dp, P, P, 8, 0, P, 7, P, P, P, None, P, big, None) == -2        # plan of 7 units
    assert f(dp, P, P, 8, 0, P, 12, P, P, P, None, P, big, None) == -2       # not a multiple of 8
    assert f(dp, None, P, 8, 2, None, 0, P, P, P, None, P, big, None) == -1
    assert f(dp, P, P, 8, 2, None, 0, P, None, P, None, P, big, None) == -1
    assert f(dp, P, P, 8, 2, None, 0, P, P, P, None, P, need - 1, None) == -4
    assert f(dp, P, P, 8, 2, None, 0, P, P, P, None, misaligned, big, None) == -4
    assert f(dp, None, None, 0, 2, None, 0, None, None, None, None, None, 0, None) == 0
