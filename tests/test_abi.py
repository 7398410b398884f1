"""Host-only checks of the C ABI: the library loads, exports every entry point
include/moba.h declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

from block_sparse_long_moba_amd import moba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "moba.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_\w+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = moba.lib()
    declared = header_functions()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(declared) == sorted(moba.EXPORTS), "binding and header disagree"


def shape(T=4096, S=1, Hq=32, Hkv=8, d=128, dtype="bf16", max_seqlen=0):
    return moba.make_shape(T, S, Hq, Hkv, d, dtype, max_seqlen)


def status_of(fn, *args):
    try:
        fn(*args)
    except moba.MobaError as e:
        return e.status, str(e)
    return 0, ""


def test_plan_sizes_and_offsets_are_consistent():
    sh = shape(T=1 << 20)
    lay = moba.moba_plan(sh, 4096, 12, 1)
    assert lay.kv_heads_per_pass == 1 and lay.q_heads_per_pass == 4
    assert lay.num_blocks_bound == 256 + 1
    offs = [lay.table_offset, lay.kbar_offset, lay.vt_offset, lay.idx_offset, lay.bins_offset,
            lay.items_offset, lay.part_o_offset, lay.part_lse_offset, lay.total_bytes]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    slots = (1 << 20) * 4 * 12
    assert lay.part_lse_offset - lay.part_o_offset >= slots * 128 * 2  # bf16 partials
    assert lay.total_bytes == moba.moba_fwd_workspace_size(sh, 4096, 12, 1)
    full = moba.moba_plan(sh, 4096, 12, 0)
    assert full.kv_heads_per_pass == 8 and full.total_bytes > lay.total_bytes
    # pass sizes are divisors of the kv head count
    assert moba.moba_plan(sh, 4096, 12, 3).kv_heads_per_pass == 2
    assert moba.moba_plan(sh, 4096, 12, 6).kv_heads_per_pass == 4


@pytest.mark.parametrize("kw,B,k,expect", [
    (dict(Hq=30, Hkv=8), 4096, 12, 1),       # Hq not a multiple of Hkv
    (dict(d=64), 4096, 12, 2),               # head_dim other than 128
    (dict(), 4000, 12, 2),                   # block size not a multiple of 64
    (dict(), 0, 12, 1),                      # block size 0
    (dict(), 4096, 0, 1),                    # topk 0
    (dict(T=1 << 20), 64, 40, 2),            # topk-1 > 32 with more blocks than topk
    (dict(T=-1), 4096, 12, 1),               # negative length
    (dict(T=10, S=0), 4096, 12, 1),          # tokens without sequences
    (dict(T=1 << 31), 4096, 12, 2),          # too many tokens
    (dict(dtype=7), 4096, 12, 1),            # unknown dtype
])
def test_plan_rejects_bad_shapes(kw, B, k, expect):
    st, msg = status_of(moba.moba_plan, shape(**kw), B, k)
    assert st == expect, msg
    assert msg


def test_large_topk_is_fine_when_it_covers_every_block():
    lay = moba.moba_plan(shape(T=4096, max_seqlen=4096), 64, 64)
    assert lay.total_bytes > 0


def test_entry_points_reject_null_arguments_without_a_device():
    L = moba.lib()
    sh = shape()
    lay = moba.moba_plan(sh, 4096, 12)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    null = None
    # moba_fwd: null q
    assert L.moba_fwd(null, fake, fake, fake, ctypes.byref(sh), 4096, 12, fake, null, null) == 1
    # moba_fwd: null cu_seqlens
    assert L.moba_fwd(fake, fake, fake, null, ctypes.byref(sh), 4096, 12, fake, null, null) == 1
    # moba_fwd_ex: workspace too small is reported before any launch
    assert L.moba_fwd_ex(fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, 0.0, fake, null,
                         fake, 16, null) == 3
    assert b"workspace" in L.moba_last_error()
    # negative softmax scale
    assert L.moba_fwd_ex(fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, -1.0, fake, null,
                         fake, 1 << 40, null) == 1
    # stage entry points: mismatched layout
    other = moba.moba_plan(shape(T=8192), 4096, 12)
    assert L.moba_gate(fake, ctypes.byref(sh), 4096, 12, ctypes.byref(other), fake, 0, null) == 1
    # kv_head_begin not aligned to the pass
    lay1 = moba.moba_plan(sh, 4096, 12, 2)
    assert L.moba_gate(fake, ctypes.byref(sh), 4096, 12, ctypes.byref(lay1), fake, 1, null) == 1
    assert L.moba_merge(ctypes.byref(sh), 4096, 12, ctypes.byref(lay), fake, 0, null, null,
                        null) == 1
    # the merged own-block stage: null out, bad scale, kv_head_begin off the pass
    assert L.moba_attn_fwd_own_merge(fake, fake, ctypes.byref(sh), 4096, 12, 0.0,
                                     ctypes.byref(lay), fake, 0, null, null, null) == 1
    assert b"out" in L.moba_last_error()
    assert L.moba_attn_fwd_own_merge(fake, fake, ctypes.byref(sh), 4096, 12, -1.0,
                                     ctypes.byref(lay), fake, 0, fake, null, null) == 1
    assert L.moba_attn_fwd_own_merge(fake, fake, ctypes.byref(sh), 4096, 12, 0.0,
                                     ctypes.byref(lay1), fake, 1, fake, null, null) == 1
    # the value-transpose stage: null v, mismatched layout
    assert L.moba_attn_prep(fake, null, ctypes.byref(sh), 4096, 12, ctypes.byref(lay), fake, 0,
                            null) == 1
    assert L.moba_attn_prep(fake, fake, ctypes.byref(sh), 4096, 12, ctypes.byref(other), fake, 0,
                            null) == 1
    # dense: bad scale / too small workspace
    assert L.moba_dense_causal_fwd(fake, fake, fake, fake, ctypes.byref(sh), float("nan"), fake,
                                   null, null, 0, null) == 1
    assert L.moba_dense_causal_fwd(fake, fake, fake, fake, ctypes.byref(sh), 0.0, fake, null,
                                   fake, 8, null) == 3


def test_empty_problem_is_a_no_op():
    L = moba.lib()
    sh = shape(T=0, S=0)
    assert L.moba_fwd(None, None, None, None, ctypes.byref(sh), 4096, 12, None, None, None) == 0
    assert L.moba_dense_causal_fwd(None, None, None, None, ctypes.byref(sh), 0.0, None, None,
                                   None, 0, None) == 0


def test_workspace_status_rejects_bad_arguments_without_a_device():
    L = moba.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert L.moba_workspace_status(2, None, None) == 1
    assert "workspace" in L.moba_last_error().decode()
    assert L.moba_workspace_status(-1, fake, None) == 1
    assert "num_seqs" in L.moba_last_error().decode()


def test_noalloc_capacity_matches_the_header():
    import re
    hdr = open(os.path.join(ROOT, "include", "moba.h")).read()
    m = re.search(r"#define MOBA_NOALLOC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == moba.NOALLOC_WORKSPACE_BYTES


def test_status_strings():
    L = moba.lib()
    for code, name in moba.STATUS.items():
        assert L.moba_status_string(code).decode() == name


def test_gate_variant_validation():
    L = moba.lib()
    sh = shape()
    lay = moba.moba_plan(sh, 4096, 12)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # window: n_sink must lie in [0, topk)
    assert L.moba_gate_window(ctypes.byref(sh), 4096, 12, 12, ctypes.byref(lay), fake, 0,
                              None) == 1
    assert L.moba_gate_window(ctypes.byref(sh), 4096, 12, -1, ctypes.byref(lay), fake, 0,
                              None) == 1
    # pooled: the own block needs a slot; extras are bounded
    assert L.moba_gate_pooled(fake, ctypes.byref(sh), 4096, 12, 6, 6, ctypes.byref(lay), fake,
                              0, None) == 1
    assert L.moba_gate_pooled(fake, ctypes.byref(sh), 4096, 12, 17, 0, ctypes.byref(lay), fake,
                              0, None) == 2
    assert L.moba_gate_pooled(None, ctypes.byref(sh), 4096, 12, 1, 1, ctypes.byref(lay), fake,
                              0, None) == 1
    # moba_fwd_gated: NULL gate, unknown kind
    assert L.moba_fwd_gated(fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, None, 0.0, fake,
                            None, fake, 1 << 40, None) == 1
    bad = moba.Gate(7, 0, 0, 0)
    assert L.moba_fwd_gated(fake, fake, fake, fake, ctypes.byref(sh), 4096, 12,
                            ctypes.byref(bad), 0.0, fake, None, fake, 1 << 40, None) == 1
    assert b"gate" in L.moba_last_error()


def test_decode_validation_and_sizes():
    L = moba.lib()
    cache = shape(T=1 << 20, S=1)
    n = moba.moba_decode_workspace_size(cache, 4096, 12)
    assert n > 0
    # workspace grows with topk (slots), and a dense topk is accepted for decode
    assert moba.moba_decode_workspace_size(cache, 4096, 256) > n
    fake = ctypes.c_void_p(0x1000)
    assert L.moba_decode(fake, fake, fake, ctypes.byref(cache), 4096, 12, 0.0, fake, None, fake,
                         16, None) == 3
    assert L.moba_decode(None, fake, fake, ctypes.byref(cache), 4096, 12, 0.0, fake, None, fake,
                         n, None) == 1
    assert L.moba_decode(fake, fake, fake, ctypes.byref(cache), 4096, 0, 0.0, fake, None, fake,
                         n, None) == 1
    assert L.moba_decode_prepare(fake, None, ctypes.byref(cache), 4096, 12, fake, n, None) == 1
    # no sequences: nothing to do
    empty = shape(T=0, S=0)
    assert L.moba_decode(None, None, None, ctypes.byref(empty), 4096, 12, 0.0, None, None, None,
                         moba.moba_decode_workspace_size(empty, 4096, 12), None) == 0


def test_bwd_plan_and_validation():
    L = moba.lib()
    sh = shape(T=1 << 20)
    f = moba.moba_plan(sh, 4096, 12, 1)
    b = moba.moba_bwd_plan(sh, 4096, 12, 1)
    # shared regions coincide; the partial-dq region holds fp32 rows
    for name in ("table_offset", "kbar_offset", "vt_offset", "idx_offset", "bins_offset",
                 "items_offset", "part_o_offset"):
        assert getattr(f, name) == getattr(b, name), name
    slots = (1 << 20) * 4 * 12
    assert b.part_lse_offset - b.part_o_offset >= slots * 128 * 4
    assert b.total_bytes - b.part_lse_offset >= (1 << 20) * 32 * 4
    assert b.total_bytes == moba.moba_bwd_workspace_size(sh, 4096, 12, 1)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    null = None
    n = b.total_bytes
    # fp32 is unsupported
    sh32 = shape(T=4096, dtype="fp32")
    assert L.moba_bwd(fake, fake, fake, fake, fake, fake, fake, ctypes.byref(sh32), 4096, 12, null,
                      0.0, fake, fake, fake, fake, 1 << 40, null) == 2
    # missing gradients, too small a workspace
    assert L.moba_bwd(fake, fake, fake, fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, null,
                      0.0, null, fake, fake, fake, n, null) == 1
    assert L.moba_bwd(fake, fake, fake, fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, null,
                      0.0, fake, fake, fake, fake, 16, null) == 3
    # stage entry points: a forward plan is not a backward plan, and vice versa
    assert L.moba_attn_bwd_dkdv(fake, fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, 0.0,
                                ctypes.byref(f), fake, 0, fake, fake, null) == 1
    assert L.moba_attn_fwd_hist(fake, fake, ctypes.byref(sh), 4096, 12, 0.0, ctypes.byref(b),
                                fake, 0, null) == 1
    assert L.moba_attn_fwd_own_merge(fake, fake, ctypes.byref(sh), 4096, 12, 0.0,
                                     ctypes.byref(b), fake, 0, fake, null, null) == 1
    assert L.moba_attn_bwd_dq(fake, fake, fake, fake, fake, ctypes.byref(sh), 4096, 12, 0.0,
                              ctypes.byref(b), fake, 0, 4, null) == 1
    # the gate and dispatch stages take either plan: the layout check passes and
    # a kv_head_begin that is not a multiple of the pass size stops them before
    # any launch
    b2 = moba.moba_bwd_plan(sh, 4096, 12, 2)
    assert L.moba_dispatch(ctypes.byref(sh), 4096, 12, ctypes.byref(b2), fake, 1, null) == 1
    assert b"multiple" in L.moba_last_error()
    empty = shape(T=0, S=0)
    assert L.moba_bwd(null, null, null, null, null, null, null, ctypes.byref(empty), 4096, 12,
                      null, 0.0, null, null, null, null,
                      moba.moba_bwd_workspace_size(empty, 4096, 12, 0), null) == 0


def test_strided_forward_validation_without_a_device():
    L = moba.lib()
    sh = shape()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first

    def call(st, q=fake, out=fake, sh=sh):
        return L.moba_fwd_strided(q, fake, fake, fake, ctypes.byref(sh),
                                  None if st is None else ctypes.byref(st), 4096, 12, None, 0.0,
                                  out, None, fake, 16, None)

    d = 128
    contiguous = moba.Strides(32 * d, d, 8 * d, d, 8 * d, d, 32 * d, d)
    # valid strides reach the workspace check (status 3), invalid ones stop before it
    assert call(None) == 3
    assert call(contiguous) == 3
    fused = moba.Strides(48 * d, d, 48 * d, d, 48 * d, d, 32 * d, d)  # views of one qkv tensor
    assert call(fused) == 3
    head_major_out = moba.Strides(32 * d, d, 8 * d, d, 8 * d, d, d, 4096 * d)
    assert call(head_major_out) == 3
    for bad in (moba.Strides(32 * d, 4, 8 * d, d, 8 * d, d, 32 * d, d),    # 8 bytes
                moba.Strides(-32 * d, d, 8 * d, d, 8 * d, d, 32 * d, d),   # negative
                moba.Strides(32 * d, d, 8 * d, 0, 8 * d, d, 32 * d, d),    # zero
                moba.Strides(32 * d, d, 8 * d, d, 8 * d, d, 32 * d, 64),   # heads overlap
                moba.Strides(32 * d, d, 8 * d, d, 8 * d, d, 31 * d, d)):   # rows overlap
        assert call(bad) == 1, (bad.q_token, bad.q_head, bad.out_token, bad.out_head)
        assert b"stride" in L.moba_last_error()
    # a block of key rows spanning 2 GiB
    huge = moba.Strides(32 * d, d, 1 << 18, d, 8 * d, d, 32 * d, d)
    assert call(huge) == 2
    assert call(moba.Strides(32 * d, d, 1 << 60, d, 8 * d, d, 32 * d, d)) == 2  # no overflow
    # fp32 rows are 16-byte aligned at multiples of 4 elements
    sh32 = shape(dtype="fp32")
    assert call(moba.Strides(36 * d + 4, d + 4, 8 * d, d, 8 * d, d, 32 * d, d), sh=sh32) == 3
    assert call(moba.Strides(36 * d + 2, d, 8 * d, d, 8 * d, d, 32 * d, d), sh=sh32) == 1
    # every pointer 16-byte aligned, with or without strides
    assert call(None, q=ctypes.c_void_p(0x1008)) == 1
    assert b"aligned" in L.moba_last_error()
