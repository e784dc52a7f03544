"""C-ABI checks that need no GPU: the library loads, exports every function
include/dcp.h declares, and rejects bad arguments on the host before any HIP
call (so nothing is enqueued)."""

import ctypes

import pytest

from mla_context_kv_amd import dcp

L = dcp.lib()
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every call below fails validation first


def test_library_exports_every_declared_function():
    names = dcp.header_functions()
    assert {"dcp_slot_map", "dcp_local_count", "dcp_kv_write", "dcp_stripe_attn",
            "dcp_stripe_attn_workspace", "dcp_lse_merge", "dcp_strerror", "dcp_relayout", "dcp_pack_heads",
            "dcp_merge_heads", "dcp_sparse_plan", "dcp_stripe_attn_multi",
            "dcp_stripe_attn_multi_workspace"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_strerror_and_version():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(dcp.strerror(code), str) and dcp.strerror(code)
    assert L.dcp_abi_version() >= 1


BAD_LAYOUTS = [dcp.layout(0, 1, 64), dcp.layout(8, 0, 64), dcp.layout(8, 1, 0), dcp.layout(8, 3, 64),
               dcp.layout(-2, 1, 64)]


@pytest.mark.parametrize("lay", BAD_LAYOUTS)
def test_bad_layout_is_rejected_everywhere(lay):
    assert L.dcp_slot_map(lay, 0, FAKE, None, 4, None, 0, 0, FAKE, FAKE, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_local_count(lay, None, FAKE, 4, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_kv_write(lay, 0, FAKE, 576, 4, FAKE, None, FAKE, 1, 1, FAKE, 1, None, None) == dcp.DCP_EINVAL
    a = _args(lay=lay)
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL


def test_slot_map_argument_errors():
    lay = dcp.layout(8, 1, 64)
    assert L.dcp_slot_map(lay, 8, FAKE, None, 4, None, 0, 0, FAKE, FAKE, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_slot_map(lay, -2, FAKE, None, 4, None, 0, 0, FAKE, FAKE, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_slot_map(lay, 0, None, None, 4, None, 0, 0, FAKE, FAKE, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_slot_map(lay, 0, FAKE, None, -1, None, 0, 0, FAKE, FAKE, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_slot_map(lay, 0, FAKE, None, 4, FAKE, 0, 4, FAKE, FAKE, FAKE, None, None) == dcp.DCP_EINVAL
    # nothing to do: success without touching the device
    assert L.dcp_slot_map(lay, 0, None, None, 0, None, 0, 0, None, None, None, None, None) == dcp.DCP_OK


def test_local_count_argument_errors():
    lay = dcp.layout(8, 64, 64)
    assert L.dcp_local_count(lay, None, None, 3, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_local_count(lay, None, FAKE, 3, None, None) == dcp.DCP_EINVAL
    assert L.dcp_local_count(lay, None, FAKE, -3, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_local_count(lay, None, None, 0, None, None) == dcp.DCP_OK


def test_kv_write_argument_errors():
    lay = dcp.layout(4, 1, 16)
    ok = dict(rank=0, kv=FAKE, row_dim=576, T=4, pos=FAKE, bt=FAKE, rows=1, cols=1, pool=FAKE, pages=1)

    def call(**kw):
        a = dict(ok, **kw)
        return L.dcp_kv_write(lay, a["rank"], a["kv"], a["row_dim"], a["T"], a["pos"], None, a["bt"],
                              a["rows"], a["cols"], a["pool"], a["pages"], None, None)

    assert call(rank=4) == dcp.DCP_EINVAL
    assert call(rank=-1) == dcp.DCP_EINVAL
    assert call(row_dim=570) == dcp.DCP_EINVAL
    assert call(T=-1) == dcp.DCP_EINVAL
    assert call(bt=None) == dcp.DCP_EINVAL
    assert call(rows=0) == dcp.DCP_EINVAL
    assert call(pool=None) == dcp.DCP_EINVAL
    assert call(pages=0) == dcp.DCP_EINVAL
    assert call(kv=None) == dcp.DCP_EINVAL
    assert call(T=0, kv=None, pos=None) == dcp.DCP_OK


def _args(lay=None, **kw):
    a = dcp.dcp_attn_args()
    a.layout = lay if lay is not None else dcp.layout(8, 1, 64)
    a.rank, a.batch, a.q_len, a.n_heads, a.head_dim, a.v_dim = 0, 2, 1, 16, 576, 512
    a.q = a.pool = a.block_table = a.seq_len = a.o = a.lse = 0x1000
    a.num_pages, a.bt_cols, a.scale, a.lse_base, a.num_splits = 4, 4, 0.07, 0, 2
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("rank", 8, dcp.DCP_EINVAL), ("rank", -1, dcp.DCP_EINVAL), ("batch", 0, dcp.DCP_EINVAL),
    ("q_len", 0, dcp.DCP_EINVAL), ("n_heads", 0, dcp.DCP_EINVAL), ("head_dim", 512, dcp.DCP_EUNSUPPORTED),
    ("v_dim", 576, dcp.DCP_EUNSUPPORTED), ("num_pages", 0, dcp.DCP_EINVAL), ("bt_cols", 0, dcp.DCP_EINVAL),
    ("lse_base", 2, dcp.DCP_EINVAL), ("num_splits", -1, dcp.DCP_EINVAL), ("q", None, dcp.DCP_EINVAL),
    ("pool", None, dcp.DCP_EINVAL), ("seq_len", None, dcp.DCP_EINVAL), ("o", None, dcp.DCP_EINVAL),
    ("window", -1, dcp.DCP_EINVAL), ("softcap", -1.0, dcp.DCP_EINVAL), ("softcap", float("nan"), dcp.DCP_EINVAL),
    ("softcap", float("inf"), dcp.DCP_EINVAL), ("partials", 2, dcp.DCP_EINVAL), ("partials", -1, dcp.DCP_EINVAL),
    ("out_records", 2, dcp.DCP_EINVAL), ("out_records", -1, dcp.DCP_EINVAL), ("lse", None, dcp.DCP_EINVAL),
])
def test_stripe_attn_argument_errors(field, value, code):
    a = _args(**{field: value})
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == code


def test_records_need_whole_head_slices():
    # records go out in head-owner order: n_heads must split evenly over the stripes
    a = _args(out_records=1, n_heads=12)
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL
    nbytes = ctypes.c_size_t(0)
    assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(nbytes)) == dcp.DCP_EINVAL


def test_softcap_and_position_bias_need_a_positive_scale():
    for kw in (dict(softcap=1.0, scale=0.0), dict(bias_slopes=0x1000, scale=-1.0)):
        a = _args(**kw)
        assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL, kw


def test_stripe_attn_workspace_size_and_missing_workspace():
    a = _args(num_splits=3, bt_cols=100)
    n = ctypes.c_size_t(0)
    assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(n)) == dcp.DCP_OK
    part = 32 * 16 * (512 * 2 + 4)      # (o bf16, lse fp32) partial of every chunk slot: 3 x 2, rounded up to 32
    assert n.value == -(-part // 256) * 256 + 2 * 2 * 4              # + the chunk table (count, first)
    a = _args(num_splits=1)
    assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(n)) == dcp.DCP_OK and n.value == 0
    assert L.dcp_stripe_attn_workspace(ctypes.byref(a), None) == dcp.DCP_EINVAL
    # splits need a workspace: rejected before launch when none is given
    a = _args(num_splits=3, bt_cols=100)
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL


def test_lse_merge_argument_errors():
    assert L.dcp_lse_merge(0, 4, 512, FAKE, FAKE, 0, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_lse_merge(8, -1, 512, FAKE, FAKE, 0, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_lse_merge(8, 4, 510, FAKE, FAKE, 0, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_lse_merge(8, 4, 512, FAKE, FAKE, 3, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_lse_merge(8, 4, 512, None, FAKE, 0, FAKE, None, None) == dcp.DCP_EINVAL
    assert L.dcp_lse_merge(8, 0, 512, None, None, 0, None, None, None) == dcp.DCP_OK


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes mirrors of dcp_layout and dcp_attn_args have the C layout:
    every field's offset and the struct sizes, as a C compiler sees dcp.h."""
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    fields = [f for f, _ in dcp.dcp_attn_args._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "dcp.h"', "int main(void) {",
           '  printf("sizeof %zu\\n", sizeof(dcp_attn_args));',
           '  printf("sizeof_layout %zu\\n", sizeof(dcp_layout));']
    src += [f'  printf("{f} %zu\\n", offsetof(dcp_attn_args, {f}));' for f in fields]
    src += ["  return 0;", "}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", inc, str(c), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                       text=True).stdout.splitlines())
    assert int(out["sizeof"]) == ctypes.sizeof(dcp.dcp_attn_args)
    assert int(out["sizeof_layout"]) == ctypes.sizeof(dcp.dcp_layout)
    for f in fields:
        assert int(out[f]) == getattr(dcp.dcp_attn_args, f).offset, f


def test_relayout_argument_errors():
    lay = dcp.layout(8, 1, 64)
    def call(**kw):
        a = dict(lay=lay, rank=1, row_dim=576, src=FAKE, src_pages=10, ps=64, sbt=FAKE, scols=4, start=FAKE,
                 len=FAKE, batch=2, max_len=100, bt=FAKE, cols=4, pool=FAKE, pages=10)
        a.update(kw)
        return L.dcp_relayout(a["lay"], a["rank"], a["row_dim"], a["src"], a["src_pages"], a["ps"], a["sbt"],
                              a["scols"], a["start"], a["len"], a["batch"], a["max_len"], a["bt"], a["cols"],
                              a["pool"], a["pages"], None, None)
    assert call(lay=dcp.layout(8, 3, 64)) == dcp.DCP_EINVAL
    for kw in (dict(rank=8), dict(rank=-1), dict(row_dim=570), dict(row_dim=0), dict(batch=-1), dict(max_len=-1),
               dict(ps=0), dict(src_pages=0), dict(scols=0), dict(cols=0), dict(pages=0), dict(src=None),
               dict(sbt=None), dict(start=None), dict(len=None), dict(bt=None), dict(pool=None)):
        assert call(**kw) == dcp.DCP_EINVAL, kw
    assert call(batch=70000) == dcp.DCP_EUNSUPPORTED
    assert call(batch=0, src=None) == dcp.DCP_OK          # nothing to move: no launch


def test_unmerged_parts_need_a_split_count_and_no_workspace():
    a = _args(partials=1, num_splits=0)
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL
    n = ctypes.c_size_t(1)
    a = _args(partials=1, num_splits=4)
    assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(n)) == dcp.DCP_OK and n.value == 0


def test_pack_and_merge_heads_argument_errors():
    assert L.dcp_pack_heads(8, 4, 12, 512, FAKE, FAKE, FAKE, None) == dcp.DCP_EINVAL     # 12 heads over 8
    assert L.dcp_pack_heads(0, 4, 16, 512, FAKE, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_pack_heads(4, 4, 16, 510, FAKE, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_pack_heads(4, -1, 16, 512, FAKE, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_pack_heads(4, 4, 16, 512, None, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_pack_heads(4, 0, 16, 512, None, None, None, None) == dcp.DCP_OK
    assert L.dcp_merge_heads(0, 4, 512, FAKE, 0, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_merge_heads(4, 4, 512, FAKE, 2, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_merge_heads(4, 4, 6, FAKE, 0, FAKE, FAKE, None) == dcp.DCP_EINVAL
    assert L.dcp_merge_heads(4, 4, 512, None, 0, FAKE, FAKE, None) == dcp.DCP_EINVAL


def test_sparse_plan_and_sparse_attention_argument_errors():
    lay = dcp.layout(8, 1, 64)
    P = dcp.dcp_layout
    call = lambda **kw: L.dcp_sparse_plan(kw.get("lay", lay), kw.get("rank", 0), kw.get("B", 2), kw.get("q_len", 1),
                                          kw.get("K", 4), kw.get("topk", FAKE), kw.get("seq", FAKE), kw.get("rows", FAKE),
                                          kw.get("bits", FAKE), kw.get("count", FAKE), kw.get("stride", 4), None)
    for kw in (dict(rank=8), dict(B=-1), dict(q_len=0), dict(K=0), dict(stride=3), dict(topk=None), dict(seq=None),
               dict(rows=None), dict(bits=None), dict(count=None), dict(lay=dcp.layout(8, 3, 64))):
        assert call(**kw) == dcp.DCP_EINVAL, kw
    assert call(q_len=33, stride=33 * 4) == dcp.DCP_EUNSUPPORTED
    assert call(B=0, topk=None) == dcp.DCP_OK
    # attention: all three sparse pointers or none; no window or position bias with a selection
    a = _args(sparse_rows=0x1000, sparse_count=0x1000, sparse_stride=4)
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL
    a = _args(sparse_rows=0x1000, sparse_bits=0x1000, sparse_count=0x1000, sparse_stride=0)
    assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EINVAL
    for kw in (dict(window=16), dict(bias_slopes=0x1000), dict(q_len=33)):
        a = _args(sparse_rows=0x1000, sparse_bits=0x1000, sparse_count=0x1000, sparse_stride=4, **kw)
        assert L.dcp_stripe_attn(ctypes.byref(a), None) == dcp.DCP_EUNSUPPORTED, kw


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No fallback: with libdcp.so absent every call raises instead of computing elsewhere."""
    monkeypatch.setattr(dcp, "LIB_PATH", str(tmp_path / "libdcp.so"))
    monkeypatch.setattr(dcp, "_lib_handle", None)
    with pytest.raises(RuntimeError, match="missing"):
        dcp.lib()


def test_multi_rank_launch_argument_errors():
    arr = (dcp.dcp_attn_args * 3)(_args(rank=0), _args(rank=1), _args(rank=2))
    n = ctypes.c_size_t(0)
    assert L.dcp_stripe_attn_multi_workspace(arr, 3, ctypes.byref(n)) == dcp.DCP_OK
    # the three ranks' chunk slots: 2 requests each, 2 splits (the _args default)
    assert n.value == -(-(32 * 16 * (512 * 2 + 4)) // 256) * 256 + 2 * 3 * 2 * 4   # 3 x 2 x 2 slots -> 32
    assert L.dcp_stripe_attn_multi_workspace(arr, 0, ctypes.byref(n)) == dcp.DCP_EINVAL
    big = (dcp.dcp_attn_args * 17)(*[_args(rank=i % 8) for i in range(17)])
    assert L.dcp_stripe_attn_multi(big, 17, None) == dcp.DCP_EUNSUPPORTED
    for field, value in (("q", 0x2000), ("batch", 3), ("num_splits", 3), ("softcap", 1.0), ("seq_len", 0x2000)):
        arr = (dcp.dcp_attn_args * 2)(_args(rank=0), _args(rank=1, **{field: value}))
        assert L.dcp_stripe_attn_multi(arr, 2, None) == dcp.DCP_EINVAL, field
    arr = (dcp.dcp_attn_args * 2)(_args(rank=0), _args(rank=9))
    assert L.dcp_stripe_attn_multi(arr, 2, None) == dcp.DCP_EINVAL
