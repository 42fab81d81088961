"""libwf's C ABI on the host (CPU only, no compute calls).

Checks that the library loads, exports every function include/wf.h declares,
and that every contract violation is rejected with its status code before any
HIP call: the device pointers passed here are fake addresses that must never
be dereferenced.
"""
import ctypes
import os
import re

import pytest

from chunk_wise_causal_amd import wf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000001000          # 16-byte aligned, never touched


def declared_functions():
    text = open(os.path.join(ROOT, "include", "wf.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wf.LIB_PATH):
        pytest.skip("libwf.so not built")
    return wf.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"wf_kv_publish", "wf_chunk_attn", "wf_last_error", "wf_device_status",
            "wf_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.wf_version().decode().startswith("libwf")


def pool(**kw):
    d = dict(k_pages=FAKE, v_pages=FAKE + 0x100000, page_table=FAKE + 0x200000,
             num_pages=10, num_logical_pages=10, page_size=256, num_heads=4, head_dim=128,
             dtype=wf.WF_BF16)
    d.update(kw)
    return wf.wf_kv_pool(**d)


def publish(L, p=None, rope=wf.wf_rope(44, 42, 42, 1e4), k=FAKE, ks=512, v=FAKE, vs=512,
            pos=FAKE, n=100, dst=0, q=None, qs=0):
    p = p or pool()
    rc = L.wf_kv_publish(ctypes.byref(p), ctypes.byref(rope) if rope else None, k, ks, v, vs,
                         pos, n, dst, q, qs, None)
    return rc, L.wf_last_error().decode()


def attn(L, p=None, segs=((0, 100, -1), (100, 50, 0), (150, 50, 1)), q=FAKE, qs=512,
         qss=(0, 50, 100), first=0, scale=0.088, out=FAKE, os_=512, n_segs=None):
    p = p or pool()
    sa = (wf.wf_segment * max(1, len(segs)))(*[wf.wf_segment(*s) for s in segs])
    qa = (ctypes.c_int32 * len(qss))(*qss)
    rc = L.wf_chunk_attn(ctypes.byref(p), sa, len(segs) if n_segs is None else n_segs, q, qs,
                         qa, len(qss) - 1, first, scale, out, os_, None, None)
    return rc, L.wf_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(page_size=48), wf.WF_ERR_INVALID, "page_size"),
    (dict(page_size=8), wf.WF_ERR_INVALID, "page_size"),
    (dict(page_size=2048), wf.WF_ERR_INVALID, "page_size"),
    (dict(head_dim=96), wf.WF_ERR_UNSUPPORTED, "head_dim"),
    (dict(head_dim=256), wf.WF_ERR_UNSUPPORTED, "head_dim"),
    (dict(num_heads=0), wf.WF_ERR_INVALID, "num_heads"),
    (dict(num_pages=0), wf.WF_ERR_INVALID, "num_pages"),
    (dict(dtype=7), wf.WF_ERR_INVALID, "dtype"),
    (dict(k_pages=0), wf.WF_ERR_INVALID, "non-NULL"),
    (dict(page_table=0), wf.WF_ERR_INVALID, "non-NULL"),
    (dict(v_pages=FAKE + 8), wf.WF_ERR_INVALID, "aligned"),
])
def test_pool_checks_both_calls(L, kw, code, msg):
    for rc, err in (publish(L, p=pool(**kw)), attn(L, p=pool(**kw))):
        assert rc == code and msg in err


@pytest.mark.parametrize("kw,msg", [
    (dict(rope=wf.wf_rope(44, 42, 40, 1e4)), "head_dim"),
    (dict(rope=wf.wf_rope(43, 43, 42, 1e4)), "even"),
    (dict(rope=wf.wf_rope(44, 42, 42, -1.0)), "theta"),
    (dict(rope=wf.wf_rope(44, 42, 42, float("inf"))), "theta"),
    (dict(pos=None), "pos_thw"),
    (dict(k=None), "k is NULL"),
    (dict(v=FAKE + 4), "aligned"),
    (dict(ks=500), "k_row_stride"),
    (dict(vs=516), "multiple of 8"),
    (dict(n=-1), "n_tok"),
    (dict(dst=-5), "dst_logical_start"),
    (dict(dst=2500, n=61), "capacity"),
    (dict(rope=None, q=FAKE, qs=512), "q_inout requires rope"),
    (dict(q=FAKE, qs=256), "q_row_stride"),
])
def test_publish_rejects(L, kw, msg):
    rc, err = publish(L, **kw)
    assert rc == wf.WF_ERR_INVALID, err
    assert msg in err


def test_publish_zero_tokens_is_noop(L):
    rc, err = publish(L, n=0, k=None, v=None)
    assert rc == wf.WF_OK and err == ""


@pytest.mark.parametrize("kw,code,msg", [
    (dict(segs=((0, 100, -1), (90, 50, 0), (150, 50, 1))), wf.WF_ERR_INVALID, "overlap"),
    (dict(segs=((0, 100, -1), (100, 50, 0))), wf.WF_ERR_INVALID, "owns no segment"),
    (dict(segs=((0, 100, -1), (100, 0, 0), (150, 50, 1))), wf.WF_ERR_INVALID, "outside"),
    (dict(segs=((0, 100, -1), (100, 50, 0), (2550, 50, 1))), wf.WF_ERR_INVALID, "outside"),
    (dict(segs=((-1, 100, -1), (100, 50, 0), (150, 50, 1))), wf.WF_ERR_INVALID, "outside"),
    (dict(n_segs=0), wf.WF_ERR_INVALID, "n_segs"),
    (dict(n_segs=65), wf.WF_ERR_INVALID, "n_segs"),
    (dict(qss=(0, 60, 50)), wf.WF_ERR_INVALID, "non-decreasing"),
    (dict(qss=(-2, 50, 100)), wf.WF_ERR_INVALID, "q_slot_start[0]"),
    (dict(qss=tuple(range(34))), wf.WF_ERR_INVALID, "n_slots"),
    (dict(first=-1), wf.WF_ERR_INVALID, "first_slot"),
    (dict(first=1), wf.WF_ERR_INVALID, "owns no segment"),
    (dict(scale=0.0), wf.WF_ERR_INVALID, "scale"),
    (dict(scale=float("nan")), wf.WF_ERR_INVALID, "scale"),
    (dict(q=None), wf.WF_ERR_INVALID, "q is NULL"),
    (dict(out=FAKE + 2), wf.WF_ERR_INVALID, "aligned"),
    (dict(os_=256), wf.WF_ERR_INVALID, "out_row_stride"),
])
def test_attn_rejects(L, kw, code, msg):
    rc, err = attn(L, **kw)
    assert rc == code, err
    assert msg in err


def test_attn_too_many_ranges_unsupported(L):
    # 32 query slots, each with its own segment, plus 32 prefix segments with
    # gaps: every slot sees >= 32 unmergeable ranges -> > 256 in total
    segs = [(i * 20, 10, -1) for i in range(32)] + [(1000 + i * 20, 10, i) for i in range(32)]
    rc, err = attn(L, segs=segs, qss=tuple(range(0, 330, 10)))
    assert rc == wf.WF_ERR_UNSUPPORTED and "ranges" in err


def test_attn_no_rows_is_noop(L):
    rc, err = attn(L, qss=(7, 7, 7), q=None, out=None)
    assert rc == wf.WF_OK and err == ""


def test_device_status_null_arg(L):
    assert L.wf_device_status(None, 0) == wf.WF_ERR_INVALID


def test_binding_raises_with_message(L):
    rc, _ = attn(L, p=pool(page_size=100))
    with pytest.raises(wf.WFError, match="page_size"):
        wf._check(rc)


# ---- the binding's own checks (before any library call) --------------------
# The C side sees raw pointers and checks strides, alignment and NULLs; the
# binding checks what only the tensors know: device, element type and rows.
# Every case here must raise ValueError without calling into the library.

@pytest.fixture
def no_lib(monkeypatch):
    def forbidden():
        raise AssertionError("the binding called the library before its own checks")
    monkeypatch.setattr(wf, "lib", forbidden)


def cpu_pool(heads=2, ps=16, D=128, pages=4, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    return wf.KVPool(torch.zeros(pages, heads, ps, D, dtype=dtype),
                     torch.zeros(pages, heads, D, ps, dtype=dtype),
                     torch.arange(pages, dtype=torch.int32))


def test_binding_checks_attention_args(no_lib):
    import torch
    P = cpu_pool()
    bf = torch.bfloat16
    q = torch.zeros(40, 2, 128, dtype=bf)
    segs, qss = [(0, 20, -1), (20, 20, 0), (40, 20, 1)], [0, 20, 40]
    cases = [
        (dict(q=torch.zeros(40, 3, 128, dtype=bf)), "q: expected"),
        (dict(q=torch.zeros(39, 2, 128, dtype=bf)), "rows"),
        (dict(q=q.float()), "dtype"),
        (dict(out=torch.zeros(40, 2, 128)), "out: dtype"),
        (dict(out=torch.zeros(30, 2, 128, dtype=bf)), "out: 30 rows"),
        (dict(lse=torch.zeros(2, 40, dtype=torch.float64)), "lse"),
        (dict(lse=torch.zeros(2, 39)), "lse: expected"),
        (dict(lse=torch.zeros(3, 40)), "lse: expected"),
        (dict(), "GPU tensor"),          # shapes fine: the pool lives on the host
    ]
    for kw, msg in cases:
        args = dict(q=q, out=None, lse=None)
        args.update(kw)
        with pytest.raises(ValueError, match=msg):
            wf.wf_chunk_attn(P, segs, args["q"], qss, out=args["out"], lse=args["lse"])
    # no rows at all: an empty [H, 0] lse passes the shape checks (torch gives
    # it a row stride of 1); only the host-resident pool is refused
    with pytest.raises(ValueError, match="GPU tensor"):
        wf.wf_chunk_attn(P, segs, q, [0, 0, 0], lse=torch.zeros(2, 0))
    with pytest.raises(ValueError, match="lse"):
        wf.wf_group_attn(P, [(0, 40)], [(0, 40, 0, 1)], q, lse=torch.zeros(2, 30))
    with pytest.raises(ValueError, match="rows"):
        wf.wf_group_attn(P, [(0, 40)], [(0, 41, 0, 1)], q)


def test_binding_checks_publish_args(no_lib):
    import torch
    P = cpu_pool()
    bf = torch.bfloat16
    k = torch.zeros(10, 2, 128, dtype=bf)
    pos = torch.zeros(10, 3, dtype=torch.int32)
    rope = ((44, 42, 42), 1e4)
    cases = [
        (dict(v=torch.zeros(9, 2, 128, dtype=bf)), "v: 9 rows"),
        (dict(v=torch.zeros(10, 2, 64, dtype=bf)), "v: expected"),
        (dict(pos=torch.zeros(10, 3, dtype=torch.int64)), "pos"),
        (dict(pos=torch.zeros(9, 3, dtype=torch.int32)), "pos"),
        (dict(pos=None), "pos: required"),
        (dict(q=torch.zeros(10, 2, 128)), "q: dtype"),
        (dict(), "GPU tensor"),
    ]
    for kw, msg in cases:
        args = dict(v=k, pos=pos, q=None)
        args.update(kw)
        with pytest.raises(ValueError, match=msg):
            wf.wf_kv_publish(P, k, args["v"], 0, pos=args["pos"], rope=rope, q=args["q"])
    x = torch.zeros(10, 256, dtype=bf)
    w = torch.zeros(3 * 2 * 128, 256, dtype=bf)
    for kw, msg in [(dict(w=torch.zeros(700, 256, dtype=bf)), "w_qkv"),
                    (dict(bias=torch.zeros(10, dtype=bf)), "bias"),
                    (dict(w=w.float()), "w_qkv: dtype"),
                    (dict(), "GPU tensor")]:
        a = dict(w=w, bias=None)
        a.update(kw)
        with pytest.raises(ValueError, match=msg):
            wf.wf_qkv_publish(P, x, a["w"], 0, pos=pos, rope=rope, bias=a["bias"])
    keys = wf.MXKeys(torch.zeros(4, 2, 8, 128, dtype=torch.uint8),
                     torch.zeros(4, 2, 8, 4, dtype=torch.uint8))
    with pytest.raises(ValueError, match="MX keys"):
        wf.wf_kv_publish_mx(P, keys, k, k, 0, pos=pos, rope=rope)
    with pytest.raises(ValueError, match="GPU tensor"):
        wf.wf_history_rotate(P, 0, 16, 2)


def gattn(L, p=None, runs=((0, 100), (100, 50), (150, 50)),
          groups=((0, 50, 0, 3), (50, 100, 0, 2)), q=FAKE, qs=512, scale=0.088, out=FAKE,
          os_=512, lse=None, lse_stride=0, n_runs=None, n_groups=None):
    p = p or pool()
    ra = (wf.wf_kv_run * max(1, len(runs)))(*[wf.wf_kv_run(*r) for r in runs])
    ga = (wf.wf_query_group * max(1, len(groups)))(*[wf.wf_query_group(*g) for g in groups])
    rc = L.wf_group_attn(ctypes.byref(p), ra, len(runs) if n_runs is None else n_runs, ga,
                         len(groups) if n_groups is None else n_groups, q, qs, scale, out, os_,
                         lse, lse_stride, None)
    return rc, L.wf_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(runs=((0, 100), (90, 50), (150, 50))), wf.WF_ERR_INVALID, "overlap"),
    (dict(runs=((0, 100), (100, 0), (150, 50))), wf.WF_ERR_INVALID, "outside"),
    (dict(runs=((0, 100), (100, 50), (2550, 50))), wf.WF_ERR_INVALID, "outside"),
    (dict(runs=((-1, 100), (100, 50), (150, 50))), wf.WF_ERR_INVALID, "outside"),
    (dict(n_runs=0), wf.WF_ERR_INVALID, "n_runs"),
    (dict(n_runs=257), wf.WF_ERR_INVALID, "n_runs"),
    (dict(n_groups=0), wf.WF_ERR_INVALID, "n_groups"),
    (dict(n_groups=33), wf.WF_ERR_INVALID, "n_groups"),
    (dict(groups=((0, 50, 0, 3), (40, 100, 0, 2))), wf.WF_ERR_INVALID, "overlap at row 40"),
    (dict(groups=((0, 50, 2, 2),)), wf.WF_ERR_INVALID, "runs"),
    (dict(groups=((0, 50, 1, 4),)), wf.WF_ERR_INVALID, "runs"),
    (dict(groups=((-1, 50, 0, 1),)), wf.WF_ERR_INVALID, "rows"),
    (dict(groups=((60, 50, 0, 1),)), wf.WF_ERR_INVALID, "rows"),
    (dict(scale=-1.0), wf.WF_ERR_INVALID, "scale"),
    (dict(q=None), wf.WF_ERR_INVALID, "q is NULL"),
    (dict(os_=256), wf.WF_ERR_INVALID, "out_row_stride"),
    (dict(lse=FAKE, lse_stride=99), wf.WF_ERR_INVALID, "lse_stride"),
])
def test_group_attn_rejects(L, kw, code, msg):
    rc, err = gattn(L, **kw)
    assert rc == code, err
    assert msg in err


def test_group_attn_shared_keys_and_noop(L):
    # groups may share runs; rows may be empty; no rows at all is a no-op
    rc, err = gattn(L, groups=((0, 0, 0, 3), (5, 5, 1, 2)), q=None, out=None)
    assert rc == wf.WF_OK and err == ""


def test_group_attn_too_many_ranges_unsupported(L):
    runs = [(i * 20, 10) for i in range(120)]
    groups = [(g, g + 1, 0, 120) for g in range(3)]   # 3 x 120 unmergeable ranges
    rc, err = gattn(L, runs=runs, groups=groups)
    assert rc == wf.WF_ERR_UNSUPPORTED and "ranges" in err


def rotate(L, table=FAKE, nlp=64, ps=256, start=512, stride=1024, n=3):
    rc = L.wf_history_rotate(table, nlp, ps, start, stride, n, None)
    return rc, L.wf_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(table=None), wf.WF_ERR_INVALID, "NULL"),
    (dict(table=FAKE + 2), wf.WF_ERR_INVALID, "aligned"),
    (dict(nlp=0), wf.WF_ERR_INVALID, "num_logical_pages"),
    (dict(ps=100), wf.WF_ERR_INVALID, "page_size"),
    (dict(ps=8), wf.WF_ERR_INVALID, "page_size"),
    (dict(start=-256), wf.WF_ERR_INVALID, "window_start"),
    (dict(start=100), wf.WF_ERR_INVALID, "window_start"),
    (dict(stride=0), wf.WF_ERR_INVALID, "chunk_stride"),
    (dict(stride=1000), wf.WF_ERR_INVALID, "chunk_stride"),
    (dict(n=0), wf.WF_ERR_INVALID, "n_chunks"),
    (dict(nlp=13), wf.WF_ERR_INVALID, "exceeds num_logical_pages"),   # window ends at page 14
    (dict(nlp=1 << 20, ps=16, start=0, stride=16, n=16385), wf.WF_ERR_UNSUPPORTED, "limit"),
])
def test_history_rotate_rejects(L, kw, code, msg):
    rc, err = rotate(L, **kw)
    assert rc == code and msg in err, (rc, err)


def test_history_rotate_single_chunk_is_noop(L):
    # one chunk: rotating by the whole window is the identity, nothing is launched
    assert rotate(L, n=1) == (wf.WF_OK, "")
    # the window may end exactly at the table's end
    assert rotate(L, nlp=14, n=1)[0] == wf.WF_OK


def mxkeys(**kw):
    d = dict(k8_pages=FAKE + 0x400000, k8_scales=FAKE + 0x500000)
    d.update(kw)
    return wf.wf_mx_keys(**d)


@pytest.mark.parametrize("keys,pkw,code,msg", [
    (None, {}, wf.WF_ERR_INVALID, "keys is NULL"),
    (dict(k8_pages=None), {}, wf.WF_ERR_INVALID, "k8_pages and k8_scales"),
    (dict(k8_scales=None), {}, wf.WF_ERR_INVALID, "k8_pages and k8_scales"),
    (dict(k8_scales=FAKE + 0x500004), {}, wf.WF_ERR_INVALID, "aligned"),
    ({}, dict(dtype=wf.WF_FP32), wf.WF_ERR_UNSUPPORTED, "mx keys"),
    ({}, dict(head_dim=64), wf.WF_ERR_UNSUPPORTED, "mx keys"),
    ({}, dict(v_pages=None), wf.WF_ERR_INVALID, "non-NULL"),
])
def test_mx_calls_reject(L, keys, pkw, code, msg):
    p = pool(**pkw)
    kp = None if keys is None else ctypes.byref(mxkeys(**keys))
    rope = wf.wf_rope(44, 42, 42, 1e4) if p.head_dim == 128 else wf.wf_rope(24, 20, 20, 1e4)
    rc = L.wf_kv_publish_mx(ctypes.byref(p), kp, ctypes.byref(rope), FAKE, 512, FAKE, 512, FAKE,
                            100, 0, None, 0, None)
    err = L.wf_last_error().decode()
    assert rc == code and msg in err, (rc, err)
    segs = (wf.wf_segment * 2)(wf.wf_segment(0, 100, -1), wf.wf_segment(100, 50, 0))
    qss = (ctypes.c_int32 * 2)(0, 50)
    rc = L.wf_chunk_attn_mx(ctypes.byref(p), kp, segs, 2, FAKE, 512, qss, 1, 0,
                            ctypes.c_float(0.088), FAKE, 512, None, None)
    err = L.wf_last_error().decode()
    assert rc == code and msg in err, (rc, err)


def test_mx_calls_need_no_bf16_keys(L):
    # the 8-bit calls never touch pool.k_pages: NULL is accepted (no-op calls)
    p = pool(k_pages=None)
    k = mxkeys()
    assert L.wf_kv_publish_mx(ctypes.byref(p), ctypes.byref(k), None, FAKE, 512, FAKE, 512,
                              None, 0, 0, None, 0, None) == wf.WF_OK
    segs = (wf.wf_segment * 1)(wf.wf_segment(0, 100, 0))
    qss = (ctypes.c_int32 * 2)(0, 0)
    assert L.wf_chunk_attn_mx(ctypes.byref(p), ctypes.byref(k), segs, 1, FAKE, 512, qss, 1, 0,
                              ctypes.c_float(0.088), FAKE, 512, None, None) == wf.WF_OK
    # the bfloat16 calls still require it
    assert L.wf_kv_publish(ctypes.byref(p), None, FAKE, 512, FAKE, 512, None, 0, 0, None, 0,
                           None) == wf.WF_ERR_INVALID


def qkv(L, p=None, rope=wf.wf_rope(44, 42, 42, 1e4), x=FAKE, xs=5120, hidden=5120, w=FAKE,
        bias=None, pos=FAKE, n=100, dst=0, q=FAKE, qs=512):
    p = p or pool()
    rc = L.wf_qkv_publish(ctypes.byref(p), ctypes.byref(rope) if rope else None, x, xs, hidden,
                          w, bias, pos, n, dst, q, qs, None)
    return rc, L.wf_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(p=pool(dtype=wf.WF_FP32)), wf.WF_ERR_UNSUPPORTED, "bfloat16"),
    (dict(p=pool(head_dim=64)), wf.WF_ERR_UNSUPPORTED, "head_dim 128"),
    (dict(hidden=100, xs=104), wf.WF_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(hidden=0, xs=0), wf.WF_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(hidden=65600, xs=65600), wf.WF_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(xs=(1 << 22) + 8), wf.WF_ERR_UNSUPPORTED, "2^22"),
    (dict(x=None), wf.WF_ERR_INVALID, "non-NULL"),
    (dict(w=None), wf.WF_ERR_INVALID, "non-NULL"),
    (dict(w=FAKE + 8), wf.WF_ERR_INVALID, "aligned"),
    (dict(xs=5000), wf.WF_ERR_INVALID, "x_row_stride"),
    (dict(xs=5124), wf.WF_ERR_INVALID, "x_row_stride"),
    (dict(bias=FAKE + 1), wf.WF_ERR_INVALID, "bias"),
    (dict(pos=None), wf.WF_ERR_INVALID, "pos_thw"),
    (dict(rope=wf.wf_rope(44, 42, 40, 1e4)), wf.WF_ERR_INVALID, "head_dim"),
    (dict(n=-1), wf.WF_ERR_INVALID, "n_tok"),
    (dict(dst=2500), wf.WF_ERR_INVALID, "capacity"),
    (dict(qs=100), wf.WF_ERR_INVALID, "q_row_stride"),
])
def test_qkv_publish_rejects(L, kw, code, msg):
    rc, err = qkv(L, **kw)
    assert rc == code and msg in err, (rc, err)


def test_qkv_publish_zero_tokens_is_noop(L):
    assert qkv(L, n=0, x=None, w=None)[0] == wf.WF_OK
