"""The C ABI on the host: the library loads without a GPU, exports every
symbol the header declares, and rejects bad arguments before any HIP call."""
import ctypes
import math
import os
import re

import pytest

import non_causal_block_amd as nb
from non_causal_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash_block_attn.h")

FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from non_causal_block_amd import build
        build.build()
    return _lib.load()


TIMELINE_BLOCK = r"#ifdef DFLASH_TIMELINE(.*?)#endif"


def _functions(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dflash_\w+)\s*\(", text, flags=re.M)))


def declared_functions():
    """Functions the product library exports (the timeline build's extra one aside)."""
    return _functions(re.sub(TIMELINE_BLOCK, "", open(HEADER).read(), flags=re.S))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 16, names
    for n in names:
        assert hasattr(lib, n), n


def test_timeline_setter_is_only_in_the_timeline_build(lib):
    blocks = re.findall(TIMELINE_BLOCK, open(HEADER).read(), flags=re.S)
    assert [_functions(b) for b in blocks] == [["dflash_timeline_set_buffer"]]
    assert not hasattr(lib, "dflash_timeline_set_buffer")


def test_stream_read_rejects_bad_arguments(lib):
    # validation happens on the host, before any HIP call
    assert nb.dflash_stream_read(None, 16, None, None) == nb.DFLASH_ERR_INVALID_ARGUMENT
    assert nb.dflash_stream_read(0x1000, 15, 0x2000, None) == nb.DFLASH_ERR_INVALID_ARGUMENT
    assert nb.dflash_stream_read(0x1008, 16, 0x2000, None) == nb.DFLASH_ERR_INVALID_ARGUMENT
    assert nb.dflash_stream_read(0x1000, 0, 0x2000, None) == nb.DFLASH_OK  # nothing to read


def test_debug_check_switch_and_argument_errors(lib):
    prev = nb.dflash_set_debug_checks(True)
    try:
        assert nb.dflash_set_debug_checks(False) is True
        assert nb.dflash_set_debug_checks(False) is False
    finally:
        nb.dflash_set_debug_checks(prev)
    expect(lib.dflash_debug_checks_result(None, None), nb.DFLASH_ERR_INVALID_ARGUMENT, "non-NULL")


def test_abi_version(lib):
    assert nb.dflash_abi_version() == 2


def test_status_strings(lib):
    for s in range(5):
        assert nb.dflash_status_string(s)
    assert nb.dflash_status_string(99) == "unknown status"


@pytest.mark.parametrize("hq,hkv,d,ok", [
    (32, 8, 512, True), (32, 4, 512, True), (8, 2, 128, True), (32, 8, 256, True), (1, 1, 8, True),
    (32, 8, 520, False), (32, 8, 100, False), (32, 7, 128, False), (0, 1, 128, False), (4, 8, 128, False),
    (32, 8, 0, False),
])
def test_supports(lib, hq, hkv, d, ok):
    assert nb.dflash_block_attn_supports(hq, hkv, d) == ok


def desc(**kw):
    base = dict(num_reqs=4, total_q=36, max_block_len=9, total_kv_len=82000, page_size=16,
                max_pages_per_req=2100, num_pages=5200, num_cus=256)
    base.update(kw)
    return nb.make_desc(**base)


def call(d, *, q=FAKE, k=FAKE, v=FAKE, pt=FAKE, ctx=FAKE, blk=FAKE, hq=32, hkv=4, hd=512, causal=None,
         window=0, scale=0.044, out=FAKE):
    return nb.dflash_block_attn(q, k, v, pt, ctx, blk, hq, hkv, hd, causal, window, scale, out, None, d)


def expect(status, want, fragment=""):
    assert status == want, (status, nb.dflash_last_error_message())
    if fragment:
        assert fragment in nb.dflash_last_error_message(), nb.dflash_last_error_message()


def test_null_desc(lib):
    st = lib.dflash_block_attn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4, 512, None, 0, 1.0, FAKE, None, None)
    expect(st, nb.DFLASH_ERR_INVALID_ARGUMENT, "desc")


def test_append_rejects_before_launch(lib):
    d = desc()
    stream = None

    def app(kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, pt=FAKE, ctx=FAKE, blk=FAKE, hkv=4, hd=512, dd=d):
        return nb.dflash_block_kv_append(kn, vn, kp, vp, pt, ctx, blk, hkv, hd, stream, dd)

    expect(app(hd=520), nb.DFLASH_ERR_UNSUPPORTED, "512")
    expect(app(hd=12), nb.DFLASH_ERR_UNSUPPORTED, "multiple of 8")
    expect(app(hkv=0), nb.DFLASH_ERR_INVALID_ARGUMENT)
    expect(app(kn=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    expect(app(vp=FAKE + 8), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    expect(app(blk=FAKE + 2), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    expect(app(dd=desc(page_size=12)), nb.DFLASH_ERR_INVALID_ARGUMENT, "page_size")
    expect(lib.dflash_block_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, None, None),
           nb.DFLASH_ERR_INVALID_ARGUMENT, "desc")
    # nothing to append: OK without touching any pointer
    expect(app(kn=0, vn=0, kp=0, vp=0, pt=0, ctx=0, blk=0, dd=desc(total_q=0)), nb.DFLASH_OK)
    # the fused call validates both halves before enqueueing either: a bad append
    # argument or a bad attention argument (no workspace) both fail up front
    fused = lambda dd=d, kn=FAKE, scale=0.044: nb.dflash_block_attn_append(
        FAKE, kn, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4, 512, None, 0, scale, FAKE, None, dd)
    expect(fused(kn=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    expect(fused(scale=math.inf), nb.DFLASH_ERR_INVALID_ARGUMENT, "scale")
    expect(fused(), nb.DFLASH_ERR_WORKSPACE_TOO_SMALL, "needs")


def test_block_conv_rejects_before_launch(lib):
    def conv(x=FAKE, base=FAKE, delta=FAKE, blk=FAKE, B=4, total=36, C=4096, G=32, taps=16, out=FAKE):
        return nb.dflash_block_conv(x, base, delta, blk, B, total, C, G, taps, out, None)

    expect(conv(C=7), nb.DFLASH_ERR_INVALID_ARGUMENT, "even")
    expect(conv(G=3), nb.DFLASH_ERR_INVALID_ARGUMENT, "divide")
    expect(conv(taps=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "taps")
    expect(conv(total=70000), nb.DFLASH_ERR_UNSUPPORTED, "65535")
    expect(conv(B=-1), nb.DFLASH_ERR_INVALID_ARGUMENT, "negative")
    expect(conv(x=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    expect(conv(out=FAKE + 2), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    expect(conv(x=0, base=0, delta=0, blk=0, out=0, total=0), nb.DFLASH_OK)  # nothing to do


def test_rejects_before_launch(lib):
    d = desc()
    expect(call(d, hd=520), nb.DFLASH_ERR_UNSUPPORTED, "512")
    expect(call(d, hd=100), nb.DFLASH_ERR_UNSUPPORTED, "multiple of 8")
    expect(call(d, hd=0), nb.DFLASH_ERR_INVALID_ARGUMENT)
    expect(call(d, hq=30, hkv=4), nb.DFLASH_ERR_INVALID_ARGUMENT, "multiple")
    expect(call(d, scale=math.inf), nb.DFLASH_ERR_INVALID_ARGUMENT, "scale")
    expect(call(d, scale=math.nan), nb.DFLASH_ERR_INVALID_ARGUMENT, "scale")
    expect(call(d, q=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    expect(call(d, out=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    expect(call(d, pt=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    expect(call(d, q=FAKE + 2), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    expect(call(d, ctx=FAKE + 1), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    # no workspace given
    expect(call(d), nb.DFLASH_ERR_WORKSPACE_TOO_SMALL, "needs")
    need = nb.dflash_block_attn_workspace_size(d, 32, 4, 512)
    d.workspace = FAKE
    d.workspace_bytes = need - 1
    expect(call(d), nb.DFLASH_ERR_WORKSPACE_TOO_SMALL)
    d.workspace = FAKE + 16
    d.workspace_bytes = need
    expect(call(d), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")


def test_spans_call_rejects_before_launch(lib):
    d = desc()

    def sp(offs=FAKE, spans=FAKE, num=3, dd=d, q=FAKE):
        return nb.dflash_block_attn_spans(q, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4, 512, FAKE, offs, spans, num, 0,
                                          0.044, FAKE, None, dd)

    expect(sp(num=-1), nb.DFLASH_ERR_INVALID_ARGUMENT, "num_spans")
    expect(sp(spans=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "spans is NULL")
    expect(sp(offs=FAKE + 2), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    expect(sp(spans=FAKE + 1), nb.DFLASH_ERR_INVALID_ARGUMENT, "aligned")
    expect(sp(q=0), nb.DFLASH_ERR_INVALID_ARGUMENT, "NULL")
    # the span checks pass with no spans at all or without span_offsets; then the
    # missing workspace is what fails
    expect(sp(spans=0, num=0), nb.DFLASH_ERR_WORKSPACE_TOO_SMALL, "needs")
    expect(sp(offs=0, spans=0, num=-1), nb.DFLASH_ERR_WORKSPACE_TOO_SMALL, "needs")
    expect(sp(dd=desc(total_q=0)), nb.DFLASH_OK)


@pytest.mark.parametrize("field,value", [
    ("page_size", 0), ("page_size", 3), ("page_size", 2048), ("max_pages_per_req", 0), ("num_pages", 0),
    ("kernel", 3), ("kernel", -1), ("num_workgroups", -1), ("num_cus", -2), ("num_reqs", -1), ("total_q", -5),
])
def test_rejects_bad_desc_fields(lib, field, value):
    d = desc()
    setattr(d, field, value)
    expect(call(d), nb.DFLASH_ERR_INVALID_ARGUMENT)


def test_empty_batch_is_a_no_op(lib):
    # nothing to do: OK without touching any pointer, workspace or device
    assert call(desc(num_reqs=0), q=0, k=0, v=0, pt=0, ctx=0, blk=0, out=0) == nb.DFLASH_OK
    assert call(desc(total_q=0), q=0, k=0, v=0, pt=0, ctx=0, blk=0, out=0) == nb.DFLASH_OK
    assert nb.dflash_block_attn_workspace_size(desc(num_reqs=0), 32, 4, 512) == 0


def test_plan_mfma_global_layer(lib):
    # head_dim 512, 9 queries x 8 q-heads per kv-head = 72 rows -> five 16-row tiles
    p = nb.dflash_block_attn_plan(desc(), 32, 4, 512)
    assert p.kernel == nb.DFLASH_KERNEL_MFMA
    assert p.rows_per_unit == 80 and p.head_dim_padded == 512 and p.tile_keys == 32
    assert p.num_workgroups == 256  # planning without a device assumes one workgroup per CU
    # merge counters (arrivals, claims per workgroup, one finish count), then two slots per
    # workgroup: bf16 partial rows and fp32 log-sum-exps, then the merge directory (8 bytes
    # per output row)
    P = p.num_workgroups
    assert p.workspace_bytes >= (2 * P + 1) * 4 + P * 2 * 80 * 512 * 2 + P * 2 * 80 * 4 + 36 * 32 * 8
    # a grid of 256: the combine kernel merges (16 units over 256 runs, about 18 pieces each,
    # so one combine workgroup per output row)
    assert p.merge_in_kernel == 0 and p.combine_workgroups == 36 * 32
    # asked for the in-kernel merge: no combine launch, same workspace
    p2 = nb.dflash_block_attn_plan(desc(merge_mode=nb.DFLASH_MERGE_IN_KERNEL), 32, 4, 512)
    assert p2.merge_in_kernel == 1 and p2.combine_workgroups == 0
    assert p2.workspace_bytes == p.workspace_bytes


def test_plan_small_problem_uses_few_workgroups(lib):
    d = desc(num_reqs=1, total_q=9, total_kv_len=521, max_pages_per_req=33, num_pages=34)
    p = nb.dflash_block_attn_plan(d, 8, 2, 128)
    # 17 tiles per kv-head, two kv-heads: two tiles per workgroup, not the whole chip
    assert p.num_workgroups == 17
    assert p.head_dim_padded == 128 and p.rows_per_unit == 48
    # a small step merges its split units inside the attention kernel (one launch)
    assert p.merge_in_kernel == 1 and p.combine_workgroups == 0
    # four such requests: ceil(2 x (65 + 4) / 2) = 69 > 64 workgroups, but 154 flat positions
    # (set-up charges of 2 included) are under 3 per CU: one workgroup per CU, merged in the kernel
    p4 = nb.dflash_block_attn_plan(desc(num_reqs=4, total_q=36, total_kv_len=4 * 521, max_pages_per_req=33,
                                        num_pages=136), 8, 2, 128)
    assert p4.num_workgroups == 256 and p4.merge_in_kernel == 1 and p4.combine_workgroups == 0
    p2 = nb.dflash_block_attn_plan(desc(num_reqs=1, total_q=9, total_kv_len=521, max_pages_per_req=33, num_pages=34,
                                        merge_mode=nb.DFLASH_MERGE_COMBINE_KERNEL), 8, 2, 128)
    assert p2.merge_in_kernel == 0 and p2.combine_workgroups > 0


def test_plan_small_step_bound(lib):
    # head_dim 256, one request of block 9, Hq 32 / Hkv 8: 36 rows, one row group.  Work =
    # 8 kv-heads x (keys // 32 + 1 tiles + a set-up charge of 2) = 8 * (keys // 32) + 24,
    # which is 768 = 3 per CU at 3007 keys and 776 at 3008; two tiles per workgroup would
    # take 376 > 64 workgroups, so the small step runs one per CU
    def plan(keys):
        return nb.dflash_block_attn_plan(desc(num_reqs=1, total_q=9, total_kv_len=keys, max_pages_per_req=256,
                                              num_pages=256), 32, 8, 256)
    small, large = plan(3007), plan(3008)
    assert small.num_workgroups == 256 and small.merge_in_kernel == 1 and small.combine_workgroups == 0
    assert large.merge_in_kernel == 0 and large.combine_workgroups > 0
    # a forced small grid still merges in the kernel; a forced merge mode wins over both rules
    forced = nb.dflash_block_attn_plan(desc(num_reqs=1, total_q=9, total_kv_len=3008, max_pages_per_req=256,
                                            num_pages=256, num_workgroups=64), 32, 8, 256)
    assert forced.num_workgroups == 64 and forced.merge_in_kernel == 1
    sep = nb.dflash_block_attn_plan(desc(num_reqs=1, total_q=9, total_kv_len=3007, max_pages_per_req=256,
                                         num_pages=256, merge_mode=nb.DFLASH_MERGE_COMBINE_KERNEL), 32, 8, 256)
    assert sep.num_workgroups == 256 and sep.merge_in_kernel == 0 and sep.combine_workgroups > 0
    # head_dim 512 keeps the general rule: ceil(4 kv-heads x (64 + 1) tiles / 2) workgroups,
    # merged by the combine kernel
    g = nb.dflash_block_attn_plan(desc(num_reqs=1, total_q=9, total_kv_len=2057, max_pages_per_req=256,
                                       num_pages=256), 32, 4, 512)
    assert g.num_workgroups == 130 and g.merge_in_kernel == 0 and g.combine_workgroups > 0


def test_plan_reference_kernel_and_forced_grid(lib):
    p = nb.dflash_block_attn_plan(desc(kernel=nb.DFLASH_KERNEL_REFERENCE, num_workgroups=37), 32, 4, 200)
    assert p.kernel == nb.DFLASH_KERNEL_REFERENCE and p.num_workgroups == 37
    assert p.rows_per_unit == 16 and p.head_dim_padded == 200
    # the reference kernel always leaves its partials to the combine kernel
    assert p.merge_in_kernel == 0 and p.combine_workgroups > 0
    p1 = nb.dflash_block_attn_plan(desc(num_workgroups=1), 32, 4, 512)
    assert p1.workspace_bytes == 0 and p1.combine_workgroups == 0


def test_plan_head_dim_padding(lib):
    for hd, want in ((8, 128), (64, 128), (136, 256), (256, 256), (264, 512), (512, 512)):
        assert nb.dflash_block_attn_plan(desc(), 32, 4, hd).head_dim_padded == want


def test_workspace_size_matches_plan(lib):
    d = desc(max_block_len=16)
    assert nb.dflash_block_attn_workspace_size(d, 32, 8, 256) == nb.dflash_block_attn_plan(d, 32, 8, 256).workspace_bytes


def test_planning_without_device_needs_cu_count(lib):
    # with num_cus = 0 the planner must ask the HIP runtime for the device; on a host
    # without a GPU that is a clean error, not a crash
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(nb.DFlashError) as e:
        nb.dflash_block_attn_plan(desc(num_cus=0), 32, 4, 512)
    assert e.value.status == nb.DFLASH_ERR_HIP


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(OSError):
        _lib.load()


def test_page_elements_limit(lib):
    # a page of one of k_pages / v_pages is addressed with 32-bit element offsets: page_size *
    # n_kv_heads * head_dim must stay below 2^31 (1024 * 4096 * 512 = 2^31 is refused)
    d = desc(page_size=1024, max_pages_per_req=100)
    expect(call(d, hq=4096, hkv=4096, hd=512), nb.DFLASH_ERR_UNSUPPORTED, "2^31")
    # just below the limit the same shape is accepted by the planner
    p = nb.dflash_block_attn_plan(desc(page_size=1024, max_pages_per_req=100), 4095, 4095, 512)
    assert p.num_workgroups >= 1


def test_merge_mode_is_checked(lib):
    d = desc()
    d.merge_mode = 3
    expect(call(d), nb.DFLASH_ERR_INVALID_ARGUMENT, "merge_mode")
