"""C-ABI checks that need no GPU: the library loads, exports every symbol include/sfa.h declares,
sizes workspaces, picks partitions, and rejects bad arguments before anything is queued.

The attention entry points are called only with arguments that fail host validation, so no
device pointer is dereferenced and no HIP call is made.
"""

import ctypes
import os
import re
import subprocess

import pytest

from mla_sparse_top_amd import sfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfa.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(sfa_\w+)\s*\(", text, flags=re.M)))


def test_header_declarations_are_exported():
    declared = _declared_functions()
    assert set(declared) == set(sfa.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", sfa.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\b(sfa_\w+)\b", out))
    for name in declared:
        assert name in exported, name
        assert getattr(sfa._lib, name) is not None


def test_library_has_gfx950_code_object():
    # the HIP fat binary embedded in our own build names its offload target
    data = open(sfa.lib_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def _dims(**kw):
    base = dict(batch=64, s1=2, n_q=128, topk=2048, max_blocks_per_batch=64, num_cache_rows=4097 * 128)
    base.update(kw)
    return sfa.make_dims(**base)


def test_partition_choice():
    # one workgroup per (token, partition): 64 x 2 tokens need 2 partitions to fill 256 CUs
    assert sfa.num_splits(_dims()) == 2
    # 32 single-token batches want 8 (256 slots each)
    assert sfa.num_splits(_dims(batch=32, s1=1)) == 8
    # 64 single-token batches want 4; a partition needs >= 256 slots: top-k 512 gives 2
    assert sfa.num_splits(_dims(batch=64, s1=1)) == 4
    assert sfa.num_splits(_dims(batch=64, s1=1, topk=512)) == 2
    # 256 tokens or more already fill the CUs
    assert sfa.num_splits(_dims(batch=128, s1=2)) == 1
    # short lists are not partitioned (a window of 128 slots, 64 slots)
    assert sfa.num_splits(_dims(batch=64, s1=2, topk=128)) == 1
    assert sfa.num_splits(_dims(batch=1, s1=1, n_q=16, topk=64)) == 1
    # at most 8 partitions unless topk needs more
    assert sfa.num_splits(_dims(batch=1, s1=1, n_q=16, topk=2048)) == 8
    assert sfa.num_splits(_dims(batch=1, s1=1, n_q=16, topk=8192)) == 8
    assert sfa.num_splits(_dims(batch=1, s1=1, n_q=16, topk=30000)) == 15
    # prefill never partitions while topk <= 2048
    assert sfa.num_splits(_dims(batch=1, s1=4096), is_prefill=True) == 1
    # topk > 2048 forces enough partitions that each compacts <= 2048 slots
    assert sfa.num_splits(_dims(batch=1, s1=4096, topk=5000), is_prefill=True) == 3
    # explicit override, raised to the minimum
    assert sfa.num_splits(_dims(num_splits=4)) == 4
    assert sfa.num_splits(_dims(topk=5000, num_splits=1)) == 3


def test_workspace_size_formula():
    d = _dims(batch=32, s1=1)  # 8 partitions
    tokens = 32
    items = tokens * 8
    part = items * 4 * 16 * 4 * 64 * 16   # 4 waves x 16 column blocks x 4 row quads x 64 lanes x float4
    ml = items * 128 * 2 * 4              # (max, sum) per head
    cnt = 82 * tokens * 8                  # counter words per token (64-bit, tagged): arrival, ready,
                                           # 64 published flags and 16 decisions of the spread merge

    def up(x):
        return (x + 255) // 256 * 256

    assert sfa.workspace_size(d) == up(part) + up(ml) + up(cnt)
    assert sfa.workspace_size(_dims(batch=128, s1=2)) == 0


@pytest.mark.parametrize("field,value", [
    ("n_kv", 2), ("kv_lora_rank", 256), ("rope_dim", 32), ("rope_dim", 0), ("block_size", 64), ("n_q", 8),
    ("n_q", 24),
    ("n_q", 144), ("topk", 0), ("topk", 40000), ("batch", -1), ("s1", -2), ("max_blocks_per_batch", 0),
    ("num_cache_rows", -1), ("num_splits", 17), ("num_splits", -1), ("kv_dtype", 3),
])
def test_bad_dims_rejected(field, value):
    d = _dims()
    setattr(d, field, value)
    with pytest.raises(sfa.SfaError) as e:
        sfa.workspace_size(d)
    assert e.value.status == -2


def _call(fn_name, dims, ptrs=None, scale=0.04, ws=None, ws_bytes=0):
    p = dict(qn=0x100000, qr=0x200000, kn=0x10000000, kr=0x20000000, sc=0x30000000, idx=0x300000,
             bt=0x400000, act=0x500000, out=0x40000000)
    if ptrs:
        p.update(ptrs)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    fn = getattr(sfa._lib, fn_name)
    return fn(ctypes.byref(dims), vp(p["qn"]), vp(p["qr"]), vp(p["kn"]), vp(p["kr"]), vp(p["sc"]), vp(p["idx"]),
              vp(p["bt"]), vp(p["act"]), ctypes.c_float(scale), vp(p["out"]), vp(ws), ctypes.c_size_t(ws_bytes),
              None)


SMALL = dict(batch=2, s1=1, n_q=16, topk=64, max_blocks_per_batch=2, num_cache_rows=512)


@pytest.mark.parametrize("fn", ["sfa_decode", "sfa_prefill"])
def test_validation_errors(fn):
    d = _dims(**SMALL)
    assert _call(fn, d, {"qn": None}) == -1
    assert _call(fn, d, {"out": None}) == -1
    assert _call(fn, d, {"qr": 0x200008}) == -3                       # misaligned
    assert _call(fn, d, {"out": 0x40000004}) == -3
    assert _call(fn, d, scale=float("inf")) == -7
    assert _call(fn, d, scale=float("nan")) == -7
    assert _call(fn, _dims(**{**SMALL, "kv_dtype": 1}), {"sc": None}) == -5
    # out overlapping query_nope
    assert _call(fn, d, {"out": 0x100000 + 4096}) == -6
    bad = _dims(**SMALL)
    bad.n_kv = 2
    assert _call(fn, bad) == -2


def test_workspace_errors():
    d = _dims(batch=1, s1=1, n_q=16, topk=2048, max_blocks_per_batch=16, num_cache_rows=4096)
    need = sfa.workspace_size(d)
    assert need > 0
    assert _call("sfa_decode", d) == -4                                  # missing
    assert _call("sfa_decode", d, ws=0x50000000, ws_bytes=need - 1) == -4  # too small
    assert _call("sfa_decode", d, ws=0x50000010, ws_bytes=need) == -4      # not 256-aligned
    # output inside the workspace
    assert _call("sfa_decode", d, {"out": 0x50000000 + 4096}, ws=0x50000000, ws_bytes=need) == -6
    assert _call("sfa_decode", d, ws=0x10000000, ws_bytes=need) == -6      # workspace over the key pool


def test_empty_batch_is_a_no_op():
    # T = 0: validated, nothing to do, no HIP call needed
    assert _call("sfa_decode", _dims(**{**SMALL, "batch": 0})) == 0


def test_resolve_validation():
    d = _dims(**SMALL)
    f = sfa._lib.sfa_resolve_rows
    vp = ctypes.c_void_p
    assert f(ctypes.byref(d), None, vp(0x400000), vp(0x500000), vp(0x600000), None) == -1
    assert f(ctypes.byref(d), vp(0x300004), vp(0x400000), vp(0x500000), vp(0x600000), None) == -3
    assert f(ctypes.byref(d), vp(0x300000), vp(0x400000), vp(0x500000), vp(0x300000), None) == -6


def test_status_strings():
    for code in range(-9, 1):
        assert sfa.status_string(code)
    assert sfa.status_string(-99) == "unknown status"


# ---- Lightning Indexer entry points: host validation only (no pointer is dereferenced) ----

def _idims(**kw):
    base = dict(batch=2, s1=2, max_blocks_per_batch=4, num_cache_rows=1024, topk=64)
    base.update(kw)
    return sfa.make_indexer_dims(**base)


def _iscores(dims, **ptrs):
    p = dict(q=0x100000, k=0x10000000, w=0x200000, bt=0x300000, act=0x400000, scores=0x40000000)
    p.update(ptrs)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return sfa._lib.sfa_indexer_scores(ctypes.byref(dims), vp(p["q"]), vp(p["k"]), vp(p["w"]), vp(p["bt"]),
                                       vp(p["act"]), vp(p["scores"]), None)


def _iselect(dims, **ptrs):
    p = dict(scores=0x40000000, act=0x400000, out=0x50000000)
    p.update(ptrs)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return sfa._lib.sfa_topk_select(ctypes.byref(dims), vp(p["scores"]), vp(p["act"]), vp(p["out"]), None)


@pytest.mark.parametrize("field,value", [("n_heads", 32), ("head_dim", 64), ("block_size", 64), ("topk", 0),
                                         ("batch", -1), ("s1", -1), ("max_blocks_per_batch", 0),
                                         ("num_cache_rows", -1)])
def test_indexer_bad_dims_rejected(field, value):
    d = _idims()
    setattr(d, field, value)
    assert _iscores(d) == -2
    assert _iselect(d) == -2


def test_indexer_validation_errors():
    d = _idims()
    assert _iscores(d, q=None) == -1
    assert _iscores(d, scores=None) == -1
    assert _iscores(d, w=0x200004) == -3                 # misaligned
    assert _iscores(d, scores=0x100000 + 4096) == -6     # scores overlapping q_index
    assert _iselect(d, out=None) == -1
    assert _iselect(d, out=0x50000008) == -3
    assert _iselect(d, out=0x40000000 + 64) == -6        # indices overlapping the scores
    empty = _idims(batch=0)
    assert _iscores(empty) == 0 and _iselect(empty) == 0


def _cw(dims, **kw):
    p = dict(nn=0x100000, nr=0x200000, pos=0x300000, bt=0x400000, kn=0x10000000, kr=0x20000000, sc=0x30000000)
    p.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return sfa._lib.sfa_cache_write(ctypes.byref(dims), vp(p["nn"]), vp(p["nr"]), vp(p["pos"]), vp(p["bt"]),
                                    vp(p["kn"]), vp(p["kr"]), vp(p["sc"]), None)


def test_cache_write_validation():
    cw = dict(batch=2, s1=2, n_q=16, topk=1, max_blocks_per_batch=2, num_cache_rows=512)
    d = _dims(**cw)
    d8 = _dims(**{**cw, "kv_dtype": 1})
    assert _cw(d, nn=None) == -1
    assert _cw(d, kr=None) == -1
    assert _cw(d8, sc=None) == -5                        # INT8 cache without scales
    assert _cw(d, pos=0x300004) == -3                    # misaligned
    assert _cw(d8, sc=0x30000008) == -3
    assert _cw(d, kn=0x100000 + 1024) == -6              # cache overlaps new_nope
    assert _cw(d8, sc=0x10000000 + 4096) == -6           # scales inside key_nope
    assert _cw(d, kr=0x10000000 + 16) == -6              # rope inside nope
    bad = _dims(**cw)
    bad.block_size = 64
    assert _cw(bad) == -2
    bad = _dims(**cw)
    bad.kv_dtype = 7
    assert _cw(bad) == -2
    # n_q, topk and num_splits are not the write's business: odd values are accepted
    odd = _dims(**cw)
    odd.n_q, odd.topk, odd.n_kv = 3, 0, 5
    assert _cw(odd, **{"nn": None}) == -1                # still validated up to the pointers
    # nothing to write: no HIP call
    assert _cw(_dims(**{**cw, "batch": 0})) == 0
    assert _cw(_dims(**{**cw, "num_cache_rows": 0})) == 0
    # rope_dim 0 (512-wide rows): new_rope and key_rope_2d are not used
    d0 = _dims(**{**cw, "rope_dim": 0})
    assert _cw(d0, nn=None, nr=None, kr=None) == -1
    assert _cw(d0, kn=0x300000 - 1024, nr=None, kr=None) == -6   # cache over positions
    assert _cw(_dims(**{**cw, "rope_dim": 0, "batch": 0}), nr=None, kr=None) == 0
    assert _cw(_dims(**{**cw, "rope_dim": 32})) == -2


def test_probe_library_is_separate_and_exports_its_entry():
    """The MFMA throughput probe is measurement context: its own library, not in libsfa.so."""
    from mla_sparse_top_amd import build as B

    assert os.path.exists(B.PROBE_LIB_PATH)
    out = subprocess.run(["nm", "-D", "--defined-only", B.PROBE_LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "sfa_probe_mfma" in out
    main = subprocess.run(["nm", "-D", "--defined-only", sfa.lib_path()], capture_output=True, text=True,
                          check=True).stdout
    assert "sfa_probe_mfma" not in main


def _wdims(**kw):
    base = dict(batch=2, s1=2, n_q=16, n_kv=1, kv_lora_rank=512, rope_dim=64, block_size=128, window=8, topk_cmp=4,
                max_blocks_ori=2, max_blocks_cmp=1, num_cache_rows=1024, kv_dtype=0, num_splits=0)
    base.update(kw)
    return sfa.SfaWindowDims(*[base[f] for f, _ in sfa.SfaWindowDims._fields_])


def _wcall(dims, ws_bytes=None, **kw):
    p = dict(qn=0x100000, qr=0x200000, kn=0x10000000, kr=0x20000000, sc=0x30000000, ci=0x400000, bo=0x500000,
             bc=0x600000, ol=0x700000, cl=0x800000, out=0x40000000, ws=0x50000000)
    p.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    if ws_bytes is None:
        ws_bytes = 1 << 30
    return sfa._lib.sfa_window_decode(ctypes.byref(dims), vp(p["qn"]), vp(p["qr"]), vp(p["kn"]), vp(p["kr"]),
                                      vp(p["sc"]), vp(p["ci"]), vp(p["bo"]), vp(p["bc"]), vp(p["ol"]), vp(p["cl"]),
                                      ctypes.c_float(0.05), vp(p["out"]), vp(p["ws"]), ctypes.c_size_t(ws_bytes), None)


def test_window_validation():
    # num_splits = 2 forces partitions, so the call needs a workspace; every call below fails
    # host validation, so nothing is ever launched
    d = _wdims(num_splits=2)
    need = sfa.window_workspace_size(d)
    assert need > 0
    assert sfa.window_workspace_size(_wdims()) == 0          # one partition: no workspace
    assert _wcall(d, qn=None) == -1
    assert _wcall(d, ci=None) == -1                          # topk_cmp > 0 needs the compressed source
    # SWA (topk_cmp == 0) takes no compressed source: the null pointers pass, and the missing
    # workspace is what fails
    assert _wcall(_wdims(topk_cmp=0, max_blocks_cmp=0, num_splits=2), ci=None, bc=None, cl=None, ws=None) == -4
    assert _wcall(_wdims(kv_dtype=1, num_splits=2), sc=None) == -5
    assert _wcall(d, bo=0x500004) == -3
    assert _wcall(d, bc=0x600004) == -3
    assert _wcall(d, ws=0x50000010) == -4                    # workspace not 256-byte aligned
    assert _wcall(d, ws_bytes=need - 1) == -4
    assert _wcall(d, out=0x100000 + 64) == -6                # out over query_nope
    assert _wcall(d, out=0x600000 - 64) == -6                # out over block_table_cmp
    assert _wcall(d, out=0x50000000 + 256) == -6             # out inside the workspace
    assert _wcall(_wdims(window=-1)) == -2
    assert _wcall(_wdims(window=0, topk_cmp=0)) == -2
    assert _wcall(_wdims(max_blocks_cmp=0)) == -2            # topk_cmp > 0 without a compressed table
    assert _wcall(_wdims(block_size=64)) == -2               # the attention's own dims are checked too
    assert _wcall(_wdims(window=40000)) == -2                # above the attention's top-k limit
    assert _wcall(_wdims(batch=0, num_splits=2), ws_bytes=need) == 0  # nothing to do, nothing queued
    # rope_dim 0 (512-wide rows): accepted by the window variants only; query_rope and key_rope
    # are then not needed (the null pointers pass, and the missing workspace is what fails)
    d0 = _wdims(rope_dim=0, num_splits=2)
    assert sfa.window_workspace_size(d0) == need
    assert _wcall(d0, qr=None, kr=None, ws=None) == -4
    assert _wcall(d0, qr=0x200004, kr=0x20000004, ws=None) == -4   # not read, so not checked
    assert _wcall(d0, qn=None, qr=None, kr=None, ws=None) == -1
    assert _wcall(d0, out=0x200000, qr=None, kr=None, ws=None) == -4  # no rope array to overlap
    assert _wcall(_wdims(rope_dim=0, batch=0, num_splits=2), qr=None, kr=None, ws_bytes=need) == 0
    assert _wcall(_wdims(rope_dim=32)) == -2
    assert _wcall(d, qr=None) == -1                          # with rope channels both are needed
    assert _wcall(d, kr=None) == -1


def _cdims(**kw):
    base = dict(batch=2, s1=2, channels=576, ratio=4, rope_positions=64, max_blocks=2, block_size=128,
                num_cache_rows=512)
    base.update(kw)
    return sfa.SfaCompressDims(**base)


def _cmp(dims, eps=1e-6, **kw):
    """sfa_compress with fake, well-separated device addresses; every case here fails validation
    (or has nothing to do), so nothing is launched."""
    p = dict(kv=0x1000000, sc=0x2000000, ape=0x3000000, g=0x3100000, cos=0x3200000, sin=0x3300000, sp=0x3400000,
             ks=0x4000000, ss=0x5000000, bt=0x6000000, kn=0x10000000, kr=0x20000000)
    p.update(kw)
    vp = lambda x: ctypes.c_void_p(x)  # noqa: E731
    return sfa._lib.sfa_compress(ctypes.byref(dims), vp(p["kv"]), vp(p["sc"]), vp(p["ape"]), vp(p["g"]),
                                 ctypes.c_float(eps), vp(p["cos"]), vp(p["sin"]), vp(p["sp"]), vp(p["ks"]),
                                 vp(p["ss"]), vp(p["bt"]), vp(p["kn"]), vp(p["kr"]), None)


def test_compress_validation():
    d = _cdims()
    for name in ("kv", "sc", "ape", "g", "cos", "sin", "sp", "ks", "ss", "bt", "kn", "kr"):
        assert _cmp(d, **{name: None}) == -1, name
    assert _cmp(d, sp=0x3400004) == -3                   # misaligned
    assert _cmp(d, kr=0x20000008) == -3
    assert _cmp(d, ks=0x1000000 + 4096) == -6            # state overlaps kv
    assert _cmp(d, ss=0x4000000 + 16) == -6              # score state inside kv state
    assert _cmp(d, kn=0x3400000) == -6                   # pool over start_pos
    assert _cmp(d, kr=0x10000000 + 1024) == -6           # rope rows inside nope rows
    for field, value in (("channels", 256), ("channels", 575), ("block_size", 64), ("ratio", 0), ("ratio", 1025), ("batch", -1),
                         ("s1", -1), ("max_blocks", 0), ("rope_positions", -1), ("num_cache_rows", -1)):
        assert _cmp(_cdims(**{field: value})) == -2, field
    assert _cmp(d, eps=-1.0) == -2
    assert _cmp(d, eps=float("nan")) == -2
    assert _cmp(d, eps=float("inf")) == -2
    assert _cmp(_cdims(batch=0)) == 0                    # nothing to do: no HIP call
    assert _cmp(_cdims(s1=0)) == 0
    # the Hadamard branch needs a power-of-two width: 128 channels only
    assert _cmp(_cdims(rotate=1)) == -2
    assert _cmp(_cdims(rotate=2)) == -2
    assert _cmp(_cdims(channels=128, rotate=2)) == -2
    # 128 channels: the row goes whole to key_nope_2d, key_rope_2d may be NULL (validated only)
    c128 = _cdims(channels=128, rotate=1)
    assert _cmp(c128, kn=None) == -1
    assert _cmp(c128, ks=0x1000000 + 1024) == -6          # state overlaps kv (2 KB at 128 channels)
    # 512 channels (rotary channels inside the row): whole to key_nope_2d, no Hadamard branch
    c512 = _cdims(channels=512)
    assert _cmp(c512, kn=None) == -1
    assert _cmp(_cdims(channels=512, rotate=1)) == -2
    assert _cmp(_cdims(channels=512, s1=0), kr=None) == 0


def test_noalloc_rejects_calls_beyond_its_scratch():
    # top-k 32768 forces 16 partitions per token: 128 tokens x 16 x 256 KB is far beyond the
    # fixed scratch, rejected on the host before any HIP call
    d = _dims(batch=64, s1=2, n_q=128, topk=32768, max_blocks_per_batch=256, num_cache_rows=4097 * 128)
    assert sfa.workspace_size(d) > sfa.NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    p = [vp(0x100000 + i * 0x10000000) for i in range(8)]
    f = sfa._lib.sfa_decode_noalloc
    assert f(ctypes.byref(d), *p, ctypes.c_float(1.0), vp(0x7000000000), None) == -9
    assert "scratch" in sfa.status_string(-9)
    # the default decode shape fits
    assert sfa.workspace_size(_dims()) <= sfa.NOALLOC_SCRATCH_BYTES
    # argument errors are sfa_decode's
    s = _dims(**SMALL)
    assert f(ctypes.byref(s), None, *p[1:], ctypes.c_float(1.0), vp(0x7000000000), None) == -1
    assert f(ctypes.byref(s), *p, ctypes.c_float(float("nan")), vp(0x7000000000), None) == -7


def _prolog_dims(**kw):
    base = dict(tokens=128, hidden=7168, q_lora_rank=1536, n_q=128, qk_nope_dim=128, rope_positions=8192, eps=1e-6)
    base.update(kw)
    return sfa.SfaPrologDims(**base)


def _prolog_call(d, over=None, ws=0x7000000000, ws_bytes=None):
    vp = ctypes.c_void_p
    names = ["x", "w_dq", "gcq", "w_uq", "w_uk", "w_dkv", "gckv", "pos", "cos", "sin", "qn", "qr", "kn", "kr", "cq"]
    p = {n: 0x100000000 * (i + 1) for i, n in enumerate(names)}
    p["cq"] = None
    p.update(over or {})
    if ws_bytes is None:
        ws_bytes = sfa.prolog_workspace_size(d)
    return sfa._lib.sfa_mla_prolog(ctypes.byref(d), *[vp(p[n]) if p[n] is not None else None for n in names],
                                   vp(ws) if ws else None, ctypes.c_size_t(ws_bytes), None)


def test_prolog_workspace_and_splits():
    # decode shape: 33 feature tiles x 7 k splits of the down-projections (231 workgroups, one
    # round on 256 compute units); partials, cq and the per-head nope parts as hi/lo pairs
    d = _prolog_dims()
    part = 7 * 128 * (1536 + 576) * 4
    cq = 2 * 128 * 1536 * 2
    qn = 2 * 128 * 128 * 128 * 2
    assert sfa.prolog_workspace_size(d) == part + cq + qn
    assert sfa.prolog_workspace_size(_prolog_dims(tokens=0)) == 0


@pytest.mark.parametrize("field,value", [("hidden", 0), ("hidden", 7200), ("q_lora_rank", 32), ("q_lora_rank", 8192),
                                         ("n_q", 0), ("n_q", 129), ("qk_nope_dim", 48), ("qk_nope_dim", 144),
                                         ("rope_positions", 0), ("eps", -1.0), ("eps", float("nan")), ("tokens", -1)])
def test_prolog_bad_dims_rejected(field, value):
    d = _prolog_dims(**{field: value})
    out = ctypes.c_size_t(0)
    assert sfa._lib.sfa_mla_prolog_workspace_size(ctypes.byref(d), ctypes.byref(out)) == -2
    assert _prolog_call(d, ws_bytes=0) == -2


def test_prolog_validation_errors():
    d = _prolog_dims()
    assert _prolog_call(d, {"x": None}) == -1
    assert _prolog_call(d, {"kr": None}) == -1
    assert _prolog_call(d, {"w_uk": 0x100000008}) == -3
    assert _prolog_call(d, ws=None) == -4
    assert _prolog_call(d, ws=0x7000000010) == -4
    need = sfa.prolog_workspace_size(d)
    assert _prolog_call(d, ws_bytes=need - 1) == -4
    assert _prolog_call(d, {"qn": 0x100000000 * 2 + 4096}) == -6     # q_nope inside w_dq
    assert _prolog_call(d, {"kn": 0x7000000000 + 4096}) == -6          # kv_nope inside the workspace
    assert _prolog_call(d, {"kr": 0x100000000 * 13 + 64}) == -6        # kv_rope inside kv_nope
    # no tokens: nothing is read, NULL pointers are fine
    assert _prolog_call(_prolog_dims(tokens=0), {n: None for n in ("x", "qn")}, ws=None, ws_bytes=0) == 0
    # the optional cq output: aligned, overlapping nothing
    assert _prolog_call(d, {"cq": 0x100000000 * 15 + 8}) == -3
    assert _prolog_call(d, {"cq": 0x100000000 * 1 + 64}) == -6      # inside x
    assert _prolog_call(d, {"cq": 0x7000000000 + 4096}) == -6        # inside the workspace


def _v4_dims(**kw):
    base = dict(tokens=128, hidden=4096, q_lora_rank=1536, n_q=128, head_dim=512, rope_positions=8192, eps=1e-6)
    base.update(kw)
    return sfa.SfaPrologV4Dims(**base)


def _v4_call(d, over=None, ws=0x7000000000, ws_bytes=None):
    """sfa_mla_prolog_v4 with fake device addresses 4 GiB apart; every case here fails validation
    (or has no tokens), so nothing is launched."""
    vp = ctypes.c_void_p
    names = ["x", "w_dq", "gcq", "w_uq", "w_dkv", "gckv", "pos", "cos", "sin", "q", "kv", "cq"]
    p = {n: 0x100000000 * (i + 1) for i, n in enumerate(names)}
    p["cq"] = None
    p.update(over or {})
    if ws_bytes is None:
        ws_bytes = sfa.prolog_v4_workspace_size(d)
    return sfa._lib.sfa_mla_prolog_v4(ctypes.byref(d), *[vp(p[n]) if p[n] is not None else None for n in names],
                                      vp(ws) if ws else None, ctypes.c_size_t(ws_bytes), None, None)


def test_prolog_v4_workspace():
    # 32 feature tiles x 8 k splits of the down-projections; cq as hi/lo; the up-projection's fp32
    # sums (256 tiles of 256 features: no split)
    d = _v4_dims()
    assert sfa.prolog_v4_workspace_size(d) == 8 * 128 * (1536 + 512) * 4 + 2 * 128 * 1536 * 2 + 128 * 65536 * 4
    assert sfa.prolog_v4_workspace_size(_v4_dims(tokens=0)) == 0


@pytest.mark.parametrize("field,value", [("hidden", 0), ("hidden", 4100), ("q_lora_rank", 32), ("q_lora_rank", 8192),
                                         ("n_q", 0), ("n_q", 129), ("head_dim", 576), ("head_dim", 128),
                                         ("rope_positions", 0), ("eps", -1.0), ("eps", float("nan")), ("tokens", -1)])
def test_prolog_v4_bad_dims_rejected(field, value):
    d = _v4_dims(**{field: value})
    out = ctypes.c_size_t(0)
    assert sfa._lib.sfa_mla_prolog_v4_workspace_size(ctypes.byref(d), ctypes.byref(out)) == -2
    assert _v4_call(d, ws_bytes=0) == -2


def test_prolog_v4_validation_errors():
    d = _v4_dims()
    assert _v4_call(d, {"x": None}) == -1
    assert _v4_call(d, {"q": None}) == -1
    assert _v4_call(d, {"kv": None}) == -1
    assert _v4_call(d, {"w_uq": 0x400000008}) == -3
    assert _v4_call(d, ws=None) == -4
    assert _v4_call(d, ws=0x7000000010) == -4
    assert _v4_call(d, ws_bytes=sfa.prolog_v4_workspace_size(d) - 1) == -4
    assert _v4_call(d, {"q": 0x100000000 * 2 + 4096}) == -6        # q inside w_dq
    assert _v4_call(d, {"kv": 0x7000000000 + 4096}) == -6           # kv inside the workspace
    assert _v4_call(d, {"kv": 0x100000000 * 10 + 64}) == -6         # kv inside q
    assert _v4_call(d, {"cq": 0x100000000 * 13 + 8}) == -3
    assert _v4_call(d, {"cq": 0x100000000 * 1 + 64}) == -6          # inside x
    assert _v4_call(_v4_dims(tokens=0), {n: None for n in ("x", "q", "kv")}, ws=None, ws_bytes=0) == 0


def _ip_dims(**kw):
    base = dict(tokens=128, hidden=7168, q_lora_rank=1536, n_heads=64, head_dim=128, rope_positions=8192, rotate=1,
                eps=1e-6)
    base.update(kw)
    return sfa.SfaIndexerPrologDims(**base)


def _ip_call(d, over=None, ws=0x7000000000, ws_bytes=None):
    vp = ctypes.c_void_p
    names = ["x", "qr", "wqb", "wk", "g", "b", "wp", "pos", "cos", "sin", "q", "k", "w"]
    p = {n: 0x100000000 * (i + 1) for i, n in enumerate(names)}
    p.update(over or {})
    if ws_bytes is None:
        ws_bytes = sfa.indexer_prolog_workspace_size(d)
    return sfa._lib.sfa_indexer_prolog(ctypes.byref(d), *[vp(p[n]) if p[n] is not None else None for n in names],
                                       vp(ws) if ws else None, ctypes.c_size_t(ws_bytes), None)


def test_indexer_prolog_workspace_and_validation():
    d = _ip_dims()
    # index query partials: 128 tiles x 2 k splits; key and weight partials: 3 tiles x 28 splits
    assert sfa.indexer_prolog_workspace_size(d) == 2 * 128 * 8192 * 4 + 28 * 128 * 192 * 4
    assert sfa.indexer_prolog_workspace_size(_ip_dims(tokens=0)) == 0
    for field, value in (("n_heads", 32), ("head_dim", 64), ("rotate", 2), ("hidden", 200), ("q_lora_rank", 100),
                         ("eps", -1.0), ("rope_positions", 0), ("tokens", -1)):
        out = ctypes.c_size_t(0)
        assert sfa._lib.sfa_indexer_prolog_workspace_size(ctypes.byref(_ip_dims(**{field: value})),
                                                          ctypes.byref(out)) == -2, field
    assert _ip_call(d, {"qr": None}) == -1
    assert _ip_call(d, {"w": None}) == -1
    assert _ip_call(d, {"wk": 0x100000000 * 4 + 2}) == -3
    assert _ip_call(d, ws=None) == -4
    assert _ip_call(d, ws_bytes=sfa.indexer_prolog_workspace_size(d) - 1) == -4
    assert _ip_call(d, {"q": 0x100000000 * 2 + 256}) == -6           # q_index inside qr
    assert _ip_call(d, {"w": 0x7000000000 + 1024}) == -6             # weights inside the workspace
    assert _ip_call(_ip_dims(tokens=0), {"x": None, "q": None}, ws=None, ws_bytes=0) == 0


def test_workspace_over_an_input_is_rejected():
    """The kernels write their workspace, so a workspace over an input is an alias error; each
    call here fails validation before any launch."""
    assert _prolog_call(_prolog_dims(), ws=0x100000000) == -6        # over x
    assert _v4_call(_v4_dims(), ws=0x100000000) == -6                # over x
    assert _v4_call(_v4_dims(), ws=0x400000000) == -6                # over w_uq
    assert _ip_call(_ip_dims(), ws=0x200000000) == -6                # over qr
    assert "workspace overlaps an input" in sfa.status_string(-6)
