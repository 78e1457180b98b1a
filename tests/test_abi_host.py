"""Host-only checks of the C ABI (no GPU needed).

* the library loads and exports every function include/ls_replay.h declares;
* ls_kv_page_table equals the oracle's page split, bit for bit;
* every argument check returns its status before any HIP call (so these run
  on a machine without a GPU).
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import response_replay_attention_amd as rra
from response_replay_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ls_replay.h")

LS_OK, INVALID, UNSUPPORTED, PAGE_RANGE, WORKSPACE = 0, -1, -2, -3, -4


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(ls_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = rra.lib()
    declared = _declared_functions()
    assert len(declared) >= 11, declared
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTS) == declared


def test_version_and_status_strings():
    assert rra.ls_version() >= 100
    for s in (0, -1, -2, -3, -4, -5):
        assert rra.ls_status_string(s)
    assert rra.ls_status_string(7) == "unknown status"


@pytest.mark.parametrize("seed", range(40))
def test_page_table_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    num_pages = int(rng.integers(0, 70))
    num_splits = int(rng.integers(1, 12))
    policy = int(rng.integers(0, 3))
    block = int(rng.integers(1, 5))
    owner = rng.integers(0, num_splits, num_pages).astype(np.int32)
    phys = num_pages + int(rng.integers(0, 5))
    l2p = rng.permutation(phys)[:num_pages].astype(np.int32)
    prompt_len = num_pages * 256 - (int(rng.integers(0, 256)) if num_pages else 0)
    order, offs = rra.ls_kv_page_table(num_pages, 256, prompt_len, l2p, phys, num_splits, policy,
                                       block, owner)
    eo, eoff = oracle.split_pages(num_pages, num_splits, policy, block, owner)
    assert list(order) == eo
    assert list(offs) == eoff


def test_page_table_oracle_properties():
    """Pins of the page-split oracle (definitions of the three policies)."""
    for n, s in ((0, 3), (1, 1), (10, 3), (8192, 8), (17408, 16), (97, 8)):
        for policy, block in ((0, 1), (1, 1), (1, 4)):
            order, offs = oracle.split_pages(n, s, policy, block)
            assert sorted(order) == list(range(n))
            assert offs[0] == 0 and offs[-1] == n and all(a <= b for a, b in zip(offs, offs[1:]))
            for c in range(s):
                pages = order[offs[c]:offs[c + 1]]
                assert pages == sorted(pages)
                if policy == 0:
                    assert pages == list(range(pages[0], pages[0] + len(pages))) if pages else True
                    sizes = [offs[i + 1] - offs[i] for i in range(s)]
                    assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)
                else:
                    assert all((p // block) % s == c for p in pages)
    # the 2M prefix over 8 splits: 1024 consecutive pages each
    order, offs = oracle.split_pages(8192, 8, 0)
    assert offs == [1024 * c for c in range(9)]


@pytest.mark.parametrize("args,status", [
    (dict(num_pages=-1), INVALID),
    (dict(num_splits=0), INVALID),
    (dict(page_size=128), UNSUPPORTED),
    (dict(prompt_len=5 * 256 + 1), INVALID),        # would need 6 pages
    (dict(policy=9), INVALID),
    (dict(policy=1, block_pages=0), INVALID),
    (dict(policy=2, owner=[0, 1, 2, 3, 4]), INVALID),  # owner out of range (3 splits)
    (dict(l2p=[0, 1, 2, 3, 9]), PAGE_RANGE),          # slot past the pool
    (dict(l2p=[0, 1, 2, 2, 3]), PAGE_RANGE),          # a slot used twice
    (dict(l2p=[0, 1, -1, 2, 3]), PAGE_RANGE),
    (dict(l2p=None, num_phys_pages=4), PAGE_RANGE),
])
def test_page_table_rejects(args, status):
    base = dict(num_pages=5, page_size=256, prompt_len=5 * 256, l2p=[4, 3, 2, 1, 0],
                num_phys_pages=6, num_splits=3, policy=0, block_pages=1, owner=None)
    base.update(args)
    with pytest.raises(B.LsError) as e:
        rra.ls_kv_page_table(**base)
    assert e.value.status == status


def test_page_table_partial_last_page_and_empty_prompt():
    order, offs = rra.ls_kv_page_table(3, 256, 2 * 256 + 1, [2, 0, 1], 3, 2, 0)
    assert list(order) == [0, 1, 2] and list(offs) == [0, 2, 3]
    order, offs = rra.ls_kv_page_table(0, 256, 0, None, 0, 4, 0)
    assert len(order) == 0 and list(offs) == [0, 0, 0, 0, 0]


# ------------------------------------------------ validation of the GPU calls
FAKE = 0x10000  # an aligned, never dereferenced "device" address


def _shape(**kw):
    d = dict(num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=256, prompt_len=4 * 256,
             resp_len=64, scale=1 / 16)
    d.update(kw)
    return B.AttnShape(**d)


_offs_keep = []


def _table(num_pages=4, num_splits=2, offs=None, **kw):
    o = np.array(offs if offs is not None else [0, 2, 4][: num_splits + 1], dtype=np.int32)
    _offs_keep.append(o)
    d = dict(l2p=FAKE, order=FAKE, split_offsets=FAKE, split_offsets_host=o.ctypes.data,
             num_pages=num_pages, num_splits=num_splits, num_phys_pages=num_pages)
    d.update(kw)
    return B.PageTable(**d)


def _fwd(sh, pt, **ptrs):
    p = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_resp=FAKE, v_resp=FAKE, part_o=FAKE,
             part_m=FAKE, part_l=FAKE, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptrs)
    return rra.lib().ls_replay_attn_fwd(ctypes.byref(sh), ctypes.byref(pt), p["q"], p["k_pool"],
                                        p["v_pool"], p["k_resp"], p["v_resp"], p["part_o"],
                                        p["part_m"], p["part_l"], p["ws"], p["ws_bytes"], None)


def _bwd(sh, pt, **ptrs):
    p = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_resp=FAKE, v_resp=FAKE, o=FAKE, lse=FAKE,
             d_o=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptrs)
    return rra.lib().ls_replay_attn_bwd(ctypes.byref(sh), ctypes.byref(pt), p["q"], p["k_pool"],
                                        p["v_pool"], p["k_resp"], p["v_resp"], p["o"], p["lse"],
                                        p["d_o"], p["dq"], p["dk"], p["dv"], p["ws"],
                                        p["ws_bytes"], None)


@pytest.mark.parametrize("shape_kw,status", [
    (dict(head_dim=64), UNSUPPORTED),
    (dict(page_size=128), UNSUPPORTED),
    (dict(num_q_heads=25), INVALID),       # Hq % Hkv != 0
    (dict(resp_len=0), INVALID),
    (dict(prompt_len=-1), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(prompt_len=5 * 256), INVALID),   # table has 4 pages, prompt needs 5
    (dict(resp_len=1 << 20), UNSUPPORTED), # Hq*R*d >= 2^31
    (dict(q_offset=-1), INVALID),
    (dict(q_offset=10, kv_rows=73), INVALID),            # kv_rows < q_offset + R
    (dict(kv_rows=-5), INVALID),
    (dict(flags=2), INVALID),                            # unknown flag
    (dict(q_offset=(1 << 21) - 64), UNSUPPORTED),        # Hkv*(q_offset+R)*d >= 2^31
    (dict(kv_rows=1 << 21), UNSUPPORTED),
])
def test_fwd_bwd_reject_bad_shapes(shape_kw, status):
    sh, pt = _shape(**shape_kw), _table()
    assert _fwd(sh, pt) == status
    assert _bwd(sh, pt) == status
    assert rra.ls_replay_attn_fwd_workspace(sh, pt) == 0


@pytest.mark.parametrize("table_kw", [
    dict(offs=[0, 3, 2]),                   # decreasing offsets
    dict(offs=[1, 2, 4]),                   # not starting at 0
    dict(offs=[0, 2, 3]),                   # not ending at num_pages
    dict(num_splits=0),
    dict(num_phys_pages=3),                 # fewer slots than pages
    dict(l2p=0),
    dict(order=0),
    dict(split_offsets=0),
    dict(split_offsets_host=0),
])
def test_fwd_bwd_reject_bad_tables(table_kw):
    sh, pt = _shape(), _table(**table_kw)
    assert _fwd(sh, pt) == INVALID
    assert _bwd(sh, pt) == INVALID


@pytest.mark.parametrize("name", ["q", "k_resp", "v_resp", "part_o", "part_m", "part_l", "k_pool"])
def test_fwd_rejects_null_or_misaligned(name):
    sh, pt = _shape(), _table()
    assert _fwd(sh, pt, **{name: 0}) == INVALID
    assert _fwd(sh, pt, **{name: FAKE + 2}) == INVALID


@pytest.mark.parametrize("name", ["q", "o", "lse", "d_o", "dq", "dk", "dv", "v_pool"])
def test_bwd_rejects_null_or_misaligned(name):
    sh, pt = _shape(), _table()
    assert _bwd(sh, pt, **{name: 0}) == INVALID
    assert _bwd(sh, pt, **{name: FAKE + 4}) == INVALID


def test_workspace_checks():
    sh, pt = _shape(), _table()
    need = rra.ls_replay_attn_bwd_workspace(sh, pt)
    assert need >= 24 * 64 * 4 + 3 * 24 * 64 * 256 * 4   # D + (2 splits + response) dQ slots
    assert _bwd(sh, pt, ws_bytes=need - 1) == WORKSPACE
    assert _bwd(sh, pt, ws=0) == WORKSPACE
    # a short prompt with 2 splits needs internal chunks -> forward workspace
    big = _shape(prompt_len=262_144, resp_len=1024)
    bt = _table(num_pages=1024, num_splits=1, offs=[0, 1024])
    need = rra.ls_replay_attn_fwd_workspace(big, bt)
    assert need > 0
    assert _fwd(big, bt, ws_bytes=need - 1) == WORKSPACE
    assert _fwd(big, bt, ws=0) == WORKSPACE


def _fwd_noalloc(sh, pt, **ptrs):
    p = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_resp=FAKE, v_resp=FAKE, part_o=FAKE,
             part_m=FAKE, part_l=FAKE)
    p.update(ptrs)
    return rra.lib().ls_replay_attn_fwd_noalloc(ctypes.byref(sh), ctypes.byref(pt), p["q"],
                                                p["k_pool"], p["v_pool"], p["k_resp"],
                                                p["v_resp"], p["part_o"], p["part_m"],
                                                p["part_l"], None)


def test_noalloc_forward_checks_before_any_hip_call():
    """The allocation-free forward returns the same validation errors as the
    forward (no GPU here: each return happens before any HIP call), and
    refuses a prompt whose resolved page list does not fit its scratch."""
    assert B.LS_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert _fwd_noalloc(_shape(head_dim=64), _table()) == UNSUPPORTED
    assert _fwd_noalloc(_shape(resp_len=0), _table()) == INVALID
    assert _fwd_noalloc(_shape(), _table(offs=[0, 3, 2])) == INVALID
    assert _fwd_noalloc(_shape(), _table(l2p=0)) == INVALID
    for name in ("q", "k_resp", "v_resp", "part_o", "part_m", "part_l", "k_pool"):
        assert _fwd_noalloc(_shape(), _table(), **{name: 0}) == INVALID
        assert _fwd_noalloc(_shape(), _table(), **{name: FAKE + 2}) == INVALID
    pages = (64 << 20) // 4 + 1      # 4 bytes per page: one page more than fits
    sh = _shape(prompt_len=pages * 256, resp_len=8)
    pt = _table(num_pages=pages, num_splits=1, offs=[0, pages])
    assert _fwd_noalloc(sh, pt) == WORKSPACE


def test_prompt_free_table_needs_no_pools():
    """P = 0: no pages, pools may be NULL; validation passes up to the launch."""
    sh = _shape(prompt_len=0)
    pt = _table(num_pages=0, num_splits=2, offs=[0, 0, 0], l2p=0, order=0)
    assert rra.ls_replay_attn_fwd_workspace(sh, pt) == 0
    assert rra.ls_replay_attn_bwd_workspace(sh, pt) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_parts=0), INVALID), (dict(rows=0), INVALID), (dict(head_dim=96), UNSUPPORTED),
    (dict(o=0), INVALID), (dict(lse=FAKE + 8), INVALID), (dict(pm=0), INVALID),
])
def test_merge_rejects(kw, status):
    p = dict(num_parts=9, rows=100, head_dim=256, po=FAKE, pm=FAKE, pl=FAKE, o=FAKE, lse=FAKE)
    p.update(kw)
    st = rra.lib().ls_lse_merge(p["num_parts"], p["rows"], p["head_dim"], p["po"], p["pm"], p["pl"],
                                p["o"], p["lse"], None)
    assert st == status


def test_timing_read_unknown_kernel_is_empty():
    rra.ls_timing_reset()
    assert rra.ls_timing_read("no_such_kernel") == (0, 0.0)


def test_calib_probe_rejects_bad_arguments_before_any_launch():
    f = ctypes.c_double(-1.0)
    call = rra.lib().ls_calib_mfma
    for mode, wgs, iters in ((4, 1, 8), (-1, 1, 8), (0, 0, 8), (0, 1, 4), (0, 1, 12)):
        assert call(mode, wgs, iters, FAKE, ctypes.byref(f), None) == INVALID
    assert call(0, 1, 8, None, ctypes.byref(f), None) == INVALID
    assert call(0, 1, 8, FAKE, None, None) == INVALID
    assert f.value == -1.0  # nothing was computed or launched


def _fwd_members(sh, pt, offs, dev=FAKE, num_members=None, **ptrs):
    p = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_resp=FAKE, v_resp=FAKE, part_o=FAKE,
             part_m=FAKE, part_l=FAKE, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptrs)
    o = np.ascontiguousarray(offs, dtype=np.int32)
    g = o.size - 1 if num_members is None else num_members
    return rra.lib().ls_replay_attn_fwd_members(
        ctypes.byref(sh), ctypes.byref(pt), g, o.ctypes.data if o.size else None, dev, p["q"],
        p["k_pool"], p["v_pool"], p["k_resp"], p["v_resp"], p["part_o"], p["part_m"],
        p["part_l"], p["ws"], p["ws_bytes"], None)


@pytest.mark.parametrize("offs", [
    [0, 64, 64],          # an empty member
    [1, 32, 64],          # does not start at row 0
    [0, 32, 63],          # does not end at resp_len
    [0, 40, 32, 64],      # decreasing
    [0, 65],              # past resp_len
])
def test_members_reject_bad_offsets(offs):
    assert _fwd_members(_shape(), _table(), offs) == INVALID


def test_members_reject_bad_counts_and_pointers():
    sh, pt = _shape(), _table()
    assert _fwd_members(sh, pt, [0, 64], num_members=0) == INVALID
    assert _fwd_members(sh, pt, [0, 32, 64], dev=0) == INVALID     # no device copy for G > 1
    assert _fwd_members(sh, pt, []) == INVALID                      # no host offsets
    # the shared checks of ls_replay_attn_fwd still apply
    assert _fwd_members(_shape(head_dim=64), pt, [0, 32, 64]) == UNSUPPORTED
    assert _fwd_members(sh, pt, [0, 32, 64], q=FAKE + 2) == INVALID
    assert _fwd_members(sh, pt, [0, 32, 64], ws_bytes=0) == WORKSPACE


# ---------------------------------------------------------------- page writer

def _append(hkv=4, d=256, tokens=300, slots=(5, 2), num_phys=8, **ptrs):
    p = dict(k=FAKE, v=FAKE, slots_dev=FAKE, k_pool=FAKE, v_pool=FAKE)
    p.update(ptrs)
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    return rra.lib().ls_kv_page_append(hkv, d, tokens, p["k"], p["v"],
                                       sl.ctypes.data if sl.size else None, p["slots_dev"],
                                       p["k_pool"], p["v_pool"], num_phys, None)


def test_page_append_rejects_bad_slots():
    assert _append(slots=(5, 8)) == PAGE_RANGE        # past the pool
    assert _append(slots=(-1, 2)) == PAGE_RANGE       # negative
    assert _append(slots=(3, 3)) == PAGE_RANGE        # one slot for two pages
    assert _append(tokens=256, slots=(7,), num_phys=7) == PAGE_RANGE


def test_page_append_rejects_bad_args():
    assert _append(tokens=0) == INVALID
    assert _append(hkv=0) == INVALID
    assert _append(num_phys=0) == INVALID
    assert _append(d=64) == UNSUPPORTED
    assert _append(slots=()) == INVALID                # no host slots
    assert _append(slots_dev=0) == INVALID
    assert _append(k=FAKE + 8) == INVALID              # misaligned chunk
    assert _append(v_pool=0) == INVALID
    assert _append(hkv=8, d=256, tokens=1 << 20, slots=tuple(range(4096)), num_phys=4096) == UNSUPPORTED


def test_page_append_wrapper_checks_slot_count():
    k = torch.zeros(2, 300, 128, dtype=torch.bfloat16)
    pool = torch.zeros(4, 2, 256, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rra.ls_kv_page_append(k, k, [0], torch.zeros(1, dtype=torch.int32), pool, pool)



# ---------------------------------------------------------- token-block shape

def test_token_block_shape_accepted_and_sized():
    """q_offset / kv_rows pass validation (the calls then stop at the missing
    workspace, before any HIP call) and size the response dK/dV partials."""
    pt = _table()
    whole = _shape()
    block = _shape(q_offset=192, kv_rows=512)
    assert _fwd(block, pt, ws_bytes=0) == WORKSPACE
    assert _bwd(block, pt, ws_bytes=0) == WORKSPACE
    assert _bwd(_shape(flags=B.LS_ACCUMULATE_KV), pt, ws_bytes=0) == WORKSPACE
    grow = rra.ls_replay_attn_bwd_workspace(block, pt) - rra.ls_replay_attn_bwd_workspace(whole, pt)
    # [2][Hq][q_offset + R][d] fp32 partials: 192 more keys
    assert grow == 2 * 24 * 192 * 256 * 4
    assert rra.ls_replay_attn_fwd_workspace(block, pt) == rra.ls_replay_attn_fwd_workspace(whole, pt)


def test_members_reject_q_offset():
    assert _fwd_members(_shape(q_offset=32), _table(), [0, 32, 64]) == INVALID


# ------------------------------------------------------ binding size checks

def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_binding_refuses_tensors_that_do_not_match_the_shape():
    """The kernels trust the shape struct; the binding refuses tensors whose
    sizes disagree with it before any library call."""
    sh = B.make_shape(6, 2, 128, 0, 40, 0.1, q_offset=24)
    pt = B.PageTable(0, 0, 0, 0, 0, 1, 0)
    q, kr = _t(6, 40, 128), _t(2, 64, 128)
    po, pm = _t(2, 6, 40, 128, dtype=torch.float32), _t(2, 6, 40, dtype=torch.float32)
    with pytest.raises(ValueError, match="k_resp"):      # needs q_offset + R = 64 rows
        B.ls_replay_attn_fwd(sh, pt, q, None, None, _t(2, 63, 128), kr, po, pm, pm)
    with pytest.raises(ValueError, match="q"):
        B.ls_replay_attn_fwd(sh, pt, _t(6, 41, 128), None, None, kr, kr, po, pm, pm)
    with pytest.raises(ValueError, match="part_o"):
        B.ls_replay_attn_fwd(sh, pt, q, None, None, kr, kr, po[:1], pm, pm)
    f32 = torch.float32
    with pytest.raises(ValueError, match="dk_resp"):
        B.ls_replay_attn_bwd(sh, pt, q, None, None, kr, kr, q, _t(6, 40, dtype=f32), q,
                             _t(6, 40, 128, dtype=f32), _t(2, 40, 128, dtype=f32),
                             _t(2, 64, 128, dtype=f32), None)
    with pytest.raises(ValueError, match="part_o"):
        B.ls_lse_merge(3, 6 * 40, 128, po, pm, pm, q, _t(6, 40, dtype=f32))
    k = _t(2, 300, 128)
    pool = _t(4, 2, 256, 128)
    with pytest.raises(ValueError, match="v_chunk"):
        B.ls_kv_page_append(k, _t(2, 299, 128), [0, 1], torch.zeros(2, dtype=torch.int32), pool, pool)
    with pytest.raises(ValueError, match="k_pool"):
        B.ls_kv_page_append(k, k, [0, 1], torch.zeros(2, dtype=torch.int32), _t(4, 2, 256, 64), pool)
