"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import joint_attention_amd as ja
from joint_attention_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "joint_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(joint_attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ja.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ja.load()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert set(declared) == set(_abi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_the_binding():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    defines = dict(re.findall(r"^#define\s+(JA_\w+)\s+(.+?)\s*$", text, flags=re.M))
    assert len(defines) >= 15
    for name, value in defines.items():
        if not re.fullmatch(r"[0-9()<\s]+", value):
            continue
        assert getattr(_abi, name) == eval(value), name      # digits, parentheses, shifts


def test_strerror_and_ld(lib):
    assert lib.joint_attn_strerror(0) == b"ok"
    assert b"invalid" in lib.joint_attn_strerror(1)
    assert lib.joint_attn_strerror(99) == b"unknown status"
    assert [lib.joint_attn_vt_ld(n) for n in (0, 1, 16, 17, 288, 16896)] == [0, 16, 16, 32, 288, 16896]


def _pack(lib, n, srcs, lens, B=1, H=2, D=128, layout=0, ld=0, dst=None):
    P = ctypes.c_void_p
    src_arr = (P * max(n, 1))(*srcs) if srcs is not None else None
    len_arr = (ctypes.c_int64 * max(n, 1))(*lens) if lens is not None else None
    offs = (ctypes.c_int64 * (max(n, 1) + 1))()
    st = lib.joint_attn_pack(n, src_arr, len_arr, B, H, D, layout, ld, dst, offs, None)
    return st, list(offs)


def test_pack_validation(lib):
    fake = 0x10000                                   # aligned, never dereferenced
    assert _pack(lib, 0, [], [])[0] == 1
    assert _pack(lib, 17, [fake] * 17, [1] * 17)[0] == 2
    assert _pack(lib, 2, [fake, fake], [4, 4], D=96)[0] == 2
    assert _pack(lib, 2, [fake, fake], [4, -1])[0] == 1
    assert _pack(lib, 2, [fake, None], [4, 4], dst=fake)[0] == 1        # NULL non-empty stream
    assert _pack(lib, 2, [fake, fake + 8], [4, 4], dst=fake)[0] == 2    # misaligned source
    assert _pack(lib, 2, [fake, fake], [4, 4], dst=None)[0] == 1        # NULL destination
    assert _pack(lib, 2, [fake, fake], [4, 4], layout=1, ld=8, dst=fake)[0] == 1   # ld < N
    assert _pack(lib, 2, [fake, fake], [4, 4], layout=1, ld=24, dst=fake)[0] == 1  # ld % 16
    assert _pack(lib, 2, [fake, fake], [4, 4], layout=7, dst=fake)[0] == 1
    # all-empty streams: a successful no-op that still reports offsets
    st, offs = _pack(lib, 3, [None, None, None], [0, 0, 0])
    assert st == 0 and offs == [0, 0, 0, 0]


def test_attention_validation(lib):
    fake = 0x10000
    f = lib.joint_attn_fwd_bf16
    assert f(fake, fake, fake, 1, 2, 64, 96, 64, 0.1, fake, None, None) == 2      # D
    assert f(fake, fake, fake, 0, 2, 64, 128, 64, 0.1, fake, None, None) == 1     # B
    assert f(fake, fake, fake, 1, 2, 64, 128, 48, 0.1, fake, None, None) == 1     # ldv < N
    assert f(fake, fake, fake, 1, 2, 64, 128, 72, 0.1, fake, None, None) == 1     # ldv % 16
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.0, fake, None, None) == 1     # scale
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, float("nan"), fake, None, None) == 1
    assert f(None, fake, fake, 1, 2, 64, 128, 64, 0.1, fake, None, None) == 1
    assert f(fake + 4, fake, fake, 1, 2, 64, 128, 64, 0.1, fake, None, None) == 2
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, fake, fake + 2, None) == 2  # lse align
    assert f(None, None, None, 1, 2, 0, 128, 0, 0.1, None, None, None) == 0       # N == 0
    # one head's V^T past JA_MAX_HEAD_ELEMS (its in-kernel offsets are 32-bit)
    big = _abi.JA_MAX_HEAD_ELEMS // 128 + 16
    assert f(fake, fake, fake, 1, 1, big, 128, big, 0.1, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 1, big - 16, 128, big, 0.1, fake, None, None) == 1   # pitch
    assert f(fake, fake, fake, 1, 1, 2 * big, 64, 2 * big, 0.1, fake, None, None) == 1
    assert lib.joint_attn_fwd_bf16_splitkv(fake, fake, fake, 1, 1, big, 128, big, 0.1, 2,
                                           fake, 1 << 30, fake, None, None) == 1
    g = lib.joint_attn_fwd_fp8
    assert g(fake, fake, fake, fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 7, None, None, fake,
             None, None) == 2                                                   # mode
    assert g(fake, fake, fake, None, fake, fake, 1, 2, 64, 128, 64, 0.1, 0, None, None, fake,
             None, None) == 1                                                   # q_scale
    assert g(fake, fake, fake, fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 1, None, fake, fake,
             None, None) == 1                                                   # split: q_hi
    q = lib.joint_attn_quant_fp8
    assert q(fake, fake, fake, 1, 2, 64, 128, 64, 0, fake, fake, fake, None, fake, fake,
             None, None, None, None, None) == 1                                  # q_scale
    assert q(fake, fake, fake, 1, 2, 64, 128, 64, 0, fake, fake, fake + 3, fake, fake, fake,
             None, None, None, None, None) == 2                                  # v8t align
    assert q(fake, fake, fake, 1, 2, 64, 128, 64, 1, fake, fake, fake, fake, fake, fake,
             fake, fake, None, fake, None) == 1                                  # split: hi_idx
    assert q(fake, fake, fake, 1, 2, 64, 128, 64, 2, fake, fake, fake, fake, fake, fake,
             None, None, None, None, None) == 2                                  # mode


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    x = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ja.joint_attn_pack([x])


def test_fwd_streams_validation(lib):
    fake = 0x10000
    P, I64 = ctypes.c_void_p, ctypes.c_int64

    def call(n, q, k, v, lens, B=1, H=2, D=128, scale=0.1, o=fake, lse=None):
        arr = lambda xs: (P * max(n, 1))(*xs) if xs is not None else None
        ln = (I64 * max(n, 1))(*lens) if lens is not None else None
        offs = (I64 * (max(n, 1) + 1))()
        st = lib.joint_attn_fwd_bf16_streams(n, arr(q), arr(k), arr(v), ln, B, H, D, scale, o,
                                             lse, offs, None)
        return st, list(offs)

    two = [fake, fake]
    assert call(0, [], [], [], [])[0] == 1
    assert call(17, [fake] * 17, [fake] * 17, [fake] * 17, [1] * 17)[0] == 2
    assert call(2, two, two, two, [4, 4], D=96)[0] == 2
    assert call(2, two, two, two, [4, -1])[0] == 1
    assert call(2, two, [fake, None], two, [4, 4])[0] == 1                # NULL non-empty k
    assert call(2, two, two, [fake, fake + 8], [4, 4])[0] == 2            # misaligned v
    assert call(2, two, two, two, [4, 4], o=None)[0] == 1
    assert call(2, two, two, two, [4, 4], o=fake + 2)[0] == 2
    assert call(2, two, two, two, [4, 4], scale=float("inf"))[0] == 1
    assert call(2, two, two, two, [4, 4], B=0)[0] == 1
    # empty streams are a successful no-op that still reports the offsets
    st, offs = call(3, [None] * 3, [None] * 3, [None] * 3, [0, 0, 0], o=None)
    assert st == 0 and offs == [0, 0, 0, 0]


def test_streams_splitkv_validation(lib, monkeypatch):
    fake = 0x10000
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    ws_query = lib.joint_attn_fwd_bf16_streams_splitkv_workspace
    # the workspace: the split partials, plus (pack_v = 1) the V^T copy, 256-byte rounded
    part = lib.joint_attn_fwd_bf16_splitkv_workspace(1, 2, 300, 128, 3)
    vt = -(-(1 * 2 * 128 * 304 * 2) // 256) * 256
    assert ws_query(1, 2, 300, 128, 3, 0) == part
    assert ws_query(1, 2, 300, 128, 3, 1) == part + vt
    assert ws_query(1, 2, 300, 128, 3, 2) == -1 and ws_query(1, 2, 300, 96, 3, 0) == -1

    def call(lens=(100, 200), n_split=3, pack_v=1, ws=fake, ws_bytes=None, o=fake, D=128,
             q=None):
        two = (P * 2)(*(q or [fake, fake]))
        ln = (I64 * 2)(*lens)
        offs = (I64 * 3)()
        need = ws_query(1, 2, sum(lens), D, max(n_split, 1), pack_v if pack_v in (0, 1) else 0)
        st = lib.joint_attn_fwd_bf16_streams_splitkv(
            2, two, two, two, ln, 1, 2, D, 0.1, n_split, pack_v, ws,
            need if ws_bytes is None else ws_bytes, o, None, offs, None)
        return st, list(offs)

    assert call(n_split=0)[0] == 1 and call(n_split=65)[0] == 1
    assert call(pack_v=2)[0] == 1 and call(pack_v=-1)[0] == 1
    assert call(ws=None)[0] == 1 and call(o=None)[0] == 1
    assert call(ws=fake + 8)[0] == 2 and call(o=fake + 2)[0] == 2
    assert call(D=96)[0] == 2
    assert call(q=[fake, None])[0] == 1                                   # NULL non-empty q
    # a workspace one byte short of the V^T copy plus the partials
    need = ws_query(1, 2, 300, 128, 3, 1)
    assert call(ws_bytes=need - 1)[0] == 1
    # too small for the V^T copy is still enough without it (it passes validation and
    # reaches the launch, which the library's failure hook refuses: nothing is launched)
    monkeypatch.setenv("JOINT_ATTN_SIMULATE_HIP_ERROR", "98")
    assert call(pack_v=0, ws_bytes=ws_query(1, 2, 300, 128, 3, 0))[0] == 3
    monkeypatch.delenv("JOINT_ATTN_SIMULATE_HIP_ERROR")
    # empty streams: a successful no-op that reports the offsets
    st, offs = call(lens=(0, 0), ws=None, o=None)
    assert st == 0 and offs == [0, 0, 0]


def test_quant_streams_validation(lib):
    fake = 0x10000
    P, I64 = ctypes.c_void_p, ctypes.c_int64

    def call(n, ptrs, lens, mode=0, ldv=16, D=128, q8=fake, hi=None):
        arr = (P * max(n, 1))(*ptrs)
        ln = (I64 * max(n, 1))(*lens)
        offs = (I64 * (max(n, 1) + 1))()
        st = lib.joint_attn_quant_fp8_streams(n, arr, arr, arr, ln, 1, 2, D, ldv, mode, q8, fake,
                                              fake, fake, fake, fake, hi, hi, hi, hi, offs, None)
        return st, list(offs)

    assert call(2, [fake, fake], [4, 4], ldv=8)[0] == 1       # ldv < N
    assert call(2, [fake, fake], [4, 4], mode=3)[0] == 2
    assert call(2, [fake, fake], [4, 4], mode=1)[0] == 1      # split without its buffers
    assert call(2, [fake, fake], [4, 4], q8=None)[0] == 1
    assert call(2, [fake, fake], [4, 4], q8=fake + 4)[0] == 2
    assert call(2, [fake, fake], [4, 4], D=80)[0] == 2
    st, offs = call(2, [None, None], [0, 0], ldv=0)
    assert st == 0 and offs == [0, 0, 0]


def test_sparse_validation(lib):
    fake = 0x10000
    f = lib.joint_attn_fwd_bf16_sparse
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, None, 0.1, fake, None, None) == 1   # mask
    assert f(fake, fake, fake, 1, 2, 64, 96, 64, fake, 0.1, fake, None, None) == 2    # D
    assert f(fake, fake, fake, 1, 2, 131073, 128, 131088, fake, 0.1, fake, None, None) == 2
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, fake, -1.0, fake, None, None) == 1
    assert f(None, None, None, 1, 2, 0, 128, 0, None, 0.1, None, None, None) == 0      # N == 0


def test_sparse_plan_sizes_and_validation(lib):
    fake = 0x10000
    assert lib.joint_attn_sparse_plan_bytes(2, 24, 16896) == 4 * 2 * 24 * 132
    assert lib.joint_attn_sparse_plan_bytes(1, 1, 1) == 4
    assert lib.joint_attn_sparse_plan_bytes(1, 1, 0) == 0
    assert lib.joint_attn_sparse_plan_bytes(0, 1, 128) == -1
    assert lib.joint_attn_sparse_plan_bytes(1, 1, 131073) == -1                  # N
    assert lib.joint_attn_sparse_plan_bytes(2048, 2, 131072) == -1               # units
    assert lib.joint_attn_sparse_plan_bytes(1024, 2, 131072) == 4 * 2097152
    p = lib.joint_attn_sparse_plan
    assert p(None, 1, 2, 300, fake, 24, None) == 1                               # mask
    assert p(fake, 1, 2, 300, None, 24, None) == 1                               # plan
    assert p(fake, 1, 2, 300, fake, 23, None) == 1                               # too small
    assert p(fake, 1, 2, 300, fake + 2, 24, None) == 2                           # alignment
    assert p(fake, 1, 2, 131073, fake, 1 << 20, None) == 2                       # N
    assert p(fake, 2048, 2, 131072, fake, 1 << 30, None) == 2                    # units
    assert p(fake, 0, 2, 300, fake, 24, None) == 1
    assert p(None, 1, 2, 0, None, 0, None) == 0                                  # N == 0
    f = lib.joint_attn_fwd_bf16_sparse_planned
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, fake, None, 0.1, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, None, fake, 0.1, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, fake, fake + 2, 0.1, fake, None, None) == 2
    assert f(fake, fake, fake, 1, 2, 64, 96, 64, fake, fake, 0.1, fake, None, None) == 2
    assert f(fake, fake, fake, 1, 2, 131073, 128, 131088, fake, fake, 0.1, fake, None, None) == 2
    assert f(fake, fake, fake, 2048, 2, 131072, 64, 131072, fake, fake, 0.1, fake, None,
             None) == 2                                                          # units
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, fake, fake, -1.0, fake, None, None) == 1
    assert f(None, None, None, 1, 2, 0, 128, 0, None, None, 0.1, None, None, None) == 0


def test_splitkv_sizes_and_validation(lib):
    fake = 0x10000
    ws = lib.joint_attn_fwd_bf16_splitkv_workspace
    # at most one round of split tiles: min(tiles, 256 slots) -- 256 without a GPU
    assert ws(2, 24, 4608, 128, 2) == 2 * 256 * 256 * 129 * 4          # 864 tiles
    assert ws(1, 2, 4608, 128, 2) == 2 * 36 * 256 * 129 * 4            # 36 tiles
    assert ws(1, 1, 40, 128, 3) == 3 * 256 * 129 * 4                  # one padded tile
    assert ws(1, 1, 40, 64, 3) == 3 * 128 * 65 * 4                   # 128-row tiles at D = 64
    assert ws(0, 24, 4608, 128, 2) == -1 and ws(1, 1, 16, 64, 0) == -1
    assert ws(1, 1, 16, 96, 2) == -1
    sug = lib.joint_attn_fwd_bf16_splitkv_suggest
    # without a GPU the plan assumes 256 slots (one 8-wave workgroup per CU)
    assert sug(2, 24, 4608, 128) == 2           # 864 tiles: 96 in the last round
    assert sug(1, 6, 16896, 128) == 7           # 396 tiles: 140 in the last round
    assert sug(1, 3, 16896, 128) == 5           # 198 tiles, all in one round
    assert sug(1, 8, 16896, 128) == 16          # 528 tiles: 16 in the last round
    assert sug(2, 24, 16896, 128) == 5          # 3168 tiles: 96 in the last round
    assert sug(2, 24, 512, 128) == 1            # 16 key tiles: the fixed cost dominates
    assert sug(1, 1, 40, 128) == 1
    f = lib.joint_attn_fwd_bf16_splitkv
    need = ws(1, 2, 64, 128, 2)
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 0, fake, need, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 2, fake, need - 1, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 2, None, need, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 2, fake + 8, need, fake, None, None) == 2
    assert f(None, None, None, 1, 2, 0, 128, 0, 0.1, 2, None, 0, None, None, None) == 0


def test_repair_count_and_validation(lib):
    fake = 0x10000
    rc = lib.joint_attn_repair_count
    assert rc(16896, 0.005) == 85 and rc(200, 0.005) == 1 and rc(9, 0.0) == 0 and rc(9, 1.0) == 9
    assert rc(9, 1.5) == -1 and rc(9, -0.1) == -1 and rc(-1, 0.5) == -1
    assert rc(9, float("nan")) == -1
    q = lib.joint_attn_quant_fp8_repair
    args = lambda n, err=fake, sel=fake: (fake, fake, fake, 1, 2, 64, 128, 64, n, fake, fake,
                                          fake, fake, fake, fake, err, err, sel, sel, sel, None)
    assert q(*args(65)) == 1                                   # n_repair > N
    assert q(*args(-1)) == 1
    assert q(*args(3, err=None)) == 1                          # residual outputs required
    assert q(*args(3, sel=None)) == 1                          # lists required when n > 0
    assert q(*args(3, err=fake + 2)) == 2                      # fp32 outputs 4-byte aligned
    f = lib.joint_attn_fwd_fp8_repair
    fa = lambda N, n, qx=fake, sel=fake, lse=fake: (fake, fake, fake, fake, fake, fake, qx, qx,
                                                    sel, sel, sel, n, 1, 2, N, 128,
                                                    (N + 15) // 16 * 16, 0.1, fake, lse, None)
    assert f(*fa(0, 0)) == 0                                   # N == 0: no-op
    assert f(*fa(131073, 5)) == 2                              # beyond JA_REPAIR_MAX_N
    assert f(*fa(64, 65)) == 1
    assert f(*fa(64, 3, qx=None)) == 1                         # exact q, k required
    assert f(*fa(64, 3, sel=None)) == 1
    assert f(*fa(64, 3, qx=fake + 8)) == 2                     # bf16 inputs 16-byte aligned
    assert f(*fa(64, 3, lse=None)) == 1                        # lse is read and rewritten


def test_fp8_splitkv_sizes_and_validation(lib):
    fake = 0x10000
    ws = lib.joint_attn_fwd_fp8_splitkv_workspace
    assert ws(2, 24, 16896, 128, 5) == 5 * 256 * 256 * 129 * 4        # one round of tiles
    assert ws(1, 2, 300, 64, 3) == 3 * 6 * 128 * 65 * 4               # 6 tiles of 128 rows
    assert ws(1, 1, 16, 96, 2) == -1 and ws(1, 1, 16, 64, 0) == -1
    sug = lib.joint_attn_fwd_fp8_splitkv_suggest
    assert sug(2, 24, 16896, 128, 0) == 5 and sug(2, 24, 16896, 128, 1) == 5
    assert sug(2, 24, 16896, 128, 7) == 1 and sug(1, 1, 40, 128, 0) == 1
    f = lib.joint_attn_fwd_fp8_splitkv
    need = ws(1, 2, 64, 128, 2)
    a = lambda mode=0, n=2, w=fake, wb=need, hi=None: (fake, fake, fake, fake, fake, fake, 1, 2, 64,
                                                       128, 64, 0.1, mode, hi, hi, n, w, wb, fake,
                                                       None, None)
    assert f(*a(n=0)) == 1 and f(*a(n=65)) == 1
    assert f(*a(wb=need - 1)) == 1 and f(*a(w=None)) == 1
    assert f(*a(mode=1)) == 1                                  # split mode needs q_hi, k_hi
    assert f(*a(mode=2)) == 2                                  # repair has its own entry point
    assert f(*a(w=fake + 4)) == 2


def test_launch_failure_is_reported(lib, monkeypatch):
    # every entry point, called with valid arguments, reports a launch failure as JA_EHIP
    # and keeps the HIP error for joint_attn_last_hip_error (the library's test hook
    # JOINT_ATTN_SIMULATE_HIP_ERROR stands in for the runtime's refusal; nothing is
    # launched)
    fake = 0x10000
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    monkeypatch.setenv("JOINT_ATTN_SIMULATE_HIP_ERROR", "98")
    two = (P * 2)(fake, fake)
    lens = (I64 * 2)(32, 96)
    offs = (I64 * 3)()
    N, ldv = 128, 128
    ws_bf = lib.joint_attn_fwd_bf16_splitkv_workspace(1, 2, N, 128, 2)
    ws_f8 = lib.joint_attn_fwd_fp8_splitkv_workspace(1, 2, N, 128, 2)
    calls = {
        "pack": lambda: lib.joint_attn_pack(2, two, lens, 1, 2, 128, 1, ldv, fake, offs, None),
        "fwd_bf16": lambda: lib.joint_attn_fwd_bf16(fake, fake, fake, 1, 2, N, 128, ldv, 0.1,
                                                    fake, fake, None),
        "fwd_bf16_sparse": lambda: lib.joint_attn_fwd_bf16_sparse(
            fake, fake, fake, 1, 2, N, 128, ldv, fake, 0.1, fake, None, None),
        "sparse_plan": lambda: lib.joint_attn_sparse_plan(fake, 1, 2, N, fake, 8, None),
        "fwd_bf16_sparse_planned": lambda: lib.joint_attn_fwd_bf16_sparse_planned(
            fake, fake, fake, 1, 2, N, 128, ldv, fake, fake, 0.1, fake, None, None),
        "fwd_bf16_splitkv": lambda: lib.joint_attn_fwd_bf16_splitkv(
            fake, fake, fake, 1, 2, N, 128, ldv, 0.1, 2, fake, ws_bf, fake, None, None),
        "fwd_bf16_splitkv_noalloc": lambda: lib.joint_attn_fwd_bf16_splitkv_noalloc(
            fake, fake, fake, 1, 2, N, 128, ldv, 0.1, 2, fake, None, None),
        "fwd_bf16_streams": lambda: lib.joint_attn_fwd_bf16_streams(
            2, two, two, two, lens, 1, 2, 128, 0.1, fake, None, offs, None),
        "fwd_bf16_streams_splitkv": lambda: lib.joint_attn_fwd_bf16_streams_splitkv(
            2, two, two, two, lens, 1, 2, 128, 0.1, 2, 1, fake,
            lib.joint_attn_fwd_bf16_streams_splitkv_workspace(1, 2, N, 128, 2, 1), fake, None,
            offs, None),
        "quant_fp8": lambda: lib.joint_attn_quant_fp8(
            fake, fake, fake, 1, 2, N, 128, ldv, 1, fake, fake, fake, fake, fake, fake, fake,
            fake, fake, fake, None),
        "quant_fp8_streams": lambda: lib.joint_attn_quant_fp8_streams(
            2, two, two, two, lens, 1, 2, 128, ldv, 0, fake, fake, fake, fake, fake, fake, None,
            None, None, None, offs, None),
        "fwd_fp8": lambda: lib.joint_attn_fwd_fp8(fake, fake, fake, fake, fake, fake, 1, 2, N, 128,
                                                  ldv, 0.1, 1, fake, fake, fake, None, None),
        "fwd_fp8_splitkv": lambda: lib.joint_attn_fwd_fp8_splitkv(
            fake, fake, fake, fake, fake, fake, 1, 2, N, 128, ldv, 0.1, 0, None, None, 2, fake,
            ws_f8, fake, None, None),
        "quant_fp8_repair": lambda: lib.joint_attn_quant_fp8_repair(
            fake, fake, fake, 1, 2, N, 128, ldv, 3, fake, fake, fake, fake, fake, fake, fake, fake,
            fake, fake, fake, None),
        "fwd_fp8_repair": lambda: lib.joint_attn_fwd_fp8_repair(
            fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, 3, 1, 2, N, 128, ldv,
            0.1, fake, fake, None),
    }
    for name, call in calls.items():
        assert call() == 3, name
        assert lib.joint_attn_last_hip_error() == 98, name
    assert offs[:] == [0, 32, 128]                # outputs of the host side are still written
    assert b"HIP" in lib.joint_attn_strerror(3)
    err = _abi.JointAttnError("joint_attn_fwd_bf16", 3, 98)
    assert "hipError 98" in str(err) and err.status == 3
    # an invalid argument is still reported as such, before the hook
    assert lib.joint_attn_fwd_bf16(None, fake, fake, 1, 2, N, 128, ldv, 0.1, fake, None, None) == 1


@pytest.mark.skipif(os.environ.get("JOINT_ATTN_STUB_LAUNCHERS") != "1",
                    reason="valid calls would launch kernels; runs only against the "
                           "host-only build with stand-in launchers (sanitizer test)")
def test_valid_calls_reach_the_launchers(lib, monkeypatch):
    # the same valid calls as above, without the failure hook: each passes validation and
    # reaches its launcher (the stand-ins check the invariants the kernels rely on)
    monkeypatch.delenv("JOINT_ATTN_SIMULATE_HIP_ERROR", raising=False)
    fake = 0x10000
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    two = (P * 2)(fake, fake)
    lens = (I64 * 2)(32, 96)
    offs = (I64 * 3)()
    for N, D, B, H in ((128, 128, 1, 2), (300, 64, 2, 3), (16896, 128, 2, 24)):
        ldv = (N + 15) // 16 * 16
        lens[0], lens[1] = 32, N - 32
        assert lib.joint_attn_pack(2, two, lens, B, H, D, 1, ldv, fake, offs, None) == 0
        assert offs[:] == [0, 32, N]
        assert lib.joint_attn_fwd_bf16(fake, fake, fake, B, H, N, D, ldv, 0.1, fake, fake,
                                       None) == 0
        for n_split in (1, 2, 5, 64):
            ws = lib.joint_attn_fwd_bf16_splitkv_workspace(B, H, N, D, n_split)
            assert lib.joint_attn_fwd_bf16_splitkv(fake, fake, fake, B, H, N, D, ldv, 0.1,
                                                   n_split, fake, ws, fake, None, None) == 0
            for mode in (0, 1):
                ws8 = lib.joint_attn_fwd_fp8_splitkv_workspace(B, H, N, D, n_split)
                assert lib.joint_attn_fwd_fp8_splitkv(
                    fake, fake, fake, fake, fake, fake, B, H, N, D, ldv, 0.1, mode, fake, fake,
                    n_split, fake, ws8, fake, None, None) == 0
        for n_split in (1, 2, 5):
            assert lib.joint_attn_fwd_bf16_splitkv_noalloc(fake, fake, fake, B, H, N, D, ldv, 0.1,
                                                           n_split, fake, fake, None) == 0
        assert lib.joint_attn_fwd_bf16_streams(2, two, two, two, lens, B, H, D, 0.1, fake,
                                               None, offs, None) == 0
        for n_split in (1, 2, 5):
            for pack_v in (0, 1):
                ws = lib.joint_attn_fwd_bf16_streams_splitkv_workspace(B, H, N, D, n_split,
                                                                       pack_v)
                assert lib.joint_attn_fwd_bf16_streams_splitkv(
                    2, two, two, two, lens, B, H, D, 0.1, n_split, pack_v, fake, ws, fake,
                    None, offs, None) == 0
        for mode in (0, 1):
            assert lib.joint_attn_quant_fp8(fake, fake, fake, B, H, N, D, ldv, mode, fake, fake,
                                            fake, fake, fake, fake, fake, fake, fake, fake,
                                            None) == 0
            assert lib.joint_attn_quant_fp8_streams(
                2, two, two, two, lens, B, H, D, ldv, mode, fake, fake, fake, fake, fake, fake,
                fake, fake, fake, fake, offs, None) == 0
            assert lib.joint_attn_fwd_fp8(fake, fake, fake, fake, fake, fake, B, H, N, D, ldv,
                                          0.1, mode, fake, fake, fake, None, None) == 0
        n = lib.joint_attn_repair_count(N, 0.005)
        assert lib.joint_attn_quant_fp8_repair(fake, fake, fake, B, H, N, D, ldv, n, fake, fake,
                                               fake, fake, fake, fake, fake, fake, fake, fake,
                                               fake, None) == 0
        assert lib.joint_attn_fwd_fp8_repair(fake, fake, fake, fake, fake, fake, fake, fake,
                                             fake, fake, fake, n, B, H, N, D, ldv, 0.1, fake,
                                             fake, None) == 0
        assert lib.joint_attn_fwd_bf16_sparse(fake, fake, fake, B, H, N, D, ldv, fake, 0.1,
                                              fake, None, None) == 0
        nbytes = lib.joint_attn_sparse_plan_bytes(B, H, N)
        assert lib.joint_attn_sparse_plan(fake, B, H, N, fake, nbytes, None) == 0
        assert lib.joint_attn_fwd_bf16_sparse_planned(fake, fake, fake, B, H, N, D, ldv, fake,
                                                      fake, 0.1, fake, None, None) == 0


def test_noalloc_validation(lib):
    # the allocation-free split-KV call: the usual argument checks, and partials beyond the
    # static scratch rejected before anything is launched (256 slots without a GPU)
    fake = 0x10000
    f = lib.joint_attn_fwd_bf16_splitkv_noalloc
    assert f(fake, fake, fake, 1, 2, 64, 96, 64, 0.1, 2, fake, None, None) == 2        # D
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 0, fake, None, None) == 1       # n_split
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 65, fake, None, None) == 1
    assert f(None, fake, fake, 1, 2, 64, 128, 64, 0.1, 2, fake, None, None) == 1
    assert f(fake, fake, fake, 1, 2, 64, 128, 64, 0.1, 2, fake + 8, None, None) == 2
    assert f(None, None, None, 1, 2, 0, 128, 0, 0.1, 2, None, None, None) == 0        # N == 0
    # one GPU's share of a 4-way head split of 2048^2: 140 split tiles x 7 ranges x 256 rows
    # x 129 floats = 129 MB > JA_SCRATCH_BYTES
    assert f(fake, fake, fake, 1, 6, 16896, 128, 16896, 0.1, 7, fake, None, None) == 4
    assert b"scratch" in lib.joint_attn_strerror(4)
    # 2048^2 T2I at the suggested split: 96 x 5 x 256 x 129 x 4 = 63.4 MB fits (reaches the
    # launch: the failure hook stands in for it here)
    import os
    os.environ["JOINT_ATTN_SIMULATE_HIP_ERROR"] = "98"
    try:
        assert f(fake, fake, fake, 2, 24, 16896, 128, 16896, 0.1, 5, fake, None, None) == 3
        assert 96 * 5 * 256 * 129 * 4 <= _abi.JA_SCRATCH_BYTES
    finally:
        del os.environ["JOINT_ATTN_SIMULATE_HIP_ERROR"]
