"""C-ABI library on the CPU: symbols, host mask builder vs the oracle, errors.

No compute is launched here: lvsa_attention is only called with arguments the
library must reject before touching a device.
"""

import ctypes
import os
import re
import time

import pytest
import torch

import block_sparse_attention_lvsa_amd as L
import oracle.mask as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "lvsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lvsa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = L.library()
    names = header_functions()
    assert set(names) == {"lvsa_version", "lvsa_last_error", "lvsa_mask_nnz", "lvsa_build_mask",
                          "lvsa_build_mask_steps", "lvsa_validate_mask", "lvsa_attention",
                          "lvsa_attention_ws", "lvsa_attention_workspace_bytes", "lvsa_attention_ws_static"}
    for n in names:
        assert hasattr(lib, n), n
    assert L.lvsa_version() == 2


def test_struct_layouts_match_header():
    # lvsa_tensor: pointer + 7 int64 + int32 (padded to 8) = 72 bytes.
    assert ctypes.sizeof(L.LvsaTensor) == 72
    assert ctypes.sizeof(L.LvsaMaskInfo) == 20


def _lib_rows(T, C, W, s, flags):
    m = L.lvsa_build_mask(T, C, W, s, flags)
    return m, m.rows()


@pytest.mark.parametrize("flags", [L.LVSA_ROT_MOD_TPER, L.LVSA_ROT_MOD_T, L.LVSA_FIXED_GRID, L.LVSA_WINDOW_ONLY])
def test_mask_bit_exact_at_workload_shapes(flags):
    for T, C, W, n in [(8, 4, 2, 8), (21, 21, 9, 50), (121, 21, 9, 50), (49, 33, 13, 50), (65, 33, 13, 50)]:
        for s in range(n):
            m = L.lvsa_build_mask(T, C, W, s, flags)
            rp, ci, info = om.build_mask(T, C, W, s, flags)
            assert m.row_ptr.tolist() == rp
            assert m.col_idx.tolist() == ci
            assert (m.c_eff, m.t_per, m.n_anchor, m.offset, m.nnz) == \
                (info.c_eff, info.t_per, info.n_anchor, info.offset, info.nnz)


@pytest.mark.parametrize("flags", [L.LVSA_ROT_MOD_TPER, L.LVSA_ROT_MOD_T])
def test_mask_bit_exact_sweep(flags):
    for T in list(range(1, 48)) + [64, 65, 100, 128, 200, 333]:
        for C in (2, 3, 4, 7, 12, 21, 33):
            for W in sorted({1, C // 2, C - 1}):
                if not 1 <= W <= C - 1:
                    continue
                for s in (0, 1, 2, 5, 13, 49):
                    m = L.lvsa_build_mask(T, C, W, s, flags)
                    rp, ci, _ = om.build_mask(T, C, W, s, flags)
                    assert m.col_idx.tolist() == ci, (T, C, W, s)
                    assert m.row_ptr.tolist() == rp


@pytest.mark.parametrize("flags", [L.LVSA_ROT_MOD_TPER, L.LVSA_ROT_MOD_T, L.LVSA_FIXED_GRID, L.LVSA_WINDOW_ONLY])
def test_mask_steps_bit_exact(flags):
    # A run of steps in one buffer: every step's block equals the oracle's
    # mask of that step, and all steps share one row_ptr.
    for T, C, W, step0, n in [(121, 21, 9, 0, 50), (49, 33, 13, 7, 13), (21, 21, 9, 0, 3), (8, 4, 2, 5, 11)]:
        ms = L.lvsa_build_mask_steps(T, C, W, step0, n, flags)
        assert tuple(ms.col_idx.shape) == (n, T * min(C, T))
        for i in range(n):
            rp, ci, info = om.build_mask(T, C, W, step0 + i, flags)
            m = ms.mask(i)
            assert m.row_ptr.tolist() == rp
            assert m.col_idx.tolist() == ci, (T, C, W, step0 + i)
            assert (m.c_eff, m.t_per, m.n_anchor, m.offset, m.nnz) == \
                (info.c_eff, info.t_per, info.n_anchor, info.offset, info.nnz)


def test_mask_steps_argument_errors():
    lib = L.library()
    rp = (ctypes.c_int32 * 200)()
    ci = (ctypes.c_int32 * 4000)()
    assert lib.lvsa_build_mask_steps(8, 4, 2, 0, 0, 0, rp, ci, 4000, None) == L.LVSA_ERR_ARG
    assert lib.lvsa_build_mask_steps(8, 4, 2, -1, 3, 0, rp, ci, 4000, None) == L.LVSA_ERR_ARG
    assert lib.lvsa_build_mask_steps(8, 4, 4, 0, 3, 0, rp, ci, 4000, None) == L.LVSA_ERR_ARG
    assert lib.lvsa_build_mask_steps(8, 4, 2, 2**31 - 2, 3, 0, rp, ci, 4000, None) == L.LVSA_ERR_ARG
    assert lib.lvsa_build_mask_steps(8, 4, 2, 0, 3, 0, None, ci, 4000, None) == L.LVSA_ERR_ARG
    for i in range(100):
        ci[i] = -7
    # 3 steps of 32 entries need 96: one short is a capacity error, nothing written
    assert lib.lvsa_build_mask_steps(8, 4, 2, 0, 3, 0, rp, ci, 95, None) == L.LVSA_ERR_CAPACITY
    assert all(ci[i] == -7 for i in range(100))
    assert lib.lvsa_build_mask_steps(8, 4, 2, 0, 3, 0, rp, ci, 96, None) == L.LVSA_OK
    assert ci[96] == -7
    with pytest.raises(IndexError):
        L.lvsa_build_mask_steps(8, 4, 2, 0, 3).mask(3)


def test_mask_nnz():
    assert L.lvsa_mask_nnz(121, 21, 9) == 121 * 21
    assert L.lvsa_mask_nnz(8, 21, 9) == 64


def test_build_mask_argument_errors():
    lib = L.library()
    rp = (ctypes.c_int32 * 200)()
    ci = (ctypes.c_int32 * 4000)()
    for (T, C, W, s, f) in [(0, 4, 2, 0, 0), (8, 1, 1, 0, 0), (8, 4, 0, 0, 0), (8, 4, 4, 0, 0),
                            (8, 4, 2, -1, 0), (8, 4, 2, 0, 9)]:
        rc = lib.lvsa_build_mask(T, C, W, s, f, rp, ci, 4000, None)
        assert rc == L.LVSA_ERR_ARG
        assert L.lvsa_last_error() != ""
    assert lib.lvsa_build_mask(8, 4, 2, 0, 0, None, ci, 4000, None) == L.LVSA_ERR_ARG
    # too small a buffer: error, nothing written
    for i in range(40):
        ci[i] = -7
    assert lib.lvsa_build_mask(8, 4, 2, 0, 0, rp, ci, 31, None) == L.LVSA_ERR_CAPACITY
    assert all(ci[i] == -7 for i in range(40))
    assert "capacity" in L.lvsa_last_error()
    assert lib.lvsa_build_mask(8, 4, 2, 0, 0, rp, ci, 32, None) == L.LVSA_OK
    assert L.lvsa_last_error() == ""
    with pytest.raises(ValueError):
        L.lvsa_build_mask(8, 4, 4, 0)


def test_validate_mask():
    m = L.lvsa_build_mask(121, 21, 9, 3)
    L.lvsa_validate_mask(121, m.row_ptr, m.col_idx)
    bad_cases = []
    ci = m.col_idx.clone(); ci[5], ci[6] = ci[6].item(), ci[5].item(); bad_cases.append((m.row_ptr, ci))
    ci = m.col_idx.clone(); ci[7] = ci[6]; bad_cases.append((m.row_ptr, ci))
    ci = m.col_idx.clone(); ci[0] = 121; bad_cases.append((m.row_ptr, ci))
    ci = m.col_idx.clone(); ci[0] = -1; bad_cases.append((m.row_ptr, ci))
    rp = m.row_ptr.clone(); rp[1] = 0; bad_cases.append((rp, m.col_idx))
    rp = m.row_ptr.clone(); rp[-1] = rp[-1] - 1; bad_cases.append((rp, m.col_idx))
    for rp, ci in bad_cases:
        with pytest.raises(ValueError) as e:
            L.lvsa_validate_mask(121, rp, ci)
        assert e.value.code == L.LVSA_ERR_MASK


def _rec(data=0x10000, B=1, H=2, N=512, D=64, sb=None, sh=None, sn=None, dtype=L.LVSA_DTYPE_BF16):
    sn = D if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = H * sh if sb is None else sb
    return L.LvsaTensor(data, B, H, N, D, sb, sh, sn, dtype)


def _attn(q, k, v, o, T=8, nnz=32, rp=0x1000, ci=0x2000, scale=0.0):
    lib = L.library()
    return lib.lvsa_attention(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                              ctypes.c_void_p(rp), ctypes.c_void_p(ci), T, nnz,
                              ctypes.byref(o), scale, None)


def test_attention_rejects_bad_arguments_before_any_device_work():
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q, k, v, o = (_rec(base + i * sz) for i in range(4))
    assert _attn(_rec(base, dtype=0), k, v, o) == L.LVSA_ERR_DTYPE
    assert _attn(_rec(base, D=96), k, v, o) == L.LVSA_ERR_SHAPE
    assert _attn(_rec(base + 2), k, v, o) == L.LVSA_ERR_SHAPE          # misaligned
    assert _attn(_rec(base, sn=68), k, v, o) == L.LVSA_ERR_SHAPE       # stride not 16 B multiple
    assert _attn(q, _rec(base + sz, N=256), v, o) == L.LVSA_ERR_SHAPE   # shape mismatch
    assert _attn(q, k, v, _rec(base + sz // 2)) == L.LVSA_ERR_SHAPE     # out overlaps q
    assert _attn(q, k, v, o, T=7) == L.LVSA_ERR_SHAPE                   # N % T != 0
    assert _attn(q, k, v, o, T=0) == L.LVSA_ERR_ARG
    assert _attn(q, k, v, o, rp=0) == L.LVSA_ERR_ARG
    assert _attn(q, k, v, o, nnz=-1) == L.LVSA_ERR_ARG
    assert _attn(q, k, v, o, scale=float("nan")) == L.LVSA_ERR_ARG
    assert _attn(_rec(0), k, v, o) == L.LVSA_ERR_ARG
    assert "overlap" in (_attn(q, k, v, _rec(base + sz // 2)) and L.lvsa_last_error())


def test_workspace_bytes():
    # key norms: B*H*T frames x 1 float, rounded up to 256 bytes; 256 bytes
    # of counters; then the partial records of the split items.  Frames of
    # >= 384 tokens: 8 XCD ranges x min(32, items / 32) items x 2 halves x 8
    # waves x 64 lanes x (3 D/4 + 8) floats, items = B*H*ceil(N/384).
    # Shorter frames: 8 x min(96, items / 32) x 2 x 4 waves x 64 lanes x
    # (D/2 + 4) floats, items = B*H*T*ceil(P/128).
    rec = 8 * 32 * 2 * 8 * 64 * 104 * 4
    assert L.lvsa_attention_workspace_bytes(1, 12, 121 * 1560, 128, 121) == 5888 + 256 + rec
    assert L.lvsa_attention_workspace_bytes(2, 40, 121 * 1560, 128, 121) == 38912 + 256 + rec
    # 1 x 2 x ceil(20 * 400 / 384) = 42 items: 1 per XCD range, 3 D/4 + 8 = 56 floats at D = 64
    assert L.lvsa_attention_workspace_bytes(1, 2, 20 * 400, 64, 20) == 256 + 256 + 8 * 1 * 2 * 8 * 64 * 56 * 4
    assert L.lvsa_attention_workspace_bytes(1, 2, 8 * 64, 64, 8) == 512  # 16 items: nothing split
    # 1 x 4 x 40 frames x 1 tile = 160 items: 5 per XCD range, (D/2 + 4) = 36 floats
    assert L.lvsa_attention_workspace_bytes(1, 4, 40 * 100, 64, 40) == 768 + 256 + 8 * 5 * 2 * 4 * 64 * 36 * 4
    lib = L.library()
    n = ctypes.c_int64(0)
    assert lib.lvsa_attention_workspace_bytes(0, 2, 512, 64, 8, ctypes.byref(n)) == L.LVSA_ERR_ARG
    assert lib.lvsa_attention_workspace_bytes(1, 2, 512, 64, 8, None) == L.LVSA_ERR_ARG
    assert lib.lvsa_attention_workspace_bytes(1, 2, 512, 32, 8, ctypes.byref(n)) == L.LVSA_ERR_SHAPE
    assert lib.lvsa_attention_workspace_bytes(1, 2, 513, 64, 8, ctypes.byref(n)) == L.LVSA_ERR_SHAPE


def _attn_ws(q, k, v, o, ws, ws_bytes, T=8, nnz=32, rp=0x1000, ci=0x2000):
    lib = L.library()
    return lib.lvsa_attention_ws(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                 ctypes.c_void_p(rp), ctypes.c_void_p(ci), T, nnz,
                                 ctypes.byref(o), 0.0, ctypes.c_void_p(ws), ws_bytes, None)


def test_workspace_errors_are_reported_before_any_device_work():
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q, k, v, o = (_rec(base + i * sz) for i in range(4))
    ws = base + 8 * sz
    need = L.lvsa_attention_workspace_bytes(1, 2, 512, 64, 8)  # 2·8 floats -> 256 bytes, + 256 of counters
    assert need == 512
    assert _attn_ws(q, k, v, o, 0, need) == L.LVSA_ERR_ARG                # NULL
    assert "NULL" in L.lvsa_last_error()
    assert _attn_ws(q, k, v, o, ws + 2, need) == L.LVSA_ERR_ARG           # misaligned
    assert _attn_ws(q, k, v, o, ws + 8, need) == L.LVSA_ERR_ARG           # 16-byte records
    assert "16-byte" in L.lvsa_last_error()
    assert _attn_ws(q, k, v, o, ws, need - 1) == L.LVSA_ERR_CAPACITY      # too small
    assert _attn_ws(q, k, v, o, base + 16, need) == L.LVSA_ERR_ARG        # inside q
    assert "overlaps" in L.lvsa_last_error()
    assert _attn_ws(_rec(base, dtype=0), k, v, o, ws, need) == L.LVSA_ERR_DTYPE  # the plain checks still apply


def _attn_static(q, k, v, o, T=8, nnz=32, rp=0x1000, ci=0x2000):
    lib = L.library()
    return lib.lvsa_attention_ws_static(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                        ctypes.c_void_p(rp), ctypes.c_void_p(ci), T, nnz,
                                        ctypes.byref(o), 0.0, None)


def test_static_scratch_entry_point_errors_before_any_device_work():
    # lvsa_attention_ws_static: the argument checks of lvsa_attention_ws, and
    # a key-norm table larger than the static scratch refused on the host.
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q, k, v, o = (_rec(base + i * sz) for i in range(4))
    assert _attn_static(q, k, v, o, T=0) == L.LVSA_ERR_ARG
    assert _attn_static(q, k, v, o, T=7) == L.LVSA_ERR_SHAPE
    assert _attn_static(_rec(base, dtype=0), k, v, o) == L.LVSA_ERR_DTYPE
    # 4,200 heads x 1,024 frames (stride-0 views): 17.2 MB of norms > 16 MiB
    big = [_rec(base + i * sz, H=4200, N=1024, sh=0) for i in range(4)]
    assert _attn_static(*big, T=1024, nnz=4096) == L.LVSA_ERR_CAPACITY
    assert "static scratch" in L.lvsa_last_error()
    assert L.LVSA_STATIC_SCRATCH_BYTES == 16 << 20


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_static_scratch_entry_point_without_device_reports_hip_error():
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q, k, v, o = (_rec(base + i * sz) for i in range(4))
    assert _attn_static(q, k, v, o) == L.LVSA_ERR_HIP


def test_attention_rejects_self_overlapping_output():
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q, k, v = (_rec(base + i * sz) for i in range(3))
    o = base + 3 * sz
    for bad in (_rec(o, sh=0),                  # two heads on the same rows
                _rec(o, sn=64, sh=64 * 256),    # heads 256 rows apart, 512 rows each
                _rec(o, B=2, H=1, sb=0, sh=0)):  # two batch entries on the same rows
        k2 = _rec(base + sz, B=bad.B, H=bad.H)
        v2 = _rec(base + 2 * sz, B=bad.B, H=bad.H)
        q2 = _rec(base, B=bad.B, H=bad.H)
        assert _attn(q2, k2, v2, bad) == L.LVSA_ERR_SHAPE
        assert "overlapping" in L.lvsa_last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers: the call must not reach a GPU")
def test_attention_accepts_interleaved_heads_and_broadcast_inputs():
    # [B, N, H, D] storage (heads interleaved within a token row) is not
    # self-overlapping, and q/k/v may broadcast a head with stride 0: all
    # argument checks pass and only the missing device is reported.
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q = _rec(base, sn=2 * 64, sh=64)
    k = _rec(base + sz, sh=0)
    v = _rec(base + 2 * sz, sh=0)
    o = _rec(base + 3 * sz, sn=2 * 64, sh=64)
    assert _attn(q, k, v, o) == L.LVSA_ERR_HIP


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_attention_without_device_reports_hip_error():
    base = 1 << 32
    sz = 2 * 512 * 64 * 2
    q, k, v, o = (_rec(base + i * sz) for i in range(4))
    assert _attn(q, k, v, o) == L.LVSA_ERR_HIP
    assert L.lvsa_last_error() != ""


def test_python_binding_rejects_host_tensors():
    x = torch.zeros(1, 2, 512, 64, dtype=torch.bfloat16)
    m = L.lvsa_build_mask(8, 4, 2, 0)
    with pytest.raises(ValueError):
        L.lvsa_attention(x, x, x, m, out=torch.empty_like(x))


def test_mask_build_time_within_pages_budget():
    # The pages put the CPU window extension at about 1.4 µs per frame and at
    # most 200 µs per step, anchor recomputation under 1 ms at 121 frames
    # (TechWalker article, §二 and §三).  One call here does both.
    lib = L.library()
    rp = (ctypes.c_int32 * 122)()
    ci = (ctypes.c_int32 * (121 * 21))()
    n = 2000
    t0 = time.perf_counter()
    for s in range(n):
        lib.lvsa_build_mask(121, 21, 9, s, 0, rp, ci, 121 * 21, None)
    per = (time.perf_counter() - t0) / n
    assert per < 200e-6, per
