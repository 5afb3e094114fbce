"""The C-ABI library loads, exports what include/ra.h declares, and rejects bad
arguments on the host (no GPU needed: only the *_validate entry points and calls
that fail validation are made, neither of which touches the device)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ra():
    import long_context_exact_tiled_amd as m
    if not os.path.exists(m.LIB_PATH):
        from long_context_exact_tiled_amd.build import build
        build()
    m.lib()
    return m


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(ra):
    names = _declared_symbols()
    assert {"ra_attn_fwd", "ra_lse_merge", "ra_ulysses_permute", "ra_attn_bwd"} <= set(names)
    L = ctypes.CDLL(ra.LIB_PATH)
    for name in names:
        assert hasattr(L, name), name


def test_version_and_status_strings(ra):
    assert ra.version() == 100
    for code, name in ra.STATUS.items():
        assert ra.status_string(code).startswith(name)
    assert ra.status_string(12345) == "unknown ra_status"


def _t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _fwd(ra, q, k, v, o=None, lse=None, **kw):
    o = torch.zeros(q.shape, dtype=q.dtype) if o is None else o
    lse = torch.zeros(q.shape[:3], dtype=torch.float32) if lse is None else lse
    return ra.STATUS[ra.attn_fwd_validate(q, k, v, o, lse, **kw)]


def test_fwd_validation(ra):
    q, k, v = _t((1, 4, 64, 128)), _t((1, 2, 64, 128)), _t((1, 2, 64, 128))
    assert _fwd(ra, q, k, v) == "RA_OK"
    assert _fwd(ra, q, k, v, causal=True, num_chunks=4, start_chunk=3, q_offset=7) == "RA_OK"
    assert _fwd(ra, q, k, v.float()) == "RA_ERR_DTYPE"
    assert _fwd(ra, q, k, v, lse=torch.zeros((1, 4, 64), dtype=torch.bfloat16)) == "RA_ERR_DTYPE"
    assert _fwd(ra, q, k, v, o=torch.zeros(q.shape)) == "RA_OK"  # fp32 partial output
    assert _fwd(ra, q, _t((1, 3, 64, 128)), _t((1, 3, 64, 128))) == "RA_ERR_SHAPE"  # Hq % Hkv
    assert _fwd(ra, q, k, _t((1, 2, 63, 128))) == "RA_ERR_SHAPE"
    assert _fwd(ra, q, k, v, num_chunks=3) == "RA_ERR_SHAPE"  # 64 % 3
    assert _fwd(ra, q, k, v, num_chunks=0) == "RA_ERR_RANGE"
    assert _fwd(ra, q, k, v, num_chunks=4, start_chunk=4) == "RA_ERR_RANGE"
    assert _fwd(ra, q, k, v, start_chunk=-1) == "RA_ERR_RANGE"
    assert _fwd(ra, q, k, v, q_offset=-1) == "RA_ERR_RANGE"
    assert _fwd(ra, q, k, v, scale=float("nan")) == "RA_ERR_RANGE"
    assert _fwd(ra, _t((1, 4, 64, 96)), _t((1, 2, 64, 96)), _t((1, 2, 64, 96))) \
        == "RA_ERR_UNSUPPORTED"
    # innermost stride != 1
    qt = _t((1, 4, 128, 64)).transpose(2, 3)
    assert _fwd(ra, qt, _t((1, 2, 64, 128)), _t((1, 2, 64, 128))) == "RA_ERR_STRIDE"
    # overlapping output rows
    o_bad = _t((1, 4, 1, 128)).expand(1, 4, 64, 128)
    assert _fwd(ra, q, k, v, o=o_bad) == "RA_ERR_STRIDE"
    # misaligned pointer (2-byte offset) and misaligned row stride
    base = _t((1 * 4 * 64 * 128 + 8,))
    q_mis = base[1:1 + 4 * 64 * 128].view(1, 4, 64, 128)
    assert _fwd(ra, q_mis, k, v) == "RA_ERR_ALIGN"
    wide = _t((1, 4, 64, 132))[..., :128]
    assert _fwd(ra, wide, k, v) == "RA_ERR_ALIGN"
    # a BSHD view (heads strided inside a token row) is a valid layout
    qb = _t((1, 64, 4, 128)).transpose(1, 2)
    assert _fwd(ra, qb, k, v) == "RA_OK"
    # empty problems are valid
    assert _fwd(ra, _t((1, 4, 0, 128)), k, v) == "RA_OK"
    assert _fwd(ra, q, _t((1, 2, 0, 128)), _t((1, 2, 0, 128))) == "RA_OK"


def test_varlen_validation(ra):
    q, k, v = _t((1, 4, 64, 128)), _t((1, 2, 64, 128)), _t((1, 2, 64, 128))
    cu = torch.tensor([0, 10, 64], dtype=torch.int32)

    def f(q=q, k=k, v=v, cu=cu, o=None, lse=None, **kw):
        o = torch.zeros(q.shape, dtype=q.dtype) if o is None else o
        lse = torch.zeros(q.shape[:3], dtype=torch.float32) if lse is None else lse
        return ra.STATUS[ra.attn_fwd_varlen_validate(q, k, v, cu, o, lse, **kw)]

    assert f() == "RA_OK"
    assert f(causal=True) == "RA_OK"
    assert f(o=torch.zeros(q.shape)) == "RA_OK"  # fp32 output
    assert f(k=_t((1, 2, 32, 128)), v=_t((1, 2, 32, 128))) == "RA_ERR_SHAPE"  # T differs
    assert f(q=q.float(), k=k.float(), v=v.float()) == "RA_ERR_UNSUPPORTED"  # bf16 only
    with pytest.raises(ra.RaError):
        f(cu=torch.tensor([0], dtype=torch.int32))
    with pytest.raises(ra.RaError):
        f(cu=torch.tensor([0, 64], dtype=torch.int64))


def test_bwd_varlen_validation(ra):
    q, k, v = _t((1, 4, 64, 128)), _t((1, 2, 64, 128)), _t((1, 2, 64, 128))
    o, do, lse = _t(q.shape), _t(q.shape), torch.zeros(1, 4, 64)
    cu = torch.tensor([0, 10, 64], dtype=torch.int32)

    def f(q=q, k=k, v=v, **kw):
        return ra.STATUS[ra.attn_bwd_varlen_validate(q, k, v, o, do, lse, cu, _t(q.shape),
                                                     _t(k.shape), _t(v.shape), **kw)]

    assert f() == "RA_OK" and f(causal=True) == "RA_OK"
    assert f(k=_t((1, 2, 32, 128)), v=_t((1, 2, 32, 128))) == "RA_ERR_SHAPE"
    # the packed forward is bf16 only, so is its backward
    fo = lambda t: t.float()
    assert ra.STATUS[ra.attn_bwd_varlen_validate(fo(q), fo(k), fo(v), fo(o), fo(do), lse, cu,
                                                 fo(q), fo(k), fo(v))] == "RA_ERR_UNSUPPORTED"


def test_fwd_rejects_before_launch(ra):
    """A failing call returns its code without touching the device (CPU tensors here)."""
    q, k = _t((1, 4, 64, 128)), _t((1, 3, 64, 128))
    with pytest.raises(ra.RaError) as e:
        ra.lib()  # loaded
        o = torch.zeros(q.shape, dtype=q.dtype)
        lse = torch.zeros(q.shape[:3])
        p = ra._params(False, 1, 0, 0, 0, None)
        ra._check(ra.lib().ra_attn_fwd(ra.desc(q), ra.desc(k), ra.desc(k), ctypes.byref(p),
                                       ra.desc(o), ra.desc(lse), None))
    assert e.value.name == "RA_ERR_SHAPE"
    assert ra.lib().ra_attn_fwd(None, None, None, None, None, None, None) == -1


def test_merge_validation(ra):
    parts = [torch.zeros(1, 2, 10, 128) for _ in range(3)]
    lses = [torch.zeros(1, 2, 10) for _ in range(3)]
    out, lse = torch.zeros(1, 2, 10, 128, dtype=torch.bfloat16), torch.zeros(1, 2, 10)
    v = lambda p, l, o=out, ls=lse: ra.STATUS[ra.lse_merge_validate(p, l, o, ls)]
    assert v(parts, lses) == "RA_OK"
    assert v([], []) == "RA_ERR_RANGE"
    assert v(parts * 22, lses * 22) == "RA_ERR_RANGE"  # 66 > 64 parts
    assert v(parts[:2] + [parts[2].bfloat16()], lses) == "RA_ERR_DTYPE"
    assert v(parts, lses[:2] + [lses[2].bfloat16()]) == "RA_ERR_DTYPE"
    assert v(parts[:2] + [torch.zeros(1, 2, 11, 128)], lses) == "RA_ERR_SHAPE"
    strided = torch.zeros(1, 2, 10, 256)[..., :128]
    assert v(parts[:2] + [strided], lses) == "RA_ERR_STRIDE"
    assert v([torch.zeros(1, 2, 10, 12)] * 3, lses, torch.zeros(1, 2, 10, 12)) \
        == "RA_ERR_UNSUPPORTED"


def test_permute_validation(ra):
    src = _t((4, 16, 28, 128))
    dst = _t((7, 64, 128))
    v = lambda s, d, P, r, dr: ra.STATUS[ra.ulysses_permute_validate(s, d, P, r, dr)]
    assert v(src, dst, 4, 0, 0) == "RA_OK"
    assert v(src, _t((4, 7, 64, 128)), 4, -1, 0) == "RA_OK"
    assert v(dst, src, 4, 3, 1) == "RA_OK"
    assert v(src, dst, 4, 4, 0) == "RA_ERR_RANGE"
    assert v(src, dst, 4, -2, 0) == "RA_ERR_RANGE"
    assert v(src, dst, 4, 0, 2) == "RA_ERR_RANGE"
    assert v(src, dst.float(), 4, 0, 0) == "RA_ERR_DTYPE"
    assert v(_t((4, 16, 30, 128)), dst, 4, 0, 0) == "RA_ERR_SHAPE"  # H % P
    assert v(src, _t((7, 63, 128)), 4, 0, 0) == "RA_ERR_SHAPE"
    assert v(_t((4, 16, 28, 4)), _t((7, 64, 4)), 4, 0, 0) == "RA_ERR_ALIGN"  # 8-byte rows


def test_permute_n_validation(ra):
    q, k, v = _t((4, 16, 28, 128)), _t((4, 16, 4, 128)), _t((4, 16, 4, 128))
    qh, kh, vh = _t((7, 64, 128)), _t((1, 64, 128)), _t((1, 64, 128))
    v_ = lambda s, d, P=4, r=0, dr=0: ra.STATUS[ra.ulysses_permute_multi_validate(s, d, P, r, dr)]
    assert v_([q, k, v], [qh, kh, vh]) == "RA_OK"
    assert v_([qh, kh, vh], [q, k, v], dr=1) == "RA_OK"
    assert v_([q, k, v], [qh, kh, _t((2, 64, 128))]) == "RA_ERR_SHAPE"  # third pair invalid
    assert v_([q] * 5, [qh] * 5) == "RA_ERR_RANGE"                      # more than 4 pairs
    assert v_([], []) == "RA_ERR_RANGE"
    # destinations overlapping each other or a source
    buf = _t((2 * 64 * 128,))
    a, b = buf[:64 * 128].view(1, 64, 128), buf[32 * 128:96 * 128].view(1, 64, 128)
    assert v_([k, v], [a, b]) == "RA_ERR_STRIDE"
    kflat = k.view(-1)
    assert v_([k, v], [kh, kflat[:64 * 128].view(1, 64, 128)]) == "RA_ERR_STRIDE"  # dst on a src


def test_bwd_validation(ra):
    q, k, v = _t((1, 4, 64, 128)), _t((1, 2, 64, 128)), _t((1, 2, 64, 128))
    o, do, lse = _t(q.shape), _t(q.shape), torch.zeros(1, 4, 64)
    dq, dk, dv = _t(q.shape), _t(k.shape), _t(k.shape)
    val = lambda *a, **kw: ra.STATUS[ra.attn_bwd_validate(*a, **kw)]
    assert val(q, k, v, o, do, lse, dq, dk, dv, causal=True) == "RA_OK"
    assert val(q, k, v, o, do, lse, dq, dk, dv.float()) == "RA_ERR_DTYPE"
    assert val(q, k, v, o, do, lse, dq, _t((1, 2, 65, 128)), dv) == "RA_ERR_SHAPE"
    f = lambda t: t.float()
    assert val(f(q), f(k), f(v), f(o), f(do), lse, f(dq), f(dk), f(dv)) == "RA_OK"  # fp32
    assert val(f(q), f(k), f(v), f(o), f(do), lse, dq, f(dk), f(dv)) == "RA_ERR_DTYPE"
    assert val(f(q)[..., :64], f(k)[..., :64], f(v)[..., :64], f(o)[..., :64], f(do)[..., :64],
               lse, f(dq)[..., :64], f(dk)[..., :64], f(dv)[..., :64]) == "RA_OK"  # D = 64
    # the D_i rows (B*Hq*Sq fp32, 256-byte rounded); with bf16 grouped heads then the
    # per-query-head fp32 dk/dv partials, 2*B*Hq*Skv*D*4 bytes
    delta = 4 * 64 * 4
    assert ra.attn_bwd_workspace_size(q, k) == delta + 2 * 4 * 64 * 128 * 4
    assert ra.attn_bwd_workspace_size(f(q), f(k)) == delta  # fp32: no partials
    assert ra.attn_bwd_workspace_size(q, _t((1, 4, 64, 128))) == delta  # one head per group
    assert ra.attn_bwd_workspace_size(q, _t((1, 3, 64, 128))) == 0


def test_bwd_accum_validation(ra):
    """The ring-backward step takes fp32 accumulators and one chunk (num_chunks = 1)."""
    q, k, v = _t((1, 4, 64, 128)), _t((1, 2, 32, 128)), _t((1, 2, 32, 128))
    o, do, lse = _t(q.shape), _t(q.shape), torch.zeros(1, 4, 64)
    f32 = lambda shape: torch.zeros(shape)
    dq, dk, dv = f32(q.shape), f32(k.shape), f32(k.shape)
    val = lambda *a, **kw: ra.STATUS[ra.attn_bwd_accum_validate(*a, **kw)]
    assert val(q, k, v, o, do, lse, dq, dk, dv, causal=True, q_offset=32, kv_offset=64) == "RA_OK"
    assert val(q, k, v, o, do, lse, dq.bfloat16(), dk, dv) == "RA_ERR_DTYPE"
    assert val(q, k, v, o, do, lse, dq, dk, dv.bfloat16()) == "RA_ERR_DTYPE"
    assert val(q, k, v, o.float(), do, lse, dq, dk, dv) == "RA_ERR_DTYPE"
    assert val(q, k, v, o, do, lse, dq, f32((1, 2, 33, 128)), dv) == "RA_ERR_SHAPE"
    assert val(q, k, v, o, do, lse, dq, dk, dv, num_chunks=2) == "RA_ERR_RANGE"
    assert val(q, k, v, o, do, lse, dq, dk, dv, q_offset=-1) == "RA_ERR_RANGE"
    # a transposed (overlapping-free but non-unit last stride) accumulator is refused
    assert val(q, k, v, o, do, lse, dq, dk, f32((1, 2, 128, 32)).transpose(2, 3)) == \
        "RA_ERR_STRIDE"


def test_fp8_validation(ra):
    f8 = lambda shape: torch.zeros(shape, dtype=torch.uint8).view(torch.float8_e4m3fn)
    q, k, vt = f8((1, 4, 64, 128)), f8((1, 2, 40, 128)), f8((1, 2, 128, 48))
    qd, kd, vd = torch.ones(1, 4), torch.ones(1, 2), torch.ones(1, 2)
    o, lse = _t((1, 4, 64, 128)), torch.zeros(1, 4, 64)
    val = lambda *a, **kw: ra.STATUS[ra.attn_fwd_fp8_validate(*a, **kw)]
    assert val(q, k, vt, qd, kd, vd, o, lse, causal=True) == "RA_OK"
    # fused ring chunks must be whole 16-key units (key tiles on 16-byte vt boundaries)
    assert val(q, k, vt, qd, kd, vd, o.float(), lse, num_chunks=2, start_chunk=1) == \
        "RA_ERR_ALIGN"  # chunks of 20 keys
    k64k, vt64k = f8((1, 2, 64, 128)), f8((1, 2, 128, 64))
    for P in (2, 4):  # chunks of 32 and 16 keys
        assert val(q, k64k, vt64k, qd, kd, vd, o.float(), lse, num_chunks=P,
                   start_chunk=1) == "RA_OK"
    k48, vt48 = f8((1, 2, 48, 128)), f8((1, 2, 128, 48))
    assert val(q, k48, vt48, qd, kd, vd, o, lse, num_chunks=2) == "RA_ERR_ALIGN"  # 24 keys
    assert val(q, k48, vt48, qd, kd, vd, o, lse, num_chunks=3) == "RA_OK"  # 16 keys
    assert val(q, k, f8((1, 2, 128, 40)), qd, kd, vd, o, lse) == "RA_ERR_ALIGN"  # rows of 40 B
    assert val(q, k, f8((1, 2, 128, 64)), qd, kd, vd, o, lse) == "RA_ERR_SHAPE"  # not S_pad
    assert val(q, k, f8((1, 2, 40, 128)), qd, kd, vd, o, lse) == "RA_ERR_SHAPE"  # not transposed
    assert val(q, k, vt, qd, kd, vd, o, lse, num_chunks=3) == "RA_ERR_SHAPE"
    assert val(q, _t((1, 2, 40, 128)), vt, qd, kd, vd, o, lse) == "RA_ERR_DTYPE"
    assert val(q, k, vt, torch.ones(1, 2), kd, vd, o, lse) == "RA_ERR_SHAPE"
    assert val(q, k, vt, qd, kd, vd, q, lse) == "RA_ERR_DTYPE"  # fp8 output refused
    q64, k64, vt64 = f8((1, 4, 64, 96)), f8((1, 2, 40, 96)), f8((1, 2, 96, 48))
    assert val(q64, k64, vt64, qd, kd, vd, _t((1, 4, 64, 96)), lse) == "RA_ERR_UNSUPPORTED"
    # fp8 inputs are refused by the bf16/fp32 entry points and the merge
    assert ra.STATUS[ra.attn_fwd_validate(q, f8((1, 2, 40, 128)), f8((1, 2, 40, 128)), o,
                                          lse)] == "RA_ERR_DTYPE"
    assert ra.STATUS[ra.lse_merge_validate([q], [lse], q, lse)] == "RA_ERR_DTYPE"


def test_fp8_quantize_validation(ra):
    x = _t((1, 3, 37, 64))
    codes, codes_t = torch.zeros(1, 3, 37, 64, dtype=torch.uint8), torch.zeros(1, 3, 64, 48,
                                                                              dtype=torch.uint8)
    as8 = lambda t: t.view(torch.float8_e4m3fn)
    desc = torch.zeros(1, 3)
    val = lambda *a, **kw: ra.STATUS[ra.fp8_quantize_validate(*a, **kw)]
    assert val(x, as8(codes), desc) == "RA_OK"
    assert val(x, as8(codes_t), desc, transpose=True) == "RA_OK"
    assert val(x, as8(codes_t), desc) == "RA_ERR_SHAPE"
    assert val(x, as8(codes), desc, transpose=True) == "RA_ERR_SHAPE"
    assert val(x.float(), as8(codes), desc) == "RA_ERR_DTYPE"
    assert val(x, _t((1, 3, 37, 64)), desc) == "RA_ERR_DTYPE"
    assert val(x, as8(codes), torch.zeros(1, 2)) == "RA_ERR_SHAPE"
    assert val(x, as8(codes), desc.bfloat16()) == "RA_ERR_DTYPE"
    assert val(_t((1, 3, 37, 8)), as8(torch.zeros(1, 3, 37, 8, dtype=torch.uint8)), desc) == \
        "RA_ERR_ALIGN"
    assert ra.lib().ra_fp8_quantize_workspace_size(ra.desc(x)) >= 3 * 4


def test_fp8_quantize_multi_validation(ra):
    """Several tensors in one call: each checked as alone; destinations (codes and
    descales) may overlap no source and no other destination; n within 1..4."""
    as8 = lambda t: t.view(torch.float8_e4m3fn)
    q, k, v = _t((1, 4, 40, 128)), _t((1, 2, 40, 128)), _t((1, 2, 40, 128))
    qc, kc = as8(torch.zeros(1, 4, 40, 128, dtype=torch.uint8)), \
        as8(torch.zeros(1, 2, 40, 128, dtype=torch.uint8))
    vt = as8(torch.zeros(1, 2, 128, 48, dtype=torch.uint8))
    qd, kd, vd = torch.zeros(1, 4), torch.zeros(1, 2), torch.zeros(1, 2)
    val = lambda *a: ra.STATUS[ra.fp8_quantize_multi_validate(*a)]
    assert val([q, k, v], [qc, kc, vt], [qd, kd, vd], [0, 0, 1]) == "RA_OK"
    assert val([q, k, v], [qc, kc, vt], [qd, kd, vd], [0, 0, 0]) == "RA_ERR_SHAPE"
    assert val([q, k], [qc, kc], [qd, qd[:, :2]], [0, 0]) == "RA_ERR_STRIDE"  # shared descale
    assert val([q, k], [qc, qc[:, :2]], [qd, kd], [0, 0]) == "RA_ERR_STRIDE"  # shared codes
    assert val([q] * 5, [qc] * 5, [qd] * 5, [0] * 5) == "RA_ERR_RANGE"
    assert val([], [], [], []) == "RA_ERR_RANGE"
    sa = (ra.RaTensor * 3)(*[ra.desc(t) for t in (q, k, v)])
    total = ra.lib().ra_fp8_quantize_n_workspace_size(3, sa)
    singles = sum(ra.lib().ra_fp8_quantize_workspace_size(ra.desc(t)) for t in (q, k, v))
    assert total == singles and total % 256 == 0


def test_params_versions_and_work_counter(ra):
    """ra_attn_params: the version-1 block (no work counter) and the version-2 block are
    both accepted; a smaller struct_size is out of range; a work counter must be 8-byte
    aligned (only its address is checked: it is device memory)."""
    assert ctypes.sizeof(ra.RaAttnParams) == 48
    assert ra.RaAttnParams.sched.offset == 40
    q, k, v = _t((1, 7, 64, 128)), _t((1, 1, 64, 128)), _t((1, 1, 64, 128))
    o, lse = torch.zeros(q.shape, dtype=q.dtype), torch.zeros(q.shape[:3])

    def check(size, sched):
        p = ra._params(True, 1, 0, 0, 0, None)
        p.struct_size = size
        p.sched = sched
        return ra.STATUS[ra.lib().ra_attn_fwd_validate(
            ra.desc(q), ra.desc(k), ra.desc(v), ctypes.byref(p), ra.desc(o), ra.desc(lse))]

    assert check(48, None) == "RA_OK"
    assert check(48, 0x10000) == "RA_OK"
    assert check(48, 0x10004) == "RA_ERR_ALIGN"
    assert check(40, None) == "RA_OK"
    assert check(40, 0x10004) == "RA_OK"  # a version-1 block has no counter field
    assert check(39, None) == "RA_ERR_RANGE"


def _raw(ra, shape, stride, dtype, ptr=1 << 20):
    """A descriptor with a fake device address: the *_validate entry points never
    dereference it, so huge strides need no memory."""
    d = ra.RaTensor()
    d.data = ptr
    d.dtype = dtype
    d.ndim = len(shape)
    for i, (n, s) in enumerate(zip(shape, stride)):
        d.shape[i] = n
        d.stride[i] = s
    return d


def _contig(shape):
    st, acc = [], 1
    for n in reversed(shape):
        st.insert(0, acc)
        acc *= n
    return st


@pytest.mark.parametrize("S,token_stride,want", [
    (256, 8_000_000, "RA_OK"),            # 127 * 8.0M * 2 + 256 B < 2^31
    (256, 8_455_000, "RA_ERR_SHAPE"),     # 127 * 8.455M * 2 B > 2^31
    (2, 8_455_000, "RA_OK"),              # a 2-token tile spans one stride only
    (128, 8_455_000, "RA_ERR_SHAPE"),
    (200, 1 << 30, "RA_ERR_SHAPE"),
])
def test_tile_offset_bound(ra, S, token_stride, want):
    """Token strides whose in-tile byte offsets would pass 2^31 are rejected on the host
    (checked only through the validate entry points; such views never reach a GPU)."""
    L = ra.lib()
    BF16 = ra.RA_BF16
    D = 128
    big = [2 * token_stride * S, token_stride * S, token_stride, 1]
    okq = lambda: _raw(ra, (1, 2, S, D), _contig((1, 2, S, D)), BF16)
    lse = _raw(ra, (1, 2, S), _contig((1, 2, S)), ra.RA_F32)
    p = ra._params(True, 1, 0, 0, 0, None)
    for which in range(4):  # q, k, v, o in turn carry the large token stride
        ts = [okq() for _ in range(4)]
        ts[which] = _raw(ra, (1, 2, S, D), big, BF16)
        rc = L.ra_attn_fwd_validate(ts[0], ts[1], ts[2], ctypes.byref(p), ts[3], lse)
        assert ra.STATUS[rc] == want, (which, ra.STATUS[rc])
    for which in range(8):  # q, k, v, o, dout, dq, dk, dv
        ts = [okq() for _ in range(8)]
        ts[which] = _raw(ra, (1, 2, S, D), big, BF16)
        rc = L.ra_attn_bwd_validate(ts[0], ts[1], ts[2], ts[3], ts[4], lse,
                                    ctypes.byref(p), ts[5], ts[6], ts[7])
        assert ra.STATUS[rc] == want, (which, ra.STATUS[rc])
