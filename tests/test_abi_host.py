"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/cpring.h declares, and
reject bad arguments before it touches the HIP runtime. Only argument
validation runs here: every call below fails validation, so nothing is
launched.
"""

import ctypes
import os
import re
import subprocess

import pytest

import context_ring_attention_zigzag_amd as cpr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpring.h")


@pytest.fixture(scope="module")
def lib():
    # CPRING_TEST_LIB: run these checks against another build of the library
    # (the host-AddressSanitizer build of tests/test_host_asan.py)
    path = os.environ.get("CPRING_TEST_LIB", cpr.LIB_PATH)
    if path == cpr.LIB_PATH and not os.path.exists(path):
        from context_ring_attention_zigzag_amd import build
        build.build()
    return cpr.load(path)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(cpr.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    path = os.environ.get("CPRING_TEST_LIB", cpr.LIB_PATH)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_padded_len(lib):
    assert lib.cp_padded_len(4096, 2, cpr.ZIGZAG) == 4096
    assert lib.cp_padded_len(4097, 2, cpr.ZIGZAG) == 4100
    assert lib.cp_padded_len(1, 4, cpr.ZIGZAG) == 8
    assert lib.cp_padded_len(65536, 8, cpr.CONTIGUOUS) == 65536
    assert lib.cp_padded_len(10, 4, cpr.CONTIGUOUS) == 12
    assert lib.cp_padded_len(1048576, 8, cpr.ZIGZAG) == 1048576
    assert lib.cp_padded_len(10, 4, cpr.STRIPED) == 12
    assert lib.cp_padded_len(32768, 4, cpr.STRIPED) == 32768
    assert lib.cp_padded_len(10, 4, 3) == -1
    for bad in ((0, 2, 0), (-5, 2, 0), (10, 0, 0), (10, 2, 5), (1 << 31, 2, 0)):
        assert lib.cp_padded_len(*bad) == -1


def test_padded_len_matches_oracle(lib):
    import oracle
    for s in (1, 3, 17, 64, 100, 257, 4096):
        for cp in (1, 2, 3, 4, 8):
            for lay in (cpr.ZIGZAG, cpr.CONTIGUOUS, cpr.STRIPED):
                assert lib.cp_padded_len(s, cp, lay) == oracle.padded_len(s, cp, lay)


def fake_ptr(n=0x100000):
    return ctypes.c_void_p(n)


def view(ptr=0x100000, sb=0, sh=0, sl=128):
    return cpr.CprView(ptr, sb, sh, sl)


def err(lib):
    return lib.cp_last_error().decode()


def test_status_strings(lib):
    for s in (0, 1, 2, 3, 99):
        assert lib.cp_status_string(s)


def test_partition_validation(lib):
    p = fake_ptr()
    assert lib.cp_zigzag_partition(100, 0, cpr.ZIGZAG, p, p, None) == cpr.EINVAL
    assert "cp_size" in err(lib)
    assert lib.cp_zigzag_partition(100, 2, 9, p, p, None) == cpr.EINVAL
    assert lib.cp_zigzag_partition(0, 2, cpr.ZIGZAG, p, p, None) == cpr.EINVAL
    assert lib.cp_zigzag_partition(100, 2, cpr.ZIGZAG, None, None, None) == cpr.EINVAL
    assert lib.cp_zigzag_partition(100, 2, cpr.ZIGZAG, ctypes.c_void_p(0x100002), None, None) == cpr.EINVAL
    assert lib.cp_zigzag_partition(1 << 31, 2, cpr.ZIGZAG, p, p, None) == cpr.EUNSUPPORTED


def step_args(**over):
    a = dict(dtype=cpr.BF16, B=1, H=2, D=128, q=view(), Lq=64, q_pos=fake_ptr(), k=view(), v=view(), Lk=64,
             kv_pos=fake_ptr(), causal=1, scale=0.0, o=fake_ptr(), m=fake_ptr(), l=fake_ptr())
    a.update(over)
    return a


def call_step(lib, a):
    return lib.cp_ring_attn_step(a["dtype"], a["B"], a["H"], a["D"], ctypes.byref(a["q"]) if a["q"] else None,
                                 a["Lq"], a["q_pos"], ctypes.byref(a["k"]) if a["k"] else None,
                                 ctypes.byref(a["v"]) if a["v"] else None, a["Lk"], a["kv_pos"], a["causal"],
                                 a["scale"], a["o"], a["m"], a["l"], None)


@pytest.mark.parametrize("over,code,needle", [
    (dict(dtype=7), cpr.EINVAL, "dtype"),
    (dict(D=96), cpr.EUNSUPPORTED, "head dim"),
    (dict(D=256), cpr.EUNSUPPORTED, "head dim"),
    (dict(B=0), cpr.EINVAL, "B and H"),
    (dict(H=-1), cpr.EINVAL, "B and H"),
    (dict(Lq=0), cpr.EINVAL, "Lq"),
    (dict(Lk=0), cpr.EINVAL, "KV length"),
    (dict(q=None), cpr.EINVAL, "q"),
    (dict(q=view(ptr=0)), cpr.EINVAL, "q: data pointer"),
    (dict(k=view(ptr=0x100008)), cpr.EINVAL, "16-byte aligned"),
    (dict(v=view(sl=132)), cpr.EINVAL, "multiples of 8"),
    (dict(k=view(sl=64)), cpr.EUNSUPPORTED, "below D"),
    (dict(q=view(sl=0)), cpr.EUNSUPPORTED, "below D"),
    (dict(D=64, v=view(sl=56)), cpr.EUNSUPPORTED, "below D"),
    (dict(v=view(sb=-8)), cpr.EINVAL, "negative stride"),
    (dict(q_pos=None), cpr.EINVAL, "position"),
    (dict(kv_pos=None), cpr.EINVAL, "position"),
    (dict(o=None), cpr.EINVAL, "state"),
    (dict(o=fake_ptr(0x100004)), cpr.EINVAL, "o_acc"),
    (dict(scale=float("nan")), cpr.EINVAL, "softmax_scale"),
    (dict(scale=float("inf")), cpr.EINVAL, "softmax_scale"),
])
def test_step_validation(lib, over, code, needle):
    assert call_step(lib, step_args(**over)) == code
    assert needle in err(lib)


def call_run(lib, cp=2, rank=0, flags=cpr.RUN_FUSED, ws=None, ws_bytes=0, out=fake_ptr(), dtype=cpr.BF16, D=128,
             Lq=64):
    q, k, v = view(), view(), view()
    return lib.cp_ring_attn_run(dtype, 1, 2, D, cp, rank, ctypes.byref(q), Lq, fake_ptr(), ctypes.byref(k),
                                ctypes.byref(v), fake_ptr(), 1, 0.0, out, None, ws, ws_bytes, flags, None)


def test_run_validation(lib):
    assert call_run(lib, cp=0) == cpr.EINVAL
    assert call_run(lib, cp=4, rank=4) == cpr.EINVAL and "rank" in err(lib)
    assert call_run(lib, rank=-1) == cpr.EINVAL
    assert call_run(lib, flags=5) == cpr.EINVAL and "flags" in err(lib)
    assert call_run(lib, out=None) == cpr.EINVAL and "o_out" in err(lib)
    assert call_run(lib, flags=cpr.RUN_STEPWISE) == cpr.EINVAL and "workspace" in err(lib)
    need = lib.cp_ring_attn_workspace_size(1, 2, 64, 128)
    assert call_run(lib, flags=cpr.RUN_STEPWISE, ws=fake_ptr(), ws_bytes=need - 1) == cpr.EINVAL
    assert call_run(lib, flags=cpr.RUN_STEPWISE, ws=fake_ptr(0x100010), ws_bytes=need) == cpr.EINVAL
    assert "256-byte" in err(lib)
    assert call_run(lib, D=32) == cpr.EUNSUPPORTED
    assert call_run(lib, Lq=(1 << 30), cp=2) == cpr.EUNSUPPORTED


def test_workspace_size(lib):
    ws = lib.cp_ring_attn_workspace_size(2, 16, 8192, 128)
    rows = 2 * 16 * 8192
    assert ws >= rows * 128 * 4 + 2 * rows * 4 and ws % 256 == 0
    assert lib.cp_ring_attn_workspace_size(0, 1, 1, 128) == 0
    assert lib.cp_ring_attn_workspace_size(1, 1, 1, 100) == 0


def state_bytes(n, rows, D):
    r256 = lambda x: (x + 255) // 256 * 256
    return r256(n * rows * D * 4) + 2 * r256(n * rows * 4)


@pytest.mark.parametrize("B,H,Lq,D,n", [
    (2, 16, 8192, 128, 1),   # 1,024 query tiles of 256: fills the GPU, one state
    (1, 32, 8192, 128, 1),   # 1,024
    (1, 4, 2048, 64, 8),     # 32 query tiles: split 8 ways (256 / 32)
    (1, 2, 250, 128, 4),     # 2 query tiles, but only 4 key tiles of 64 per block
    (1, 1, 64, 128, 1),      # a single key tile per block: nothing to split
    (1, 128, 256, 128, 2),   # 128 query tiles: half the GPU, split 2 ways
    (1, 100, 256, 64, 2),    # 100 query tiles: split 2 ways
    (1, 129, 256, 128, 1),   # 129 query tiles: more than half the GPU, no split
    (1, 1, 100000, 64, 1),   # 391 query tiles of one head: no split
])
def test_workspace_size_covers_the_key_split(lib, B, H, Lq, D, n):
    """The workspace holds n float32 states: n > 1 when a bf16 fused run splits the keys of a grid of at
    most 128 query tiles (half of the 256 compute units) into min(256 // grid, key tiles per block, 16)
    slices."""
    grid = -(-Lq // 256) * B * H
    n_kt = -(-Lq // 64)
    expect = 1 if (2 * grid > 256 or n_kt <= 1) else min(256 // grid, n_kt, 16)
    assert expect == n
    assert lib.cp_ring_attn_workspace_size(B, H, Lq, D) == state_bytes(expect, B * H * Lq, D)


def test_state_call_validation(lib):
    p = fake_ptr()
    assert lib.cp_ring_attn_init(1, 1, 0, 128, p, p, p, None) == cpr.EINVAL
    assert lib.cp_ring_attn_init(1, 1, 8, 128, None, p, p, None) == cpr.EINVAL
    assert lib.cp_ring_attn_merge(1, 1, 8, 128, p, p, p, None, p, p, None) == cpr.EINVAL
    assert lib.cp_ring_attn_merge(1, 1, 8, 100, p, p, p, p, p, p, None) == cpr.EUNSUPPORTED
    assert lib.cp_ring_attn_finalize(cpr.BF16, 1, 1, 8, 128, p, p, p, None, None, None) == cpr.EINVAL
    assert lib.cp_ring_attn_finalize(5, 1, 1, 8, 128, p, p, p, p, None, None) == cpr.EINVAL
    assert lib.cp_ring_attn_finalize(cpr.F32, 1, 1, 8, 128, p, p, p, fake_ptr(0x100008), None, None) == cpr.EINVAL


def test_gather_validation(lib):
    v = view()
    p = fake_ptr()
    assert lib.cp_shard_gather(cpr.BF16, 1, 1, 100, 128, ctypes.byref(v), None, 10, p, None) == cpr.EINVAL
    assert lib.cp_shard_gather(cpr.BF16, 1, 1, 100, 128, ctypes.byref(v), p, 10, None, None) == cpr.EINVAL
    assert lib.cp_shard_gather(cpr.BF16, 1, 1, 100, 128, ctypes.byref(v), p, 0, p, None) == cpr.EINVAL
    bad = view(sl=130)
    assert lib.cp_shard_gather(cpr.F32, 1, 1, 100, 128, ctypes.byref(bad), p, 10, p, None) == cpr.EINVAL


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(cpr, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        cpr.load(str(tmp_path / "nope.so"))


def test_extension_validation(lib):
    """cp_ring_attn_run_ex rejects K/V head counts that do not divide H, before touching any memory."""
    q, k, v = view(), view(), view()
    p = fake_ptr()
    for h_kv in (3, -1, 5):
        ext = cpr.CprAttnExt(h_kv, None, None)
        st = lib.cp_ring_attn_run_ex(cpr.BF16, 1, 4, 128, 2, 0, ctypes.byref(q), 128, p, ctypes.byref(k),
                                     ctypes.byref(v), p, 1, 0.0, ctypes.byref(ext), p, None, None, 0,
                                     cpr.RUN_FUSED, None)
        assert st == cpr.EINVAL
    ext = cpr.CprAttnExt(2, ctypes.c_void_p(0x100002), None)   # misaligned window array
    st = lib.cp_ring_attn_run_ex(cpr.BF16, 1, 4, 128, 2, 0, ctypes.byref(q), 128, p, ctypes.byref(k), ctypes.byref(v),
                                 p, 1, 0.0, ctypes.byref(ext), p, None, None, 0, cpr.RUN_FUSED, None)
    assert st == cpr.EINVAL



def test_step_flags_validation(lib):
    """cp_ring_attn_step_ex checks its first/last-hop flags and their outputs before launching anything."""
    q, k, v = view(), view(), view()
    p = fake_ptr()

    def step(ext, state=p):
        return lib.cp_ring_attn_step_ex(cpr.BF16, 1, 2, 128, ctypes.byref(q), 64, p, ctypes.byref(k), ctypes.byref(v),
                                        64, p, 1, 0.0, ctypes.byref(ext), state, state, state, None)

    assert step(cpr.CprAttnExt(2, None, None, 4)) == cpr.EINVAL                   # unknown bit
    assert step(cpr.CprAttnExt(2, None, None, cpr.STEP_LAST)) == cpr.EINVAL       # no o_out
    assert step(cpr.CprAttnExt(2, None, None, cpr.STEP_LAST, fake_ptr(0x100008))) == cpr.EINVAL   # misaligned
    assert step(cpr.CprAttnExt(2, None, None, cpr.STEP_LAST, p, fake_ptr(0x100002))) == cpr.EINVAL
    # the state is needed unless both flags are set
    assert step(cpr.CprAttnExt(2, None, None, cpr.STEP_FIRST), state=None) == cpr.EINVAL
    assert step(cpr.CprAttnExt(2, None, None, cpr.STEP_LAST, p), state=None) == cpr.EINVAL


def test_bwd_workspace_size(lib):
    ws = lib.cp_ring_attn_bwd_workspace_size(2, 16, 8192)
    assert ws >= 2 * 16 * 8192 * 8 + 8192 * 8 and ws % 256 == 0
    assert lib.cp_ring_attn_bwd_workspace_size(0, 1, 8) == 0
    assert lib.cp_ring_attn_bwd_workspace_size(1, 1, 0) == 0


def test_bwd_validation(lib):
    """The backward entry points reject bad arguments before launching anything."""
    p = fake_ptr()
    q, k, v, o, g = view(), view(), view(), view(), view()
    need = lib.cp_ring_attn_bwd_workspace_size(1, 2, 64)

    def prep(dtype=cpr.BF16, D=128, lse=p, ws=p, nbytes=need, ov=o):
        return lib.cp_ring_attn_bwd_prep(dtype, 1, 2, D, 64, ctypes.byref(ov), ctypes.byref(g), lse, p, 1, None, ws,
                                         nbytes, None)
    assert prep(lse=None) == cpr.EINVAL and "lse" in err(lib)
    assert prep(ws=None) == cpr.EINVAL and "workspace" in err(lib)
    assert prep(nbytes=need - 1) == cpr.EINVAL
    assert prep(ws=fake_ptr(0x100010)) == cpr.EINVAL and "256-byte" in err(lib)
    assert prep(D=96) == cpr.EUNSUPPORTED
    assert prep(dtype=cpr.F32, ov=view(sl=130)) == cpr.EINVAL and "16-byte" in err(lib)

    def step(h_kv=0, dq=p, ws=p, nbytes=need, scale=0.0):
        return lib.cp_ring_attn_bwd_step(cpr.BF16, 1, 2, 128, h_kv, ctypes.byref(q), ctypes.byref(g), 64,
                                         ctypes.byref(k), ctypes.byref(v), 64, p, scale, ws, nbytes, dq, p, p, None)
    assert step(h_kv=3) == cpr.EINVAL and "H_kv" in err(lib)
    assert step(dq=None) == cpr.EINVAL and "dq_acc" in err(lib)
    assert step(dq=fake_ptr(0x100004)) == cpr.EINVAL and "16-byte" in err(lib)
    assert step(nbytes=0) == cpr.EINVAL and "workspace" in err(lib)
    assert step(scale=float("nan")) == cpr.EINVAL

    def run(cp=2, rank=0, dk=p):
        return lib.cp_ring_attn_bwd_run(cpr.BF16, 1, 2, 128, cp, rank, ctypes.byref(q), 64, p, ctypes.byref(k),
                                        ctypes.byref(v), p, ctypes.byref(o), ctypes.byref(g), p, 1, 0.0, None, p, dk,
                                        p, p, need, None)
    assert run(cp=0) == cpr.EINVAL
    assert run(rank=2) == cpr.EINVAL and "rank" in err(lib)
    assert run(dk=None) == cpr.EINVAL and "dk_ring" in err(lib)


def test_rope_validation(lib):
    p = fake_ptr()
    x = view()

    def call(dtype=cpr.BF16, D=128, pos=p, base=10000.0, style=cpr.ROPE_INTERLEAVED, out=p, xv=x):
        return lib.cp_rope_apply(dtype, 1, 2, 64, D, ctypes.byref(xv), pos, base, style, out, None)
    assert call(pos=None) == cpr.EINVAL and "pos" in err(lib)
    assert call(base=0.0) == cpr.EINVAL and "base" in err(lib)
    assert call(base=float("inf")) == cpr.EINVAL
    assert call(style=7) == cpr.EINVAL and "style" in err(lib)
    assert call(out=None) == cpr.EINVAL
    assert call(out=fake_ptr(0x100008)) == cpr.EINVAL and "16-byte" in err(lib)
    assert call(D=80) == cpr.EUNSUPPORTED
    assert call(dtype=cpr.F32, xv=view(sl=130)) == cpr.EINVAL


def test_bwd_workspace_size_ex(lib):
    base = lib.cp_ring_attn_bwd_workspace_size
    ex = lib.cp_ring_attn_bwd_workspace_size_ex
    # the glossary example's rank: small grids, room for partial gradients
    assert ex(1, 4, 4, 64, 2048, 4096) > base(1, 4, 2048)
    assert ex(1, 4, 0, 64, 2048, 4096) == ex(1, 4, 4, 64, 2048, 4096)
    # the non-causal 65,536-token share: large grids, no split
    assert ex(2, 16, 16, 128, 8192, 65536) == base(2, 16, 8192)
    for bad in ((0, 4, 4, 64, 2048, 4096), (1, 4, 3, 64, 2048, 4096), (1, 4, 4, 96, 2048, 4096),
                (1, 4, 4, 64, 0, 4096), (1, 4, 4, 64, 2048, 0), (1, 4, -1, 64, 2048, 4096)):
        assert ex(*bad) == 0, bad
