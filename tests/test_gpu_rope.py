"""GPU parity of the rotary embedding (cp_rope_apply) against the fp64 oracle.

Bars: float32 max |out - ref| <= 1e-5 (sin/cos and the products in float32 of
an angle reduced in double precision); bf16 |out - ref| <= 2^-8 |ref| + 1e-5
elementwise (one rounding of the result to bf16 is at most half a unit in the
last place, 2^-9 relative; the float32 arithmetic before it can move the result
across a rounding boundary, hence one full unit). Rotating the natural sequence
and gathering a rank's rows must be bit-identical to gathering first and
rotating with the rank's global position ids.
"""

import numpy as np
import pytest
import torch

import oracle
import context_ring_attention_zigzag_amd as cpr
from context_ring_attention_zigzag_amd import device_inputs as di

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
STYLES = {"interleaved": (cpr.ROPE_INTERLEAVED, oracle.INTERLEAVED), "half": (cpr.ROPE_HALF, oracle.HALF)}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpr.load()
    yield


def note(msg):
    print(f"[gpu-rope] {msg}", flush=True)


def check(out, ref, dtype, what):
    err = np.abs(out - ref)
    note(f"{what}: max|err|={err.max():.3e}")
    if dtype == "f32":
        assert err.max() <= 1e-5, what
    else:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), what


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_rope_rank_queries_and_ring_keys(dtype, d, style):
    """A rank's queries with q_pos and the ring-ordered keys with ring_pos (pads included) of a zigzag layout."""
    s, cp, rank = 1000, 4, 1
    rng = np.random.default_rng(400 + d)
    x = torch.from_numpy(rng.standard_normal((2, 3, s, d)).astype(np.float32)).to(TDT[dtype])
    host = x.float().numpy().astype(np.float64)
    tok, pos = di.layout_arrays(s, cp, cpr.ZIGZAG)
    lq = tok.numel() // cp
    cs, os_ = STYLES[style]
    for name, idx, p in (("q_local", tok[rank * lq:(rank + 1) * lq], pos[rank * lq:(rank + 1) * lq]),
                         ("k_ring", tok, pos)):
        local = di.gather(x.cuda(), s, idx)
        out = cpr.cp_rope_apply(local, p.contiguous(), style=cs)
        torch.cuda.synchronize()
        ref = oracle.rope(local.float().cpu().numpy().astype(np.float64), p.cpu().numpy(), style=os_)
        check(out.float().cpu().numpy(), ref, dtype, f"{dtype} D={d} {style} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_million_token_positions(dtype):
    """Positions up to 2^20 (the million-token share): angles of 10^6 radians stay accurate."""
    L, d = 512, 128
    rng = np.random.default_rng(410)
    pos = np.sort(rng.choice(1 << 20, size=L, replace=False)).astype(np.int32)
    pos[-3:] = [(1 << 20) - 1, (1 << 20) - 2, -1]
    x = torch.from_numpy(rng.standard_normal((1, 2, L, d)).astype(np.float32)).to(TDT[dtype]).cuda()
    out = cpr.cp_rope_apply(x, torch.from_numpy(pos).cuda(), base=10000.0)
    torch.cuda.synchronize()
    ref = oracle.rope(x.float().cpu().numpy().astype(np.float64), pos)
    check(out.float().cpu().numpy(), ref, dtype, f"{dtype} positions to 2^20")
    assert torch.equal(out[:, :, -1], x[:, :, -1])   # pad row unchanged


def test_rope_commutes_with_layout_bit_exact():
    """Rotate-then-gather == gather-then-rotate with global positions (Megatron page, implementation quirk)."""
    s, cp, d = 4096, 4, 128
    rng = np.random.default_rng(420)
    x = torch.from_numpy(rng.standard_normal((1, 4, s, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    nat_pos = torch.arange(s, dtype=torch.int32, device="cuda")
    rotated = cpr.cp_rope_apply(x, nat_pos)
    for lay in (cpr.ZIGZAG, cpr.STRIPED):
        tok, pos = di.layout_arrays(s, cp, lay)
        lq = tok.numel() // cp
        for r in range(cp):
            idx = tok[r * lq:(r + 1) * lq]
            a = di.gather(rotated, s, idx)
            b = cpr.cp_rope_apply(di.gather(x, s, idx), pos[r * lq:(r + 1) * lq].contiguous())
            assert torch.equal(a, b), (lay, r)


def test_rope_in_place_and_strided_input():
    s, d = 300, 64
    rng = np.random.default_rng(430)
    x = torch.from_numpy(rng.standard_normal((2, 6, s, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    pos = torch.arange(5, 5 + s, dtype=torch.int32, device="cuda")
    want = cpr.cp_rope_apply(x.contiguous(), pos)
    y = x.clone()
    cpr.cp_rope_apply(y, pos, out=y)              # in place
    sub = cpr.cp_rope_apply(x[:, ::2], pos)       # every other head of a larger tensor
    torch.cuda.synchronize()
    assert torch.equal(y, want)
    assert torch.equal(sub, want[:, ::2])


def test_rope_is_deterministic():
    x = torch.randn((2, 4, 777, 128), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    pos = torch.arange(100, 877, dtype=torch.int32, device="cuda")
    a = cpr.cp_rope_apply(x, pos, style=cpr.ROPE_HALF)
    b = cpr.cp_rope_apply(x, pos, style=cpr.ROPE_HALF)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
