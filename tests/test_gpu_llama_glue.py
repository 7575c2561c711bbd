"""The decoder stack's fused elementwise kernels (libllama_glue.so) against
plain PyTorch fp32 references of the same operations.  The residual add rounds
exactly as a bf16 tensor add does (bit for bit); normalised, rotated and gated
values may differ from the reference by one bf16 rounding step (the reference
reduces and evaluates cos / sin / exp in a different order)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from sparse_attention_long_fwht_amd import llama_glue as G
    return torch, G


def within_one_ulp(torch, got, ref_f32):
    """got (bf16) is ref rounded to bf16, or one of its bf16 neighbours."""
    ref = ref_f32.to(torch.bfloat16)
    a = got.view(torch.int16).to(torch.int32)
    b = ref.view(torch.int16).to(torch.int32)
    # adjacent bf16 values of one sign differ by 1 in their bit patterns
    ok = ((a - b).abs() <= 1) | (got.float() == ref.float())
    assert bool(ok.all()), "max diff %g" % (got.float() - ref_f32).abs().max().item()


@pytest.mark.parametrize("rows,hidden", [(1, 4096), (3, 4096), (5, 256), (2, 14336)])
def test_add_rmsnorm(env, rows, hidden):
    torch, G = env
    g = torch.Generator(device="cuda").manual_seed(rows * hidden)
    x = (torch.randn(rows, hidden, generator=g, device="cuda") * 3).to(torch.bfloat16)
    d = torch.randn(rows, hidden, generator=g, device="cuda").to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(hidden, generator=g, device="cuda")).to(torch.bfloat16)
    x_sum = x + d  # bf16 add: the exact reference of the residual
    ref = x_sum.float() * torch.rsqrt(x_sum.float().pow(2).mean(-1, keepdim=True) + 1e-5) * w.float()
    xo, h = x.clone(), torch.empty_like(x)
    G.add_rmsnorm(xo, d, xo, w, h, 1e-5)  # in place, as the decoder uses it
    torch.cuda.synchronize()
    assert torch.equal(xo, x_sum)
    within_one_ulp(torch, h, ref)
    h2 = torch.empty_like(x)
    G.add_rmsnorm(x, None, None, w, h2, 1e-5)  # no residual, no store
    torch.cuda.synchronize()
    ref2 = x.float() * torch.rsqrt(x.float().pow(2).mean(-1, keepdim=True) + 1e-5) * w.float()
    within_one_ulp(torch, h2, ref2)


def test_rope_append(env):
    torch, G = env
    B, Hq, Hkv, cap = 3, 32, 8, 40000
    g = torch.Generator(device="cuda").manual_seed(7)
    qkv = torch.randn(B, (Hq + 2 * Hkv) * 128, generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.tensor([0, 32768, 39999], dtype=torch.int32, device="cuda")
    inv = 1.0 / (500000.0 ** (torch.arange(0, 128, 2, device="cuda", dtype=torch.float32) / 128))
    kc = torch.randn(B, Hkv, cap, 128, generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn(B, Hkv, cap, 128, generator=g, device="cuda").to(torch.bfloat16)
    kc0, vc0 = kc.clone(), vc.clone()
    q = torch.empty(B, Hq, 128, dtype=torch.bfloat16, device="cuda")
    G.rope_append(qkv, pos, inv, q, kc, vc)
    torch.cuda.synchronize()
    ang = pos.float()[:, None] * inv[None, :]
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rot(x):
        x1, x2 = x[..., :64].float(), x[..., 64:].float()
        return torch.cat((x1 * c - x2 * s, x2 * c + x1 * s), -1)

    qr = rot(qkv[:, :Hq * 128].view(B, Hq, 128))
    kr = rot(qkv[:, Hq * 128:(Hq + Hkv) * 128].view(B, Hkv, 128))
    vr = qkv[:, (Hq + Hkv) * 128:].view(B, Hkv, 128)
    within_one_ulp(torch, q, qr)
    for b in range(B):
        p = int(pos[b])
        within_one_ulp(torch, kc[b, :, p], kr[b])
        assert torch.equal(vc[b, :, p], vr[b])
        kc0[b, :, p] = kc[b, :, p]
        vc0[b, :, p] = vc[b, :, p]
    assert torch.equal(kc, kc0) and torch.equal(vc, vc0)  # no other row touched


@pytest.mark.parametrize("rows,ffn", [(1, 14336), (16, 14336), (2, 512)])
def test_silu_mul(env, rows, ffn):
    torch, G = env
    g = torch.Generator(device="cuda").manual_seed(rows + ffn)
    gu = (torch.randn(rows, 2 * ffn, generator=g, device="cuda") * 4).to(torch.bfloat16)
    out = torch.empty(rows, ffn, dtype=torch.bfloat16, device="cuda")
    G.silu_mul(gu, out)
    torch.cuda.synchronize()
    gf, uf = gu[:, :ffn].float(), gu[:, ffn:].float()
    within_one_ulp(torch, out, gf * torch.sigmoid(gf) * uf)
