"""sageattn as a drop-in for torch.nn.functional.scaled_dot_product_attention
(deployment guide sec. 5.1 assigns it to F.scaled_dot_product_attention): a
small torch attention module calls F.scaled_dot_product_attention with SDPA's
keywords or positional order; with sageattn assigned in its place the module's
attention output equals a direct sageattn call bit for bit, is within the
parity tolerance of the oracle on the module's own q, k, v, and within the
method's accuracy of exact attention.  A call with a mask raises
NotImplementedError, which the module catches to fall back.  Needs an MI355X."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import quantized_attention_smooth_amd as sage
from parity_utils import ABS_TOL, COS_EMU, COS_EXACT, EXP_BAND, cosine, out_ulp

pytestmark = pytest.mark.gpu


class TinySelfAttention(torch.nn.Module):
    """x (B, N, dim) -> attention of its H heads, (B, H, N, D), through
    F.scaled_dot_product_attention as model code calls it."""

    def __init__(self, dim=512, heads=4, positional=False, mask=False):
        super().__init__()
        self.h, self.d = heads, dim // heads
        self.qkv = torch.nn.Linear(dim, 3 * dim, bias=False)
        self.positional, self.mask = positional, mask
        self.fallbacks = 0

    def forward(self, x):
        b, n, _ = x.shape
        q, k, v = self.qkv(x).view(b, n, 3, self.h, self.d).permute(2, 0, 3, 1, 4).contiguous()
        self.last_qkv = (q, k, v)
        if self.mask:
            m = torch.ones(n, n, dtype=torch.bool, device=x.device).tril()
            try:
                return F.scaled_dot_product_attention(q, k, v, attn_mask=m)
            except NotImplementedError:
                self.fallbacks += 1                  # torch's attention, computed in fp32
                return _ORIGINAL_SDPA(q.float(), k.float(), v.float(), attn_mask=m).half()
        if self.positional:
            return F.scaled_dot_product_attention(q, k, v, None, 0.0, True)
        return F.scaled_dot_product_attention(q, k, v, attn_mask=None, dropout_p=0.0, is_causal=True,
                                              scale=1 / math.sqrt(self.d))


_ORIGINAL_SDPA = F.scaled_dot_product_attention


@pytest.mark.parametrize("positional", [False, True])
def test_module_with_sageattn_as_sdpa(monkeypatch, positional):
    print(f"[gpu-case] SDPA drop-in: tiny module B2 N600 dim512 H4 fp16 causal positional={positional} seed 61",
          flush=True)
    torch.manual_seed(61)
    mod = TinySelfAttention(positional=positional).cuda().half()
    x = torch.randn(2, 600, 512, device="cuda").half()
    monkeypatch.setattr(torch.nn.functional, "scaled_dot_product_attention", sage.sageattn)
    with torch.no_grad():
        out = mod(x)
    q, k, v = mod.last_qkv
    direct = sage.sageattn(q, k, v, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, direct)
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    ref = oracle.reference_forward(qn, kn, vn, dtype="fp16", causal=True, exp_band=EXP_BAND)
    ex = oracle.exact_forward(qn, kn, vn, causal=True)
    got = out.float().cpu().numpy()
    for b in range(2):
        r = ref["out"][b]
        assert np.all(np.abs(got[b] - r) <= ABS_TOL + out_ulp(r, "fp16") + ref["allow"][b])
    assert cosine(got, np.stack(ref["out"])) >= COS_EMU
    assert cosine(got, np.stack(ex["out"])) >= COS_EXACT


def test_masked_call_falls_back(monkeypatch):
    print("[gpu-case] SDPA drop-in: masked call falls back to torch", flush=True)
    torch.manual_seed(62)
    mod = TinySelfAttention(mask=True).cuda().half()
    x = torch.randn(1, 100, 512, device="cuda").half()
    monkeypatch.setattr(torch.nn.functional, "scaled_dot_product_attention", sage.sageattn)
    with torch.no_grad():
        out = mod(x)
    torch.cuda.synchronize()
    assert mod.fallbacks == 1 and out.shape == (1, 4, 100, 128)
