"""attn_decode_noalloc (static device scratch, no allocation) against attn_decode through the
C ABI: two calls in a row on the same GPU, the second smaller, each equal to attn_decode's
result and within the oracle's bound; plus the size limit."""
import numpy as np
import pytest

from causal_attention_02_amd import binding as bd
from causal_attention_02_amd.inputs import WORKLOADS, make_decode_inputs
from oracle import attention_decode
from tests.util import TOL_O, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu


def _opts(w):
    return bd.AttnOptions(softcap=w.softcap, rope=w.rope, rope_base=w.rope_base,
                          qk_norm=w.qk_norm, norm_eps=w.norm_eps)


def _case(w, split_len):
    import torch
    print(f"noalloc case B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} Lmax={w.T} split={split_len}",
          flush=True)
    q, kc, vc, lens = make_decode_inputs(w)
    tq, tkc, tvc = (to_dev(x, torch.bfloat16) for x in (q, kc, vc))
    tl = torch.from_numpy(lens).to("cuda")
    out = torch.full_like(tq, float("nan"))
    bd.attn_decode_noalloc(tq, tkc, tvc, tl, out, _opts(w), split_len=split_len)
    ref = bd.attn_decode(tq, tkc, tvc, tl, _opts(w), split_len=split_len)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    kw = dict(softcap=w.softcap, rope=w.rope, rope_base=w.rope_base, qk_norm=w.qk_norm,
              norm_eps=w.norm_eps)
    assert rel_l2(to_host(out), attention_decode(q, kc, vc, lens, **kw)) <= TOL_O


def test_noalloc_decode_matches_decode_twice_second_smaller():
    big = WORKLOADS["gqa181m_decode"]                     # one chunk per cache
    small = big.with_(B=5, T=700)                         # chunked: tickets and partials used
    _case(big, 0)
    _case(small, 128)
    _case(small.with_(B=3, T=300), 64)


def test_noalloc_decode_rejects_configs_beyond_the_scratch():
    import torch
    w = WORKLOADS["gqa181m_decode"].with_(B=64, T=8192)
    cfg = bd.make_decode_cfg(w.B, w.Hq, w.Hkv, w.D, w.T, _opts(w), 64)
    import ctypes
    assert bd.lib().attn_decode_workspace_bytes(ctypes.byref(cfg)) > bd.DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((w.B, w.Hkv, w.T, w.D), dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(bd.AttnError) as ei:
        bd.attn_decode_noalloc(q, kc, kc, lens, out, _opts(w), split_len=64)
    assert ei.value.status == bd.ATTN_ESCRATCH
