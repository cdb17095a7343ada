"""GPU: swa_decode_noalloc (decode with the library's per-GPU scratch array
instead of a caller workspace) against swa_decode with a caller workspace.

Both run the same kernels with the same split configuration, so the outputs
must be identical bit for bit; both are also held to the oracle at the bf16 /
fp32 bar.  Two calls in a row, the second with a smaller input, check that the
scratch contents one call leaves behind do not leak into the next.  The
shapes use the workspace path (few (request, key/value head) groups: one
workgroup per split, partial states through the scratch, then the combine).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


def _case(dtype, B, W, Hq, Hkv, D, seed):
    c = inp.DecodeCase(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, cur_lo=0, cur_hi=3 * W, dtype=dtype,
                       seed=seed)
    return [dev(x) for x in inp.decode_inputs(c)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_decode_two_calls(dtype):
    shapes = [(3, 1000, 8, 2, 128, 5), (1, 300, 4, 1, 64, 6)]   # second call smaller
    for B, W, Hq, Hkv, D, seed in shapes:
        need = bd.decode_workspace_size(B, Hq, Hkv, W, D)
        assert 0 < need <= bd.DECODE_NOALLOC_SCRATCH_BYTES
        q, kc, vc, sp, cur = _case(dtype, B, W, Hq, Hkv, D, seed)
        banner(f"decode_noalloc {dtype} B={B} W={W} Hq={Hq} Hkv={Hkv} D={D}")
        o1, l1 = bd.decode_noalloc(q, kc, vc, sp, cur, return_lse=True)
        torch.cuda.synchronize()
        o2, l2 = bd.decode(q, kc, vc, sp, cur, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert torch.equal(torch.nan_to_num(l1, neginf=-1e30), torch.nan_to_num(l2, neginf=-1e30))
        ro, _ = oracle.swa_decode(inp.widen(q.cpu()), inp.widen(kc.cpu()), inp.widen(vc.cpu()),
                                  sp.cpu().numpy(), cur.cpu().numpy(), W)
        assert max_err(host(o1), ro) <= (TOL_BF16 if dtype == "bf16" else TOL_F32)


def test_noalloc_merge_path_matches_decode():
    # many (request, key/value head) groups: the splits merge inside the
    # workgroup and the scratch is not read at all
    q, kc, vc, sp, cur = _case("bf16", 64, 512, 32, 8, 128, 7)
    banner("decode_noalloc merge path B=64 W=512")
    o1 = bd.decode_noalloc(q, kc, vc, sp, cur)
    o2 = bd.decode(q, kc, vc, sp, cur)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # host-side rejection, nothing launched
    B, W, Hq, Hkv, D = 512, 32768, 8, 8, 128
    assert bd.decode_workspace_size(B, Hq, Hkv, W, D) > bd.DECODE_NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p(4096)
    rc = bd.lib().swa_decode_noalloc(0, P, P, P, P, P, P, None, B, W, Hq, Hkv, D, 0.1, None)
    assert rc == 3  # SWA_ERR_WORKSPACE
