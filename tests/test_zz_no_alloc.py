"""fa_fwd_splitkv_static, the split-KV forward that allocates nothing (its
partials live in the library's static device scratch), against
fa_fwd_splitkv with a caller's workspace, through the C ABI.

Both run the same kernels with the same chunks, so O and L must agree bit for
bit. The calls come in pairs on one device, the second on a smaller problem,
so that the second reads a scratch still holding the first call's partials:
every partial the merge reads must have been written by the call itself. One
small causal case is also held to the fp64 oracle (bf16 tolerance 1e-2 plus
the bf16 rounding floor of the exact answer on O, 1e-3 on L), and a problem
whose partials exceed the scratch must be refused before anything runs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, dtype, seed):
    q, k, v = make_qkv(B, H, N, d, "f32" if dtype == "f32" else "bf16", seed=seed)
    dev = [t.cuda().contiguous() for t in (q, k, v)]
    if dtype != "fp8":
        return dev, None, (q, k, v)
    q8, k8, v8, ds = fa.quantize_qkv_fp8(*dev)
    return [q8, k8, v8], ds, None


def _pair(B, H, N, d, dtype, causal, splits, seed):
    (q, k, v), ds, host = _inputs(B, H, N, d, dtype, seed)
    need = fa.splitkv_workspace_bytes(B, H, N, d, splits)
    assert 0 < need <= fa.STATIC_SCRATCH_BYTES
    print(f"  static split-KV {dtype} B={B} H={H} N={N} d={d} causal={causal} splits={splits} "
          f"({need / 2**20:.1f} MiB of partials)", flush=True)
    o_s, l_s = fa.fwd_splitkv_static(q, k, v, splits, causal=causal, descales=ds)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_w, l_w = fa.fwd(q, k, v, causal=causal, descales=ds, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_s.view(torch.int16 if o_s.dtype == torch.bfloat16 else torch.int32),
                       o_w.view(torch.int16 if o_w.dtype == torch.bfloat16 else torch.int32)), "O differs"
    assert torch.equal(l_s.view(torch.int32), l_w.view(torch.int32)), "L differs"
    return o_s, l_s, host


@pytest.mark.parametrize("first,second", [
    # bf16, head dim 128: the largest accepted split (8 x 4096 in 3 chunks,
    # 50.7 MB), then a small ragged causal one
    (dict(B=1, H=8, N=4096, d=128, dtype="bf16", causal=False, splits=3),
     dict(B=2, H=3, N=777, d=128, dtype="bf16", causal=True, splits=2)),
    # fp8 per-head scales
    (dict(B=1, H=4, N=2000, d=128, dtype="fp8", causal=False, splits=4),
     dict(B=1, H=2, N=300, d=128, dtype="fp8", causal=True, splits=2)),
    # the generic kernel: fp32 and bf16 at head dim 64
    (dict(B=1, H=3, N=1500, d=64, dtype="f32", causal=True, splits=3),
     dict(B=1, H=2, N=129, d=64, dtype="bf16", causal=False, splits=2)),
])
def test_static_matches_workspace_path_on_two_calls(first, second):
    _pair(**first, seed=1)
    o, l, host = _pair(**second, seed=2)
    if second["dtype"] == "bf16" and second["causal"]:
        q, k, v = (t.double().numpy() for t in host)
        O_ref, L_ref = oracle.attention(q, k, v, scale=1.0 / math.sqrt(q.shape[-1]), causal=True)
        floor = float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))
        assert np.max(np.abs(o.double().cpu().numpy() - O_ref)) <= 1e-2 + floor
        assert np.max(np.abs(l.double().cpu().numpy() - L_ref)) <= 1e-3


def test_oversized_problem_is_refused():
    # 4 chunks of 8 x 4096 need 67.6 MB of partials, above the 64 MiB scratch
    (q, k, v), _, _ = _inputs(1, 8, 4096, 128, "bf16", seed=3)
    with pytest.raises(fa.FAError) as e:
        fa.fwd_splitkv_static(q, k, v, 4)
    assert e.value.status == -11
