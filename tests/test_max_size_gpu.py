"""The forward at the largest sequence fa_fwd accepts for one bf16 head of
d = 128: N = 8388479 tokens, where (N + 128) * 256 bytes still fits the 32-bit
byte offsets a head is addressed with (one token more is refused, checked on
the CPU in test_abi). Causal, unsplit, through the C ABI, against the fp64
oracle on sampled rows: 0 and 1, the rows either side of the first key-tile and
query-tile boundaries, the middle, the last rows of the sequence (the highest
offsets Q, K, V and O are read or written at, inside the ragged last query
tile) and 8 uniform draws. Tolerances as for the other long sequences: O 1e-2
plus the bf16 output floor, L 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_qkv_long

pytestmark = pytest.mark.gpu

D = 128
N_MAX = (2 ** 31 - 1) // (D * 2) - 128          # largest N with (N + 128) * 256 <= INT_MAX


def test_largest_accepted_sequence_causal():
    assert (N_MAX + 128) * D * 2 <= 2 ** 31 - 1 < (N_MAX + 129) * D * 2
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(777)
    rows = {0, 1, 31, 32, 127, 128, N_MAX // 2, N_MAX - 129, N_MAX - 128, N_MAX - 2, N_MAX - 1}
    rows.update(int(r) for r in rng.integers(0, N_MAX, size=8))
    rows = np.array(sorted(rows), dtype=np.int64)
    print(f"[case] N={N_MAX} d={D} bf16 causal, {len(rows)} sampled rows", flush=True)
    q, k, v = make_qkv_long(N_MAX, D, seed=51)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.fwd(qd, kd, vd, causal=True, scale=scale, num_splits=1)
    idx = torch.from_numpy(rows).cuda()
    got_o = o[:, :, idx].float().cpu().double().numpy()
    got_l = lse[:, :, idx].cpu().double().numpy()
    torch.cuda.synchronize()
    del qd, kd, vd, o, lse
    print("    kernel done; oracle on the sampled rows", flush=True)
    O_ref, L_ref = oracle.attention(q, k, v, scale=scale, causal=True, rows=rows)
    err_o = float(np.max(np.abs(got_o - O_ref)))
    err_l = float(np.max(np.abs(got_l - L_ref)))
    floor = float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))
    print(f"    max|dO|={err_o:.3e} (tol {1e-2 + floor:.3e}) max|dL|={err_l:.3e}", flush=True)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    assert err_o <= 1e-2 + floor and err_l <= 1e-3
