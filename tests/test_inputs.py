"""The seeded input generators (CPU): the chunked long-sequence generator
depends on its seed and chunking only, not on how many threads draw it, and
gives distinct, roughly N(0, 1) bf16 tensors."""
import torch

from tiled_attention_fa2_amd.inputs import make_qkv_long


def test_long_generator_is_thread_count_independent():
    a = make_qkv_long(1000, 64, seed=5, chunk_rows=96, threads=1)
    b = make_qkv_long(1000, 64, seed=5, chunk_rows=96, threads=7)
    for x, y in zip(a, b):
        assert x.shape == (1, 1, 1000, 64) and x.dtype == torch.bfloat16
        assert torch.equal(x, y)
    c = make_qkv_long(1000, 64, seed=6, chunk_rows=96)
    assert not torch.equal(a[0], c[0])
    q, k, v = a
    assert not torch.equal(q, k) and not torch.equal(k, v)
    # chunks are not copies of one another
    assert not torch.equal(q[0, 0, :96], q[0, 0, 96:192])
    x = torch.cat([t.float().ravel() for t in a])
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
