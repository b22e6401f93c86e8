"""recap_block_scores_noalloc (fixed library-held scratch, no allocation inside the call)
against recap_block_scores (caller's workspace) on the GPU, through the C ABI: the same
kernels on the same inputs, so the block probabilities must agree bit for bit. Two calls in a
row, the second smaller, so the second runs on a scratch that still holds the first call's
means; and a third at the first size again."""
import pytest
import torch

import block_sparse_attention_top_amd as bsa
from block_sparse_attention_top_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, N, D, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B, H, N, D), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, H, N, D), generator=g, device=DEV).to(torch.bfloat16)
    # a shared low-frequency component so that the scores are not uniform
    pos = torch.linspace(0, 6.28, N, device=DEV).view(1, 1, N, 1)
    f = torch.arange(D, device=DEV).view(1, 1, 1, D) % 8 + 1
    q = (q.float() + 2.0 * torch.sin(pos * f)).to(torch.bfloat16)
    k = (k.float() + 2.0 * torch.sin(pos * f)).to(torch.bfloat16)
    return q, k


@pytest.mark.parametrize("shape", [
    [(1, 40, 75600, 128, 64), (2, 3, 1000, 64, 128), (1, 40, 75600, 128, 64)],
])
def test_block_scores_noalloc_matches_workspace_call(shape):
    bsa.load()
    for i, (B, H, N, D, blk) in enumerate(shape):
        print(f"[case] call {i}: B={B} H={H} N={N} D={D} block={blk}", flush=True)
        q, k = _inputs(B, H, N, D, 100 + i)
        desc = bsa.make_desc(q, blk)
        need = bsa.recap_workspace_size(_lib.OP_BLOCK_SCORES, desc)
        assert need <= _lib.NOALLOC_SCRATCH_BYTES
        M = -(-N // blk)
        ref = bsa.recap_block_scores(desc, q, k)
        got = torch.full((B, H, M, M), float("nan"), dtype=torch.float32, device=DEV)
        bsa.recap_block_scores_noalloc(desc, q, k, probs=got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: {(got != ref).sum().item()} values differ"
        rows = got.sum(-1)
        assert torch.all((rows - 1).abs() <= 1e-5)


def test_block_scores_noalloc_rejects_oversize():
    """A call needing more than the fixed scratch is rejected before any launch (no write)."""
    bsa.load()
    B, H, N, D, blk = 1, 64, 75600, 128, 64  # 77.5 MB of pooled means
    q = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device=DEV)
    desc = bsa.make_desc(q, blk)
    M = -(-N // blk)
    probs = torch.full((B, H, M, M), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(bsa.RecapError) as ei:
        bsa.recap_block_scores_noalloc(desc, q, q, probs=probs)
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert torch.all(probs == 7.0)
