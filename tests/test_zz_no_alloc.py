"""topk_select_noalloc (the top-k call that allocates nothing: its workspace is
a fixed device array the library owns) against topk_select with a caller
workspace, through the C-ABI: bit-exact selections on two calls in a row, the
second with a smaller input, on the split path (few long BF16 rows, decode)
and the row path (many rows), plus the refusal of a shape beyond the array."""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev, down, up

pytestmark = pytest.mark.gpu


def _scores(rng, B, T, N):
    s = np.round(rng.standard_normal((B, T, N)) * 8, 1).astype(np.float32)    # many ties in BF16
    s[:, :, ::7] = -np.inf
    return up(s).to(torch.bfloat16)


def _both(L, sc, ne, qp, k):
    B, T, _ = sc.shape
    a = torch.full((B, T, k), -7, dtype=torch.int32, device=dev())     # sentinels no result can hold
    b = torch.full((B, T, k), -9, dtype=torch.int32, device=dev())
    L.topk_select_noalloc(sc, ne, qp, 4, k, a)
    L.topk_select(sc, ne, qp, 4, k, b)
    torch.cuda.synchronize()
    return a, b


def test_topk_select_noalloc_matches_topk_select():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(90)
    cases = [
        # (B, T, N, k, q_pos, n_entries): decode shape, then a smaller split-path input, then the row path
        (8, 1, 262208, 1024, [4 * 262144 + 3] * 6 + [4 * 9000 + 1, 5], [262144] * 8),
        (3, 1, 40000, 512, [4 * 40000, 4 * 30000 + 2, 4 * 40000], [40000, 40000, 20000]),
        (1, 64, 5000, 256, list(range(4 * 5000 - 64, 4 * 5000)), [5000]),
    ]
    for B, T, N, k, qp, ne in cases:
        need = L.topk_workspace_size(B, T, N, k, L.CSA_BF16)
        print(f"topk_select_noalloc B={B} T={T} N={N} k={k}: workspace {need} bytes", flush=True)
        assert need <= L.TOPK_NOALLOC_MAX_BYTES
        sc = _scores(rng, B, T, N)
        a, b = _both(L, sc, up(np.array(ne, np.int32)), up(np.array(qp, np.int64).reshape(B, T)), k)
        assert torch.equal(a, b)
        assert (down(a) >= -1).all()


def test_topk_select_noalloc_refuses_shapes_beyond_its_array():
    from long_context_compressed_compress_amd import libcsa as L
    B, N, k = 120, 1 << 20, 1024      # split path, 120 rows of 2^20 scores: about 33 MiB of workspace
    assert L.topk_workspace_size(B, 1, N, k, L.CSA_BF16) > L.TOPK_NOALLOC_MAX_BYTES
    sc = torch.zeros(B, 1, N, dtype=torch.bfloat16, device=dev())
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=dev())
    with pytest.raises(L.CsaError) as ex:
        L.topk_select_noalloc(sc, up(np.full(B, N, np.int32)), up(np.full((B, 1), 4 * N, np.int64)), 4, k, idx)
    assert ex.value.status == L.CSA_ERR_WORKSPACE
