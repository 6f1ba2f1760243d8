"""moe_permute_noalloc (no workspace: the library's fixed device buffer holds
the per-block counts) against moe_permute with a caller workspace, bit for
bit, on two calls in a row, the second smaller, so stale contents of the
fixed buffer from the first call would show."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_routed_expert_moe_amd import moe
    return moe


def _skewed_idx(g, T, k, E):
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    return np.stack([g.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _run(m, idx, E, noalloc):
    T, k = idx.shape
    d_idx = torch.from_numpy(idx).cuda()
    out = [torch.full((E,), -7, dtype=torch.int32, device="cuda"),
           torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
           torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
           torch.full((T * k,), -7, dtype=torch.int32, device="cuda")]
    if noalloc:
        m.moe_permute_noalloc(d_idx, E, *out)
    else:
        ws = torch.empty(max(1, m.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device="cuda")
        m.moe_permute(d_idx, E, *out, ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("first,second", [
    ((8192, 8, 384), (3001, 7, 100)),      # block path twice, smaller second call
    ((32768, 8, 1024), (2100, 8, 384)),    # at the buffer's limit (256 blocks x 1024 experts), then smaller
    ((4096, 8, 384), (64, 8, 384)),        # block path, then the one-workgroup path
])
def test_noalloc_permute_matches_workspace_permute(m, first, second):
    g = np.random.default_rng(0)
    for T, k, E in (first, second):
        print(f"[gpu-case] permute_noalloc T={T} k={k} E={E}", flush=True)
        idx = _skewed_idx(g, T, k, E)
        got = _run(m, idx, E, True)
        ref = _run(m, idx, E, False)
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)


def test_noalloc_permute_rejects_sizes_beyond_its_buffer(m):
    # 1024 experts and 262,145+ slots need more than the fixed 262,144 count entries
    T, k, E = 32769, 8, 1024
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    bufs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    with pytest.raises(m.MoEError) as ei:
        m.moe_permute_noalloc(idx, E, *bufs)
    assert ei.value.status == m.MOE_ERR_UNSUPPORTED
