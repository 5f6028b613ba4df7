"""ftq_moe_q4_0_q8_1_noalloc: the matmul with the library's fixed per-device
scratch instead of a caller workspace, for callers that cannot allocate.  Its
output must equal ftq_moe_q4_0_q8_1's bit for bit (the same kernels) and the
oracle within the stated tolerance, on consecutive calls that share the
scratch, the second with a smaller batch."""
import numpy as np
import pytest
import torch

from quantized_moe_expert_quantize_amd import ftq
from tests._cases import Case, assert_matches_oracle, say

pytestmark = pytest.mark.gpu


def _both(c: Case, path):
    wq, aq, ids = c.gpu()
    ref = ftq.moe(wq, aq, ids, c.E, c.N, c.K, path=path)
    out = torch.full_like(ref, float("nan"))
    ftq.moe_noalloc(wq, aq, ids, c.E, c.N, c.K, out, path=path)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("path", [ftq.PATH_GROUPED, ftq.PATH_GEMV, ftq.PATH_AUTO])
def test_noalloc_equals_workspace_call_on_two_calls(path):
    # page-1 rows (K = 2816, 128 experts, top-8) at two batch sizes: the first
    # call fills the scratch, the second (smaller) reuses it
    E, N, K, k = 128, 200, 2816, 8
    for T in (600, 70):
        say(f"[noalloc] path={path} E={E} N={N} K={K} T={T} top_k={k}")
        c = Case(E, N, K, T, k, seed=T)
        need = ftq.workspace_bytes(E, N, K, T, k, path)
        ref, out = _both(c, path)
        assert torch.equal(out, ref), f"T={T}: differs from the workspace call"
        pairs = np.unique(np.concatenate([np.arange(0, T * k, 37), [T * k - 1]]))
        r, ab = c.oracle_out(pairs)
        assert_matches_oracle(out[torch.from_numpy(pairs).cuda()].cpu().numpy(), r, ab, c.nb)
        say(f"[noalloc]   workspace it replaces: {need} bytes")


def test_noalloc_rejects_what_does_not_fit():
    # 1.6 M pairs need more than the 4 MiB scratch; nothing is launched
    E, N, K, T, k = 128, 64, 64, 200_000, 8
    assert ftq.workspace_bytes(E, N, K, T, k, ftq.PATH_GROUPED) > 4 << 20
    w = torch.zeros(E * N * (K // 32) * 18, dtype=torch.uint8, device="cuda")
    a = torch.zeros(T * (K // 32) * 36, dtype=torch.uint8, device="cuda")
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T * k, N), dtype=torch.float32, device="cuda")
    with pytest.raises(ftq.FtqError) as ei:
        ftq.moe_noalloc(w, a, ids, E, N, K, out, path=ftq.PATH_GROUPED)
    assert ei.value.status == ftq.ERR_UNSUPPORTED and "scratch" in str(ei.value)
    # invalid sizes report the same error as the workspace call
    with pytest.raises(ftq.FtqError) as ei:
        ftq.moe_noalloc(w, a, ids, E, N, K + 1, out)
    assert ei.value.status == ftq.ERR_INVALID_ARG
