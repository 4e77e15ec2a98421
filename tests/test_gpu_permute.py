"""The device grouping (moe_permute: chunk histograms, the column scan split
over up to 16 threads per expert, the stable scatter) against the oracle's
stable counting sort, integer-exact, over expert counts and batch sizes
that take every split of the scan: fewer chunks than threads per expert,
16 threads per expert, a non-power-of-two share, one thread per expert at
E = 1000 and 1024, and every row on one expert."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import custom, say
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


# (E, T, k, pattern): rows = T * k
CASES = [
    (3, 400, 3, "uniform"),      # 1200 rows: 5 chunks, 5 threads per expert
    (8, 2000, 4, "uniform"),     # 8000 rows: 32 chunks, 16 threads per expert
    (100, 5000, 8, "uniform"),   # 40000 rows: 157 chunks, 10 threads per expert
    (128, 8192, 8, "skewed"),    # 65536 rows: 256 chunks, 8 threads per expert
    (1000, 4096, 8, "uniform"),  # one thread per expert
    (1024, 9000, 8, "uniform"),  # 72000 rows, one thread per expert
    (64, 3000, 6, "one_expert"),  # every row on expert 37
]


def _idx(E, T, k, pattern, rng):
    if pattern == "one_expert":
        return np.full((T, k), 37, np.int32)
    if pattern == "skewed":
        # a tenth of the experts take most rows
        p = np.full(E, 1.0)
        p[: E // 10] = 40.0
        return rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    return rng.integers(0, E, size=(T, k), dtype=np.int32)


@pytest.mark.parametrize("E,T,k,pattern", CASES)
def test_permute_matches_oracle(E, T, k, pattern):
    cfg = synth.layer_keys(custom(T=T, hidden_size=64, num_experts=E, num_experts_per_tok=k,
                                  moe_intermediate_size=64, num_shared_experts=0))
    rng = np.random.default_rng(E * 7 + k)
    idx = _idx(E, T, k, pattern, rng)
    rows = T * k
    ws = moe.alloc_workspace(cfg, T)
    d_idx = torch.from_numpy(idx.reshape(-1)).cuda()
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sr = torch.empty(rows, dtype=torch.int32, device="cuda")
    rp = torch.empty(rows, dtype=torch.int32, device="cuda")
    say(f"permute E={E} T={T} k={k} {pattern}")
    for _ in range(2):  # the workspace's scratch is reused as is by a second call
        moe.moe_permute(cfg, T, d_idx, offs, sr, rp, ws)
        torch.cuda.synchronize()
        _, r_offs, r_sr, r_rp = O.permute(idx, E)
        assert np.array_equal(offs.cpu().numpy(), r_offs)
        assert np.array_equal(sr.cpu().numpy(), r_sr)
        assert np.array_equal(rp.cpu().numpy(), r_rp)
