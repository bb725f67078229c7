"""The splitter's two selection rules on caller-supplied values ("Spark-H3"
blog, 01 / Method: Spark-Reblock, the partitioner paragraph: every group is
split by the distance while the child capacities are enforced; the two-pole
rule and its tie rules -- -0 equals +0, NaN ranks last, ties to the lower
token id -- are the reading both implementations take), through the C ABI's
test hooks, bit for bit against the oracle's capacity_partition and
argmin_lowest_id.

* spark_debug_partition_level: rows whose groups take each of the top
  level's two kernel paths (the one-workgroup select up to 64 blocks, the
  many-workgroup radix rounds and segmented partition above), on both sides
  of the boundary (64 and 65 blocks: a second segment of one position) and
  with unaligned rows, with values drawn from a tie-heavy set (+-0, +-inf,
  NaN, repeated numbers) and from a continuous distribution, and ragged
  last blocks.
* spark_debug_argmin: the pole choice's (value, id) ordering on the same
  kinds of rows, 1 to 5,000 values.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()


def say(msg):
    print(msg, flush=True)


TIES = np.array([-1.5, -0.0, 0.0, 0.25, 2.0, np.nan, np.inf, -np.inf], dtype=np.float32)


def _rows(rng, count, n, kind):
    if kind == "ties":
        s = rng.choice(TIES, size=(count, n))
    elif kind == "few":
        s = rng.integers(-3, 4, size=(count, n)).astype(np.float32)
        s[rng.random((count, n)) < 0.05] = np.nan
        s[s == 0] = np.where(rng.random(int((s == 0).sum())) < 0.5, -0.0, 0.0)
    else:
        s = rng.standard_normal((count, n)).astype(np.float32)
    ids = np.stack([np.sort(rng.choice(4 * n + 8, size=n, replace=False)) for _ in range(count)])
    return s.astype(np.float32), ids.astype(np.int32)


@pytest.mark.parametrize("n,block", [(37, 8), (1000, 64), (8192, 128), (8193, 128), (9000, 64), (70000, 128),
                                     (70001, 128)])
@pytest.mark.parametrize("kind", ["ties", "few", "normal"])
def test_capacity_partition_matches_oracle(n, block, kind):
    rng = np.random.default_rng(n * 7 + block + len(kind))
    count = 3
    s, ids = _rows(rng, count, n, kind)
    nbg = -(-n // block)
    cL = ((nbg + 1) // 2) * block
    say(f"[partition] n={n} block={block} ({nbg} blocks, left capacity {cL}) kind={kind}")
    got = L.spark_debug_partition_level(torch.from_numpy(s).to(DEV), torch.from_numpy(ids).to(DEV), block)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for r in range(count):
        left, right = O.capacity_partition(s[r].astype(np.float64), ids[r], cL)
        assert np.array_equal(got[r], np.concatenate([left, right])), r


@pytest.mark.parametrize("n", [1, 5, 64, 300, 5000])
@pytest.mark.parametrize("kind", ["ties", "few", "normal"])
def test_argmin_matches_oracle(n, kind):
    rng = np.random.default_rng(n * 11 + len(kind))
    count = 16
    v, ids = _rows(rng, count, n, kind)
    # shuffle the ids within each row: the argmin does not rely on their order
    ids = np.stack([rng.permutation(r) for r in ids]).astype(np.int32)
    got = L.spark_debug_argmin(torch.from_numpy(v).to(DEV), torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for r in range(count):
        want = ids[r][O.argmin_lowest_id(v[r].astype(np.float64), ids[r])]
        assert got[r] == want, (r, got[r], want)
    say(f"[argmin] n={n} kind={kind}: {count} rows equal")


def test_signed_zero_and_nan_cases():
    v = torch.tensor([[0.0, -0.0], [-0.0, 0.0], [float("nan"), 5.0], [float("nan"), float("nan")]],
                     device=DEV)
    ids = torch.tensor([[3, 7], [3, 7], [0, 1], [9, 4]], dtype=torch.int32, device=DEV)
    got = L.spark_debug_argmin(v, ids).cpu().tolist()
    assert got == [3, 3, 1, 4]
    # one block of capacity: ceil(ceil(4/2)/2)*2 = 2 go left
    s = torch.tensor([[-0.0, 0.0, float("nan"), 1.0]], device=DEV)
    pid = torch.tensor([[1, 2, 3, 4]], dtype=torch.int32, device=DEV)
    got = L.spark_debug_partition_level(s, pid, 2).cpu().tolist()
    assert got == [[1, 4, 2, 3]]
