"""A wide seeded parity sweep: the random generators of the gather and indexer
tests at fresh seeds (50000 on), every output compared byte for byte with the
oracle.  Each seed draws a batch for the medium, page-size and dense
generators and one corrupted indexer batch; every tenth seed adds ten small
workloads.  PKVG_SWEEP_SEEDS sets the number of seeds (default 100, about 15 s
on one MI355X); 2783 seeds are 13,922 cases."""
import os

import numpy as np
import pytest
import torch

import oracle_pins
import paged_kv_cache_device_amd as pkvg
import test_gather_gpu as tg
import test_indexer_gpu as ti
import workloads
from gpu_util import check_parity, log

pytestmark = pytest.mark.gpu

FIRST_SEED = 50000
SEEDS = int(os.environ.get("PKVG_SWEEP_SEEDS", "100"))


def indexer_batch(seed: int):
    """One random indexer batch with corrupted ids and table entries (the
    generator of the indexer's small random test)."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    layout = int(rng.integers(0, 2))
    bs = int(rng.choice([16, 32, 64])) if layout else int(rng.choice([1, 2, 7, 16, 64]))
    hd = int(rng.choice([64, 128, 256]))
    lens = rng.integers(0, 5 * bs + 3, size=B).tolist()
    lens = [0 if rng.random() < 0.15 else n for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    iw = workloads.make_indexer_workload(
        f"ix_sweep{seed}", lens, bs, hd, max(pages, 1) + int(rng.integers(0, 5)), seed=seed,
        layout=layout, record_pad=4 * int(rng.integers(0, 9)), pad_rows=int(rng.integers(0, 70)),
        value_cols=hd + int(rng.choice([0, 0, 1, 3, 16])), scale_cols=int(rng.choice([1, 2, 3])),
        allow_alias=bool(rng.random() < 0.3))
    return ti.corrupt(iw, rng)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkvg.library()  # fail loudly if the HIP library is missing


def test_wide_seeded_sweep():
    cases = 0
    for seed in range(FIRST_SEED, FIRST_SEED + SEEDS):
        check_parity(tg.medium_random_workload(seed), tg.DEV)
        check_parity(tg.page_size_random_workload(seed), tg.DEV)
        check_parity(tg.dense_random_workload(seed), tg.DEV)
        ti.check_indexer_parity(indexer_batch(seed))
        cases += 4
        if seed % 10 == 0:
            for wl in oracle_pins.random_small_workloads(seed, 10):
                check_parity(wl, tg.DEV)
                cases += 1
    log(f"[sweep] {cases} cases over seeds {FIRST_SEED}..{FIRST_SEED + SEEDS - 1}: identical to the oracle")
