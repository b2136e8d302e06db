"""GPU: seeded random configurations of the R-SWA step and of the K-draft
verify, through the oracle-checked drivers of test_gpu_parity.py (rswa_run:
[P3] write_decode_step then decode_attention, ring slots bit for bit) and
test_gpu_verify.py (run_verify: [P3] verify_attention against K sequential
decodes, nothing written).  Each case draws the kind (f32 or the int8
mirror), KV heads, group size, batch, reference length (empty, one row,
tile edges, a few thousand rows), the number of steps before the verify
(warm-up, a ring that fills during the drafts, steady state) and the draft
count."""
import numpy as np
import pytest
import torch

from gpu_cases import say
from int8_kv_cache_decode_amd import kvq as K
from test_gpu_parity import rswa_run
from test_gpu_verify import run_verify

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


PREFILLS = [0, 1, 15, 16, 17, 127, 128, 129, 500, 2047, 3001]


@pytest.mark.parametrize("seed", range(8))
def test_random_rswa_steps(seed):
    r = np.random.default_rng(5000 + seed)
    kind = (K.KIND_F32, K.KIND_I8)[seed % 2]
    nh = int(r.integers(1, 9))
    hpk = int(r.choice([1, 2, 4, 8]))
    batch = int(r.integers(1, 4))
    prefill = int(r.choice(PREFILLS)) if r.random() < 0.6 else int(r.integers(0, 2500))
    steps = int(r.choice([1, 2, 127, 128, 129, 200])) if r.random() < 0.6 else int(r.integers(1, 260))
    say("case: random rswa seed", seed, "kind", kind, "nh", nh, "hpk", hpk, "batch", batch, "prefill", prefill,
        "steps", steps)
    rswa_run(nh, prefill, steps, seed=5100 + seed, check_every=max(1, steps // 6), batch=batch, hpk=hpk, kind=kind)


@pytest.mark.parametrize("seed", range(8))
def test_random_verify(seed):
    r = np.random.default_rng(6000 + seed)
    kind = (K.KIND_F32, K.KIND_I8)[seed % 2]
    hkv = int(r.integers(1, 7))
    hpk = int(r.choice([1, 2, 4, 8]))
    n_draft = int(r.integers(1, 16 // hpk + 1))
    batch = int(r.integers(1, 4))
    prefill = int(r.choice(PREFILLS)) if r.random() < 0.6 else int(r.integers(0, 2500))
    n_hist = int(r.choice([0, 1, 120, 127, 128, 300])) if r.random() < 0.6 else int(r.integers(0, 300))
    say("case: random verify seed", seed, "kind", kind, "hkv", hkv, "hpk", hpk, "n_draft", n_draft, "batch", batch,
        "prefill", prefill, "n_hist", n_hist)
    run_verify(batch, hkv, hpk, prefill, n_hist, n_draft, seed=6100 + seed, kind=kind)
