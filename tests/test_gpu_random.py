"""Randomized parity against the oracle: 3000 small problems from fixed seeds, each drawing its
sequence form (offsets, per-token IDs, batch rows), channel count (1..2050, partial strips and
odd counts), sequence count (0..140, both levels of the offsets lookup), lengths (1..1000), filter
width (2..8), slot pool (both layouts, -1 slots, 3..6 positions) or history rows, d(tail),
activation, tap and bias dtypes, and empty sequences.  Forward always, backward without a pool.
A failure names its seed; the case is rebuilt by make_case(seed)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402
from causal_depthwise_conv1d_width_amd import workloads as wl  # noqa: E402

CHANNELS = [1, 2, 3, 7, 8, 13, 64, 127, 128, 130, 256, 510, 512, 514, 1000, 1024, 1032, 1536, 2048, 2050]
SEEDS = range(20000, 23000)


def make_case(seed):
    """(case, dtail, has_pool) for one seed; problems stay under ~3M elements."""
    rng = np.random.default_rng(seed)
    mode = str(rng.choice(["cu", "cu", "idx", "batch"]))
    C = int(rng.choice(CHANNELS))
    nseq = int(rng.choice([0, 1, 2, 5, 9, 30, 126, 127, 140]))
    max_len = int(rng.choice([1, 2, 3, 5, 10, 40, 300, 1000]))
    while nseq * max_len * C > 3_000_000 and max_len > 1:
        max_len //= 2
    pool = mode in ("cu", "batch") and rng.random() < 0.35
    hist = mode in ("cu", "batch") and not pool and rng.random() < 0.5
    W = 4 if pool else int(rng.choice([2, 3, 4, 4, 5, 6, 7, 8]))  # the pool form is width four
    case = wl.random_case(rng, C=C, nseq=nseq, max_len=max_len, mode=mode,
                          pool_layout_name=(str(rng.choice(["hist", "chan"])) if pool else None),
                          L=int(rng.choice([3, 4, 6])), with_hist=hist, w_f32=bool(rng.integers(0, 2)),
                          act=str(rng.choice(["silu", "silu", "none"])), force_empty=bool(rng.random() < 0.3),
                          sentinel=bool(rng.random() < 0.5))
    if W != 4:
        w = wl.uniform_f32(rng, (C, W))
        case["w"] = w if case["w"].dtype == np.float32 else wl.to_bf16_bits(w)
        if case.get("hist") is not None:
            case["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], W - 1, C))
    dtail = wl.normal_bf16(rng, (W - 1, C)) if mode == "cu" and not pool and rng.random() < 0.3 else None
    case["name"] = (f"seed{seed}-{mode}-C{C}-n{nseq}-L{max_len}-W{W}-"
                    f"{'pool' if pool else ('hist' if hist else 'plain')}{'-dtail' if dtail is not None else ''}")
    return case, dtail, pool


def test_random_problems(oracle):
    print(f"[gpu] random problems, seeds {SEEDS.start}..{SEEDS.stop - 1}", flush=True)
    failures = []
    for seed in SEEDS:
        case, dtail, pool = make_case(seed)
        try:
            gh.check_fwd(oracle, case)
            if not pool:
                gh.check_bwd(oracle, case, dtail=dtail)
        except AssertionError as e:
            failures.append(f"{case['name']}: {str(e)[:200]}")
    assert not failures, f"{len(failures)} of {len(SEEDS)} random problems differ:\n" + "\n".join(failures[:20])
