"""GPU check of the no-allocation decode (swa_decode_noalloc): the same output
bits as swa_decode with a caller workspace, on two calls in a row, the second
with a smaller batch and another split count (the static scratch keeps the
first call's partials, which the second must not read)."""

import numpy as np
import pytest
import torch

from sliding_window_attention_swa_amd import workloads as WL

from gpu_path import TOL, DeviceWorkload, check, oracle_decode, run_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sliding_window_attention_swa_amd import swa  # noqa: F401  (fails loudly if libswa.so is missing)
    yield
    torch.cuda.synchronize()


def _noalloc(dw, splits, out_dtype=torch.float32):
    from sliding_window_attention_swa_amd import swa
    wl = dw.wl
    out = torch.empty((wl.batch, wl.q_heads, wl.head_dim), dtype=out_dtype, device="cuda")
    swa.swa_decode_noalloc(dw.q, dw.layer, dw.index, wl.window, out, sinks=dw.sinks, num_splits=splits,
                           use_map=False)
    torch.cuda.synchronize()
    return out


def test_decode_noalloc_matches_workspace_decode():
    cases = [("first", 51, [1, 700, 3000, 9000], 16, 2, "bf16", 8),     # larger batch, 8 splits
             ("second", 52, [5, 900], 16, 2, "e4m3", 3)]                # smaller, another split count
    for name, seed, lens, hq, hkv, kvd, splits in cases:
        say(f"noalloc decode {name}: B={len(lens)}, {kvd}, {splits} splits")
        wl = WL.decode_workload(f"noalloc_{name}", seed, lens, hq, hkv, -1, 16, "bf16", kvd, sinks=True)
        dw = DeviceWorkload(wl)
        want = run_decode(dw, "f32", num_splits=splits)
        got = _noalloc(dw, splits)
        assert torch.equal(got, want), name
        check(got, oracle_decode(wl), TOL[kvd], f"noalloc {name}")
        got_bf = _noalloc(dw, splits, torch.bfloat16)
        assert torch.equal(got_bf, want.to(torch.bfloat16)), name
    # one split: no scratch at all
    wl = WL.decode_workload("noalloc_one", 53, [3, 40], 16, 2, -1, 16, "bf16", "bf16", sinks=False)
    dw = DeviceWorkload(wl)
    assert torch.equal(_noalloc(dw, 1), run_decode(dw, "f32", num_splits=1))
