"""The allocation-free FOID entry point (adahop_detect_noalloc, static
device scratch) against adahop_detect with a caller workspace, through the C
ABI: indices bit-identical on two calls in a row, the second on a smaller
input, both large enough that the selection uses its scratch (more than one
selection level)."""
import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def tensor(rows, cols, axis, seed):
    dim = rows if axis == "ROWS" else cols
    lines = synth.pick_lines(seed, 77, dim, max(1, dim // 100))
    x = synth.fill_bf16(rows, cols, seed, 70, 1.0, 0 if axis == "ROWS" else 1, lines, 30.0)
    return torch.from_numpy(x.view(np.int16)).to(DEV)


def test_noalloc_matches_workspace_entry_point():
    lib = A.lib()
    assert lib.adahop_detect_noalloc_max_bytes() == 1 << 20
    cases = [(64, 14336, "COLS", 64, 0),    # 14 chunks, then the final selection
             (70000, 64, "ROWS", 300, 1),   # k > 256: chunks of 4096, two levels
             (9000, 128, "ROWS", 40, 2)]    # smaller than the one before
    for rows, cols, axis, k, seed in cases:
        print("noalloc FOID", rows, cols, axis, k, flush=True)
        assert A.adahop_detect_workspace_size(rows, cols, axis, k) > 0
        t = tensor(rows, cols, axis, seed)
        want = A.adahop_detect(t, axis, k).cpu().numpy()
        out = torch.full((k,), -1, dtype=torch.int32, device=DEV)
        got = A.adahop_detect_noalloc(t, axis, k, idx_out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert np.array_equal(got.cpu().numpy(), want), (rows, cols, axis, k)
        assert np.all(np.diff(want) > 0)


def test_noalloc_rejects_selections_beyond_the_static_scratch():
    # k = 1024 over 400 000 candidates needs ~2.3 MiB of survivor lists: a
    # clear error before any launch, nothing written.
    lib = A.lib()
    need = A.adahop_detect_workspace_size(400000, 64, "ROWS", 1024)
    assert need > lib.adahop_detect_noalloc_max_bytes()
    t = torch.zeros((400000, 64), dtype=torch.int16, device=DEV)
    out = torch.full((1024,), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(A.AdahopError) as e:
        A.adahop_detect_noalloc(t, "ROWS", 1024, idx_out=out)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == -7).all())
