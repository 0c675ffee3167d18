"""tfb_softmax_cross_entropy_noalloc, the entry point for callers that cannot
allocate device memory, through the C ABI: its loss against
tfb_softmax_cross_entropy's on the same logits (and against the oracle), on two
calls in a row, the second smaller (the fixed scratch array keeps the first
call's contents); sizes past its limit are rejected on the host."""
import ctypes

import numpy as np
import pytest

import synthetic as S
from oracle import ops as O
from parity import FWD_TOL, assert_close

pytestmark = pytest.mark.gpu

T = pytest.importorskip("transformer_fwd_bwd_amd")


def _noalloc(ctx, logits_dev, ld, targets_dev, rows, cols, loss_dev):
    lib = T.load_library()
    return lib.tfb_softmax_cross_entropy_noalloc(ctypes.c_void_p(logits_dev.data_ptr()), ld,
                                                 ctypes.c_void_p(targets_dev.data_ptr()), rows, cols,
                                                 ctypes.c_void_p(loss_dev.data_ptr()),
                                                 ctypes.c_void_p(ctx.stream.cuda_stream))


def test_noalloc_cross_entropy_matches_the_arena_entry_point(ctx):
    import torch
    # the first call fills 3000 rows of scratch; the second, smaller one (ragged row
    # length, padded row stride) must not see them
    for i, (rows, cols, pad) in enumerate([(3000, 1000, 0), (37, 517, 3)]):
        logits = S.random_array(160 + i, (rows, cols), 3.0)
        targets = S.random_ids(162 + i, (rows,), cols)
        lt = ctx.tensor(logits.shape, logits)
        want = T.softmax_cross_entropy(lt, targets).item()
        ld = cols + pad
        padded = np.full((rows, ld), 1e30, np.float32)       # the padding must never be read
        padded[:, :cols] = logits
        ldev = torch.from_numpy(padded).to("cuda:0")
        tdev = torch.from_numpy(targets).to("cuda:0")
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda:0")
        rc = _noalloc(ctx, ldev, ld, tdev, rows, cols, loss)
        assert rc == 0, T.load_library().tfb_last_error().decode()
        ctx.sync()
        got = float(loss.cpu().numpy()[0])
        ref = float(np.mean(O.softmax_ce_fwd(logits.astype(np.float64), targets)[0]))
        assert abs(got - want) <= FWD_TOL["fp32"] * max(abs(want), 1), (rows, got, want)
        assert_close(np.array([got]), np.array([ref]), FWD_TOL["fp32"], f"loss vs oracle, {rows} rows")
        ctx.tape_reset()
        lt.release()


def test_noalloc_cross_entropy_rejects_sizes_past_its_scratch(ctx):
    import torch
    lib = T.load_library()
    rows = 65536 + 1
    ldev = torch.zeros((1, 4), dtype=torch.float32, device="cuda:0")   # never read: rejected on the host
    tdev = torch.zeros((1,), dtype=torch.int32, device="cuda:0")
    loss = torch.zeros((1,), dtype=torch.float32, device="cuda:0")
    rc = _noalloc(ctx, ldev, 4, tdev, rows, 4, loss)
    assert rc == -2 and "at most 65536 rows" in lib.tfb_last_error().decode()
    assert _noalloc(ctx, ldev, 4, tdev, 0, 4, loss) == -2
    assert lib.tfb_softmax_cross_entropy_noalloc(None, 4, None, 1, 4, None, None) == -1
