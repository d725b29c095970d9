"""Slot assignment and base read-back through the C ABI: the pool keeps each
d_k x B_V value tile of a base contiguous, callers exchange states in the
natural [d_k, d_v] layout.  Copies are exact (byte for byte)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TILES = [(128, 128), (128, 64), (128, 32), (128, 16), (64, 64), (64, 32), (32, 32), (16, 16)]


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,bv", TILES)
def test_assign_read_roundtrip_and_tile_layout(d, bv, state_dtype):
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import say

    say(f"[gpu] state layout d={d} B_V={bv} {state_dtype}")
    P, Hv, Hk = 7, 4, 2
    pool = dl.DeltaLogPool(P, Hv, Hk, d, 4, "scalar", "delta", state_dtype, "f32", max_batch=3,
                           value_tile=bv)
    dt = torch.float32 if state_dtype == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(d * 1000 + bv)
    init = torch.randn((P, Hv, d, d), generator=g).to(dt)
    ids = np.array([5, 0, 3, 6, 1, 2, 4], dtype=np.int32)
    for lo in range(0, P, 3):
        pool.assign(ids[lo: lo + 3], init[lo: lo + 3].cuda().contiguous())
    torch.cuda.synchronize()
    # read-back in the natural layout is byte-exact, in any slot order
    back = pool.read_base(ids).cpu()
    assert torch.equal(back.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       init.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    order = np.array([2, 4, 6], dtype=np.int32)
    sub = pool.read_base(order).cpu()
    pos = {int(s): j for j, s in enumerate(ids)}
    assert torch.equal(sub, init[[pos[int(s)] for s in order]])
    # the raw buffer is value-tile major: [P, H_v, d / B_V, d_k, B_V]
    raw = pool.base_tiles.cpu()
    nat = raw.permute(0, 1, 3, 2, 4).reshape(P, Hv, d, d)
    assert torch.equal(nat[torch.from_numpy(ids.astype(np.int64))], init)
    # a zero assignment clears only its slots; reading leaves the counters alone
    pool.decode_step([1], torch.randn(1, Hk, d).cuda(), torch.randn(1, Hk, d).cuda(),
                     torch.randn(1, Hv, d).cuda(), torch.rand(1, Hv).cuda() * -0.1,
                     torch.rand(1, Hv).cuda())
    pool.assign([3])
    after = pool.read_base(np.arange(P, dtype=np.int32)).cpu()
    assert torch.count_nonzero(after[3]) == 0
    assert torch.equal(after[5], init[0])
    n_dev = pool.device_log_len()
    assert n_dev[1].tolist() == [1] * (Hv * (d // bv))
    assert int(n_dev.sum()) == Hv * (d // bv)
    pool.close()
