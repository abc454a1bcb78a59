"""rwkv7_greedy_noalloc (partials in the library's static device array)
against rwkv7_greedy (partials in a caller workspace): ids, occurrence rows
and error flags bit for bit, on two calls in a row, the second smaller, then
a call with a repeated slot, and the size limit rejected on the host."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    import rwkv_linear_attention_decode_amd as R
    return R


def _case(R, B, V, n_slots, seed, slots=None):
    g = torch.Generator().manual_seed(seed)
    logits = (torch.randn(B, V, generator=g) * 3).cuda()
    logits[0, 5] = logits[0].max() + 1.0          # a clear winner that the penalty may remove
    occ = (torch.rand(n_slots, V, generator=g) * (torch.rand(n_slots, V, generator=g) < 0.05) * 4).cuda()
    occ[0, 5] = 2.0
    if slots is None:
        slots = torch.randperm(n_slots, generator=g)[:B].to(torch.int32)
    slot_idx = torch.as_tensor(slots, dtype=torch.int32).cuda()
    pres = (torch.rand(B, generator=g) * 2).cuda()
    freq = (torch.rand(B, generator=g) * 2).cuda()
    dec = (0.9 + 0.1 * torch.rand(B, generator=g)).cuda()
    return logits, occ, slot_idx, pres, freq, dec


def _both(R, B, V, n_slots, seed, slots=None):
    logits, occ, slot_idx, pres, freq, dec = _case(R, B, V, n_slots, seed, slots)
    occ_a, occ_b = occ.clone(), occ.clone()
    ids_a = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ids_b = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(R.rwkv7_greedy_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    R.rwkv7_greedy(logits, occ_a, n_slots, slot_idx, pres, freq, dec, ids_a, ws)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    R.rwkv7_greedy_noalloc(logits, occ_b, n_slots, slot_idx, pres, freq, dec, ids_b, flags)
    torch.cuda.synchronize()
    fa = R.rwkv7_poll_error(ws)
    fb = int(flags.item())
    assert torch.equal(ids_a, ids_b), (B, V)
    assert torch.equal(occ_a.view(torch.int32), occ_b.view(torch.int32)), (B, V)
    assert fa == fb, (fa, fb)
    return ids_b.cpu().numpy(), fb


def test_noalloc_matches_workspace_greedy_two_calls(R):
    ids, f = _both(R, 256, 65536, 300, 1)             # the largest call the scratch holds
    assert f == 0 and ids.min() >= 0
    ids, f = _both(R, 3, 1000, 5, 2)                  # then a smaller one: same array, fewer blocks
    assert f == 0 and ids.min() >= 0


def test_noalloc_flags_repeated_slot(R):
    ids, f = _both(R, 4, 4096, 8, 3, slots=[1, 6, 1, 2])
    assert f == R.ERR_SLOT_DUP


def test_noalloc_rejects_oversize(R):
    logits = torch.zeros(257, 65536, device="cuda")
    occ = torch.zeros(300, 65536, device="cuda")
    one = torch.ones(257, device="cuda")
    slots = torch.arange(257, dtype=torch.int32, device="cuda")
    ids = torch.zeros(257, dtype=torch.int32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(R.RWKV7Error) as e:
        R.rwkv7_greedy_noalloc(logits, occ, 300, slots, one, one, one, ids, flags)
    assert e.value.status == R.RWKV7_ESHAPE
