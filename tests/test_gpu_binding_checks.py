"""The binding rejects caller-supplied outputs and workspaces that the C ABI
could not check (it sees only pointers): wrong shape, dtype, device or
layout raise DFlashError before anything is launched, so the tensors keep
their contents."""

import pytest
import torch

pytestmark = pytest.mark.gpu


def _filled(shape, dtype, dev):
    return torch.full(shape, 7, dtype=dtype, device=dev)


def test_head_outputs_checked(dfl, dev):
    h = torch.randn(5, 64, device=dev).to(torch.bfloat16)
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    good = (torch.empty(5, 16, device=dev), torch.empty(5, 16, dtype=torch.int32, device=dev))
    bad_cases = [
        (_filled((4, 16), torch.float32, dev), good[1]),          # too few rows
        (good[0], _filled((5, 16), torch.int64, dev)),            # wrong dtype
        (_filled((5, 32), torch.float32, dev)[:, :16], good[1]),  # not contiguous
        (torch.empty(5, 16), good[1]),                            # host tensor
        (good[0],),                                               # not a pair
    ]
    for out in bad_cases:
        with pytest.raises(dfl.DFlashError):
            dfl.head_topk(h, W, out=out)
    torch.cuda.synchronize()
    assert torch.all(bad_cases[0][0] == 7) and torch.all(bad_cases[1][1] == 7)
    with pytest.raises(dfl.DFlashError):
        dfl.head_topk(h, W, workspace=torch.empty(1 << 20, dtype=torch.float32, device=dev))
    with pytest.raises(dfl.DFlashError):
        dfl.head_topk(h, W.cpu())                                 # inputs on two devices
    tv, ti = dfl.head_topk(h, W, out=good)                        # the right ones pass
    assert tv.data_ptr() == good[0].data_ptr()


def test_verify_and_select_outputs_checked(dfl, dev):
    B, T, V = 3, 8, 500
    logits = torch.randn(B, T, V, device=dev)
    draft = torch.randint(0, V, (B, T - 1), dtype=torch.int32, device=dev)
    rid = torch.arange(B, dtype=torch.int64, device=dev)
    small = _filled((B, T - 1), torch.int32, dev)
    with pytest.raises(dfl.DFlashError):
        dfl.verify_greedy(logits, draft, out=(small, torch.empty(B, dtype=torch.int32, device=dev)))
    with pytest.raises(dfl.DFlashError):
        dfl.verify_sample(logits, draft, 1.0, 0, rid, rid,
                          out=(torch.empty(B, T, dtype=torch.int32, device=dev), _filled((B, 1), torch.int32, dev)))
    torch.cuda.synchronize()
    assert torch.all(small == 7)
    tv = torch.randn(B, T - 1, 16, device=dev)
    ti = torch.randint(0, V, (B, T - 1, 16), dtype=torch.int32, device=dev)
    F = torch.randn(V, 32, device=dev)
    with pytest.raises(dfl.DFlashError):
        dfl.select_path(tv, ti, F, F, out=(small, small.clone(), torch.empty(B, dtype=torch.float64, device=dev)))
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    rank, tok, score = (torch.empty(B, T - 1, dtype=torch.int32, device=dev),
                        torch.empty(B, T - 1, dtype=torch.int32, device=dev), torch.empty(B, device=dev))
    with pytest.raises(dfl.DFlashError):
        dfl.bind_select_path(tv, ti, F, F, rank, tok, score[:2], ws)
    with pytest.raises(dfl.DFlashError):
        dfl.bind_verify_greedy(logits, draft, small, torch.empty(B, dtype=torch.int32, device=dev), ws)
    dfl.bind_select_path(tv, ti, F, F, rank, tok, score, ws)()   # the right ones pass
