"""graft_lmhead_topk_noalloc (the lm-head + top-k entry point that takes no
workspace: its scratch is an array built into the library) equals the
workspace entry point graft_lmhead_topk bit for bit, on two calls in a row,
the second smaller than the first (the array keeps the first call's
contents)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _case(api, M, H, V, k, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    hidden = torch.randn(M, H, generator=g).to(torch.bfloat16).cuda()
    w = (0.02 * torch.randn(V, H, generator=g)).to(torch.bfloat16).cuda()
    wp = torch.empty(api.graft_lmhead_pack_bytes(V, H) // 2, dtype=torch.bfloat16, device="cuda")
    api.graft_lmhead_pack(V, H, w, wp)
    return hidden, wp


def test_noalloc_equals_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_tree_verification_parent_amd import api
    from draft_tree_verification_parent_amd._native import W_PACKED

    # 960 rows (256 x 256 tiles, four m tiles) then 60 rows (the 64-row kernel)
    for M, H, V, k, seed in ((960, 1024, 20011, 8, 1), (60, 512, 9000, 16, 2)):
        need = api.graft_lmhead_topk_noalloc_bytes(M, k)
        assert 0 < need <= api.graft_lmhead_topk_noalloc_bytes(16384, 16) <= 8 << 20
        print(f"[noalloc] M={M} H={H} V={V} k={k}: {need} bytes of built-in scratch", flush=True)
        hidden, wp = _case(api, M, H, V, k, seed)
        ref_id = torch.empty(M, k, dtype=torch.int32, device="cuda")
        ref_val = torch.empty(M, k, dtype=torch.float32, device="cuda")
        ws = torch.empty(api.graft_lmhead_topk_workspace_bytes(M, V, k), dtype=torch.uint8, device="cuda")
        api.graft_lmhead_topk(M, H, V, k, hidden, wp, None, ref_id, ref_val, ws, w_layout=W_PACKED)
        got_id = torch.full((M, k), -5, dtype=torch.int32, device="cuda")
        got_val = torch.full((M, k), -5.0, dtype=torch.float32, device="cuda")
        api.graft_lmhead_topk_noalloc(M, H, V, k, hidden, wp, got_id, got_val)
        torch.cuda.synchronize()
        assert torch.equal(got_id, ref_id)
        assert torch.equal(got_val, ref_val)
        # the planted structure is real: each row's top ids are distinct and sorted by value
        v = got_val.cpu().numpy()
        assert np.all(np.diff(v, axis=1) <= 0)
