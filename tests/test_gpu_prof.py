"""The library's opt-in kernel timing: records per step of work, on the
launch stream, in launch order; nothing recorded while it is off."""
import numpy as np
import pytest

from oft_inputs import CONFIGS, make_dense, make_moe
from tests.helpers import dev

pytestmark = pytest.mark.gpu


def test_prof_records_dense_and_moe_steps():
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = CONFIGS["tiny_qkv"].with_(x_dtype="bf16", M=300)
    inp = make_dense(cfg, seed=0)
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, oft.OFT_DT_BF16, oft.OFT_W_INT4, cfg.g)
    Rf = torch.empty((cfg.nblk, cfg.b, cfg.b), dtype=torch.float32, device="cuda")
    Rops = torch.empty((cfg.nblk, 2, cfg.b, cfg.b), dtype=torch.int16, device="cuda")
    x, wc, ws, dy = dev(inp["x"]), dev(inp["w_codes"]), dev(inp["w_scales"]), dev(inp["dy"])
    y = torch.empty((cfg.M, cfg.N), dtype=torch.int16, device="cuda")
    dx = torch.empty((cfg.M, cfg.K), dtype=torch.int16, device="cuda")
    dq = torch.empty((cfg.nblk, cfg.npair), dtype=torch.float32, device="cuda")
    nb = oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD)
    work = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")

    def step():
        oft.cayley_build(dev(inp["p"]), cfg.nblk, cfg.b, Rf, Rops)
        oft.oft_linear_fwd(d, x, wc, ws, Rops, y)
        oft.oft_linear_bwd(d, dy, y, wc, ws, Rf, Rops, dx, dq, work, nb)

    step()
    torch.cuda.synchronize()
    oft.prof_enable(False)
    assert oft.prof_records() == []
    oft.prof_enable(True)
    step()
    step()
    torch.cuda.synchronize()
    oft.prof_enable(False)
    recs = oft.prof_records()
    names = [n for n, _ in recs]
    print(recs, flush=True)
    assert names[:2] == ["cayley", "dense.fwd"] and names.count("dense.fwd") == 2
    assert "dense.dq" in names and "dense.dx" in names
    assert all(ms > 0.0 for _, ms in recs)
    step()  # off again: nothing more is recorded
    torch.cuda.synchronize()
    assert len(oft.prof_records()) == len(recs)

    mcfg = CONFIGS["moe_30b_a3b"].with_(T=256, E=8)
    minp = make_moe(mcfg, seed=0)
    md = oft.moe_desc(mcfg.T, mcfg.E, mcfg.k, mcfg.H, mcfg.I, mcfg.g, mcfg.b, mcfg.chunk)
    P = mcfg.T * mcfg.k
    i32 = dict(dtype=torch.int32, device="cuda")
    rtt = dict(topk_idx=torch.empty((mcfg.T, mcfg.k), **i32),
               topk_w=torch.empty((mcfg.T, mcfg.k), dtype=torch.float32, device="cuda"),
               counts=torch.empty(mcfg.E, **i32), offsets=torch.empty(mcfg.E + 1, **i32),
               perm=torch.empty(P, **i32), inv_perm=torch.empty(P, **i32), active=torch.empty(mcfg.E, **i32),
               n_active=torch.empty(4, **i32), chunk_of_expert=torch.empty(mcfg.E, **i32))
    rt = oft.moe_routing(**rtt)
    mRf = torch.empty((mcfg.E, mcfg.nblk_e, mcfg.b, mcfg.b), dtype=torch.float32, device="cuda")
    mRops = torch.empty((mcfg.E, mcfg.nblk_e, 2, mcfg.b, mcfg.b), dtype=torch.int16, device="cuda")
    oft.cayley_build(dev(minp["p"]), mcfg.E * mcfg.nblk_e, mcfg.b, mRf, mRops)
    W = {n: dev(minp[n]) for n in ("wgu_codes", "wgu_scales", "wd_codes", "wd_scales")}
    hs = torch.empty((P, 2 * mcfg.I), dtype=torch.int16, device="cuda")
    my = torch.empty((mcfg.T, mcfg.H), dtype=torch.int16, device="cuda")
    mdx = torch.empty((mcfg.T, mcfg.H), dtype=torch.int16, device="cuda")
    mdq = torch.empty((mcfg.E, mcfg.nblk_e, mcfg.npair), dtype=torch.float32, device="cuda")
    mdw = torch.empty((mcfg.T, mcfg.k), dtype=torch.float32, device="cuda")
    nbf = oft.oft_moe_workspace_bytes(md, oft.OFT_PASS_FWD)
    nbb = oft.oft_moe_workspace_bytes(md, oft.OFT_PASS_BWD)
    wsf = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(nbb, dtype=torch.uint8, device="cuda")
    oft.prof_enable(True)
    oft.oft_moe_grouped_fwd(md, dev(minp["x"]), dev(minp["logits"]), W["wgu_codes"], W["wgu_scales"],
                            W["wd_codes"], W["wd_scales"], mRops, rt, hs, my, wsf, nbf)
    oft.oft_moe_grouped_bwd(md, dev(minp["dy"]), rt, hs, W["wgu_codes"], W["wgu_scales"], W["wd_codes"],
                            W["wd_scales"], mRf, mRops, mdx, mdq, mdw, wsb, nbb)
    torch.cuda.synchronize()
    oft.prof_enable(False)
    names = [n for n, _ in oft.prof_records()]
    print(names, flush=True)
    assert names == ["moe.route", "moe.gateup", "moe.down", "moe.combine", "moe.worklist", "moe.dA",
                     "moe.dw_reduce", "moe.dq", "moe.dX", "moe.unpermute"]
