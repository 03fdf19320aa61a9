"""GPU checks of the double-buffered adapter slots (oft_slots_switch,
oft_linear_fwd_slots).

The forward on the active slot must equal the plain forward on that slot's
rotation pack bit for bit (the same kernels read the same operands), the
latch must name the slot and version the switch published, and the output
must match the oracle for the adapter in that slot.  A forward captured
once in a HIP graph must follow every later switch: each replay is checked
against an eager forward on the slot the switch made active, with eager
work and synchronisations between the replays.
"""
import numpy as np
import pytest

from oft_inputs import make_dense
from oracle import dense as odense
from tests.helpers import bf16_to_f64, dev, err, host
from tests.test_gpu_dense import SMALL, _wfmt

pytestmark = pytest.mark.gpu
TOL = 2e-2

# one case per forward kernel: copy ring (FP8), register prefetch (fp32 x),
# skinny (fp32 x, few tokens), 256-wide-step decode (INT4, FP4), FP8 decode
CASES = ["fp8_b32_ragged", "int4_f32x_wide", "int4_g32_f32x_b32", "decode_int4_g32", "decode_split_fp8_b16",
         "fp4_decode_g32"]


def _ctx(name):
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = SMALL[name]
    inp = make_dense(cfg, seed=0, with_dy=False)
    # one base layer and input, three adapters (A from the same draw)
    ps = [inp["p"]] + [make_dense(cfg, seed=s, with_dy=False)["p"] for s in (1, 2)]
    xdt = oft.OFT_DT_F32 if cfg.x_dtype == "f32" else oft.OFT_DT_BF16
    c = {
        "cfg": cfg, "inp": inp, "ps": ps,
        "d": oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, xdt, _wfmt(oft, cfg.w_fmt), cfg.g),
        "tdt": torch.float32 if cfg.x_dtype == "f32" else torch.int16,
        "x": dev(inp["x"]), "wc": dev(inp["w_codes"]), "ws": dev(inp["w_scales"]),
        "Rf": torch.empty((cfg.nblk, cfg.b, cfg.b), dtype=torch.float32, device="cuda"),
        "slots": [torch.empty((cfg.nblk, 2, cfg.b, cfg.b), dtype=torch.int16, device="cuda") for _ in range(2)],
        "state": torch.zeros(4, dtype=torch.int32, device="cuda"),
        "latch": torch.full((4,), -1, dtype=torch.int32, device="cuda"),
    }
    return c


def _publish(c, slot, adapter, version):
    """Cayley build of adapter into the slot, then the switch to it."""
    import orthogonal_fine_tuning_amd as oft

    cfg = c["cfg"]
    oft.cayley_build(dev(c["ps"][adapter]), cfg.nblk, cfg.b, c["Rf"], c["slots"][slot])
    oft.oft_slots_switch(c["state"], slot, version)


def _out(c):
    import torch

    return torch.full((c["cfg"].M, c["cfg"].N), -3, dtype=c["tdt"], device="cuda")


def _fwd_slots(c, y):
    import orthogonal_fine_tuning_amd as oft

    oft.oft_linear_fwd_slots(c["d"], c["x"], c["wc"], c["ws"], c["slots"][0], c["slots"][1], c["state"],
                             c["latch"], y)


def _fwd_plain(c, slot):
    import torch
    import orthogonal_fine_tuning_amd as oft

    y = _out(c)
    oft.oft_linear_fwd(c["d"], c["x"], c["wc"], c["ws"], c["slots"][slot], y)
    torch.cuda.synchronize()
    return host(y)


def _oracle_err(c, y, adapter):
    inp = dict(c["inp"])
    inp["p"] = c["ps"][adapter]
    ref = odense.run(inp)["y"]
    got = host(y) if c["cfg"].x_dtype == "f32" else bf16_to_f64(host(y))
    return err(np.asarray(got, dtype=np.float64), ref)


@pytest.mark.parametrize("name", CASES)
def test_slots_forward_follows_the_switch(name):
    import torch

    print(f"[slots] {name}", flush=True)
    c = _ctx(name)
    seen = []
    for slot, adapter, version in [(0, 0, 1), (1, 1, 2), (0, 2, 3), (1, 0, 4)]:
        _publish(c, slot, adapter, version)
        y = _out(c)
        _fwd_slots(c, y)
        torch.cuda.synchronize()
        assert host(c["latch"])[:2].tolist() == [slot, version]
        assert np.array_equal(host(y), _fwd_plain(c, slot))
        e = _oracle_err(c, y, adapter)
        print(f"  slot {slot} adapter {adapter} version {version}: err {e:.2e}", flush=True)
        assert e <= TOL
        seen.append(host(y))
    assert not np.array_equal(seen[0], seen[1])  # the adapters differ, so do the outputs
    assert np.array_equal(seen[0], seen[3])      # adapter 0 again, now from slot 1


def test_slots_zero_tokens_still_latch():
    import torch
    import orthogonal_fine_tuning_amd as oft

    c = _ctx("decode_int4_g32")
    _publish(c, 1, 1, 7)
    d0 = oft.linear_desc(0, c["cfg"].K, c["cfg"].segs, c["cfg"].b, oft.OFT_DT_BF16, oft.OFT_W_INT4, c["cfg"].g)
    oft.oft_linear_fwd_slots(d0, None, None, None, None, None, c["state"], c["latch"], None)
    torch.cuda.synchronize()
    assert host(c["latch"])[:2].tolist() == [1, 7]


@pytest.mark.parametrize("name", ["decode_int4_g32", "fp8_b32_ragged"])
def test_slots_graph_replay_follows_the_switch(name):
    import torch

    print(f"[slots graph] {name}", flush=True)
    c = _ctx(name)
    _publish(c, 0, 0, 1)
    y = _out(c)
    _fwd_slots(c, y)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fwd_slots(c, y)
    torch.cuda.synchronize()
    for slot, adapter, version in [(0, 0, 1), (1, 1, 2), (0, 2, 3), (1, 0, 4)]:
        if version > 1:
            _publish(c, slot, adapter, version)
            torch.cuda.synchronize()
        for rep in range(2):
            c["latch"].fill_(-1)
            g.replay()
            torch.cuda.synchronize()
            assert host(c["latch"])[:2].tolist() == [slot, version], (slot, version, rep)
            assert np.array_equal(host(y), _fwd_plain(c, slot)), (slot, version, rep)
        print(f"  slot {slot} version {version}: two replays match", flush=True)


@pytest.mark.parametrize("name", ["decode_int4_g32", "fp8_b32_ragged"])
def test_slots_two_streams_own_latches(name):
    """Two streams, each with its own latch, run the slot forward at the
    same time, before and after a switch published on a third stream that
    waits for both: each call's output equals the plain forward on the slot
    its own latch names (calls in flight never share a latch)."""
    import torch
    import orthogonal_fine_tuning_amd as oft

    print(f"[slots two streams] {name}", flush=True)
    c = _ctx(name)
    _publish(c, 0, 0, 1)
    _publish(c, 1, 1, 1)  # builds slot 1, publishes it ...
    _publish(c, 0, 0, 2)  # ... then slot 0 again: active slot 0, version 2
    torch.cuda.synchronize()
    want = {0: _fwd_plain(c, 0), 1: _fwd_plain(c, 1)}
    sa, sb, sw = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    latches = [torch.full((4,), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    for rnd, (slot, version) in enumerate([(0, 2), (1, 3)]):
        if rnd == 1:
            # the switch waits for both streams' previous calls, then both wait for it
            ev = [torch.cuda.Event() for _ in range(2)]
            ev[0].record(sa)
            ev[1].record(sb)
            sw.wait_event(ev[0])
            sw.wait_event(ev[1])
            oft.oft_slots_switch(c["state"], slot, version, stream=sw.cuda_stream)
            done = torch.cuda.Event()
            done.record(sw)
            sa.wait_event(done)
            sb.wait_event(done)
        ys = []
        for st, latch in zip((sa, sb), latches):
            y = _out(c)
            oft.oft_linear_fwd_slots(c["d"], c["x"], c["wc"], c["ws"], c["slots"][0], c["slots"][1], c["state"],
                                     latch, y, stream=st.cuda_stream)
            ys.append(y)
        torch.cuda.synchronize()
        for y, latch in zip(ys, latches):
            got = host(latch)[:2].tolist()
            assert got == [slot, version], (rnd, got)
            assert np.array_equal(host(y), want[slot])
