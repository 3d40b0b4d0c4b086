"""Two handles of different shapes driven at the same time on two streams,
their calls interleaved on the host: layout, FP8 or bf16 dispatch and combine
on each, every result compared with the oracle.  The library keeps no state
outside a handle (no device globals, no shared workspace), so the two must
not disturb each other."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import say, dev, to_dev_bf16, bits_of, ulp_diff, compare_layout
from synth import Config, generate, bf16_from_f32

pytestmark = pytest.mark.gpu


def test_two_handles_on_two_streams():
    import combine_ep_layout_amd as ep
    cfgs = [Config("a", 3000, 1024, 8, 64, 64, 64, fp8=True),
            Config("b", 1700, 768, 4, 24, 24, 32)]
    say("[two handles] 3000 tokens FP8 top-8 / 1700 tokens bf16 top-4, two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]       # default priority
    hs, ds, Ls, pools, ys, eos, epochs = [], [], [], [], [], [], []
    for i, cfg in enumerate(cfgs):
        d = generate(cfg, 20 + i)
        hs.append(ep.EpHandle(cfg.tokens, cfg.top_k, cfg.num_experts, cfg.block_m))
        ds.append(d)
        Ls.append(oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m))
        rng = np.random.default_rng(30 + i)
        eo = bf16_from_f32(rng.standard_normal((hs[i].capacity_rows, cfg.hidden), dtype=np.float32))
        eos.append(eo)
    torch.cuda.synchronize()
    dev_in = [(torch.from_numpy(d["topk_idx"]).to(dev()), torch.from_numpy(d["topk_weights"]).to(dev()),
               to_dev_bf16(d["x"]), to_dev_bf16(eo)) for d, eo in zip(ds, eos)]
    torch.cuda.synchronize()
    # interleave: layout a, layout b, dispatch a, dispatch b, combine a, combine b
    for i in range(2):
        epochs.append(hs[i].layout(dev_in[i][0], dev_in[i][1], stream=streams[i]))
    for i, cfg in enumerate(cfgs):
        pool, scales = hs[i].new_pool(cfg.hidden, fp8=cfg.fp8)
        hs[i].dispatch(dev_in[i][2], pool, scales, fp8=cfg.fp8, stream=streams[i])
        pools.append((pool, scales))
    for i in range(2):
        ys.append(hs[i].combine(epochs[i], dev_in[i][3], stream=streams[i]))
    torch.cuda.synchronize()
    for i, cfg in enumerate(cfgs):
        compare_layout(hs[i], Ls[i])
        recv = Ls[i]["pool_recv_token"]
        real = recv >= 0
        pool, scales = pools[i]
        if cfg.fp8:
            op, osc = oracle.dispatch_fp8(ds[i]["x"], recv)
            assert np.array_equal(pool.cpu().numpy()[real], op[real])
            assert np.array_equal(scales.cpu().numpy()[real], osc[real])
        else:
            op = oracle.dispatch_bf16(ds[i]["x"], recv)
            assert np.array_equal(bits_of(pool)[real], op[real])
        y_or = oracle.combine(eos[i], Ls[i]["slot_to_pool_row"], ds[i]["topk_weights"])
        assert ulp_diff(bits_of(ys[i]), y_or).max(initial=0) <= 1
        assert hs[i].sync_status() == ep.EP_OK
        say(f"  handle {cfg.name}: layout, dispatch and combine match")
    for h in hs:
        h.close()
