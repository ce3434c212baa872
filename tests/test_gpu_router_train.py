"""GPU parity of the training steps around the routing (moe_route_bwd,
moe_bias_update) against the oracle (oracle.router_train), stage-wise: the
oracle consumes the forward's own logits, expert lists and expert output
rows, so only the router backward's arithmetic is compared.

* dlogits (fp32 on both sides, the GPU's sigmoid in fp32): relative L2 1e-5;
* dx_router, dw_router (bf16 matrix cores, dlogits rounded to bf16): the
  bf16 bar 1e-2;
* the balance loss value: relative 1e-5;
* the bias update: bit for bit.
Reduced batch (3 sequences of 100 tokens, ragged against the 128-wide
tiles) and the full 4096-token DeepSeek-V3-dims batch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from moe_synth import configs, gen
from oracle import router_train as rtr
from tests.gpu_util import dev, device_inputs, host, log, rel_l2

pytestmark = pytest.mark.gpu


def _run(cfg, x_d, wr_d, b_d, w1, w2, w1s, w2s, dout_d, seq_len, alpha):
    ew = moe.ExpertWeights.from_dense(w1, w2, cfg.fmt)
    sw = moe.ExpertWeights.from_dense(w1s, w2s, cfg.fmt) if w1s is not None else None
    fw = moe.MoEForward.for_config(cfg, keep_logits=True)
    fw(x_d, wr_d, b_d, ew, sw)
    rb = moe.RouterBackward(fw, seq_len=seq_len, aux_alpha=alpha)
    rb(dout_d, x_d, wr_d)
    torch.cuda.synchronize()
    return fw, rb


def _check(cfg, fw, rb, x, wr, dout, seq_len, alpha):
    idx = host(fw.topk_idx)
    rm = host(fw.row_map)
    y_sel = host(fw.y_rows[torch.from_numpy(rm.ravel().astype(np.int64)).cuda()]).reshape(
        cfg.T, cfg.k, cfg.H)
    ref = rtr.router_backward(x, wr, host(fw.logits), idx, dout, y_sel, cfg.routed_scale,
                              seq_len=seq_len, aux_alpha=alpha)
    e_dl = rel_l2(host(rb.dlogits), ref["dlogits"])
    e_dx = rel_l2(host(rb.dx), ref["dx"])
    e_dw = rel_l2(host(rb.dw), ref["dw_router"])
    log(f"  dlogits {e_dl:.2e}, dx {e_dx:.2e}, dW_r {e_dw:.2e}")
    assert e_dl < 1e-5 and e_dx < 1e-2 and e_dw < 1e-2
    if alpha:
        got, want = float(host(rb.aux_loss)[0]), float(ref["aux_loss"])
        log(f"  balance loss {got:.7f} (oracle {want:.7f})")
        assert abs(got - want) <= 1e-5 * abs(want)


@pytest.mark.parametrize("alpha", [0.0, 0.01])
def test_router_backward_reduced(gpu_lib, alpha):
    cfg = configs.get("mini_bf16")
    log(f"router backward {cfg.name} alpha={alpha}")
    h, d = device_inputs(cfg)
    g = np.random.default_rng(4)
    dout = gen.round_to_storage(g.standard_normal((cfg.T, cfg.H)), "bf16")
    fw, rb = _run(cfg, d["x"], d["w_router"], d["bias"], d["w1"], d["w2"], d["w1s"], d["w2s"],
                  dev(dout, "bf16"), 100, alpha)
    _check(cfg, fw, rb, h["x"], h["w_router"], dout, 100, alpha)


@pytest.mark.timeout(600)
def test_router_backward_full_size(gpu_lib):
    cfg = configs.get("dsv3_bf16_t4096")
    log(f"router backward {cfg.name} with the balance loss over 2 sequences")
    x, wr, b = gen.host_x(cfg), gen.host_router(cfg), gen.host_bias(cfg)
    wts = gen.device_expert_weights(cfg, "cuda")
    sh = gen.device_shared_weights(cfg, "cuda")
    g = np.random.default_rng(5)
    dout = gen.round_to_storage(g.standard_normal((cfg.T, cfg.H)), "bf16")
    fw, rb = _run(cfg, dev(x, "bf16"), dev(wr, "bf16"), dev(b), wts["w1"], wts["w2"], sh["w1s"],
                  sh["w2s"], dev(dout, "bf16"), 2048, 1e-3)
    del wts, sh
    _check(cfg, fw, rb, x, wr, dout, 2048, 1e-3)


def test_bias_update(gpu_lib):
    cfg = configs.get("mini_bf16")
    h, d = device_inputs(cfg)
    fw = moe.MoEForward.for_config(cfg)
    fw.route(d["x"], d["w_router"], d["bias"])
    fw.permute()
    out = torch.empty_like(d["bias"])
    moe.bias_update(fw, d["bias"], 1e-3, out=out)
    torch.cuda.synchronize()
    want = rtr.bias_update(h["bias"], host(fw.counts), cfg.k, 1e-3)
    assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32))
    # in place
    b2 = d["bias"].clone()
    moe.bias_update(fw, b2, 1e-3)
    torch.cuda.synchronize()
    assert np.array_equal(host(b2).view(np.uint32), want.view(np.uint32))
