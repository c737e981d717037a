"""Library calls captured in a HIP graph and replayed.

The captured step holds three wide-window linears sharing one workspace with
three different grids (63 workgroups with one tile each, 128 with the token
blocks split, 178 with groups of 6 tiles: the cross-workgroup flags advance by
one per launch, replay or not, on every slot), a one-launch linear, the 4-bit
wide linear, the LM head with the accept step, and a chained layer.  It
is replayed several times with new inputs copied in between, with eager calls
on the same workspaces and synchronizations between the replays; every replay
must give the eager calls' bits, and the wide and one-launch linears the
oracle's.
"""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16
from tests.test_parity_chain import build_chain, layer

pytestmark = pytest.mark.gpu


def lin(M, N, K, key, bits=8):
    x, w, s = synth.linear_case(M, K, N, key)
    wd, sd = dev_bf16(w), dev(s)
    if bits == 8:
        wq, sw = binding.quasar_quantize_weights(wd, sd)
    else:
        wq, sw = binding.quasar_quantize_weights_w4(wd, sd)
    return w, s, sd, wq, sw


def test_calls_replayed_in_a_graph_match_the_eager_calls():
    announce("graph replay")
    binding.device_check()
    Mw, Nw, Kw = 48, 1000, 2048            # wide kernel, one tile per workgroup
    Ms, Ns, Ks = 64, 2048, 1024            # wide kernel, token blocks split
    Mg, Ng, Kg = 48, 17000, 512            # wide kernel, groups of 6 tiles
    Mf, Nf, Kf = 6, 3000, 1024             # one-launch kernel
    M4, N4, K4 = 20, 700, 1024             # 4-bit wide kernel
    B, k, V, Kh = 1, 5, 5000, 1024         # LM head + accept
    ww, sw_, swd, wqw, sww = lin(Mw, Nw, Kw, (120, 0))
    wsp, ssp_, sspd, wqsp, swsp = lin(Ms, Ns, Ks, (120, 5))
    wg6, sg6_, sg6d, wqg6, swg6 = lin(Mg, Ng, Kg, (120, 6))
    wf, sf_, sfd, wqf, swf = lin(Mf, Nf, Kf, (120, 1))
    w4, s4_, s4d, wq4, sw4 = lin(M4, N4, K4, (120, 2), bits=4)
    wh, sh_, shd, wqh, swh = lin(B * (k + 1), V, Kh, (120, 3))
    reps = 3
    xs_w = [synth.activations(Mw, Kw, (121, r)) for r in range(reps)]
    xs_s = [synth.activations(Ms, Ks, (127, r)) for r in range(reps)]
    xs_g = [synth.activations(Mg, Kg, (128, r)) for r in range(reps)]
    xs_f = [synth.activations(Mf, Kf, (122, r)) for r in range(reps)]
    xs_4 = [synth.activations(M4, K4, (123, r)) for r in range(reps)]
    xs_h = [synth.activations(B * (k + 1), Kh, (124, r)) for r in range(reps)]
    drafts = [np.random.default_rng(125 + r).integers(0, V, (B, k)).astype(np.int32)
              for r in range(reps)]

    xw, xf, x4, xh = (dev_bf16(xs_w[0]), dev_bf16(xs_f[0]), dev_bf16(xs_4[0]),
                      dev_bf16(xs_h[0]))
    draft = dev(drafts[0])
    xsp, xg6 = dev_bf16(xs_s[0]), dev_bf16(xs_g[0])
    ws_w = binding.new_workspace(max(binding.workspace_bytes_linear(*shape) for shape in
                                     ((Mw, Nw, Kw), (Ms, Ns, Ks), (Mg, Ng, Kg))))
    ws_4 = binding.new_workspace(binding.workspace_bytes_w4(M4, N4, K4))
    ws_h = binding.new_workspace(binding.workspace_bytes_lm_head_verify(B, k, V, Kh))
    yw = torch.empty((Mw, Nw), dtype=torch.bfloat16, device="cuda")
    aw = torch.empty((Mw, Nw), dtype=torch.int32, device="cuda")
    ysp = torch.empty((Ms, Ns), dtype=torch.bfloat16, device="cuda")
    yg6 = torch.empty((Mg, Ng), dtype=torch.bfloat16, device="cuda")
    yf = torch.empty((Mf, Nf), dtype=torch.bfloat16, device="cuda")
    af = torch.empty((Mf, Nf), dtype=torch.int32, device="cuda")
    y4 = torch.empty((M4, N4), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((B, k + 1, V), dtype=torch.bfloat16, device="cuda")
    acc_len = torch.empty((B,), dtype=torch.int32, device="cuda")
    nxt = torch.empty((B,), dtype=torch.int32, device="cuda")
    Mc = 6
    layers = [layer(1024, 1024, 256, 1536, (126, 0))]
    xc = dev_bf16(synth.activations(Mc, 1024, (126, 9)))
    ch, recs = build_chain(Mc, layers, xc)

    def step():
        binding.quasar_w8a8_linear(xw, swd, wqw, sww, out=yw, acc_out=aw, workspace=ws_w)
        binding.quasar_w8a8_linear(xsp, sspd, wqsp, swsp, out=ysp, workspace=ws_w)
        binding.quasar_w8a8_linear(xg6, sg6d, wqg6, swg6, out=yg6, workspace=ws_w)
        binding.quasar_w8a8_linear(xf, sfd, wqf, swf, out=yf, acc_out=af)
        binding.quasar_w4a8_linear(x4, s4d, wq4, sw4, out=y4, workspace=ws_4)
        binding.quasar_lm_head_verify(xh, shd, wqh, swh, B, draft, logits=logits,
                                      workspace=ws_h, accept_len=acc_len, next_token=nxt)
        ch.run()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # prime outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    outs = lambda: [t.clone() for t in (yw, aw, yf, af, y4, logits, acc_len, nxt, ysp, yg6)] + \
        [r[3].clone() for r in recs]
    for r in range(reps):
        xw.copy_(dev_bf16(xs_w[r]))
        xsp.copy_(dev_bf16(xs_s[r]))
        xg6.copy_(dev_bf16(xs_g[r]))
        xf.copy_(dev_bf16(xs_f[r]))
        x4.copy_(dev_bf16(xs_4[r]))
        xh.copy_(dev_bf16(xs_h[r]))
        draft.copy_(dev(drafts[r]))
        for t in (yw, aw, yf, af, y4, logits, ysp, yg6):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs()
        # the same calls eagerly, on the same workspaces
        step()
        torch.cuda.synchronize()
        want = outs()
        for i, (g, e) in enumerate(zip(got, want)):
            assert torch.equal(g.view(torch.uint8) if g.dtype == torch.bfloat16 else g,
                               e.view(torch.uint8) if e.dtype == torch.bfloat16 else e), (r, i)
        ref = orc.w8a8_linear_rows(xs_w[r], sw_, ww)
        assert np.array_equal(host(got[1]), ref["acc"].astype(np.int32))
        assert np.array_equal(host_bf16(got[0]), ref["y"])
        assert np.array_equal(host_bf16(got[8]), orc.w8a8_linear_rows(xs_s[r], ssp_, wsp)["y"])
        assert np.array_equal(host_bf16(got[9]), orc.w8a8_linear_rows(xs_g[r], sg6_, wg6)["y"])
        ref = orc.w8a8_linear_rows(xs_f[r], sf_, wf)
        assert np.array_equal(host(got[3]), ref["acc"].astype(np.int32))
        assert np.array_equal(host_bf16(got[2]), ref["y"])
        ref = orc.w4a8_linear_rows(xs_4[r], s4_, w4)
        assert np.array_equal(host_bf16(got[4]), ref["y"])
        lg = orc.w8a8_linear_rows(xs_h[r], sh_, wh)["y"].reshape(B, k + 1, V)
        assert np.array_equal(host_bf16(got[5]).reshape(B, k + 1, V), lg)
        L_ref, n_ref, _ = orc.greedy_accept(lg, drafts[r])
        assert np.array_equal(host(got[6]), L_ref) and np.array_equal(host(got[7]), n_ref)
    assert binding.device_check() == (binding.QUASAR_OK, 0)
    del graph
