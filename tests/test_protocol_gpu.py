"""The cross-workgroup protocol of the persistent kernels, on the GPU.

* Every bounded wait that gives up is reported: with the forced-expiry hook on
  (wait targets the kernels can never reach, a short spin bound; every kernel
  still runs to its end and stays inside its buffers), the next
  quasar_device_check returns QUASAR_ERR_INCOMPLETE with the kinds of wait
  that gave up.  With the hook off, the same workspace gives oracle-exact
  results again and the check is clean: the flag header stays consistent
  through launches whose waits gave up.
* Calls on two streams with two workspaces do not interfere through memory:
  two wide-window linears issued back to back on two streams either both
  match the oracle with a clean check, or -- when their grids could not be
  resident at once -- the check reports it.
"""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16

pytestmark = pytest.mark.gpu


def case(M, N, K, key):
    x, w, s = synth.linear_case(M, K, N, key)
    wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
    return x, w, s, wq, sw


def run(x, s, wq, sw, N, ws=None):
    acc = torch.empty((x.shape[0], N), dtype=torch.int32, device="cuda")
    y = binding.quasar_w8a8_linear(dev_bf16(x), dev(s), wq, sw, acc_out=acc, workspace=ws)
    return y, acc


def exact(x, s, w, y, acc):
    ref = orc.w8a8_linear_rows(x, s, w)
    return (np.array_equal(host(acc), ref["acc"].astype(np.int32))
            and np.array_equal(host_bf16(y), ref["y"]))


def test_forced_wait_expiry_is_reported_and_the_workspace_recovers():
    binding.device_check()  # start from a clean word
    wide = case(48, 520, 1024, (91, 0))
    small = case(6, 512, 1024, (91, 1))
    ws = binding.new_workspace(binding.workspace_bytes_linear(48, 520, 1024))
    announce("forced expiry: wide 48x520x1024, fused 6x512x1024")
    binding.force_wait_expiry(True)
    try:
        run(*[wide[i] for i in (0, 2, 3, 4)], 520, ws)
        run(*[small[i] for i in (0, 2, 3, 4)], 512)
    finally:
        binding.force_wait_expiry(False)
    st, bits = binding.device_check()
    assert st == binding.QUASAR_ERR_INCOMPLETE
    assert bits & binding.QUASAR_WAIT_ROWS and bits & binding.QUASAR_WAIT_LDS, bits
    # the same workspace, hook off: exact again, and nothing reported
    announce("after forced expiry: the same calls, hook off")
    for _ in range(2):
        x, w, s, wq, sw = wide
        y, acc = run(x, s, wq, sw, 520, ws)
        torch.cuda.synchronize()
        assert exact(x, s, w, y, acc)
        x, w, s, wq, sw = small
        y, acc = run(x, s, wq, sw, 512)
        torch.cuda.synchronize()
        assert exact(x, s, w, y, acc)
    assert binding.device_check() == (binding.QUASAR_OK, 0)


def test_forced_expiry_with_4bit_weights_is_reported_and_the_workspace_recovers():
    """The wide kernel's 4-bit instantiation follows the same protocol."""
    binding.device_check()
    M, N, K = 40, 700, 1024
    x, w, s = synth.linear_case(M, K, N, (94, 0))
    wq4, sw4 = binding.quasar_quantize_weights_w4(dev_bf16(w), dev(s))
    ws = binding.new_workspace(binding.workspace_bytes_w4(M, N, K))
    xd, sd = dev_bf16(x), dev(s)
    announce("forced expiry: wide 4-bit 40x700x1024")
    binding.force_wait_expiry(True)
    try:
        binding.quasar_w4a8_linear(xd, sd, wq4, sw4, workspace=ws)
    finally:
        binding.force_wait_expiry(False)
    st, bits = binding.device_check()
    assert st == binding.QUASAR_ERR_INCOMPLETE and bits & binding.QUASAR_WAIT_ROWS, bits
    ref = orc.w4a8_linear_rows(x, s, w)
    for _ in range(2):
        acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
        y = binding.quasar_w4a8_linear(xd, sd, wq4, sw4, acc_out=acc, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), ref["acc"].astype(np.int32))
        assert np.array_equal(host_bf16(y), ref["y"])
    assert binding.device_check() == (binding.QUASAR_OK, 0)


def test_launches_of_different_grids_share_one_workspace():
    """Wide launches whose grids differ (one workgroup per group of weight
    tiles where the groups fit: 100, 192 or 32 workgroups here; two per pair
    of tiles with the token blocks split: 128 or 256; else one per compute
    unit), back to back on ONE workspace, a small grid first and a full
    one after it, in two rounds: each matches the oracle and no wait gives up.
    A launch advances the flag slots beyond its own grid too, so the next
    launch with a larger grid finds every slot counting the same launches."""
    cases = [(96, 1600, 4096), (48, 4096, 4096), (48, 6144, 4096), (16, 500, 4096),
             (64, 2048, 4096), (20, 1000, 8208), (48, 3072, 4096), (96, 4096, 4096)]
    ws = binding.new_workspace(max(binding.workspace_bytes_linear(M, N, K) for M, N, K in cases))
    data = [case(M, N, K, (17, i)) for i, (M, N, K) in enumerate(cases)]
    assert binding.device_check() == (0, 0)
    for rnd in range(2):
        outs = []
        for (M, N, K), (x, w, s, wq, sw) in zip(cases, data):
            announce("protocol_mixed_grids", rnd, M, N, K)
            outs.append(run(x, s, wq, sw, N, ws))
        torch.cuda.synchronize()
        assert binding.device_check() == (0, 0), f"a wait gave up in round {rnd}"
        for (x, w, s, wq, sw), (y, acc) in zip(data, outs):
            assert exact(x, s, w, y, acc)


def test_workspace_init_resets_a_junk_header():
    """quasar_workspace_init zeroes the flag header with a kernel: a workspace
    whose header holds junk gives exact results after it."""
    binding.device_check()
    x, w, s, wq, sw = case(33, 300, 2048, (92, 0))
    ws = binding.new_workspace(binding.workspace_bytes_linear(33, 300, 2048))
    hdr = binding.lib().quasar_workspace_header_bytes()
    ws[:hdr] = (torch.arange(hdr, device="cuda", dtype=torch.int32) * 37 % 251).to(torch.uint8)
    binding.workspace_init(ws)
    torch.cuda.synchronize()
    assert int(ws[:hdr].count_nonzero()) == 0
    announce("after quasar_workspace_init, 33x300x2048")
    y, acc = run(x, s, wq, sw, 300, ws)
    torch.cuda.synchronize()
    assert exact(x, s, w, y, acc)
    assert binding.device_check() == (binding.QUASAR_OK, 0)


def test_two_streams_two_workspaces():
    binding.device_check()
    a = case(96, 4096, 4096, (93, 0))
    b = case(48, 6144, 4096, (93, 1))
    ws_a = binding.new_workspace(binding.workspace_bytes_linear(96, 4096, 4096))
    ws_b = binding.new_workspace(binding.workspace_bytes_linear(48, 6144, 4096))
    xa, xb = dev_bf16(a[0]), dev_bf16(b[0])
    sa, sb = dev(a[2]), dev(b[2])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    announce("two streams: wide 96x4096x4096 and 48x6144x4096")
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            acc_a = torch.empty((96, 4096), dtype=torch.int32, device="cuda")
            ya = binding.quasar_w8a8_linear(xa, sa, a[3], a[4], acc_out=acc_a, workspace=ws_a)
        with torch.cuda.stream(s2):
            acc_b = torch.empty((48, 6144), dtype=torch.int32, device="cuda")
            yb = binding.quasar_w8a8_linear(xb, sb, b[3], b[4], acc_out=acc_b, workspace=ws_b)
        outs.append((ya, acc_a, yb, acc_b))
    torch.cuda.synchronize()
    st, bits = binding.device_check()
    if st == binding.QUASAR_ERR_INCOMPLETE:
        print(f"[protocol] the two grids could not be resident at once: reported, bits={bits}")
        return
    assert st == binding.QUASAR_OK
    for ya, acc_a, yb, acc_b in outs:
        assert exact(a[0], a[2], a[1], ya, acc_a)
        assert exact(b[0], b[2], b[1], yb, acc_b)
