"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any
launch (no GPU is touched by these calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from w8a8_quantized_speculative_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quasar.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(quasar_\w+)\s*\(", text)))


def test_header_declares_the_three_calls_and_diagnostics():
    names = declared_functions()
    for must in ("quasar_quantize_weights", "quasar_w8a8_linear", "quasar_verify_accept",
                 "quasar_quantize_activations", "quasar_w8a8_workspace_bytes",
                 "quasar_accept_workspace_bytes", "quasar_status_string"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (quasar_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    assert set(binding._SIGNATURES) == set(declared_functions())


def test_status_strings(L):
    for code in range(6):
        assert L.quasar_status_string(code).decode().startswith("QUASAR_")
    assert b"UNKNOWN" in L.quasar_status_string(99)
    assert L.quasar_abi_version() == 11


def test_workspace_header_and_init_errors(L):
    hdr = L.quasar_workspace_header_bytes()
    assert hdr == 65536
    # every workspace that carries flags starts with the header
    for M, N, K in [(96, 4096, 12288), (9, 16, 16), (6, 64, 16384)]:
        assert L.quasar_w8a8_workspace_bytes(M, N, K) >= hdr + M * K
    init = L.quasar_workspace_init
    assert init(None, 1 << 20, None) == WORKSPACE
    assert init(FAKE, hdr - 1, None) == WORKSPACE
    assert init(FAKE + 16, 1 << 20, None) == WORKSPACE


def test_workspace_queries_are_pure_host_and_monotone(L):
    assert L.quasar_w8a8_workspace_bytes(0, 100, 64) == 0
    assert L.quasar_w8a8_workspace_bytes(6, 0, 64) == 0
    assert L.quasar_w8a8_workspace_bytes(6, 100, 60) == 0          # K % 16 != 0
    # the one-launch kernel (M <= 8, K <= 12288) needs no workspace
    for M, N, K in [(6, 6144, 4096), (8, 4096, 12288), (1, 16, 16), (6, 151936, 4096)]:
        assert L.quasar_w8a8_workspace_bytes(M, N, K) == 0
    # the wide path stages the quantized activations and INT32 partial sums
    for M, N, K in [(96, 4096, 12288), (9, 16, 16), (128, 151936, 4096), (6, 64, 16384)]:
        b = L.quasar_w8a8_workspace_bytes(M, N, K)
        assert b >= M * K + 4 * M and b % 256 == 0
    assert L.quasar_accept_workspace_bytes(0, 5, 10) == 0
    assert L.quasar_accept_workspace_bytes(1, 5, 151936) > 0
    assert L.quasar_accept_workspace_bytes(1, 64, 10) == 0          # k > QUASAR_MAX_DRAFT


def linear(L, x=FAKE, s=FAKE, wq=FAKE, sw=FAKE, M=16, N=32, K=64, y=FAKE, acc=None, ws=FAKE,
           wsb=1 << 20):
    return L.quasar_w8a8_linear(x, s, wq, sw, M, N, K, y, acc, ws, wsb, None)


def test_linear_argument_errors(L):
    assert linear(L, M=-1) == INVALID
    assert linear(L, K=0) == INVALID
    assert linear(L, K=72) == INVALID                      # not a multiple of 16
    assert linear(L, K=65536 + 16) == UNSUPPORTED
    assert linear(L, M=129) == UNSUPPORTED
    assert linear(L, M=0) == OK and linear(L, N=0) == OK   # empty calls are no-ops
    assert linear(L, x=None) == INVALID
    assert linear(L, y=None) == INVALID
    assert linear(L, x=FAKE + 8) == INVALID                # not 16-byte aligned
    assert linear(L, wq=FAKE + 4) == INVALID
    assert linear(L, sw=FAKE + 2) == INVALID
    assert linear(L, acc=FAKE + 2) == INVALID
    need = L.quasar_w8a8_workspace_bytes(16, 32, 64)
    assert need > 0
    assert linear(L, ws=None) == WORKSPACE
    assert linear(L, wsb=need - 1) == WORKSPACE
    assert linear(L, ws=FAKE + 16) == WORKSPACE            # not 256-byte aligned


def test_quantizer_argument_errors(L):
    qw = L.quasar_quantize_weights
    assert qw(FAKE, FAKE, -1, 64, FAKE, FAKE, None) == INVALID
    assert qw(FAKE, FAKE, 10, 8, FAKE, FAKE, None) == INVALID
    assert qw(FAKE, FAKE, 10, 1 << 17, FAKE, FAKE, None) == UNSUPPORTED
    assert qw(FAKE, FAKE, 0, 64, None, None, None) == OK
    assert qw(None, FAKE, 10, 64, FAKE, FAKE, None) == INVALID
    assert qw(FAKE, FAKE + 4, 10, 64, FAKE, FAKE, None) == INVALID
    qa = L.quasar_quantize_activations
    assert qa(FAKE, FAKE, 3, 64, FAKE, None, None, None) == INVALID
    assert qa(FAKE, FAKE, 3, 64, FAKE, FAKE, FAKE + 4, None) == INVALID
    assert qa(FAKE, FAKE, 0, 64, None, None, None, None) == OK


def accept(L, logits=FAKE, draft=FAKE, B=1, k=5, V=100, T=0.0, u=None, acc=FAKE, nxt=FAKE,
           ws=FAKE, wsb=1 << 20):
    return L.quasar_verify_accept(logits, draft, B, k, V, T, u, acc, nxt, None, None, ws, wsb, None)


def test_accept_argument_errors(L):
    assert accept(L, B=-1) == INVALID
    assert accept(L, V=0) == INVALID
    assert accept(L, k=-1) == INVALID
    assert accept(L, k=64) == UNSUPPORTED
    assert accept(L, T=-1.0) == INVALID
    assert accept(L, T=float("nan")) == INVALID
    assert accept(L, T=float("inf")) == INVALID
    assert accept(L, T=1.0, u=None) == INVALID             # rejection needs uniforms
    assert accept(L, draft=None) == INVALID                # k > 0 needs drafts
    assert accept(L, B=0) == OK
    assert accept(L, logits=None) == INVALID
    assert accept(L, nxt=FAKE + 2) == INVALID
    assert accept(L, ws=None) == WORKSPACE
    assert accept(L, wsb=16) == WORKSPACE


def lm_head_verify(L, x=FAKE, s=FAKE, wq=FAKE, sw=FAKE, B=1, k=5, V=1000, K=64, draft=FAKE,
                   T=0.0, u=None, logits=FAKE, acc=FAKE, nxt=FAKE, ws=FAKE, wsb=1 << 20):
    return L.quasar_lm_head_verify(x, s, wq, sw, B, k, V, K, draft, T, u, logits, acc, nxt, None,
                                   None, ws, wsb, None)


def test_lm_head_verify_argument_errors(L):
    assert lm_head_verify(L, B=-1) == INVALID
    assert lm_head_verify(L, V=0) == INVALID
    assert lm_head_verify(L, K=72) == INVALID
    assert lm_head_verify(L, T=-1.0) == INVALID
    assert lm_head_verify(L, T=float("nan")) == INVALID
    assert lm_head_verify(L, T=1.0, u=None) == INVALID
    assert lm_head_verify(L, draft=None) == INVALID
    assert lm_head_verify(L, x=FAKE + 8) == INVALID
    assert lm_head_verify(L, logits=None) == INVALID
    assert lm_head_verify(L, k=64) == UNSUPPORTED
    assert lm_head_verify(L, B=22, k=5) == UNSUPPORTED       # 132 token rows > 128
    assert lm_head_verify(L, K=65536 + 16) == UNSUPPORTED
    assert lm_head_verify(L, B=0) == OK
    assert lm_head_verify(L, ws=None) == WORKSPACE
    need = L.quasar_lm_head_verify_workspace_bytes(1, 5, 1000, 64)
    assert need > 0 and lm_head_verify(L, wsb=need - 1) == WORKSPACE


def test_lm_head_verify_workspace(L):
    q = L.quasar_lm_head_verify_workspace_bytes
    assert q(0, 5, 1000, 64) == 0 and q(1, 64, 1000, 64) == 0 and q(22, 5, 1000, 64) == 0
    # fused: three [rows][workgroups] arrays of 4-byte partials
    fused = q(1, 5, 151936, 4096)
    assert 3 * 6 * 256 * 4 <= fused <= 3 * 6 * 256 * 4 + 3 * 256
    # fallbacks: the linear's workspace plus the accept step's
    for B, k, V, K in [(3, 5, 20000, 512), (1, 5, 3000, 16384), (1, 1, 600000, 64)]:
        assert q(B, k, V, K) >= L.quasar_w8a8_workspace_bytes(B * (k + 1), V, K) + \
            L.quasar_accept_workspace_bytes(B, k, V)


def test_w4_argument_errors_and_sizes(L):
    qw4 = L.quasar_quantize_weights_w4
    assert qw4(FAKE, FAKE, 10, 64, FAKE, FAKE, None) == INVALID     # K % 128 != 0
    assert qw4(FAKE, FAKE, 10, 8, FAKE, FAKE, None) == INVALID
    assert qw4(FAKE, FAKE, 0, 128, None, None, None) == OK
    assert qw4(FAKE, FAKE + 4, 10, 128, FAKE, FAKE, None) == INVALID
    lin4 = lambda M=6, N=32, K=128, x=FAKE, y=FAKE, ws=None, nb=0: L.quasar_w4a8_linear(
        x, FAKE, FAKE, FAKE, M, N, K, y, None, ws, nb, None)
    assert lin4(K=192) == INVALID
    assert lin4(M=97) == UNSUPPORTED                                # 4-bit weights: M <= 96
    assert lin4(M=129) == UNSUPPORTED
    assert lin4(M=9) == WORKSPACE                                   # the wide kernel needs one
    assert lin4(K=12288 + 128) == WORKSPACE
    need = L.quasar_w4a8_workspace_bytes(9, 32, 128)
    assert need >= L.quasar_workspace_header_bytes()
    assert lin4(M=9, ws=FAKE, nb=need - 256) == WORKSPACE
    assert lin4(M=9, ws=FAKE + 16, nb=need) == WORKSPACE             # not 256-byte aligned
    assert lin4(M=0) == OK and lin4(N=0) == OK
    assert lin4(x=None) == INVALID and lin4(y=FAKE + 1) == INVALID
    ws4 = L.quasar_w4a8_workspace_bytes
    assert ws4(6, 4096, 4096) == 0 and ws4(8, 4096, 12288) == 0     # one launch, no workspace
    assert ws4(48, 4096, 4096) > 0 and ws4(96, 24576, 4096) > 0 and ws4(6, 64, 16384) > 0
    assert ws4(97, 16, 128) == 0 and ws4(48, 16, 192) == 0 and ws4(0, 16, 128) == 0
    assert L.quasar_packed_weight_bytes_w4(4096, 4096) == 4096 * 4096 // 2
    assert L.quasar_packed_weight_bytes_w4(17, 256) == 2 * 2 * 1024
    assert L.quasar_packed_weight_bytes_w4(16, 192) == 0
    name = lambda M, N, K: L.quasar_w4a8_kernel_name(M, N, K).decode()
    assert name(6, 4096, 4096) == "w4a8_linear_fused_kernel<6, 4, 1>"
    assert name(6, 4096, 12288) == "w4a8_linear_fused_kernel<6, 4, 3>"
    assert name(1, 16, 8192) == "w4a8_linear_fused_kernel<2, 4, 2>"
    # wider windows: the wide kernel with 4-bit weights, <token blocks, tiles per group>
    assert name(9, 16, 128) == "w4a8_linear_wide_kernel<1, 1>"
    assert name(48, 4096, 4096) == "w4a8_linear_wide_kernel<3, 1>"
    assert name(96, 4096, 4096) == "w4a8_linear_wide_split_kernel<3, 2>"
    assert name(64, 2048, 4096) == "w4a8_linear_wide_split_kernel<2, 2>"
    assert name(96, 6144, 4096) == "w4a8_linear_wide_split_kernel<3, 3>"   # triples from 96 tokens
    assert name(64, 6144, 4096) == "w4a8_linear_wide_kernel<4, 2>"
    assert name(16, 24576, 4096) == "w4a8_linear_wide_kernel<1, 6>"     # 4-bit: groups of 6 below 48 tokens too
    assert name(96, 24576, 4096) == "w4a8_linear_wide_kernel<6, 6>"
    assert name(6, 64, 16384) == "w4a8_linear_wide_kernel<1, 2>"
    assert name(97, 16, 128) == "" and name(6, 16, 192) == ""


def test_packed_weight_bytes(L):
    assert L.quasar_packed_weight_bytes(4096, 4096) == 4096 * 4096
    assert L.quasar_packed_weight_bytes(17, 80) == 2 * 2 * 1024     # padded to 16 rows x 64 cols
    assert L.quasar_packed_weight_bytes(151936, 4096) == 151936 * 4096
    assert L.quasar_packed_weight_bytes(0, 64) == 0
    assert L.quasar_packed_weight_bytes(16, 72) == 0                # K % 16 != 0


def test_kernel_name_names_the_launch_plan(L):
    name = lambda M, N, K: L.quasar_w8a8_kernel_name(M, N, K).decode()
    # one-launch kernel: <token rows compiled for, streamer wavefronts, phases per streamer>
    assert name(6, 4096, 4096) == "w8a8_linear_fused_kernel<6, 4, 2>"
    assert name(6, 4096, 12288) == "w8a8_linear_fused_kernel<6, 4, 6>"
    assert name(1, 16, 16) == "w8a8_linear_fused_kernel<2, 4, 2>"
    assert name(8, 4096, 8192) == "w8a8_linear_fused_kernel<8, 4, 4>"
    # wider windows (or K > 12288): one launch over ceil(M / 16) token blocks,
    # or half of them per workgroup where two workgroups share each pair of
    # tiles (an even block count from 64 tokens, up to 256 tiles in a multiple
    # of 8 pairs, K <= 8192, or 256 tiles from 96 tokens, or more than
    # 96 x 12288 codes); otherwise
    # <token blocks, tiles per group>, while the code matrix is at most
    # 96 x 12288 bytes: K > 8192 pairs up to 512 tiles; otherwise one tile up to
    # 256 tiles, pairs up to 512, pairs below 1024 tiles up to 64 tokens, pairs
    # up to 2048 tiles up to 32 tokens; groups of 4 tiles beyond
    assert name(48, 4096, 4096) == "w8a8_linear_wide_kernel<3, 1>"
    assert name(96, 4096, 4096) == "w8a8_linear_wide_split_kernel<3, 2>"  # token blocks split in two
    assert name(96, 4096, 12288) == "w8a8_linear_wide_split_kernel<3, 2>"  # split: 256 tiles
    assert name(48, 4096, 12288) == "w8a8_linear_wide_kernel<3, 2>"
    assert name(128, 4096, 12288) == "w8a8_linear_wide_split_kernel<4, 2>"  # beyond 96 x 12288
    assert name(64, 4096, 12288) == "w8a8_linear_wide_kernel<4, 2>"    # no split: K-split pairs
    assert name(96, 2048, 12288) == "w8a8_linear_wide_kernel<6, 2>"    # no split: 128 tiles
    assert name(64, 2048, 4096) == "w8a8_linear_wide_split_kernel<2, 2>"  # split
    assert name(80, 4096, 4096) == "w8a8_linear_wide_kernel<5, 1>"     # odd block count: no split
    assert name(128, 4000, 4096) == "w8a8_linear_wide_kernel<8, 1>"    # 125 pairs: no split
    assert name(96, 6144, 4096) == "w8a8_linear_wide_split_kernel<3, 3>"  # groups of 3 tiles
    assert name(64, 6144, 4096) == "w8a8_linear_wide_split_kernel<2, 3>"
    assert name(96, 6152, 4096) == "w8a8_linear_wide_kernel<6, 2>"        # 129 triples
    assert name(48, 6144, 4096) == "w8a8_linear_wide_kernel<3, 2>"
    assert name(9, 16, 16) == "w8a8_linear_wide_kernel<1, 1>"
    assert name(6, 64, 16384) == "w8a8_linear_wide_kernel<1, 2>"
    assert name(96, 24576, 4096) == "w8a8_linear_wide_kernel<6, 6>"     # groups of 6 tiles
    assert name(48, 151936, 4096) == "w8a8_linear_wide_kernel<3, 6>"
    assert name(96, 151936, 4096) == "w8a8_linear_wide_kernel<6, 6>"
    assert name(128, 151936, 4096) == "w8a8_linear_wide_kernel<8, 4>"
    assert name(48, 12288, 4096) == "w8a8_linear_wide_kernel<3, 2>"     # 768 tiles, <= 64 tokens
    assert name(96, 12288, 4096) == "w8a8_linear_wide_kernel<6, 4>"     # 768 tiles, > 64 tokens
    assert name(64, 16384, 4096) == "w8a8_linear_wide_kernel<4, 4>"     # 1024 tiles
    assert name(32, 16384, 4096) == "w8a8_linear_wide_kernel<2, 2>"     # <= 2048 tiles, <= 32 tokens
    assert name(16, 24576, 4096) == "w8a8_linear_wide_kernel<1, 2>"
    assert name(32, 24576, 4096) == "w8a8_linear_wide_kernel<2, 6>"     # 32 tokens: groups of 6
    assert name(32, 151936, 4096) == "w8a8_linear_wide_kernel<2, 4>"
    assert name(48, 24576, 4096) == "w8a8_linear_wide_kernel<3, 6>"
    assert name(112, 24576, 4096) == "w8a8_linear_wide_kernel<7, 4>"    # 7 blocks: groups of 4
    assert name(16, 49152, 4096) == "w8a8_linear_wide_kernel<1, 4>"     # 3072 tiles
    # invalid or unsupported sizes
    assert name(0, 16, 16) == "" and name(6, 16, 17) == "" and name(129, 16, 16) == ""


def test_stream_copy_argument_errors(L):
    buf = ctypes.create_string_buffer(64)
    base = ctypes.addressof(buf)
    aligned = base + (-base % 16)
    assert L.quasar_stream_copy(None, None, 0, None) == 0              # empty copy is a no-op
    assert L.quasar_stream_copy(None, aligned, 16, None) == 1          # null source
    assert L.quasar_stream_copy(aligned, aligned, 15, None) == 1       # not a multiple of 16
    assert L.quasar_stream_copy(aligned + 1, aligned, 16, None) == 1   # misaligned


# ------------------------------------------------------- decoder steps (host checks)
def test_embed_and_rmsnorm_argument_errors(L):
    emb = lambda tok=FAKE, tab=FAKE, M=6, V=100, H=64, h=FAKE: L.quasar_embed(tok, tab, M, V, H, h, None)
    assert emb(M=0) == OK
    assert emb(M=-1) == INVALID and emb(V=0) == INVALID and emb(H=0) == INVALID
    assert emb(H=65537) == UNSUPPORTED
    assert emb(tok=None) == INVALID and emb(h=FAKE + 2) == INVALID
    rms = lambda h=FAKE, d=None, g=FAKE, M=6, H=64, eps=1e-6, o=FAKE: L.quasar_rmsnorm(
        h, d, g, M, H, eps, o, None)
    assert rms(M=0) == OK
    assert rms(eps=0.0) == INVALID and rms(eps=float("nan")) == INVALID
    assert rms(eps=float("inf")) == INVALID and rms(H=0) == INVALID
    assert rms(h=FAKE + 4) == INVALID and rms(g=FAKE + 8) == INVALID  # 16-byte aligned
    assert rms(o=FAKE + 2) == INVALID and rms(d=FAKE + 4) == INVALID  # 8-byte aligned
    assert rms(g=None) == INVALID and rms(H=65537) == UNSUPPORTED


def test_rope_attention_silu_argument_errors(L):
    def rope(qkv=FAKE, B=1, T=6, Hq=32, Hkv=8, D=128, pos0=10, Lmax=16, base=1e6, eps=1e-6,
             kc=FAKE, vc=FAKE):
        return L.quasar_qk_rope_cache(qkv, FAKE, FAKE, B, T, Hq, Hkv, D, pos0, Lmax, base, eps,
                                      FAKE, kc, vc, None)
    assert rope(B=0) == OK
    assert rope(D=64) == UNSUPPORTED                 # head dim 128 only
    assert rope(Hq=30) == UNSUPPORTED                # Hq % Hkv != 0
    assert rope(pos0=11) == UNSUPPORTED              # pos0 + T > Lmax
    assert rope(base=1.0) == INVALID and rope(pos0=-1) == INVALID and rope(T=0) == INVALID
    assert rope(qkv=None) == INVALID and rope(kc=FAKE + 1) == INVALID

    assert L.quasar_attention_workspace_bytes(1, 6, 32, 8, 2048) > 0
    assert L.quasar_attention_workspace_bytes(0, 6, 32, 8, 2048) == 0
    assert L.quasar_attention_workspace_bytes(1, 6, 32, 5, 2048) == 0  # Hq % Hkv != 0
    need = L.quasar_attention_workspace_bytes(1, 6, 32, 8, 10)

    def attn(q=FAKE, B=1, T=6, Hq=32, Hkv=8, D=128, pos0=10, Lmax=16, ws=FAKE, wsb=None,
             kc=FAKE):
        return L.quasar_attention(q, kc, FAKE, B, T, Hq, Hkv, D, pos0, Lmax, FAKE, ws,
                                  need if wsb is None else wsb, None)
    assert attn(B=0) == OK
    assert attn(D=96) == UNSUPPORTED
    assert attn(T=17) == UNSUPPORTED                 # (Hq / Hkv) * T > 64 rows per KV head
    assert attn(pos0=11) == UNSUPPORTED              # the window passes Lmax
    assert attn(wsb=need - 1) == WORKSPACE and attn(ws=None) == WORKSPACE
    assert attn(ws=FAKE + 16) == WORKSPACE           # 256-byte aligned
    assert attn(q=FAKE + 8) == INVALID and attn(kc=FAKE + 2) == INVALID  # 16-byte aligned
    assert attn(q=None) == INVALID

    silu = lambda gu=FAKE, M=6, I=12288, o=FAKE: L.quasar_silu_mul(gu, M, I, o, None)
    assert silu(M=0) == OK
    assert silu(I=0) == INVALID and silu(M=-1) == INVALID and silu(gu=None) == INVALID
    assert silu(M=65536) == UNSUPPORTED and silu(o=FAKE + 1) == INVALID


def chain_links(n=2, **over):
    """n links of 64 x 64; link i > 0 reads link i - 1's output (x = y_prev)."""
    arr = (binding.ChainLink * n)()
    for i in range(n):
        x = FAKE if i == 0 else FAKE + 0x1000 * i
        arr[i] = binding.ChainLink(x, FAKE, FAKE, FAKE, FAKE + 0x1000 * (i + 1), None, 64, 64, 64,
                                   i - 1, 0)
    for k, v in over.items():
        i, field = k.split("_", 1)
        setattr(arr[int(i[1:])], field, v)
    return arr


def chain(L, links, n=None, dev=FAKE, M=6, ws=FAKE, wsb=1 << 24):
    n = len(links) if n is None else n
    return L.quasar_w8a8_chain(ctypes.cast(links, ctypes.c_void_p), dev, n, M, ws, wsb, None)


def test_chain_argument_errors(L):
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    hdr = L.quasar_workspace_header_bytes()
    lk = chain_links()
    assert L.quasar_w8a8_chain_workspace_bytes(P(lk), 2, 6) == hdr  # the flag header
    assert L.quasar_w8a8_chain_workspace_bytes(P(chain_links(l1_dep=-1)), 2, 6) == hdr
    assert L.quasar_w8a8_chain_workspace_bytes(P(lk), 2, 9) == 0
    assert L.quasar_w8a8_chain_kernel_name(6).decode().startswith("w8a8_chain_kernel<6")
    assert chain(L, chain_links(), n=0) == OK                       # empty chain: no-op
    assert chain(L, chain_links(), M=0) == INVALID
    assert chain(L, chain_links(), M=9) == UNSUPPORTED
    assert chain(L, chain_links(l0_N=40)) == INVALID                 # N % 16 != 0
    assert chain(L, chain_links(l1_K=12304, l1_ldx=12304, l1_dep=-1)) == UNSUPPORTED
    assert chain(L, chain_links(l1_ldx=48)) == INVALID               # ldx < K
    assert chain(L, chain_links(l1_ldx=68, l1_dep=-1)) == INVALID    # ldx % 8 != 0
    assert chain(L, chain_links(l0_dep=0)) == INVALID                # a link cannot wait for itself
    assert chain(L, chain_links(3, l2_dep=0)) == INVALID             # only the previous link
    assert chain(L, chain_links(l1_dep=-2)) == INVALID
    assert chain(L, chain_links(l1_x=FAKE + 0x1000 + 16)) == INVALID  # slice past the row end
    assert chain(L, chain_links(l1_x=FAKE + 0x1000 + 8, l1_K=48)) == INVALID  # col0 % 16 != 0
    assert chain(L, chain_links(l1_ldx=128, l0_N=64)) == INVALID     # ldx != the row length
    assert chain(L, chain_links(l1_flags=2)) == INVALID
    assert chain(L, chain_links(l1_flags=1, l1_acc_out=FAKE)) == INVALID  # SWIGLU without acc
    assert chain(L, chain_links(l0_x=FAKE + 8)) == INVALID
    assert chain(L, chain_links(l0_y=FAKE + 4)) == INVALID
    assert chain(L, chain_links(l1_s=None)) == INVALID
    assert chain(L, chain_links(), dev=None) == INVALID
    assert chain(L, chain_links(), ws=None) == WORKSPACE
    assert chain(L, chain_links(), wsb=hdr - 256) == WORKSPACE
    assert chain(L, chain_links(), n=5000) == UNSUPPORTED


def test_chain_verify_argument_errors(L):
    links = chain_links()
    cv = lambda n=2, B=1, k=5, T=0.0, u=None, draft=FAKE, lk=links: L.quasar_chain_verify(
        ctypes.cast(lk, ctypes.c_void_p), FAKE, n, B, k, draft, T, u, FAKE, FAKE, None, None,
        FAKE, 1 << 24, None)
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert L.quasar_chain_verify_workspace_bytes(P(links), 2, 1, 5) > \
        L.quasar_w8a8_chain_workspace_bytes(P(links), 2, 6)          # + the accept partials
    assert L.quasar_chain_verify_workspace_bytes(P(links), 2, 2, 5) == 0  # 12 rows > 8
    assert cv(n=0) == INVALID
    assert cv(B=2) == UNSUPPORTED
    assert cv(T=-1.0) == INVALID
    assert cv(T=float("nan")) == INVALID
    assert cv(T=1.0, u=None) == INVALID
    assert cv(draft=None) == INVALID
    assert cv(lk=chain_links(l1_flags=1)) == INVALID                 # the head is not gated


def test_noalloc_argument_errors(L):
    na = lambda M=16, N=32, K=64, x=FAKE, y=FAKE: L.quasar_w8a8_linear_noalloc(
        x, FAKE, FAKE, FAKE, M, N, K, y, None, None)
    assert na(M=-1) == INVALID
    assert na(K=72) == INVALID
    assert na(M=0) == OK
    assert na(x=None) == INVALID
    assert na(y=FAKE + 1) == INVALID
    assert na(M=129) == UNSUPPORTED
    # the scratch holds the workspace of M <= 128 at K <= 16384, not more
    assert na(M=128, N=64, K=65536) == UNSUPPORTED
    assert L.quasar_w8a8_workspace_bytes(128, 151936, 16384) <= 12 << 20
