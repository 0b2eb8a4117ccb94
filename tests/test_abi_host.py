"""C ABI checks that need no GPU: symbols, workspace layout, host-side validation.

The validation tests pass fake, never-dereferenced device addresses.  Each of
them expects the call to be rejected on the host; if a check were missing,
the call would go on to launch kernels on those addresses.  So they run only
in a child process in which no GPU is visible (``test_fake_address_calls``
starts it; there a call that wrongly passes its checks fails to find a device
and returns MOE_FFN_ERR_HIP), never in a process that can reach a GPU.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

import routed_expert_ffn_topk_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")

A = 0x7f0000000000  # fake, 256-byte aligned device address

CHILD_ENV = "MOE_FFN_ABI_NO_GPU_CHILD"
IN_CHILD = os.environ.get(CHILD_ENV) == "1"
# fake-address tests: only in the child, and only if it really sees no GPU
# (torch.cuda.device_count() counts devices without initialising one)
fake = pytest.mark.skipif(not IN_CHILD or torch.cuda.device_count() > 0,
                          reason="fake device addresses: run by test_fake_address_calls "
                                 "in a child process with no visible GPU")


@pytest.mark.skipif(IN_CHILD, reason="this is the child")
def test_fake_address_calls():
    """Run this file's fake-address tests in a child process that sees no GPU."""
    env = dict(os.environ, **{CHILD_ENV: "1", "HIP_VISIBLE_DEVICES": "-1",
                              "CUDA_VISIBLE_DEVICES": "-1", "ROCR_VISIBLE_DEVICES": "-1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-rs", os.path.abspath(__file__)],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout[-6000:] + r.stderr[-2000:]
    assert r.returncode == 0, out
    # in the child only this launcher itself is skipped
    assert "1 skipped" in out.splitlines()[-1], "fake-address tests skipped in the child:\n" + out


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moe_[a-z0-9_]+)\s*\(",
                      text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"moe_ffn_forward", "moe_ffn_forward_int8", "moe_ffn_forward_logits", "moe_route_topk",
            "moe_ffn_workspace_bytes", "moe_ffn_workspace_layout", "moe_ffn_check_status",
            "moe_ffn_status_string"} <= set(names)
    assert "moe_ffn_device_check" in names
    here = os.path.dirname(moe.__file__)
    for path in (os.path.join(here, "libmoe_ffn.so"), os.path.join(here, "libmoe_ffn_debug.so")):
        L = ctypes.CDLL(path)
        for n in names:
            assert hasattr(L, n), (path, n)


def test_status_strings():
    for code in range(-7, 1):
        s = moe.moe_ffn_status_string(code)
        assert s and s != "unknown status"
    assert moe.moe_ffn_status_string(-99) == "unknown status"


def test_workspace_layout_regions_fit_and_align():
    T, H, I, E, k = 16, 7168, 2048, 256, 8
    L = moe.moe_ffn_workspace_layout(T, H, I, E, k)
    regions = [("meta", 8 * 4), ("counts", E * 4), ("offsets", (E + 1) * 4),
               ("active", E * 4), ("large", E * 4), ("sorted_slot", T * k * 4),
               ("h", T * k * I * 2),
               ("y", L["y_parts"] * T * k * H * 4)]
    end = 0
    for name, size in regions:
        assert L[name] % 256 == 0
        assert L[name] >= end
        end = L[name] + size
    assert L["total_bytes"] >= end and L["total_bytes"] % 256 == 0
    assert moe.moe_ffn_workspace_bytes(T, H, I, E, k) == L["total_bytes"]


def test_down_k_parts():
    """y holds one plane per K part of the tiled down product: one for batches
    of at most 64 tokens (no tiled product) and for shapes with many tiles
    (Qwen3-235B, DeepSeek-V3 at 2048 / 4096 tokens), more for few long tiles
    (Mixtral-8x7B prefill); the tiled parity cases run 1, 2 and 4 parts."""
    parts = lambda *a: moe.moe_ffn_workspace_layout(*a)["y_parts"]  # noqa: E731
    assert parts(64, 4096, 14336, 8, 2) == 1
    assert parts(2048, 4096, 1536, 128, 8) == 1
    assert parts(4096, 7168, 2048, 256, 8) == 1
    assert parts(2048, 4096, 14336, 8, 2) == 4
    assert parts(512, 4096, 14336, 8, 2) == 2
    assert {parts(129, 32, 32, 1, 1), parts(1000, 96, 160, 2, 1),
            parts(400, 64, 1024, 2, 2)} == {1, 2, 4}
    # never more parts than K stages of 32
    assert parts(65, 4096, 32, 8, 2) == 1 and parts(65, 4096, 64, 8, 2) <= 2


@pytest.mark.parametrize("args", [(-1, 64, 64, 8, 2), (4, 0, 64, 8, 2), (4, 64, 64, 0, 1),
                                  (4, 64, 64, 8, 9), (4, 64, 64, 2000, 2), (4, 64, 64, 8, 0)])
def test_workspace_bytes_rejects_bad_shapes(args):
    assert moe.moe_ffn_workspace_bytes(*args) == 0
    with pytest.raises(moe.MoeFfnError):
        moe.moe_ffn_workspace_layout(*args)


def fwd(**kw):
    a = dict(x=A, ids=A + 0x100000, w=A + 0x200000, wg=A + 0x1000000, wu=A + 0x2000000,
             wd=A + 0x3000000, out=A + 0x300000, T=4, H=64, I=96, E=8, k=2,
             ws=A + 0x4000000, wsb=1 << 30)
    a.update(kw)
    return moe.lib().moe_ffn_forward(a["x"], a["ids"], a["w"], a["wg"], a["wu"], a["wd"],
                                     a["out"], a["T"], a["H"], a["I"], a["E"], a["k"],
                                     a["ws"], a["wsb"], None)


@fake
def test_forward_host_validation():
    assert fwd(T=0) == moe.MOE_FFN_OK                       # empty batch: no-op
    assert fwd(H=48) == moe.MOE_FFN_ERR_BAD_SHAPE            # H not a multiple of 32
    assert fwd(I=100) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd(k=9) == moe.MOE_FFN_ERR_BAD_SHAPE             # top_k > E
    assert fwd(E=0) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd(T=-1) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd(x=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert fwd(wd=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert fwd(ws=None) == moe.MOE_FFN_ERR_WORKSPACE
    assert fwd(wsb=128) == moe.MOE_FFN_ERR_WORKSPACE
    assert fwd(x=A + 8) == moe.MOE_FFN_ERR_MISALIGNED
    assert fwd(wg=A + 0x1000000 + 2) == moe.MOE_FFN_ERR_MISALIGNED
    assert fwd(ws=A + 0x4000000 + 16) == moe.MOE_FFN_ERR_MISALIGNED
    assert fwd(out=A + 64) == moe.MOE_FFN_ERR_ALIAS          # out overlaps x
    assert fwd(ws=A + 0x300000 - 256) == moe.MOE_FFN_ERR_ALIAS  # workspace overlaps out


def fwd_logits(**kw):
    a = dict(x=A, lg=A + 0x500000, ids=A + 0x100000, w=A + 0x200000, wg=A + 0x1000000,
             wu=A + 0x2000000, wd=A + 0x3000000, out=A + 0x300000, T=4, H=64, I=96, E=8, k=2,
             ws=A + 0x4000000, wsb=1 << 30)
    a.update(kw)
    return moe.lib().moe_ffn_forward_logits(a["x"], a["lg"], a["ids"], a["w"], a["wg"], a["wu"],
                                            a["wd"], a["out"], a["T"], a["H"], a["I"], a["E"],
                                            a["k"], a["ws"], a["wsb"], None)


def fwd_noalloc(**kw):
    a = dict(x=A, ids=A + 0x100000, w=A + 0x200000, wg=A + 0x1000000, wu=A + 0x2000000,
             wd=A + 0x3000000, out=A + 0x300000, T=4, H=64, I=96, E=8, k=2)
    a.update(kw)
    return moe.lib().moe_ffn_forward_noalloc(a["x"], a["ids"], a["w"], a["wg"], a["wu"],
                                             a["wd"], a["out"], a["T"], a["H"], a["I"], a["E"],
                                             a["k"], None)


@fake
def test_forward_noalloc_host_validation():
    """The no-allocation entry point refuses sizes whose workspace exceeds the
    array it holds (before any device call), and otherwise checks as
    moe_ffn_forward does."""
    big = dict(T=4096, H=4096, I=14336, E=8, k=2)
    assert moe.moe_ffn_workspace_bytes(4096, 4096, 14336, 8, 2) > moe.MOE_FFN_NOALLOC_WORKSPACE_BYTES
    assert fwd_noalloc(**big) == moe.MOE_FFN_ERR_WORKSPACE
    assert fwd_noalloc(T=0) == moe.MOE_FFN_OK
    assert fwd_noalloc(H=48) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd_noalloc(k=9) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd_noalloc(x=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert fwd_noalloc(wd=None) == moe.MOE_FFN_ERR_NULL_ARG


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    assert "#define MOE_FFN_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)" in text
    assert moe.MOE_FFN_NOALLOC_WORKSPACE_BYTES == 32 << 20
    # decode-sized batches of every workload shape fit
    for T, H, I, E, k in [(64, 4096, 14336, 8, 2), (16, 7168, 2048, 256, 8),
                          (16, 6144, 16384, 8, 2), (16, 4096, 1536, 128, 8)]:
        assert moe.moe_ffn_workspace_bytes(T, H, I, E, k) <= moe.MOE_FFN_NOALLOC_WORKSPACE_BYTES


@fake
def test_forward_logits_host_validation():
    assert fwd_logits(T=0) == moe.MOE_FFN_OK
    assert fwd_logits(k=65, E=128) == moe.MOE_FFN_ERR_BAD_SHAPE    # router handles k <= 64
    assert fwd_logits(k=9) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd_logits(H=48) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert fwd_logits(lg=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert fwd_logits(ids=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert fwd_logits(wu=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert fwd_logits(lg=A + 0x500002) == moe.MOE_FFN_ERR_MISALIGNED
    assert fwd_logits(ids=A + 0x100002) == moe.MOE_FFN_ERR_MISALIGNED
    # written routing outputs may not overlap each other, logits, x, out or the workspace
    assert fwd_logits(w=A + 0x100004) == moe.MOE_FFN_ERR_ALIAS
    assert fwd_logits(ids=A + 0x500010) == moe.MOE_FFN_ERR_ALIAS
    assert fwd_logits(w=A + 0x40) == moe.MOE_FFN_ERR_ALIAS
    assert fwd_logits(ids=A + 0x300010) == moe.MOE_FFN_ERR_ALIAS
    assert fwd_logits(w=A + 0x4000100) == moe.MOE_FFN_ERR_ALIAS
    assert fwd_logits(lg=A + 0x300000 - 16) == moe.MOE_FFN_ERR_ALIAS
    assert fwd_logits(out=A + 64) == moe.MOE_FFN_ERR_ALIAS


@fake
def test_forward_int8_requires_group_multiples():
    L = moe.lib()
    rc = L.moe_ffn_forward_int8(A, A + 0x100000, A + 0x200000, A + 0x1000000, A + 0x1800000,
                                A + 0x2000000, A + 0x2800000, A + 0x3000000, A + 0x3800000, 128,
                                A + 0x300000, 4, 96, 256, 8, 2, A + 0x4000000, 1 << 30, None)
    assert rc == moe.MOE_FFN_ERR_BAD_SHAPE
    rc = L.moe_ffn_forward_int8(A, A + 0x100000, A + 0x200000, A + 0x1000000, None,
                                A + 0x2000000, A + 0x2800000, A + 0x3000000, A + 0x3800000, 128,
                                A + 0x300000, 4, 128, 256, 8, 2, A + 0x4000000, 1 << 30, None)
    assert rc == moe.MOE_FFN_ERR_NULL_ARG


@fake
@pytest.mark.parametrize("group", [0, 64, 256, -128])
def test_forward_int8_rejects_other_groups(group):
    L = moe.lib()
    rc = L.moe_ffn_forward_int8(A, A + 0x100000, A + 0x200000, A + 0x1000000, A + 0x1800000,
                                A + 0x2000000, A + 0x2800000, A + 0x3000000, A + 0x3800000,
                                group, A + 0x300000, 4, 128, 256, 8, 2, A + 0x4000000, 1 << 30,
                                None)
    assert rc == moe.MOE_FFN_ERR_BAD_SHAPE


@fake
def test_route_host_validation():
    L = moe.lib()
    assert L.moe_route_topk(A, 0, 8, 2, A + 0x1000, A + 0x2000, None) == moe.MOE_FFN_OK
    assert L.moe_route_topk(A, 4, 8, 9, A + 0x1000, A + 0x2000, None) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert L.moe_route_topk(A, 4, 2048, 2, A + 0x10000, A + 0x20000, None) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert L.moe_route_topk(None, 4, 8, 2, A + 0x1000, A + 0x2000, None) == moe.MOE_FFN_ERR_NULL_ARG
    assert L.moe_route_topk(A, 4, 8, 2, A + 0x1000, A + 0x1010, None) == moe.MOE_FFN_ERR_ALIAS
    assert L.moe_route_topk(A, 4, 8, 2, A + 0x1001, A + 0x2000, None) == moe.MOE_FFN_ERR_MISALIGNED


def test_launch_probe_rejects_bad_counts():
    # rejected before any device call; no address involved
    assert moe.lib().moe_ffn_launch_probe(-1, None) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert moe.lib().moe_ffn_launch_probe(1000001, None) == moe.MOE_FFN_ERR_BAD_SHAPE


@fake
def test_read_probe_host_validation():
    L = moe.lib()
    assert L.moe_ffn_read_probe(None, 1 << 20, A + 0x100000, None) == moe.MOE_FFN_ERR_NULL_ARG
    assert L.moe_ffn_read_probe(A, 1 << 20, None, None) == moe.MOE_FFN_ERR_NULL_ARG
    assert L.moe_ffn_read_probe(A, 0, A + 0x100000, None) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert L.moe_ffn_read_probe(A, 1000, A + 0x100000, None) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert L.moe_ffn_read_probe(A + 8, 1 << 20, A + 0x100000, None) == moe.MOE_FFN_ERR_MISALIGNED
    assert L.moe_ffn_read_probe(A, 1 << 20, A + 0x100002, None) == moe.MOE_FFN_ERR_MISALIGNED


def test_set_split_validation():
    L = moe.lib()
    for v in (0, 1, 2, 4):
        assert L.moe_ffn_set_split(v, v) == moe.MOE_FFN_OK
    for bad in (3, 8, -1):
        assert L.moe_ffn_set_split(bad, 0) == moe.MOE_FFN_ERR_BAD_SHAPE
        assert L.moe_ffn_set_split(0, bad) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert L.moe_ffn_set_split(0, 0) == moe.MOE_FFN_OK


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises((TypeError, moe.MoeFfnError)):
        moe.moe_ffn_forward(x, torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2),
                            torch.zeros(8, 96, 64, dtype=torch.bfloat16),
                            torch.zeros(8, 96, 64, dtype=torch.bfloat16),
                            torch.zeros(8, 64, 96, dtype=torch.bfloat16),
                            workspace=torch.zeros(16, dtype=torch.uint8))


def attn(**kw):
    a = dict(q=A, k=A + 0x1000000, v=A + 0x2000000, lens=A + 0x100000, out=A + 0x200000, B=2,
             h_q=8, h_kv=2, d=128, L=64, scale=0.125, ws=A + 0x4000000, wsb=1 << 30)
    a.update(kw)
    return moe.lib().moe_attn_decode(a["q"], a["k"], a["v"], a["lens"], a["out"], a["B"],
                                     a["h_q"], a["h_kv"], a["d"], a["L"], a["scale"], a["ws"],
                                     a["wsb"], None)


@fake
def test_attn_host_validation():
    assert attn(B=0) == moe.MOE_FFN_OK
    assert attn(d=96) == moe.MOE_FFN_ERR_BAD_SHAPE            # d in {64, 128, 256}
    assert attn(h_q=6, h_kv=4) == moe.MOE_FFN_ERR_BAD_SHAPE    # not a multiple
    assert attn(h_q=34, h_kv=2) == moe.MOE_FFN_ERR_BAD_SHAPE   # group of 17
    assert attn(L=-1) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert attn(q=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert attn(k=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert attn(ws=None) == moe.MOE_FFN_ERR_WORKSPACE
    assert attn(wsb=256) == moe.MOE_FFN_ERR_WORKSPACE
    assert attn(q=A + 8) == moe.MOE_FFN_ERR_MISALIGNED
    assert attn(lens=A + 0x100002) == moe.MOE_FFN_ERR_MISALIGNED
    assert attn(ws=A + 0x4000000 + 64) == moe.MOE_FFN_ERR_MISALIGNED
    assert attn(out=A + 0x200) == moe.MOE_FFN_ERR_ALIAS       # out overlaps q
    assert attn(out=A + 0x1000100) == moe.MOE_FFN_ERR_ALIAS   # out overlaps the keys
    assert attn(ws=A + 0x2000000) == moe.MOE_FFN_ERR_ALIAS    # workspace on the values


def test_attn_workspace_bytes():
    n = moe.moe_attn_decode_workspace_bytes(32, 32, 4, 128, 32768)
    assert n > 0 and n % 256 == 0
    assert moe.moe_attn_decode_workspace_bytes(0, 8, 2, 64, 16) == 256
    assert moe.moe_attn_decode_workspace_bytes(1, 8, 2, 100, 16) == 0
    assert moe.moe_attn_decode_workspace_bytes(1, 8, 3, 64, 16) == 0


def resplit(**kw):
    """moe_ffn_forward_resplit with fake addresses (T=4, H=128, I=256, E=8,
    k=2); keyword arguments replace single arguments by name."""
    args = dict(x=A, ids=A + 0x100000, w=A + 0x200000, Pg=A + 0x1000000, Sg=A + 0x1100000,
                Rg=A + 0x1200000, SRg=A + 0x1300000, Pu=A + 0x1400000, Su=A + 0x1500000,
                Ru=A + 0x1600000, SRu=A + 0x1700000, Pd=A + 0x1800000, Sd=A + 0x1900000,
                Qd=A + 0x1a00000, Sdh=A + 0x1b00000, crit=A + 0x1c00000, group=128,
                out=A + 0x300000, T=4, H=128, I=256, E=8, k=2, ws=A + 0x4000000,
                ws_bytes=1 << 30)
    args.update(kw)
    return moe.lib().moe_ffn_forward_resplit(*args.values(), None)


@fake
def test_forward_resplit_host_validation():
    assert resplit(group=64) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert resplit(H=96) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert resplit(I=160) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert resplit(crit=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert resplit(SRu=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert resplit(Qd=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert resplit(Rg=A + 0x1200008) == moe.MOE_FFN_ERR_MISALIGNED
    assert resplit(Sdh=A + 0x1b00002) == moe.MOE_FFN_ERR_MISALIGNED   # scales: 4 bytes
    assert resplit(ws_bytes=1024) == moe.MOE_FFN_ERR_WORKSPACE
    assert resplit(out=A + 0x40) == moe.MOE_FFN_ERR_ALIAS
    assert resplit(T=0) == moe.MOE_FFN_OK


@fake
def test_route_grouped_host_validation():
    L = moe.lib()

    def call(T=4, E=256, ng=8, tg=4, k=8, lg=A, bias=None, ids=A + 0x100000, w=A + 0x200000):
        return L.moe_route_grouped(lg, bias, T, E, ng, tg, k, 1.0, ids, w, None)

    assert call(E=250) == moe.MOE_FFN_ERR_BAD_SHAPE          # groups do not divide E
    assert call(ng=128, E=256) == moe.MOE_FFN_ERR_BAD_SHAPE   # more than 64 groups
    assert call(tg=9) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert call(tg=0) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert call(tg=1, k=33) == moe.MOE_FFN_ERR_BAD_SHAPE      # more than one group holds
    assert call(k=65, ng=1, tg=1) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert call(E=2048, ng=64) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert call(T=-1) == moe.MOE_FFN_ERR_BAD_SHAPE
    assert call(T=0) == moe.MOE_FFN_OK
    assert call(lg=None) == moe.MOE_FFN_ERR_NULL_ARG
    assert call(bias=A + 0x300002) == moe.MOE_FFN_ERR_MISALIGNED
    assert call(ids=A + 0x200010) == moe.MOE_FFN_ERR_ALIAS     # ids overlap w
    assert call(ids=A + 0x40) == moe.MOE_FFN_ERR_ALIAS         # ids overlap logits
    assert call(bias=A + 0x200000 - 512) == moe.MOE_FFN_ERR_ALIAS


def _z(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def _layer_inputs(T=4, H=128, I=256, E=8, k=2):
    """CPU tensors of a small layer (the binding checks shapes before it
    looks at devices, so none of these reach the library)."""
    return dict(x=_z(T, H), ids=_z(T, k, dtype=torch.int32), w=_z(T, k, dtype=torch.float32),
                T=T, H=H, I=I, E=E, k=k)


BAD_ROUTING = [
    ("ids_rows", lambda a: dict(ids=_z(a["T"] + 1, a["k"], dtype=torch.int32))),
    ("ids_1d", lambda a: dict(ids=_z(a["T"] * a["k"], dtype=torch.int32))),
    ("w_cols", lambda a: dict(w=_z(a["T"], a["k"] + 1, dtype=torch.float32))),
    ("w_rows", lambda a: dict(w=_z(a["T"] - 1, a["k"], dtype=torch.float32))),
    ("out", lambda a: dict(out=_z(a["T"], a["H"] + 32))),
    ("x_3d", lambda a: dict(x=_z(1, a["T"], a["H"]))),
]


@pytest.mark.parametrize("fmt", ["bf16", "int8", "int4", "resplit"])
@pytest.mark.parametrize("bad", [b[0] for b in BAD_ROUTING])
def test_binding_rejects_wrong_routing_and_out_shapes(fmt, bad):
    """topk_ids / topk_w must be [T, top_k] and out [T, H]: the kernels index
    them by those sizes, so the binding refuses anything else (ValueError)
    before any library call."""
    a = _layer_inputs()
    a.update(dict(BAD_ROUTING)[bad](a))
    E, I, H = a["E"], a["I"], a["H"]
    G = 128
    out = a.get("out")
    with pytest.raises(ValueError):
        if fmt == "bf16":
            moe.moe_ffn_forward(a["x"], a["ids"], a["w"], _z(E, I, H), _z(E, I, H), _z(E, H, I),
                                out=out)
        elif fmt == "int8":
            i8, f32 = torch.int8, torch.float32
            moe.moe_ffn_forward_int8(a["x"], a["ids"], a["w"], _z(E, I, H, dtype=i8),
                                     _z(E, I, H // G, dtype=f32), _z(E, I, H, dtype=i8),
                                     _z(E, I, H // G, dtype=f32), _z(E, H, I, dtype=i8),
                                     _z(E, H, I // G, dtype=f32), out=out)
        elif fmt == "int4":
            u8, f32 = torch.uint8, torch.float32
            moe.moe_ffn_forward_int4(a["x"], a["ids"], a["w"], _z(E, I, H // 2, dtype=u8),
                                     _z(E, I, H // G, dtype=f32), _z(E, I, H // 2, dtype=u8),
                                     _z(E, I, H // G, dtype=f32), _z(E, H, I // 2, dtype=u8),
                                     _z(E, H, I // G, dtype=f32), out=out)
        else:
            u8, f32 = torch.uint8, torch.float32
            p, sg = _z(E, I, H // 2, dtype=u8), _z(E, I, H // G, dtype=f32)
            moe.moe_ffn_forward_resplit(a["x"], a["ids"], a["w"], p, sg, p, sg, p, sg, p, sg,
                                        _z(E, H, I // 2, dtype=u8), _z(E, H, I // G, dtype=f32),
                                        _z(E, H, I, dtype=torch.int8),
                                        _z(E, H, I // G, dtype=f32), _z(E, dtype=u8), out=out)


@pytest.mark.parametrize("name", ["Q_up", "S_gate", "S_down"])
def test_binding_rejects_wrong_int8_tensor_shapes(name):
    """Every INT8 weight and scale tensor is checked against [E, N, K] and the
    row-major scale shape [E, N, K/128]; a group-major table is refused."""
    a = _layer_inputs()
    E, I, H, G = a["E"], a["I"], a["H"], 128
    i8, f32 = torch.int8, torch.float32
    t = dict(Q_gate=_z(E, I, H, dtype=i8), S_gate=_z(E, I, H // G, dtype=f32),
             Q_up=_z(E, I, H, dtype=i8), S_up=_z(E, I, H // G, dtype=f32),
             Q_down=_z(E, H, I, dtype=i8), S_down=_z(E, H, I // G, dtype=f32))
    t[name] = {"Q_up": _z(E, I + 16, H, dtype=i8), "S_gate": _z(E, H // G, I, dtype=f32),
               "S_down": _z(E, I // G, H, dtype=f32)}[name]
    with pytest.raises(ValueError):
        moe.moe_ffn_forward_int8(a["x"], a["ids"], a["w"], t["Q_gate"], t["S_gate"], t["Q_up"],
                                 t["S_up"], t["Q_down"], t["S_down"])


def test_binding_rejects_wrong_router_and_attention_outputs():
    with pytest.raises(ValueError):
        moe.moe_route_topk(_z(4, 8, dtype=torch.float32), 2,
                           topk_ids=_z(4, 3, dtype=torch.int32))
    with pytest.raises(ValueError):
        moe.moe_route_grouped(_z(4, 256, dtype=torch.float32), 8, 8, 4,
                              topk_w=_z(5, 8, dtype=torch.float32))
    with pytest.raises(ValueError):
        moe.moe_ffn_forward_logits(_z(4, 128), _z(4, 8, dtype=torch.float32), 2,
                                   _z(8, 256, 128), _z(8, 256, 128), _z(8, 128, 256),
                                   out=_z(4, 64))
    with pytest.raises(ValueError):
        moe.moe_attn_decode(_z(2, 8, 128), _z(2, 2, 64, 128), _z(2, 2, 64, 128),
                            _z(2, dtype=torch.int32), out=_z(2, 8, 64))
