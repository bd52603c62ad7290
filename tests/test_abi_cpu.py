"""The C-ABI library loads and exports every symbol include/rlq.h declares.

CPU only: nothing here launches a kernel or touches a device.  The calls made
are the host-only helpers and argument validation that fails before any HIP
call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from decode_attention_rlq_amd import rlq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlq_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rlq.LIB_PATH):
        from decode_attention_rlq_amd import build
        build.build()
    return rlq.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(rlq.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_defaults(lib):
    assert rlq.abi_version() == 1
    p = rlq.default_params()
    assert (p.tau, p.gain, p.level_inner, p.level_outer) == (
        np.float32(0.9816), 1.0, np.float32(0.4528), np.float32(1.510))


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert lib.rlq_status_string(s).startswith(b"RLQ_")
    assert lib.rlq_status_string(7) == b"unknown rlq status"


def test_coupled_gain_matches_oracle(lib):
    tau, a, b, _ = oracle.lloyd_max_gaussian()
    for t in (0.85, 0.91, tau, 1.1):
        g = rlq.coupled_gain(t, a, b)
        assert abs(g - oracle.coupled_gain(t, np.float32(a), np.float32(b))) < 1e-6
    assert np.isnan(rlq.coupled_gain(0.9, 0.0, 1.5))


def test_workspace_size(lib):
    n1 = rlq.decode_workspace_size(4, 16, 262144)
    n2 = rlq.decode_workspace_size(4, 32, 262144)
    assert n1 > 0 and n2 > 0 and n1 % 16 == 0 and n2 % 16 == 0
    assert rlq.decode_workspace_size(1, 16, 0) > 0
    with pytest.raises(ValueError):
        rlq.decode_workspace_size(1, 24, 100)
    with pytest.raises(ValueError):
        rlq.decode_workspace_size(0, 16, 100)
    with pytest.raises(ValueError):
        rlq.decode_workspace_size(1, 144, 100)
    # The 16-head kernel's grid holds at most 65535 (request, head group)
    # pairs; the many-head kernel (heads a multiple of 64) has no such bound.
    assert rlq.decode_workspace_size(65535, 16, 100) > 0
    assert rlq.decode_workspace_size(21845, 48, 100) > 0
    assert rlq.decode_workspace_size(100000, 64, 100) > 0
    for bad in ((65536, 16, 100), (21846, 48, 100)):
        with pytest.raises(ValueError):
            rlq.decode_workspace_size(*bad)


@pytest.mark.parametrize("batch,heads,ctx", [(32, 112, 59297), (1, 16, 1 << 20), (4, 16, 262144),
                                              (256, 16, 20000), (2, 16, 5000)])
def test_workspace_splits_cover_the_context(lib, batch, heads, ctx):
    """The workspace holds (splits + 1) partials of 16 x 512 fp32 + 32 floats
    per request and 16-head group, and a split covers at most 16,384 tokens:
    the split count implied by the size must cover the longest context."""
    per = (16 * 512 + 32) * 4
    parts, rem = divmod(rlq.decode_workspace_size(batch, heads, ctx), per)
    assert rem == 0
    splits = parts // (batch * (heads // 16)) - 1
    assert splits >= 1 and splits * 16384 >= ctx


@pytest.mark.parametrize("batch,heads,ctx", [(32, 128, 59297), (4, 64, 262144), (1, 128, 1 << 22),
                                              (200, 128, 1000), (3, 128, 0), (300, 64, 70000)])
def test_workspace_many_heads_holds_every_item(lib, batch, heads, ctx):
    """With a multiple of 64 heads the workspace holds, per work-item slot and
    16-head tile, a 16 x 512 fp32 partial + 32 floats, then two ints per
    request.  The slots cover one round of workgroups (256 per 64 heads),
    and at least ceil(tiles / 2046) items per request (an item spans at most
    2046 tiles of 32 tokens), in a multiple of 8."""
    per = (16 * 512 + 32) * 4
    size = rlq.decode_workspace_size(batch, heads, ctx)
    parts, rem = divmod(size - 8 * batch, per)
    assert rem == 0 and parts % (heads // 16) == 0
    slots = parts // (heads // 16)
    tiles = -(-ctx // 32)
    assert slots % 8 == 0
    assert slots >= 256 // (heads // 64)
    assert slots >= batch * max(1, -(-tiles // 2046))


def test_validation_rejects_before_any_launch(lib):
    p = rlq.default_params()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    good = rlq.CacheDesc(0x100000, 0x100000, 0x100000, 4, 64, None, None, 0, 0, 0)
    bad_page = rlq.CacheDesc(0x100000, 0x100000, 0x100000, 4, 32, None, None, 0, 0, 0)
    misaligned = rlq.CacheDesc(0x100004, 0x100000, 0x100000, 4, 64, None, None, 0, 0, 0)
    no_max_batch = rlq.CacheDesc(0x100000, 0x100000, 0x100000, 4, 64, 0x100000, None, 4, 0, 0)
    A = lib.rlq_quantize_append
    # neither latent form
    assert A(ctypes.byref(p), ctypes.byref(good), None, None, None, fake, fake, fake, fake, 1, 1, 8, None, None) == -1
    # both latent forms
    assert A(ctypes.byref(p), ctypes.byref(good), fake, fake, fake, fake, fake, fake, fake, 1, 1, 8, None, None) == -1
    # latent without rotation
    assert A(ctypes.byref(p), ctypes.byref(good), fake, None, None, fake, fake, fake, fake, 1, 1, 8, None, None) == -1
    for c in (bad_page, misaligned, no_max_batch):
        assert A(ctypes.byref(p), ctypes.byref(c), None, fake, None, fake, fake, fake, fake, 1, 1, 8, None, None) == -1
    assert A(ctypes.byref(p), ctypes.byref(good), None, fake, None, fake, fake, fake, fake, 1, 0, 8, None, None) == -1
    assert A(None, ctypes.byref(good), None, fake, None, fake, fake, fake, fake, 1, 1, 8, None, None) == -1
    for bad_tau in (-0.5, float("nan"), float("inf")):  # the code assignment needs tau >= 0
        q = rlq.default_params()
        q.tau = bad_tau
        assert A(ctypes.byref(q), ctypes.byref(good), None, fake, None, fake, fake, fake, fake, 1, 1, 8, None,
                 None) == -1
    D = lib.rlq_mla_decode
    args = lambda heads, mcl, ws: (ctypes.byref(p), ctypes.byref(good), fake, fake, 1, heads, 0.1,
                                   fake, 4, fake, mcl, fake, None, fake, ws, None)
    assert D(*args(8, 64, 1 << 30)) == -1       # heads not a multiple of 16
    assert D(*args(256, 64, 1 << 30)) == -1     # too many heads
    assert D(*args(16, 257, 1 << 30)) == -1     # context beyond the block table
    assert D(*args(16, 256, 16)) == -3          # workspace too small


def test_extend_workspace_and_validation(lib):
    """rlq_mla_extend: (query, head) rows per request padded to 64, partials
    per item slot and 16-row tile; validation fails before any launch."""
    per = (16 * 512 + 32) * 4
    for batch, heads, max_q, ctx in [(4, 16, 512, 33280), (2, 128, 7, 1000), (3, 16, 1, 64)]:
        size = rlq.extend_workspace_size(batch, heads, max_q, ctx)
        rows = -(-max_q * heads // 64) * 64
        parts, rem = divmod(size - 8 * batch, per)
        assert rem == 0 and parts % (rows // 16) == 0 and (parts // (rows // 16)) % 8 == 0
    for bad in [(1, 24, 4, 100), (0, 16, 4, 100), (1, 16, 0, 100), (1, 16, 101, 100), (1, 144, 4, 100),
                (1, 128, 40000, 40000)]:  # the last exceeds the launch grid (rows / 64 > 65535)
        with pytest.raises(ValueError):
            rlq.extend_workspace_size(*bad)
    p = rlq.default_params()
    fake = ctypes.c_void_p(0x100000)
    good = rlq.CacheDesc(0x100000, 0x100000, 0x100000, 4, 64, None, None, 0, 0, 0)
    E = lib.rlq_mla_extend
    args = lambda cuq, heads, mq, mcl, ws: (ctypes.byref(p), ctypes.byref(good), fake, fake, cuq, 1, heads, mq, 0.1,
                                            fake, 4, fake, mcl, fake, None, fake, ws, None)
    assert E(*args(None, 16, 4, 64, 1 << 30)) == -1   # no cu_seqlens_q
    assert E(*args(fake, 8, 4, 64, 1 << 30)) == -1    # heads not a multiple of 16
    assert E(*args(fake, 16, 0, 64, 1 << 30)) == -1   # no queries
    assert E(*args(fake, 16, 65, 64, 1 << 30)) == -1  # more queries than context
    assert E(*args(fake, 16, 4, 257, 1 << 30)) == -1  # context beyond the block table
    assert E(*args(fake, 16, 4, 64, 16)) == -3        # workspace too small
