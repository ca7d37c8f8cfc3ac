"""The C ABI on the host (no GPU): the library loads, exports every function
include/pa.h declares, and rejects invalid arguments before launching anything."""

import ctypes
import os
import re

import pytest

import paged_kv_attention_decode_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(pa.SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code, name in pa._STATUS.items():
        assert pa.status_string(code).startswith(name)
    assert "unknown" in pa.status_string(99)
    assert pa.version() == 10000


def test_workspace_size_layout(lib):
    # split: fp32 max_logits and exp_sums [rows][P], partial outputs [rows][P][d], each region 256-byte aligned
    S, q_len, n_h, n_kv, d, MB, ps = 8, 1, 32, 8, 128, 8192, 512
    P = -(-MB * 16 // ps)
    rows = S * q_len * n_h
    stats = -(-rows * P * 4 // 256) * 256
    assert pa.decode_workspace_size(S, q_len, n_h, n_kv, d, MB, ps) == 2 * stats + -(-rows * P * d * 4 // 256) * 256
    assert pa.decode_workspace_size(3, 5, 7, 7, 64, 3, 48) == 2 * 512 + -(-105 * 1 * 64 * 4 // 256) * 256
    assert pa.decode_workspace_size(S, q_len, n_h, n_kv, d, MB, 0) == 0
    assert pa.decode_workspace_size(S, q_len, n_h, n_kv, d, MB, 24) == 0  # not a multiple of the block size
    assert pa.decode_workspace_size(S, q_len, n_h, n_kv, d, MB, -2) == 0
    # balanced: counters int32[S * n_kv], then 2 * 1024 pieces of (n_h / n_kv) * q_len rows of d + 2 floats
    got = pa.decode_workspace_size(64, 1, 32, 8, 128, 256, pa.PA_BALANCED)
    assert got == 64 * 8 * 4 + -(-2 * 1024 * 4 * 130 * 4 // 256) * 256


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation first


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, q_len=1, S=2, n_h=4, n_kv=2, d=64,
             NB=16, bs=16, MB=3, ps=0, ws=None, wsb=0, dt=pa.PA_F32, stream=None)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"], a["q_len"], a["S"],
                         a["n_h"], a["n_kv"], a["d"], a["NB"], a["bs"], a["MB"], a["ps"], a["ws"], a["wsb"], a["dt"],
                         a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(bt=None), 1),
    (dict(n_h=5), 2),
    (dict(q_len=0), 2),
    (dict(q_len=9), 2),
    (dict(ps=24), 2),
    (dict(d=96), 3),
    (dict(bs=32), 3),
    (dict(dt=7), 3),
    (dict(n_h=18, n_kv=2), 3),          # 9 rows per KV head in fp32
    (dict(n_h=18, n_kv=2, q_len=8, dt=pa.PA_BF16), 3),  # 72 rows per KV head in bf16 (at most 64)
    (dict(n_h=130, n_kv=2, dt=pa.PA_BF16), 3),          # 65 rows per KV head in bf16
    (dict(ps=512, ws=None), 4),
    (dict(ps=512, ws=FAKE, wsb=16), 4),
    (dict(ps=-1, ws=None), 4),
    (dict(ps=-1, ws=FAKE, wsb=1024), 4),
    (dict(ps=-2), 2),
    (dict(q=ctypes.c_void_p(0x10008)), 2),  # not 16-byte aligned
])
def test_decode_rejects_invalid_arguments(lib, kw, status):
    assert _decode(lib, **kw) == status


def test_zero_sequences_is_a_no_op(lib):
    assert _decode(lib, S=0, q=None, out=None) == 0


def test_cache_write_rejects_invalid_arguments(lib):
    f = lib.pa_cache_write
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 16, 16, 2, 64, pa.PA_BF16, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 2, 64, pa.PA_BF16, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 16, 2, 80, pa.PA_BF16, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 16, 16, 2, 64, pa.PA_BF16, None) == 2
    assert f(None, None, None, None, None, 0, 16, 16, 2, 64, pa.PA_BF16, None) == 0  # nothing to write


def test_cache_write_fp8_rejects_invalid_arguments(lib):
    f = lib.pa_cache_write_fp8
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 16, 16, 2, 64, pa.PA_BF16, None) == 1  # no k_scale
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 2, 64, pa.PA_BF16, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 16, 2, 96, pa.PA_BF16, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 16, 16, 2, 64, pa.PA_BF16, None) == 2
    assert f(None, None, None, None, None, None, None, 0, 16, 16, 2, 64, pa.PA_BF16, None) == 0


def _decode_fp8(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, cl=FAKE, scale=0.1, q_len=1, S=2, n_h=4,
             n_kv=2, d=64, NB=16, bs=16, MB=3, ps=0, ws=None, wsb=0, dt=pa.PA_BF16, stream=None)
    a.update(kw)
    return lib.pa_decode_fp8(a["out"], a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["bt"], a["cl"], a["scale"],
                             a["q_len"], a["S"], a["n_h"], a["n_kv"], a["d"], a["NB"], a["bs"], a["MB"], a["ps"],
                             a["ws"], a["wsb"], a["dt"], a["stream"])


def test_decode_fp8_rejects_invalid_arguments(lib):
    assert _decode_fp8(lib, dt=pa.PA_F32) == 3          # q/out must be bf16
    assert _decode_fp8(lib, ks=None) == 1
    assert _decode_fp8(lib, vs=None) == 1
    assert _decode_fp8(lib, n_h=130, n_kv=2) == 3       # 65 rows per KV head
    assert _decode_fp8(lib, ps=-1, ws=None) == 4
    assert _decode_fp8(lib, S=0, q=None, out=None) == 0


def _decode_tree(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, par=FAKE, scale=0.1, T=15, S=2, n_h=4, n_kv=1,
             d=128, NB=16, bs=16, MB=3, ps=0, ws=None, wsb=0, dt=pa.PA_BF16, stream=None)
    a.update(kw)
    return lib.pa_decode_tree(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["par"], a["scale"], a["T"],
                              a["S"], a["n_h"], a["n_kv"], a["d"], a["NB"], a["bs"], a["MB"], a["ps"], a["ws"],
                              a["wsb"], a["dt"], a["stream"])


def test_decode_tree_rejects_invalid_arguments(lib):
    assert _decode_tree(lib, dt=pa.PA_F32) == 3          # bf16 only
    assert _decode_tree(lib, par=None) == 1              # the tree is required
    assert _decode_tree(lib, T=65, n_h=1) == 2           # at most 64 nodes
    assert _decode_tree(lib, T=0) == 2
    assert _decode_tree(lib, T=17, n_h=4) == 3           # 68 rows per KV head
    assert _decode_tree(lib, d=96) == 3
    assert _decode_tree(lib, ps=-1, ws=None) == 4
    assert _decode_tree(lib, S=0, q=None, out=None) == 0


def test_reduce_accepts_tree_sized_q_len_only_up_to_64(lib):
    f = lib.pa_reduce
    assert f(FAKE, FAKE, 8, FAKE, 2, 64, 4, 64, 3, 16, 32, pa.PA_BF16, None) == 4      # q_len 64 valid: workspace small
    assert f(FAKE, FAKE, 1 << 30, FAKE, 2, 65, 4, 64, 3, 16, 32, pa.PA_BF16, None) == 2


def _prefill(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, qs=FAKE, scale=0.1, S=2, T=600, mq=512, n_h=32,
             n_kv=8, d=128, NB=64, bs=16, MB=40, dt=pa.PA_BF16, stream=None)
    a.update(kw)
    return lib.pa_prefill(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["qs"], a["scale"], a["S"], a["T"],
                          a["mq"], a["n_h"], a["n_kv"], a["d"], a["NB"], a["bs"], a["MB"], a["dt"], a["stream"])


def test_prefill_rejects_invalid_arguments(lib):
    assert _prefill(lib, dt=pa.PA_F32) == 3            # bf16 only
    assert _prefill(lib, d=96) == 3
    assert _prefill(lib, bs=32) == 3
    assert _prefill(lib, n_h=30) == 2                  # not a multiple of the KV heads
    assert _prefill(lib, mq=(1 << 20) + 1) == 3
    # workgroups past 2^31 - 1: 2^20 tokens x 8 heads per KV head = 32768 chunks of 256 rows, x 8 x 8192
    assert _prefill(lib, mq=1 << 20, n_h=64, n_kv=8, S=8192, T=1 << 20) == 3
    assert _prefill(lib, mq=1 << 20, n_h=64, n_kv=8, S=8191, T=1 << 20, qs=None) == 1  # one fewer fits
    # query rows of one (sequence, KV head) past 2^31 - 1: 2^20 tokens x 2048 heads per KV head
    assert _prefill(lib, mq=1 << 20, n_h=2048, n_kv=1, S=1, T=1 << 20) == 3
    assert _prefill(lib, qs=None) == 1
    assert _prefill(lib, out=None) == 1
    assert _prefill(lib, S=0, q=None, out=None) == 0   # nothing to do
    assert _prefill(lib, T=0, q=None, out=None) == 0


def test_copy_blocks_rejects_invalid_arguments(lib):
    f = lib.pa_copy_blocks
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 16, 16, 8, None) == 2       # block bytes not a multiple of 16
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 0, 16, 4096, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, None, 3, 16, 16, 4096, None) == 1
    assert f(None, None, None, None, None, 0, 16, 16, 4096, None) == 0    # nothing to copy


def test_reduce_rejects_invalid_arguments(lib):
    f = lib.pa_reduce
    assert f(FAKE, FAKE, 1 << 30, FAKE, 2, 1, 4, 64, 3, 16, 0, pa.PA_F32, None) == 2     # partition_size 0
    assert f(FAKE, None, 0, FAKE, 2, 1, 4, 64, 3, 16, 32, pa.PA_F32, None) == 4
    assert f(FAKE, FAKE, 8, FAKE, 2, 1, 4, 64, 3, 16, 32, pa.PA_F32, None) == 4
    assert f(None, FAKE, 1 << 30, FAKE, 2, 1, 4, 64, 3, 16, 32, pa.PA_F32, None) == 1


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError, match="GPU"):
        pa.decode(q, torch.zeros(16, 16, 2, 64), torch.zeros(16, 16, 2, 64), torch.zeros(2, 3, dtype=torch.int32),
                  torch.ones(2, dtype=torch.int32), 0.125)


def _layout(lib, nb, bs, n_kv, d, eb):
    total, voff = ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = lib.pa_kv_cache_layout(nb, bs, n_kv, d, eb, ctypes.byref(total), ctypes.byref(voff))
    return st, total.value, voff.value


def test_kv_cache_layout_places_v_one_head_slice_off(lib):
    # the 8B layer's pools (20,000 blocks of 16 tokens x 8 heads x 128): bf16 and fp8 codes
    assert _layout(lib, 20000, 16, 8, 128, 2) == (0, 2 * 655360000 + 256, 655360000 + 256)
    assert _layout(lib, 20000, 16, 8, 128, 1) == (0, 2 * 327680000 + 128, 327680000 + 128)
    # a pool that is not a multiple of 2 KiB rounds up first; a 64-byte slice rounds up to 128
    assert _layout(lib, 1, 16, 1, 64, 1) == (0, 2048 + 128 + 1024, 2048 + 128)
    for nb in (1, 3, 1000):
        for n_kv in (1, 2, 8):
            for d in (64, 128):
                for eb in (1, 2, 4):
                    st, total, voff = _layout(lib, nb, 16, n_kv, d, eb)
                    pool = nb * 16 * n_kv * d * eb
                    slice_ = -(-d * eb // 128) * 128 % 2048
                    assert st == 0 and voff % 128 == 0 and voff >= pool and total == voff + pool
                    assert voff % 2048 == slice_, (nb, n_kv, d, eb)
    # with 2 KiB token rows (8 heads of 128 bf16) no head has K and V at the same offset within 1 KiB
    _, _, voff = _layout(lib, 20000, 16, 8, 128, 2)
    assert all((256 * g) % 1024 != (voff + 256 * g) % 1024 for g in range(8))


def test_kv_cache_layout_rejects_invalid_arguments(lib):
    total, voff = ctypes.c_int64(0), ctypes.c_int64(0)
    assert lib.pa_kv_cache_layout(16, 16, 8, 128, 2, None, ctypes.byref(voff)) == 1
    assert lib.pa_kv_cache_layout(16, 16, 8, 128, 2, ctypes.byref(total), None) == 1
    assert _layout(lib, 0, 16, 8, 128, 2)[0] == 2
    assert _layout(lib, 16, 16, 0, 128, 2)[0] == 2
    assert _layout(lib, 16, 16, 8, 128, 3)[0] == 2
    assert _layout(lib, 16, 32, 8, 128, 2)[0] == 3          # block_size other than 16
    assert _layout(lib, 1 << 50, 16, 8, 128, 2)[0] == 3     # past 2^62 bytes
